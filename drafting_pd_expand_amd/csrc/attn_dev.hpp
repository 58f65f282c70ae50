// Device side of the paged split-KV attention: configuration, LDS layouts,
// one split work item and one merge wave, shared by the attention kernels and
// the persistent decode kernel.
//
// Paged causal multi-query attention of the drafter, split over the KV
// sequence, on CDNA4 MFMA.
//
// [Blog] = "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding
// in vLLM" (summary page): every draft position of a request -- the copied
// verify window and the K-1 MASK slots -- attends in the same pass, through
// the request's KV pages ("P-EAGLE core method": all positions go through the
// layers together; "vLLM engineering details": slot mapping over a paged KV
// cache). [arXiv] = ScienceStack page of arXiv 2602.01469, Theorem 2.3: the
// score of rotated q and k depends on positions only through their
// difference, so the cache stores keys already rotated.
//
// Work split. A plan kernel (once per forward) picks one split length for
// the whole batch from the total context, so every workgroup streams about
// the same number of pages whatever the length mix, and lists the
// (request, split) units. Work unit = (unit, kv head). All query vectors of
// the request that share the kv head (GQA group x rows, e.g. 8 x 14 = 112)
// are packed into 16-wide MFMA tiles, two per wave.
//
// Per pair of 16-token pages (32 keys), per query tile:
//   S^T(16 x 16) = K_rows (16 x dh) * Q^T, twice (16x16x32 MFMA). The A
//     operand rows are picked so that lane group g (lanes 16g..16g+15) ends up
//     holding the scores of keys 8g..8g+7 of the pair in its 8 accumulators;
//   online softmax per query column in fp32, exp2 domain, with a lazy running
//     max: the column max is exchanged (two row-swap permutes) and the accumulators
//     rescaled only when a wave vote finds a score more than 2^8 above it;
//   O^T(dh x 16) += V^T (dh x 32 keys) * P^T: a lane's 8 probabilities
//     (rounded to bf16) are its B operand as they are, and its A operand is
//     one 16-byte read of the dim-major V page (keys 8g..8g+7 of one dim
//     row); one more MFMA with an all-ones A operand accumulates the column
//     sums of the same rounded weights, so no VALU adds or shuffles are
//     spent on the running sum.
// Pages are staged global -> LDS directly (global_load_lds, 16 B per lane) in
// a 4-deep ring of chunks shared by all waves; the LDS layouts are XOR
// swizzles of the page layout chosen so that every 8-lane group of a 16-byte
// fragment read touches 8 different bank groups. Pages past the split or
// with a bad block-table entry are read from a zero page and masked.
// Each split writes an unnormalized partial (O, running max, running sum);
// a merge kernel combines the splits in a fixed order (deterministic). A request
// with a single split writes its normalized bf16 output directly.
#pragma once

#include <math.h>

#include <algorithm>
#include <type_traits>

#include "attn_plan.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace pd {

namespace {

constexpr float kNegInf = -INFINITY;
// Running maxima are raised only when a new score exceeds them by more than
// this (log2 units); exp2 arguments then stay <= kRescale, the final O / l is
// unchanged, and the accumulator rescales are skipped on most pages.
constexpr float kRescale = 8.0f;
constexpr int kBtMax = kAttnBtMax;        // block-table entries of one split cached in LDS
constexpr int kMaxSplitKeys = kAttnMaxSplitKeys;
constexpr int kMaxSplits = 128;           // splits of one request the merge combines
// merge-kernel workgroups resident at once with one head per wave (four per
// CU, register-bound)
constexpr int kMergeRoundWgs = 1024;

// K and V of pages that are past the split end or invalid come from here
// (zero-initialised at load; nothing writes it).
__device__ __align__(16) uint16_t g_zero_page[PD_PAGE * 128];

// Per head size and cache type: waves per workgroup, query tiles per wave
// (one pass covers 128 queries), pages per LDS stage, stages in the ring,
// 1 KB loads per page (K then V^T) and per wave per stage. fp8 pages at dh 64
// (CONV): a stage holds as many pages as a bf16 one, in half the bytes; after
// it lands, one pass of the whole workgroup turns it into bf16 pages (each
// code once, not once per wave) in the layout the bf16 fragment reads use
// (C = 64 over ~4k-key contexts: 125-128 vs 134 us per launch on a bf16 cache).
// fp8 pages at dh 128: a stage holds twice the pages of a bf16 one (the same
// bytes) and every wave converts the fragments it reads (the conversion pass
// measured slower there: 149 vs 135 us on 16 x 20000 keys, its LDS round
// trip and second barrier per 2-page stage cost more than the conversions
// it saves). At dh 64 over a bf16 cache
// a 3-stage ring (~51 KB of LDS) lets three workgroups share a CU instead of
// two, with the same bytes in flight per CU: the kernel is bound by issue
// (MFMA, softmax, LDS reads) as much as by the KV stream, and the third
// workgroup's waves fill the gaps (64 requests x 4k keys: 144 -> 136 us).
template <int DH, bool F8 = false, int NS = 0>
struct AttnCfg {
    static constexpr int NW = 4;
    static constexpr int TPW = 2;
    static constexpr int EB = F8 ? 1 : 2;          // bytes per cached element
    static constexpr bool CONV = F8 && DH == 64;   // fp8 stage converted by a workgroup pass
    static constexpr int CH = (DH == 64 ? 4 : 2) * (F8 && !CONV ? 2 : 1);   // pages per stage
    static constexpr int NST = NS ? NS : ((DH == 64 && !F8) ? 3 : 4);
    static constexpr int PE = 16 * DH;             // elements of one page of K (or V)
    static constexpr int LPP = 2 * PE * EB / 1024; // 1 KB blocks per page: K half, V half
    static constexpr int L = CH * LPP / NW;        // loads per wave per stage
    static_assert(CH * LPP % NW == 0, "stage loads split evenly over the waves");
    static_assert(CH % 2 == 0, "pages are consumed in pairs");
};

// LDS swizzles (element offsets inside one staged page). A K row keeps its
// 16-byte chunks XOR-permuted by key_sw(key); the fragment reads of one
// 8-lane group are keys {0-3, 8-11} (or {4-7, 12-15}) at one chunk, which
// key_sw maps to 8 distinct chunk positions. At dh 128 a K row is a whole
// 256-byte bank line and the 16 lanes of a read are those 8 keys in both
// pages of a pair: the odd page's rows also flip chunk bit 3 (key_swp), so
// the 16 reads land on 16 distinct slots (without it, 30% of the LDS cycles
// of the 20000-key, 16-request batch were bank conflicts). A V^T row (one
// dim, 16 keys) keeps its two 16-byte halves swapped on rows 4-7 of every 8,
// so the reads of rows 0..7 at one half cover 8 distinct 16-byte positions.
__device__ __forceinline__ int key_sw(int key) { return (key & 3) | ((key >> 1) & 4); }
template <int DH>
__device__ __forceinline__ int key_swp(int key, int page) {
    return key_sw(key) | (DH == 128 ? (page & 1) << 3 : 0);
}
__device__ __forceinline__ int v_half(int row, int half) { return half ^ ((row >> 2) & 1); }

// fp8 pages with the conversion pass are staged as they are cached (K
// [16][dh], V^T [dh][16] codes, no permutation): only that pass reads them,
// 16 bytes per lane in order. fp8 pages read directly (dh 128): a K row (one
// key, 128 bytes) keeps its 16-byte chunks XOR-permuted by key_sw8; the 16
// lanes of one fragment read are keys {0-3, 8-11} of both pages of a pair at
// one chunk, and the permutation puts them on 16 distinct 16-byte slots of a
// 256-byte bank line. V^T rows are 16 bytes (16 keys) and are read 8 bytes at
// a time: no permutation needed.
__device__ __forceinline__ int key_sw8(int key, int page) {
    return ((key >> 1) & 1) | (((key >> 3) & 1) << 1) | ((page & 1) << 2);
}

// 8 E4M3 codes -> 8 bf16 (exact: every E4M3 value is a bf16 value)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// The ring's global -> LDS copies are ordered by hand: wait_vmcnt<N> (own
// copies), then barrier_lds (every wave's copies visible, every wave done
// with the slot about to be refilled). The LDS destination is passed to the
// copy as a plain 32-bit address, and the barrier as its own instruction, so
// that the compiler adds no wait of its own for copies still in flight into
// other ring slots (it cannot tell the slots apart and would wait for all).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// max over the four lanes l, l^16, l^32, l^48 (one query column of a 16x16
// MFMA tile): the gfx950 row-swap permutes exchange rows 0<->1, 2<->3 and
// halves 0<->1 without going through LDS
__device__ __forceinline__ float col_max(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// LDS address of a pointer into a __shared__ array, as a plain (wave-uniform)
// 32-bit offset
__device__ __forceinline__ unsigned lds_addr(void* p) {
    return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)p);
}

}  // namespace

// LDS of one split work item: the page ring, the split's block-table entries
// and the per-page valid flags.
template <int DH, bool F8, int NS>
struct AttnSmem {
    using Cf = AttnCfg<DH, F8, NS>;
    using ET = typename std::conditional<F8, uint8_t, uint16_t>::type;
    __align__(16) ET kv[Cf::NST][Cf::CH][2][Cf::PE];   // [stage][page][K, V^T]
    // CONV: the stage being consumed, converted to bf16 pages (bf16 layout)
    __align__(16) uint16_t cv[Cf::CONV ? Cf::CH : 1][2][Cf::CONV ? Cf::PE : 8];
    int btc[kBtMax + Cf::CH];
    int pv[Cf::NST][Cf::CH];
};

// One split work item (unit blk / Hkv of the plan, kv head blk % Hkv) on the
// calling workgroup. CG: the plan, q and the cached pages may have been written
// by other workgroups of the same launch, and the outputs are read by them
// (coherent accesses, see ldc / stc).
template <int DH, bool F8, bool CG, int NS>
__device__ __forceinline__ void attn_split_item(const AttnArgs& a, int blk, AttnSmem<DH, F8, NS>& sm) {
    using Cf = AttnCfg<DH, F8, NS>;
    using ET = typename std::conditional<F8, uint8_t, uint16_t>::type;   // cached element
    constexpr int KB = DH / 32;  // 16x16x32 steps over dh for the scores
    constexpr int OT = DH / 16;  // 16-dim output tiles
    constexpr int TPW = Cf::TPW, NW = Cf::NW, NT = 64 * NW, CH = Cf::CH, NST = Cf::NST;
    constexpr bool CONV = Cf::CONV;
    auto& kv = sm.kv;
    auto& btc = sm.btc;
    auto& pv = sm.pv;
    // The page copies need no coherent bit even inside the decode kernel: a
    // layer's pages are first read in this launch after the RoPE phase wrote
    // the new keys, so no XCD can hold a stale copy of them.

    const int g = blk % a.Hkv, u = blk / a.Hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;

    const int nunits = ldc<CG>(a.plan);
    const int4* recp = reinterpret_cast<const int4*>(a.plan + kPlanUnits + (size_t)u * kPlanRec);
    const int4 ra = ldc<CG>(recp), rb = ldc<CG>(recp + 1);   // in bounds for every u < max_units
    if (u >= nunits) return;
    const int r = ra.x, s = ra.y, ns = ra.z, row0 = ra.w;
    const int row1 = rb.x, kb = rb.y, ke = rb.z;
    const int npages = (ke - kb + PD_PAGE - 1) / PD_PAGE;   // 1 .. kBtMax
    const int nchunks = (npages + CH - 1) / CH;
    const int G = a.Hq / a.Hkv;
    const int nq = (row1 - row0) * G;
    // an fp8 cache holds K / k_scale and V / v_scale: the scores take k_scale
    // with the softmax scale, the outputs v_scale
    const float scale = a.scale_log2 * (F8 ? a.k_scale : 1.0f), inv_scale = 1.0f / scale;
    const float osc = F8 ? a.v_scale : 1.0f;

    bf16x8 qv[TPW][KB];
    int qrow[TPW], qh[TPW], lim[TPW];
    bool qok[TPW], qrej[TPW];
    auto load_q = [&](int qbase) {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int qi = qbase + (wave + NW * tt) * 16 + r16;
            qok[tt] = qi < nq;
            qrow[tt] = row0 + (qok[tt] ? qi / G : 0);
            qh[tt] = g * G + (qok[tt] ? qi % G : 0);
            // row0 <= qrow < row1 <= T: both loads are in bounds for every lane
            const bool rej = a.is_rejected && a.is_rejected[qrow[tt]] != 0;   // (null: none rejected)
            const int pos = a.positions[qrow[tt]];
            qrej[tt] = !qok[tt] || rej;
            // keys this query may see: t <= lim (rejected / padding queries: no limit, not used)
            lim[tt] = qrej[tt] ? 0x7fffffff : min(ke - 1, pos);
            const uint16_t* qp = a.q + ((size_t)qrow[tt] * a.Hq + qh[tt]) * DH;
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                // fp8 read directly: the dims of a score step are regrouped so that
                // one 16-byte read of a key row feeds two steps (the q side follows)
                const int dim = (F8 && !CONV) ? 64 * (kk >> 1) + 16 * g4 + 8 * (kk & 1) : 32 * kk + 8 * g4;
                qv[tt][kk] = qok[tt] ? ldc<CG>(reinterpret_cast<const bf16x8*>(qp + dim)) : zero_bf16x8();
            }
        }
    };
    load_q(0);
    // block-table entries of the split, padded with -1 to whole chunks
    const int32_t* bt = a.block_table + (size_t)r * a.max_blocks + kb / PD_PAGE;
    for (int i = tid; i < nchunks * CH; i += NT) btc[i] = i < npages ? bt[i] : -1;
    __syncthreads();

    // Load assignment: the wave's qd-th 1 KB load of a chunk is block
    // qd*NW + wave of the chunk's CH*LPP blocks, i.e. page qd*NW/LPP (known at
    // compile time) and part (qd*NW) % LPP + wave of that page (wave-uniform).
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint16_t* zp = g_zero_page;
    int loff[Cf::L];   // per-lane source offset (elements) inside the page
    // the wave's qd-th block of a stage: page and part (wave-uniform)
    auto blk_page = [&](int qd) {
        if constexpr (Cf::LPP % NW == 0) return qd * NW / Cf::LPP;
        else return (qd * NW + wv) / Cf::LPP;
    };
    auto blk_part = [&](int qd) {
        if constexpr (Cf::LPP % NW == 0) return (qd * NW) % Cf::LPP + wv;
        else return (qd * NW + wv) % Cf::LPP;
    };
#pragma unroll
    for (int qd = 0; qd < Cf::L; ++qd) {
        const int part = blk_part(qd);
        if constexpr (!F8) {
            if (part < Cf::LPP / 2) {               // K: 512 / DH keys per 1 KB block
                const int key = (512 / DH) * part + lane / (DH / 8);
                loff[qd] = key * DH + (((lane % (DH / 8)) ^ key_swp<DH>(key, blk_page(qd))) << 3);
            } else {                                // V^T: 32 dim rows of 16 keys per 1 KB block
                const int row = 32 * (part - Cf::LPP / 2) + lane / 2;
                loff[qd] = row * PD_PAGE + (v_half(row, lane & 1) << 3);
            }
        } else if constexpr (CONV) {   // the block's 1 KB in order (K part, then V^T part)
            loff[qd] = (part % (Cf::LPP / 2)) * 1024 + lane * 16;
        } else {
            if (part < Cf::LPP / 2) {               // K: 1024 / DH keys per 1 KB block
                const int key = (1024 / DH) * part + lane / (DH / 16);
                loff[qd] = key * DH + (((lane % (DH / 16)) ^ key_sw8(key, blk_page(qd))) << 4);
            } else {                                // V^T: 64 dim rows of 16 keys per 1 KB block
                loff[qd] = (64 * (part - Cf::LPP / 2) + lane) * PD_PAGE;
            }
        }
    }
    // global -> LDS for chunk c into ring slot `slot`: every wave issues exactly
    // Cf::L 1 KB loads (pages past the split or with a bad block-table entry
    // read the zero page and are marked invalid), so vmcnt counts agree
    auto issue = [&](int c, int slot) {
#pragma unroll
        for (int qd = 0; qd < Cf::L; ++qd) {
            const int p = blk_page(qd);
            const int part = blk_part(qd);
            const int blk = __builtin_amdgcn_readfirstlane(btc[c * CH + p]);
            const bool ok = (unsigned)blk < (unsigned)a.num_blocks;
            const bool isk = part < Cf::LPP / 2;
            const ET* base = ok ? static_cast<const ET*>(isk ? a.kplane : a.vplane) + ((size_t)blk * a.Hkv + g) * Cf::PE
                                : reinterpret_cast<const ET*>(zp);
            ET* dst = &kv[slot][p][isk ? 0 : 1][(isk ? part : part - Cf::LPP / 2) * (1024 / Cf::EB)];
            // each cached page is read once per layer; non-temporal copies
            // (cache policy 2) measured faster for bf16 pages of dh 128 (16 x
            // 20000-key batch: 142 -> 134 us) and slower for dh 64 and fp8 pages
            __builtin_amdgcn_global_load_lds((void*)(base + loff[qd]),
                                             (__attribute__((address_space(3))) void*)(uintptr_t)lds_addr(dst),
                                             16, 0, (DH == 128 && !F8) ? 2 : 0);
        }
        if (tid < CH) {
            const int pg = c * CH + tid;
            const int blk = btc[pg];
            const int ok = (unsigned)blk < (unsigned)a.num_blocks;
            if (pg < npages && !ok) flag(a.status, PD_STATUS_BAD_PAGE);
            pv[slot][tid] = ok;
        }
    };

    // fragment read offsets (elements) inside a staged page pair
    const int kpage = r16 >> 3;                              // A-operand row -> page of the pair
    const int key0 = (r16 & 3) | ((r16 & 4) << 1);           // keys 0-3, 8-11 (+4 for the second MFMA)
    const int ksw = key_swp<DH>(key0, kpage);                // the same for key0 + 4
    const int vpage = g4 >> 1;                               // lane group -> page of its 8 keys
    const int voff = r16 * PD_PAGE + (v_half(r16, g4 & 1) << 3);
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

    // CONV: ring slot b's pages -> bf16 pages in sm.cv, in the bf16 layout
    // (K rows permuted by key_swp, V^T halves by v_half). Thread t converts
    // one 16-code K chunk (key, chunk) and one V^T row (16 keys) of page
    // t / DH: 16 keys x DH / 16 chunks = DH rows = DH threads per page.
    auto convert = [&](int b) {
        if constexpr (CONV) {
            static_assert(NT == CH * DH, "one K chunk and one V^T row per thread");
            const int p = tid / DH, idx = tid % DH;
            const int key = idx / (DH / 16), c16 = idx % (DH / 16);
            const uint4 kw = *reinterpret_cast<const uint4*>(&kv[b][p][0][key * DH + 16 * c16]);
            const uint4 vw = *reinterpret_cast<const uint4*>(&kv[b][p][1][idx * PD_PAGE]);
            const int ks = key_swp<DH>(key, p);
            uint16_t* kd = &sm.cv[p][0][key * DH];
            uint16_t* vd = &sm.cv[p][1][idx * PD_PAGE];
            *reinterpret_cast<bf16x8*>(kd + (((2 * c16) ^ ks) << 3)) = fp8x8_to_bf16(kw.x, kw.y);
            *reinterpret_cast<bf16x8*>(kd + (((2 * c16 + 1) ^ ks) << 3)) = fp8x8_to_bf16(kw.z, kw.w);
            *reinterpret_cast<bf16x8*>(vd + (v_half(idx, 0) << 3)) = fp8x8_to_bf16(vw.x, vw.y);
            *reinterpret_cast<bf16x8*>(vd + (v_half(idx, 1) << 3)) = fp8x8_to_bf16(vw.z, vw.w);
        }
    };

    for (int qbase = 0; qbase < nq; qbase += NW * TPW * 16) {
        if (qbase > 0) load_q(qbase);
        const bool wave_has = qbase + wave * 16 < nq;   // wave-uniform
        f32x4 o[TPW][OT], lacc[TPW];
        float mrun[TPW], mb[TPW], thr[TPW];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
            for (int j = 0; j < OT; ++j) o[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            mrun[tt] = kNegInf;
            mb[tt] = 0.f;
            thr[tt] = kNegInf;
            lacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        wait_vmcnt<0>();   // query fragments in registers before the ring starts counting

        for (int st = 0; st < NST - 1 && st < nchunks; ++st) issue(st, st);
        for (int c = 0; c < nchunks; ++c) {
            // loads of chunk c done (later chunks may stay in flight), then all waves' loads
            const int later = min(NST - 2, nchunks - 1 - c);
            if (later >= 2) wait_vmcnt<2 * Cf::L>();
            else if (later == 1) wait_vmcnt<Cf::L>();
            else wait_vmcnt<0>();
            barrier_lds();
            if (c + NST - 1 < nchunks) issue(c + NST - 1, (c + NST - 1) % NST);
            const int b = c % NST;
            if constexpr (CONV) {
                // every wave converts its share (the chunk's slot landed; the
                // previous chunk's converted pages are no longer read), then all
                convert(b);
                barrier_lds();
            }
            if (!wave_has) continue;
#pragma unroll
            for (int pi = 0; pi < CH; pi += 2) {
                const int p0 = kb + (c * CH + pi) * PD_PAGE;
                if (p0 >= ke) break;
                const bool pgok = pv[b][pi + vpage] != 0;   // this lane group's page
                bf16x8 k0[KB], k1[KB], vf[OT];
                if constexpr (!F8 || CONV) {
                    // bf16 pages: the ring slot's, or (CONV) their conversion
                    const uint16_t* Kp;
                    const uint16_t* Vp;
                    if constexpr (CONV) {
                        Kp = sm.cv[pi + kpage][0];
                        Vp = sm.cv[pi + vpage][1];
                    } else {
                        Kp = reinterpret_cast<const uint16_t*>(kv[b][pi + kpage][0]);
                        Vp = reinterpret_cast<const uint16_t*>(kv[b][pi + vpage][1]);
                    }
#pragma unroll
                    for (int kk = 0; kk < KB; ++kk) {
                        const int ch = ((4 * kk + g4) ^ ksw) << 3;
                        k0[kk] = *reinterpret_cast<const bf16x8*>(Kp + key0 * DH + ch);
                        k1[kk] = *reinterpret_cast<const bf16x8*>(Kp + (key0 + 4) * DH + ch);
                    }
#pragma unroll
                    for (int j = 0; j < OT; ++j)
                        vf[j] = *reinterpret_cast<const bf16x8*>(Vp + 16 * PD_PAGE * j + voff);
                } else {
                    const uint8_t* Kp = reinterpret_cast<const uint8_t*>(kv[b][pi + kpage][0]);
                    const uint8_t* Vp = reinterpret_cast<const uint8_t*>(kv[b][pi + vpage][1]);
                    // K: one 16-byte read per key row feeds score steps 2m and 2m + 1
                    const int sw = key_sw8(key0, kpage);   // the same for key0 + 4
#pragma unroll
                    for (int m2 = 0; m2 < KB / 2; ++m2) {
                        const int ch = ((4 * m2 + g4) ^ sw) << 4;
                        const uint4 a0 = *reinterpret_cast<const uint4*>(Kp + key0 * DH + ch);
                        const uint4 a1 = *reinterpret_cast<const uint4*>(Kp + (key0 + 4) * DH + ch);
                        k0[2 * m2] = fp8x8_to_bf16(a0.x, a0.y);
                        k0[2 * m2 + 1] = fp8x8_to_bf16(a0.z, a0.w);
                        k1[2 * m2] = fp8x8_to_bf16(a1.x, a1.y);
                        k1[2 * m2 + 1] = fp8x8_to_bf16(a1.z, a1.w);
                    }
                    // V^T: keys 8 (g4 & 1) .. + 7 of one dim row
#pragma unroll
                    for (int j = 0; j < OT; ++j) {
                        const uint2 w = *reinterpret_cast<const uint2*>(Vp + (16 * j + r16) * PD_PAGE + 8 * (g4 & 1));
                        vf[j] = fp8x8_to_bf16(w.x, w.y);
                    }
                }
                const int t0 = p0 + 8 * g4;   // keys t0 .. t0+7 in this lane's scores (and V fragments)
                if (p0 + 2 * PD_PAGE > ke) {
                    // the pair reaches past the split's last key: the slots from ke on
                    // are not part of the context and may hold anything (NaN / Inf
                    // codes included), and a masked key's zero weight would not
                    // cancel them in the PV product, so their V elements are zeroed
                    const int nin = ke - t0;   // keys t0 .. t0+nin-1 are inside
#pragma unroll
                    for (int j = 0; j < OT; ++j)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (e >= nin) vf[j][e] = (__bf16)0.0f;
                }
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KB; ++kk) {
                        s0 = mfma_16x16x32(k0[kk], qv[tt][kk], s0);
                        s1 = mfma_16x16x32(k1[kk], qv[tt][kk], s1);
                    }
                    float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
                    const int vis = lim[tt] - t0;   // key t0+e is visible iff e <= vis
                    if (__any(!pgok || vis < 7)) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) sc[e] = (pgok && e <= vis) ? sc[e] : kNegInf;
                    }
                    const float lm = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
                    if (__any(lm > thr[tt])) {
                        // the column max (4 lane groups), raised only by more than kRescale
                        const float mnew = col_max(lm) * scale;   // -inf stays -inf
                        const bool raise = mnew > mrun[tt] + kRescale;
                        const float alpha = raise ? __builtin_amdgcn_exp2f(mrun[tt] - mnew) : 1.0f;
                        if (raise) {
                            mrun[tt] = mnew;
                            mb[tt] = -mnew;
                            thr[tt] = (mnew + kRescale) * inv_scale;
                        }
                        lacc[tt] = lacc[tt] * alpha;
#pragma unroll
                        for (int j = 0; j < OT; ++j) o[tt][j] = o[tt][j] * alpha;
                    }
                    bf16x8 pb;
#pragma unroll
                    for (int e = 0; e < 8; ++e)   // raw v_exp_f32: weights below 2^-126 flush to zero
                        pb[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[e], scale, mb[tt]));
#pragma unroll
                    for (int j = 0; j < OT; ++j) o[tt][j] = mfma_16x16x32(vf[j], pb, o[tt][j]);
                    // running sums of the same rounded weights: an all-ones A operand makes
                    // every row of the product the column sum over the pair's 32 keys
                    lacc[tt] = mfma_16x16x32(ones, pb, lacc[tt]);
                }
            }
        }
        __syncthreads();   // ring slots are free again before a next query pass reuses them

#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const float l = lacc[tt][0];
            if (!qok[tt]) continue;
            if (ns == 1) {
                // the only split: normalized bf16 output (rejected rows: zeros)
                const float inv = (!qrej[tt] && l > 0.f) ? osc / l : 0.f;
                uint16_t* op = a.out + ((size_t)qrow[tt] * a.Hq + qh[tt]) * DH + 4 * g4;
#pragma unroll
                for (int j = 0; j < OT; ++j) {
                    const uint32_t lo = f2bf(o[tt][j][0] * inv) | (uint32_t(f2bf(o[tt][j][1] * inv)) << 16);
                    const uint32_t hi = f2bf(o[tt][j][2] * inv) | (uint32_t(f2bf(o[tt][j][3] * inv)) << 16);
                    stc<CG>(reinterpret_cast<uint2*>(op + 16 * j), make_uint2(lo, hi));
                }
            } else {
                const size_t base = ((size_t)s * a.T + qrow[tt]) * a.Hq + qh[tt];
#pragma unroll
                for (int j = 0; j < OT; ++j)
                    stc<CG>(reinterpret_cast<f32x4*>(a.part_o + base * DH + 16 * j + 4 * g4), o[tt][j] * osc);
                if (g4 == 0) stc<CG>(reinterpret_cast<float2*>(a.part_ml + base * 2), make_float2(mrun[tt], l));
            }
        }
    }
}

// out[row][h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s. One wave per
// HPW q heads of one row: the row's request and split count are found once;
// then the (m, l) pairs and the first chunk of partial outputs of all HPW
// heads are loaded together (one round trip), the partial outputs as float4s,
// DH/4 lanes per split and 64/(DH/4) splits per load instruction. The split
// weights are formed across lanes (lane s holds split s); each lane sums its
// splits in order and the lane groups are then added in a fixed tree
// (deterministic). Requests with one split were written by the split kernel.

// Merge of the HPW (row, head) pairs starting at pair0 on the calling wave.
template <int DH, int HPW, bool CG>
__device__ __forceinline__ void attn_merge_wave(const AttnArgs& a, int pair0) {
    constexpr int LPS = DH / 4;        // lanes per split
    constexpr int SPI = 64 / LPS;      // splits per load instruction
    constexpr int CHUNK = 16 / HPW;    // load instructions in flight per head
    const int lane = threadIdx.x & 63;
    if (pair0 >= a.T * a.Hq) return;
    const int row = pair0 / a.Hq, h0 = pair0 % a.Hq;
    // request of the row = the last r with cu_out[r] <= row, found by the
    // whole wave: lane l tests start l * step, then the 64 starts after the
    // last hit (two dependent loads for up to 4096 requests, not log2 C)
    int r = 0;
    bool found = true;
    {
        const int step = (a.C + 63) / 64;
        const int i1 = lane * step;
        const uint64_t m1 = __ballot(i1 < a.C && a.cu_out[i1] <= row);
        if (m1 == 0) {
            found = false;
        } else {
            const int b = (63 - __clzll((long long)m1)) * step;
            const int i2 = b + lane;
            const uint64_t m2 = __ballot(lane < step && i2 < a.C && a.cu_out[i2] <= row);
            r = b + (63 - __clzll((long long)m2));   // m2 holds lane 0: cu_out[b] <= row
        }
    }
    const bool inr = found && row < a.cu_out[r + 1];
    const int nsr = ldc<CG>(a.plan + kPlanNs + r);
    if (inr && nsr == 1) return;
    const int ns = (inr && !(a.is_rejected && a.is_rejected[row])) ? min(nsr, kMaxSplits) : 0;
    const size_t stride = (size_t)a.T * a.Hq;   // between splits, in (row, head) units
    const size_t base0 = (size_t)row * a.Hq + h0;
    const int sub = lane / LPS, dq = lane % LPS;   // split within an instruction, dim quad
    float2 ml0[HPW], ml1[HPW];
    float4 v[HPW][CHUNK];
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
        const size_t base = base0 + j;
        ml0[j] = lane < ns ? ldc<CG>(reinterpret_cast<const float2*>(a.part_ml + (lane * stride + base) * 2))
                           : make_float2(kNegInf, 0.f);
        ml1[j] = lane + 64 < ns ? ldc<CG>(reinterpret_cast<const float2*>(a.part_ml + ((lane + 64) * stride + base) * 2))
                                : make_float2(kNegInf, 0.f);
#pragma unroll
        for (int k = 0; k < CHUNK; ++k) {
            const int sp = k * SPI + sub;
            v[j][k] = sp < ns ? ldc<CG>(reinterpret_cast<const float4*>(a.part_o + (sp * stride + base) * DH + 4 * dq))
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    const int ninst = (ns + SPI - 1) / SPI;
    float w0[HPW], w1[HPW], L[HPW];
    float4 acc[HPW];
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
        const float M = wave_max(fmaxf(ml0[j].x, ml1[j].x));
        w0[j] = 0.f;
        w1[j] = 0.f;
        L[j] = 0.f;
        if (M != kNegInf) {
            w0[j] = __builtin_amdgcn_exp2f(ml0[j].x - M);   // -inf -> 0 for missing splits
            w1[j] = __builtin_amdgcn_exp2f(ml1[j].x - M);
            L[j] = w0[j] * ml0[j].y + w1[j] * ml1[j].y;
        }
        L[j] = wave_sum(L[j]);
        acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int i0 = 0; i0 < ninst; i0 += CHUNK) {
        if (i0 > 0) {   // more splits than a chunk holds: the next chunk of every head at once
#pragma unroll
            for (int j = 0; j < HPW; ++j)
#pragma unroll
                for (int k = 0; k < CHUNK; ++k) {
                    const int sp = (i0 + k) * SPI + sub;
                    v[j][k] = sp < ns ? ldc<CG>(reinterpret_cast<const float4*>(a.part_o + (sp * stride + base0 + j) * DH +
                                                                                4 * dq))
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
                }
        }
#pragma unroll
        for (int j = 0; j < HPW; ++j)
#pragma unroll
            for (int k = 0; k < CHUNK; ++k) {
                const int s0 = (i0 + k) * SPI;   // first split of this instruction (uniform; 64 | s0 + SPI)
                const int sp = s0 + sub;
                const float w = __shfl(s0 < 64 ? w0[j] : w1[j], sp & 63, kWave);
                if (sp < ns) {
                    acc[j].x += w * v[j][k].x;
                    acc[j].y += w * v[j][k].y;
                    acc[j].z += w * v[j][k].z;
                    acc[j].w += w * v[j][k].w;
                }
            }
    }
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
#pragma unroll
        for (int off = LPS; off < 64; off <<= 1) {
            acc[j].x += __shfl_xor(acc[j].x, off, kWave);
            acc[j].y += __shfl_xor(acc[j].y, off, kWave);
            acc[j].z += __shfl_xor(acc[j].z, off, kWave);
            acc[j].w += __shfl_xor(acc[j].w, off, kWave);
        }
        if (sub == 0) {
            const float inv = L[j] > 0.f ? 1.0f / L[j] : 0.f;
            uint2 pk;
            pk.x = uint32_t(f2bf(acc[j].x * inv)) | (uint32_t(f2bf(acc[j].y * inv)) << 16);
            pk.y = uint32_t(f2bf(acc[j].z * inv)) | (uint32_t(f2bf(acc[j].w * inv)) << 16);
            stc<CG>(reinterpret_cast<uint2*>(a.out + (base0 + j) * DH + 4 * dq), pk);
        }
    }
}

}  // namespace pd
