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
// Work unit = (request, kv head, KV split). All query vectors of the request
// that share the kv head (GQA group x rows, e.g. 8 x 13 = 104) are packed
// into 16-wide MFMA tiles (two per wave at dh 64, one at dh 128). For each
// pair of 16-token pages:
//   S^T(16 keys x 16 queries) = K_page (16 x dh) * Q^T  -- 16x16x32 MFMA,
//       the K page is token-major so a lane's 16-byte load is one key's
//       8 consecutive dims;
//   online softmax per query column (fp32, exp2 domain; the four lane groups
//       of a column are combined with two xor shuffles);
//   O^T(dh x 16 queries) += V^T (dh x 32 keys) * P^T -- one 16x16x32 MFMA
//       per pair of pages: a lane's S^T accumulators (keys 4*g4..+3 of each
//       page) are its B operand once the MFMA's k slots are mapped to
//       (page A keys 4*g4..+3, page B keys 4*g4..+3); the V page is
//       dim-major so the matching A operand is two 8-byte reads;
//   softmax bookkeeping per 32 keys: one max and one sum exchange, scores
//       scaled inside a single FMA, masking and accumulator rescaling only
//       when a wave vote says some lane needs them.
// The workgroup stages each chunk of pages into LDS once (all waves share it;
// the next chunk's global loads are in flight while the current one is
// used). Nothing is transposed: the LDS layout is the page layout, with K rows
// padded by 16 bytes and V^T rows to 48 bytes so the fragment reads hit
// distinct banks. Each split writes an
// unnormalized partial (O, running max, running sum) per query; a merge
// kernel combines the splits in order (deterministic) and writes bf16 output.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pd {

namespace {

constexpr float kNegInf = -INFINITY;
// Running maxima are raised only when a new score exceeds them by more than
// this (log2 units); exp2 arguments then stay <= kRescale, the final O / l is
// unchanged, and the accumulator rescales are skipped on most pages.
constexpr float kRescale = 8.0f;
constexpr int kBtMax = 512;   // block-table entries of one split cached in LDS

// Per head size: waves per workgroup, query tiles per wave (one workgroup
// holds 128 queries), pages per LDS stage, stages in the ring, 1 KB loads per
// page (K then V^T) and per wave per stage.
template <int DH>
struct AttnCfg {
    static constexpr int NW = DH == 64 ? 4 : 8;
    static constexpr int TPW = DH == 64 ? 2 : 1;
    static constexpr int CH = DH == 64 ? 4 : 2;
    static constexpr int NST = 4;
    static constexpr int LPP = DH / 16;            // 1 KB blocks per page: K DH/32, V DH/32
    static constexpr int L = CH * LPP / NW;        // loads per wave per stage
    static constexpr int PE = 16 * DH;             // elements of one page of K (or V)
    static_assert(CH * LPP % NW == 0, "stage loads split evenly over the waves");
};

__device__ __forceinline__ int num_splits(int seq, int nsmax, int min_split) {
    const int ns = (seq + min_split - 1) / min_split;
    return ns < nsmax ? ns : nsmax;
}

__device__ __forceinline__ int split_len(int seq, int ns) {
    const int l = (seq + ns - 1) / ns;
    return (l + PD_PAGE - 1) & ~(PD_PAGE - 1);
}

// LDS swizzles (element offsets inside one page of the stage): a K row of key
// `key` keeps its 16-byte chunks XOR-permuted, a V^T row (one dim, 16 keys)
// keeps its two 16-byte halves swapped on every other group of 8 rows, so the
// MFMA fragment reads of 16 lanes hit 16 different bank groups.
template <int DH>
__device__ __forceinline__ int k_lds(int key, int chunk) {
    const int sw = DH == 64 ? ((key & 7) ^ (key >> 3)) : key;
    return key * DH + ((chunk ^ sw) << 3);
}
__device__ __forceinline__ int v_lds(int row, int unit /* 4-key unit 0..3 */) {
    const int half = (unit >> 1) ^ ((row >> 3) & 1);
    return row * PD_PAGE + (half << 3) + ((unit & 1) << 2);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int DH>
__global__ __launch_bounds__(64 * AttnCfg<DH>::NW) void attn_split_kernel(AttnArgs a) {
    using Cf = AttnCfg<DH>;
    constexpr int KB = DH / 32;  // 16x16x32 steps over dh for the scores
    constexpr int OT = DH / 16;  // 16-dim output tiles
    constexpr int TPW = Cf::TPW, NW = Cf::NW, NT = 64 * NW, CH = Cf::CH, NST = Cf::NST;
    __shared__ __align__(16) uint16_t kv[NST][CH][2][Cf::PE];   // [stage][page][K, V^T]
    __shared__ int btc[kBtMax];
    __shared__ int pv[NST][CH];

    const int r = blockIdx.z, g = blockIdx.y, s = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;

    const int row0 = a.cu_out[r], row1 = a.cu_out[r + 1];
    const int seq = a.seq_lens[r];
    if (row0 < 0 || row1 > a.T || row1 < row0 || seq < 1 || seq > a.max_blocks * PD_PAGE) {
        if (s == 0 && g == 0 && tid == 0) flag(a.status, PD_STATUS_BAD_ROW);
        return;
    }
    const int ns = num_splits(seq, a.nsmax, a.min_split);
    if (s >= ns) return;
    const int sl = split_len(seq, ns);
    const int kb = s * sl;
    const int ke = min(seq, kb + sl);
    int npages = ke > kb ? (ke - kb + PD_PAGE - 1) / PD_PAGE : 0;
    if (npages > kBtMax) {  // the host sizes splits below this; never read past the cache
        if (tid == 0) flag(a.status, PD_STATUS_BAD_ROW);
        npages = 0;
    }
    const int nchunks = (npages + CH - 1) / CH;
    const int G = a.Hq / a.Hkv;
    const int nq = (row1 - row0) * G;
    const int32_t* bt = a.block_table + (size_t)r * a.max_blocks + kb / PD_PAGE;
    for (int i = tid; i < npages; i += NT) btc[i] = bt[i];
    __syncthreads();

    // global -> LDS for chunk c into ring slot `slot`: every wave issues exactly
    // Cf::L 1 KB loads (pages past the split or with a bad block-table entry
    // read page 0 of the pool and are marked invalid), so vmcnt counts agree
    auto issue = [&](int c, int slot) {
#pragma unroll
        for (int q = 0; q < Cf::L; ++q) {
            const int inst = wave + NW * q;
            const int p = inst / Cf::LPP, part = inst % Cf::LPP;
            const int pg = c * CH + p;
            const int blk = pg < npages ? btc[pg] : -1;
            const bool ok = blk >= 0 && blk < a.num_blocks;
            const size_t pbase = ((size_t)(ok ? blk : 0) * a.Hkv + g) * Cf::PE;
            const uint16_t* src;
            uint16_t* dst;
            if (part < Cf::LPP / 2) {           // K: rows of 64 / DH*2/16 keys per 1 KB block
                constexpr int KPB = 512 / DH;   // keys per block
                const int key = KPB * part + lane / (DH / 8);
                const int chunk = lane % (DH / 8);
                const int sw = DH == 64 ? ((key & 7) ^ (key >> 3)) : key;
                src = a.kplane + pbase + key * DH + ((chunk ^ sw) << 3);
                dst = &kv[slot][p][0][part * 512];
            } else {                            // V^T: 32 dim rows of 16 keys per 1 KB block
                const int b = part - Cf::LPP / 2;
                const int row = 32 * b + lane / 2;
                const int half = (lane & 1) ^ ((row >> 3) & 1);
                src = a.vplane + pbase + row * PD_PAGE + (half << 3);
                dst = &kv[slot][p][1][b * 512];
            }
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
        if (tid < CH) {
            const int pg = c * CH + tid;
            const int blk = pg < npages ? btc[pg] : -1;
            const int ok = blk >= 0 && blk < a.num_blocks;
            if (pg < npages && !ok) flag(a.status, PD_STATUS_BAD_PAGE);
            pv[slot][tid] = ok;
        }
    };

    for (int qbase = 0; qbase < nq; qbase += NW * TPW * 16) {
        const bool wave_has = qbase + wave * 16 < nq;   // wave-uniform
        bf16x8 qv[TPW][KB];
        int qpos[TPW], qrow[TPW], qh[TPW];
        bool qok[TPW];
        f32x4 o[TPW][OT];
        float mrun[TPW], lrun[TPW];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int qi = qbase + (wave + NW * tt) * 16 + r16;
            qok[tt] = qi < nq;
            qrow[tt] = row0 + (qok[tt] ? qi / G : 0);
            qh[tt] = g * G + (qok[tt] ? qi % G : 0);
            qpos[tt] = (qok[tt] && !a.is_rejected[qrow[tt]]) ? a.positions[qrow[tt]] : -1;
            const uint16_t* qp = a.q + ((size_t)qrow[tt] * a.Hq + qh[tt]) * DH;
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
                qv[tt][kk] = qok[tt] ? ld_bf16x8(qp + 32 * kk + 8 * g4) : zero_bf16x8();
#pragma unroll
            for (int j = 0; j < OT; ++j) o[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            mrun[tt] = kNegInf;
            lrun[tt] = 0.f;
        }
        wait_vmcnt<0>();   // query fragments in registers before the ring starts counting

        for (int st = 0; st < NST - 1 && st < nchunks; ++st) issue(st, st);
        for (int c = 0; c < nchunks; ++c) {
            // loads of chunk c done (later chunks may stay in flight), then all waves' loads
            const int later = min(NST - 2, nchunks - 1 - c);
            if (later >= 2) wait_vmcnt<2 * Cf::L>();
            else if (later == 1) wait_vmcnt<Cf::L>();
            else wait_vmcnt<0>();
            __syncthreads();
            if (c + NST - 1 < nchunks) issue(c + NST - 1, (c + NST - 1) % NST);
            const int b = c % NST;
            if (!wave_has) continue;
            // pages in pairs: 32 keys per softmax step and per PV MFMA
            for (int pi = 0; pi < CH; pi += 2) {
                const int p0 = kb + (c * CH + pi) * PD_PAGE;
                if (p0 >= ke) break;
                const bool okA = pv[b][pi] != 0;
                const bool okB = p0 + PD_PAGE < ke && pv[b][pi + 1] != 0;
                const uint16_t* KA = kv[b][pi][0];
                const uint16_t* KBp = kv[b][pi + 1][0];
                const uint16_t* VA = kv[b][pi][1];
                const uint16_t* VBp = kv[b][pi + 1][1];
                bf16x8 kA[KB], kB[KB], vab[OT];
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) {
                    kA[kk] = *reinterpret_cast<const bf16x8*>(KA + k_lds<DH>(r16, 4 * kk + g4));
                    kB[kk] = *reinterpret_cast<const bf16x8*>(KBp + k_lds<DH>(r16, 4 * kk + g4));
                }
                // V^T fragments of both pages: k slots 0-3 = page A keys 4*g4.., 4-7 = page B keys 4*g4..
#pragma unroll
                for (int j = 0; j < OT; ++j) {
                    uint2 va = *reinterpret_cast<const uint2*>(VA + v_lds(16 * j + r16, g4));
                    uint2 vb = *reinterpret_cast<const uint2*>(VBp + v_lds(16 * j + r16, g4));
                    if (!okA) va = make_uint2(0, 0);
                    if (!okB) vb = make_uint2(0, 0);
                    vab[j] = __builtin_bit_cast(bf16x8, make_uint4(va.x, va.y, vb.x, vb.y));
                }
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    f32x4 sA = f32x4{0.f, 0.f, 0.f, 0.f}, sB = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KB; ++kk) {
                        sA = mfma_16x16x32(kA[kk], qv[tt][kk], sA);
                        sB = mfma_16x16x32(kB[kk], qv[tt][kk], sB);
                    }
                    // raw scores of keys p0+4*g4+i (page A) and p0+16+4*g4+i (page B)
                    float sc[8] = {sA[0], sA[1], sA[2], sA[3], sB[0], sB[1], sB[2], sB[3]};
                    // keys this query may see: t <= lim (invalid queries: no limit, don't care)
                    const int lim = qok[tt] && qpos[tt] >= 0 ? min(ke - 1, qpos[tt]) : 0x7fffffff;
                    if (__any(p0 + 2 * PD_PAGE - 1 > lim || !okA || !okB)) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const int t = p0 + (i >> 2) * PD_PAGE + 4 * g4 + (i & 3);
                            const bool ok = (i < 4 ? okA : okB) && t <= lim;
                            sc[i] = ok ? sc[i] : kNegInf;
                        }
                    }
                    float mx = sc[0];
#pragma unroll
                    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
                    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
                    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
                    const float mnew = mx * a.scale_log2;   // -inf stays -inf
                    const bool raise = mnew > mrun[tt] + kRescale;
                    if (__any(raise)) {
                        const float alpha = raise ? __builtin_amdgcn_exp2f(mrun[tt] - mnew) : 1.0f;
                        if (raise) mrun[tt] = mnew;
                        lrun[tt] *= alpha;
#pragma unroll
                        for (int j = 0; j < OT; ++j) o[tt][j] = o[tt][j] * alpha;
                    }
                    const float muse = (mrun[tt] == kNegInf) ? 0.f : mrun[tt];
                    float p[8], ls = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        // raw v_exp_f32: weights below 2^-126 flush to zero
                        p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], a.scale_log2, -muse));
                        ls += p[i];
                    }
                    ls += __shfl_xor(ls, 16, kWave);
                    ls += __shfl_xor(ls, 32, kWave);
                    lrun[tt] += ls;
                    bf16x8 pb;
#pragma unroll
                    for (int i = 0; i < 8; ++i) pb[i] = (__bf16)p[i];
#pragma unroll
                    for (int j = 0; j < OT; ++j) o[tt][j] = mfma_16x16x32(vab[j], pb, o[tt][j]);
                }
            }
        }
        __syncthreads();   // ring slots are free again before a next query pass reuses them

#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            if (!qok[tt]) continue;
            const size_t base = ((size_t)s * a.T + qrow[tt]) * a.Hq + qh[tt];
#pragma unroll
            for (int j = 0; j < OT; ++j)
                *reinterpret_cast<f32x4*>(a.part_o + base * DH + 16 * j + 4 * g4) = o[tt][j];
            if (g4 == 0) {
                a.part_ml[base * 2] = mrun[tt];
                a.part_ml[base * 2 + 1] = lrun[tt];
            }
        }
    }
}

// out[row][h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, splits in
// order. One wave per (row, q head): the split weights are formed across
// lanes, then each lane accumulates its dims over the splits.
template <int DH>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pair = blockIdx.x * 4 + wave;
    if (pair >= a.T * a.Hq) return;
    const int row = pair / a.Hq, h = pair % a.Hq;
    int lo = 0, hi = a.C - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu_out[mid] <= row) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int seq = a.seq_lens[r];
    const bool ok = !a.is_rejected[row] && seq >= 1 && seq <= a.max_blocks * PD_PAGE &&
                    a.cu_out[r] <= row && row < a.cu_out[r + 1];
    const int ns = ok ? num_splits(seq, a.nsmax, a.min_split) : 0;  // <= 128
    constexpr int PER = DH / 64;
    const size_t stride = (size_t)a.T * a.Hq;   // between splits, in (row, head) units
    const size_t base = (size_t)row * a.Hq + h;
    float2 ml0 = make_float2(kNegInf, 0.f), ml1 = make_float2(kNegInf, 0.f);
    if (lane < ns) ml0 = *reinterpret_cast<const float2*>(a.part_ml + (lane * stride + base) * 2);
    if (lane + 64 < ns) ml1 = *reinterpret_cast<const float2*>(a.part_ml + ((lane + 64) * stride + base) * 2);
    const float M = wave_max(fmaxf(ml0.x, ml1.x));
    float w0 = 0.f, w1 = 0.f, L = 0.f;
    if (M != kNegInf) {
        w0 = __builtin_amdgcn_exp2f(ml0.x - M);   // -inf -> 0 for missing splits
        w1 = __builtin_amdgcn_exp2f(ml1.x - M);
        L = w0 * ml0.y + w1 * ml1.y;
    }
    L = wave_sum(L);
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    // all split loads of a lane are independent: issue them 32 at a time
#pragma unroll 32
    for (int sp = 0; sp < ns; ++sp) {
        const float w = __shfl(sp < 64 ? w0 : w1, sp & 63, kWave);
        const float* po = a.part_o + (sp * stride + base) * DH;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += w * po[lane + 64 * i];
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    uint16_t* op = a.out + base * DH;
#pragma unroll
    for (int i = 0; i < PER; ++i) op[lane + 64 * i] = f2bf(acc[i] * inv);
}

template <int DH>
int launch_dh(const AttnArgs& a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    constexpr int NW = AttnCfg<DH>::NW;
    if (e0) (void)hipEventRecord(e0, s);
    // splits a request can have: bounded by nsmax and by the block table's reach
    const int reach = (a.max_blocks * PD_PAGE + a.min_split - 1) / a.min_split;
    const int gx = reach < a.nsmax ? reach : a.nsmax;
    hipLaunchKernelGGL(attn_split_kernel<DH>, dim3(gx, a.Hkv, a.C), dim3(64 * NW), 0, s, a);
    if (e1) (void)hipEventRecord(e1, s);
    if (hipGetLastError() != hipSuccess) return PD_EHIP;
    hipLaunchKernelGGL(attn_merge_kernel<DH>, dim3((a.T * a.Hq + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

}  // namespace

int launch_attention(int dh, const AttnArgs& a, hipStream_t s, hipEvent_t split_begin,
                     hipEvent_t split_end) {
    if (a.C <= 0 || a.T <= 0) return PD_OK;
    if (dh == 64) return launch_dh<64>(a, s, split_begin, split_end);
    if (dh == 128) return launch_dh<128>(a, s, split_begin, split_end);
    return PD_EINVAL;
}

}  // namespace pd
