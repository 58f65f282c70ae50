// bf16 GEMMs of the drafter, Y = X W^T with fp32 accumulation on CDNA4 MFMA.
//
// The drafter's projections (fc 3d->d, QKV, O, gate/up, down, LM head;
// [Paper] = "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training" summary
// page, sec. 2 architecture; [arXiv] = its ScienceStack page, Figure 2) see
// few rows per step: the draft batch has v_r + K - 1 computed rows per
// request and the LM head C*K rows. Three kernels:
//
//  * M <= 64 rows (low concurrency; the LM head up to 128 rows): every
//    projection is a stream of its weight matrix. A persistent ring kernel
//    (one workgroup per CU) copies W and the matching X columns straight from
//    HBM into a ring of LDS stages and runs v_mfma_f32_16x16x32_bf16 on them
//    (W rows are the A operand, X rows the B operand, so a lane ends with 4
//    consecutive output columns of one row); the projections of 17..64 rows
//    stage only W (X fragments go straight to registers);
//  * more rows: persistent tiles fed by a global -> LDS ring, 256 x 256 from
//    384 rows on (the LM head from 129), 128 x 128 (two workgroups per CU)
//    below.
//
// Projections with few output columns are split over workgroups along K.
// Those splits never meet inside the GEMM: each writes an fp32 partial plane,
// and the row kernel that consumes the projection (layer-0 input, RoPE + KV
// write, residual + RMSNorm) sums the planes in split order. No workgroup ever
// waits on another, so no device-wide fence is needed, and the result is
// deterministic. Epilogues: fp32 partial plane, SwiGLU on a pair of matrices
// (gate and up rows streamed side by side, one bf16 rounding), and LM-head
// max/argmax (lowest index on ties) with optional fp32 logits: one partial
// per column tile, or in the few-row kernel one per wave, which keeps its
// best over every column it computes.
#include <float.h>
#include <limits.h>

#include <utility>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace pd {

namespace {


__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ void better(float& bv, int& bi, float ov, int oi) {
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

// ---------------------------------------------------------------------------
// Persistent ring kernel for few rows (M <= 64): the weight stream goes
// straight from HBM into LDS (global_load_lds, 16 B per lane) through a ring
// of NST stages of 128 reduction elements, so each CU keeps ~100 KB of
// weights in flight with a single workgroup and no staging registers. A
// stage holds the workgroup's W rows (NM groups of 16 output columns per
// wave: for SwiGLU one group per matrix, otherwise NM adjacent column
// groups of the one matrix) and the matching X columns of all M rows. Two
// column groups per wave halve the X bytes staged per W byte (the X rows are
// shared by every column of the tile), at the cost of fewer ring stages; the
// waves read
// their MFMA fragments from it (W is the A operand, X the B operand, in every
// kernel of this file, so the epilogues agree). Rows are stored with
// their 16-byte chunks XOR-permuted by (row & 15): the 16 lanes that one LDS
// cycle serves (rows r..r+15, one chunk) read 16 different 16-byte slots of
// the 256-byte bank line. Workgroups are persistent: each
// walks the work items (column tile, K split) blockIdx.x, +gridDim.x, ... and
// the ring runs on across item boundaries, so a CU never waits for a new
// workgroup's first loads.
constexpr int kRS = 128;   // reduction elements per ring stage (256 B of each row)
// Waves per column group of the LM head on 8 X tiles (65..128 rows) and on 2
// (17..32 rows): two, each taking half of the X tiles, so that two waves
// share a SIMD and hide each other's waits (C = 16, 112 rows: 136 vs 157 us,
// 4.6 vs 4.0 TB/s; four waves per group 138 us; C = 4, 28 rows: 174.5 vs
// 176.4 us)
constexpr int kRingLmRowSplit = 2;
constexpr int kRingLm2RowSplit = 2;

// 16 zero bytes: the source of out-of-range chunks (zero-initialised at load)
__device__ __align__(16) uint16_t g_gemm_zero[8];

// KRS: reduction elements per stage (128: rows of 16 16-byte chunks; 64: rows
// of 8 chunks, for 8 X tiles, whose X rows would otherwise crowd the ring).
// RS: waves per column group, each taking MT / RS of the X tiles (2 for the
// LM head on 8 or 2 X tiles: two waves per SIMD)
template <int WN, int NM, int MT, int KRS = kRS, int RS = 1>
struct RingCfg {
    static constexpr int NT = 64 * WN * RS;
    static constexpr int CH = KRS / 8;        // 16-byte chunks per staged row
    static constexpr int WR = 16 * WN * NM;   // W rows per stage (64 or 128)
    static constexpr int XR = 16 * MT;        // X rows per stage
    static constexpr int WL = WR * CH / NT;   // 16-byte W loads per thread per stage
    static constexpr int XL = XR * CH / NT;   // 16-byte X loads per thread per stage
    static constexpr int L = WL + XL;
    static constexpr int SE = (WR + XR) * KRS;   // elements per stage
    // ring stages. One X tile: 4 (the 1-request step with 6, 4, 3, 2 stages
    // in one same-box run: 495.7, 484.5, 495.0, 666.1 us; 5 in another: 489.6
    // against 494.8; the LM head the same at 6 and 4): more stages in flight
    // per CU do not stream faster
    static constexpr int NST = KRS == 64 ? 4
                               : (WR == 64 ? (MT == 1 ? 4 : (MT == 2 ? 5 : 4)) : (MT == 1 ? 4 : 3));
    static_assert(WL * NT == WR * CH && XL * NT == XR * CH, "whole loads per thread");
};

// Chunk permutation of a staged row: the 16 lanes one LDS cycle serves read
// rows r .. r+15 at one chunk. With 16 chunks a row fills a 256-byte bank
// line and the chunk is XORed with r & 15; with 8 chunks two rows share a
// line (the row's parity picks the half) and the chunk is XORed with
// (r >> 1) & 7. Either way the 16 lanes hit 16 distinct 16-byte slots.
template <int CH>
__device__ __forceinline__ int ring_sw(int row) {
    if constexpr (CH == 16) return row & 15;
    else return (row >> 1) & 7;
}

template <int N>
__device__ __forceinline__ void ring_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most `later` stages of L loads each are still in flight
template <int L, int MAXN>
__device__ __forceinline__ void ring_wait_later(int later) {
    if constexpr (MAXN == 0) {
        ring_wait<0>();
    } else {
        if (later >= MAXN) ring_wait<L * MAXN>();
        else ring_wait_later<L, MAXN - 1>(later);
    }
}
__device__ __forceinline__ void ring_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// LDS address of a pointer into a __shared__ array as a wave-uniform 32-bit
// offset: the copies into the ring are then ordered only by the explicit
// waits above (the compiler would otherwise wait for all of them at every
// LDS read, not knowing the ring slots apart)
__device__ __forceinline__ unsigned ring_lds(void* p) {
    return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)p);
}

template <int WN, int NM, int MT, int EPI, int KRS = kRS, int RS = 1>
__global__ __launch_bounds__(64 * WN * RS) void gemm_ring_kernel(GemmArgs a) {
    using Cf = RingCfg<WN, NM, MT, KRS, RS>;
    constexpr int MTW = MT / RS;   // X tiles of each wave
    static_assert(MT % RS == 0 && (RS == 1 || EPI == EPI_ARGMAX), "row split: the LM head only");
    constexpr int NT = Cf::NT, NST = Cf::NST, L = Cf::L, WL = Cf::WL, XL = Cf::XL, CH = Cf::CH;
    constexpr bool PAIR = (EPI == EPI_SWIGLU);          // row groups = gate, up of the same columns
    constexpr int TW = 16 * WN * (PAIR ? 1 : NM);       // output columns per tile
    __shared__ __align__(16) uint16_t ring[NST * Cf::SE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, tb = (wave / WN) * MTW;   // column group of the wave, its first X tile
    const int r16 = lane & 15, g4 = lane >> 4;

    const int ksteps = (a.K + KRS - 1) / KRS;
    const int per = (ksteps + a.splits - 1) / a.splits;
    const int ntn = (a.N + TW - 1) / TW;   // column tiles
    const int nitems = ntn * a.splits;
    const int G = gridDim.x;

    // this thread's fixed share of every stage: W (row within the tile,
    // chunk) and X (row pointer, chunk)
    int wrr[WL], wgq[WL], wch[WL], wofs[WL];
#pragma unroll
    for (int j = 0; j < WL; ++j) {
        const int u = tid + NT * j, wr = u / CH;
        wrr[j] = wr % (16 * WN);
        wgq[j] = wr / (16 * WN);   // row group of this load
        wch[j] = ((u % CH) ^ ring_sw<CH>(wr)) * 8;
        wofs[j] = wrr[j] * a.K + wch[j];   // element offset from the tile's first row, k = 0
    }
    const uint16_t* xp[XL];
    int xch[XL];
#pragma unroll
    for (int j = 0; j < XL; ++j) {
        const int u = tid + NT * j, m = u / CH;
        xch[j] = ((u % CH) ^ ring_sw<CH>(m)) * 8;
        int row = m;
        bool ok = m < a.M;
        if (ok && a.xrows) {
            row = a.xrows[m];
            if (row < 0 || row >= a.xrows_limit) {
                ok = false;
                flag(a.status, PD_STATUS_BAD_ROW);
            }
        }
        xp[j] = ok ? a.X + (size_t)row * a.ldx : nullptr;
    }
    const uint16_t* zp = g_gemm_zero;
    const unsigned lds0 = ring_lds(ring);

    // stages this workgroup consumes, item by item
    int total = 0;
    for (int it = blockIdx.x; it < nitems; it += G) {
        const int sp = it / ntn;
        total += max(0, min(ksteps, (sp + 1) * per) - sp * per);
    }

    // issue cursor: (item, stage) of the next stage to load; the W sources
    // of the item (row pointers at each load's chunk, or null past N) are set
    // once per item, so a stage only adds its K offset
    int iitem = blockIdx.x, iks = 0, ike = 0;
    const uint16_t* wp[WL];
    bool wfull = true;   // the item's tile lies inside N
    auto set_item = [&]() {
        const int sp = iitem / ntn;
        iks = sp * per;
        ike = min(ksteps, (sp + 1) * per);
        const int n0 = (iitem % ntn) * TW;
        wfull = n0 + TW <= a.N;
#pragma unroll
        for (int j = 0; j < WL; ++j) {
            const int q = wgq[j];
            const int nq = n0 + (PAIR ? 0 : q * 16 * WN);
            const uint16_t* base = (PAIR && q == 1) ? a.W2 : a.W;
            wp[j] = (nq + wrr[j] < a.N) ? base + (size_t)nq * a.K + wofs[j] : nullptr;
        }
    };
    if (iitem < nitems) set_item();
    auto issue = [&](int slot) {
        // skip items without stages (not produced by the planner)
        while (iitem < nitems && iks >= ike) {
            iitem += G;
            if (iitem < nitems) set_item();
        }
        const int k0 = iks * KRS;
        const unsigned sbase = lds0 + (unsigned)(slot * Cf::SE) * 2u;
        // whole tile inside N and whole stage inside K: no per-lane bounds
        const bool kin = k0 + KRS <= a.K;
        const bool inner = wfull && kin;
#pragma unroll
        for (int j = 0; j < WL; ++j) {
            const uint16_t* src;
            if (inner)
                src = wp[j] + k0;
            else
                src = (wp[j] && k0 + wch[j] < a.K) ? wp[j] + k0 : zp;
            // every weight is read once: non-temporal (cache policy 2), so the
            // stream does not evict the X columns all workgroups re-read
            __builtin_amdgcn_global_load_lds((void*)src,
                (__attribute__((address_space(3))) void*)(uintptr_t)(sbase + (unsigned)(wave * 64 + NT * j) * 16u),
                16, 0, 2);
        }
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const int k = k0 + xch[j];
            const uint16_t* src = (xp[j] && (kin || k < a.K)) ? xp[j] + k : zp;
            __builtin_amdgcn_global_load_lds((void*)src,
                (__attribute__((address_space(3))) void*)(uintptr_t)(sbase + (unsigned)(Cf::WR * KRS * 2) +
                                                                      (unsigned)(wave * 64 + NT * j) * 16u),
                16, 0, 0);
        }
        ++iks;
    };

    ring_wait<0>();   // row gathers done before the ring starts counting
    for (int st = 0; st < NST - 1 && st < total; ++st) issue(st);

    // LM head: a lane's best (value, lowest index) of row 16t + r16 over every
    // column it sees, across all of the workgroup's items
    float runv[MTW];
    int runi[MTW];
#pragma unroll
    for (int t = 0; t < MTW; ++t) {
        runv[t] = -FLT_MAX;
        runi[t] = INT_MAX;
    }
    int qc = 0;   // stages consumed
    for (int it = blockIdx.x; it < nitems; it += G) {
        const int sp = it / ntn;
        const int kb = sp * per, ke = min(ksteps, (sp + 1) * per);
        if (kb >= ke) continue;
        f32x4 acc[MTW][NM];
#pragma unroll
        for (int t = 0; t < MTW; ++t)
#pragma unroll
            for (int q = 0; q < NM; ++q) acc[t][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int ks = kb; ks < ke; ++ks, ++qc) {
            // loads of stage qc done (later stages may stay in flight), then every wave's
            ring_wait_later<L, NST - 2>(min(NST - 2, total - 1 - qc));
            ring_barrier();
            if (qc + NST - 1 < total) issue((qc + NST - 1) % NST);
            const uint16_t* Ws = ring + (qc % NST) * Cf::SE;
            const uint16_t* Xs = Ws + Cf::WR * KRS;
#pragma unroll
            for (int j = 0; j < KRS / 32; ++j) {
                // every staged row here is 16t + r16 for some t: its permutation
                // depends on r16 alone
                const int pos = ((4 * j + g4) ^ ring_sw<CH>(r16)) * 8;
                bf16x8 wf[NM];
#pragma unroll
                for (int q = 0; q < NM; ++q)
                    wf[q] = *reinterpret_cast<const bf16x8*>(Ws + (q * 16 * WN + 16 * wn + r16) * KRS + pos);
#pragma unroll
                for (int t = 0; t < MTW; ++t) {
                    const bf16x8 xf = *reinterpret_cast<const bf16x8*>(Xs + (16 * (tb + t) + r16) * KRS + pos);
#pragma unroll
                    for (int q = 0; q < NM; ++q) acc[t][q] = mfma_16x16x32(wf[q], xf, acc[t][q]);
                }
            }
        }

        // lane holds rows m = 16 (tb + t) + r16 and columns n .. n+3 of each column group q
        const int n0 = (it % ntn) * TW + 16 * wn + 4 * g4;
        if constexpr (EPI == EPI_ARGMAX) {
#pragma unroll
            for (int q = 0; q < NM; ++q) {
                const int n = n0 + q * 16 * WN;
                if (n >= a.N) continue;
#pragma unroll
                for (int t = 0; t < MTW; ++t) {
                    const int m = 16 * (tb + t) + r16;
#pragma unroll
                    for (int e = 0; e < 4; ++e) better(runv[t], runi[t], acc[t][q][e], n + e);
                    if (a.logits && m < a.M)
                        *reinterpret_cast<f32x4*>(a.logits + (size_t)m * a.ldlog + n) = acc[t][q];
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < MTW; ++t) {
                const int m = 16 * (tb + t) + r16;
                if (m >= a.M) continue;
                if constexpr (EPI == EPI_PARTIAL) {
#pragma unroll
                    for (int q = 0; q < NM; ++q) {
                        const int n = n0 + q * 16 * WN;
                        if (n < a.N) *reinterpret_cast<f32x4*>(a.ws + ((size_t)sp * a.M + m) * a.N + n) = acc[t][q];
                    }
                } else {
                    if (n0 >= a.N) continue;
                    float h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[e] = silu(acc[t][0][e]) * acc[t][NM - 1][e];
                    uint2 pk;
                    pk.x = uint32_t(f2bf(h[0])) | (uint32_t(f2bf(h[1])) << 16);
                    pk.y = uint32_t(f2bf(h[2])) | (uint32_t(f2bf(h[3])) << 16);
                    *reinterpret_cast<uint2*>(a.yb + (size_t)m * a.ldyb + n0) = pk;
                }
            }
        }
    }
    if constexpr (EPI == EPI_ARGMAX) {
        // one (value, index) per row per column group: entry blockIdx.x * WN + wn
#pragma unroll
        for (int t = 0; t < MTW; ++t) {
            float bv = runv[t];
            int bi = runi[t];
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float ov = __shfl_xor(bv, off, kWave);
                const int oi = __shfl_xor(bi, off, kWave);
                better(bv, bi, ov, oi);
            }
            const int m = 16 * (tb + t) + r16;
            if (g4 == 0 && m < a.M) {
                a.amax_v[(size_t)m * a.ntiles + blockIdx.x * WN + wn] = bv;
                a.amax_i[(size_t)m * a.ntiles + blockIdx.x * WN + wn] = bi;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Weight-only ring (17..64 rows: the projections of the few-request steps).
// The ring kernel above stages the X columns in its LDS stages next to the
// weights; at 33..64 rows they fill half of every stage (the gate/up stream
// ran ~1.5x slower at 56 rows than at 7). Here the LDS ring holds weights
// only: NST stages of 64 W rows x 128 reduction elements (16 KB each). Each
// of the four waves owns one 16-row X tile
// and all 64 columns of the stage, and loads its X fragments straight into
// registers, from L2 (X is a few hundred KB that every workgroup re-reads).
// The X loads of a stage are issued with the stage's weight loads, NST - 1
// stages ahead, so the ring's in-order vmcnt waits cover them too; the
// register slot of stage q is q mod NST, and the stage loop runs in whole
// passes of NST stages, unrolled, so that every slot index is a compile-time
// constant. Padding rows of a partial X tile read zeros; their MFMAs cost
// nothing in a stream this far below the ridge.
//
// The compiler adds its own waits before the X registers are used; they stay
// partial (NST - 2 stages of loads may remain in flight) because the weight
// copies use the buffer form (see below). A workgroup owns exactly one
// (column tile, K split) item and writes it after the loop. Projections
// only (fp32 partial planes, SwiGLU): measured on the 4-request step (56
// projection rows) with 8 stages, the projections ran 24 us faster per step
// than on the ring kernel, the 28-row LM head 20 us slower. Stages: 4 (three
// same-box runs of that step against 8 stages at 598-602 us: 6 594.0, 5
// 577.9, 4 572.6, 3 568.7-574.6, 2 668.1 us; 3 and 4 are within 1%).
constexpr int kWRingStages = 4;
// word 3 of a raw buffer descriptor on gfx9 (no format conversion, no swizzle)
constexpr int kBufferRsrcWord3 = 0x00020000;

// f(integral_constant<int, I>) for I = 0, 1, ... in order
template <int... I, class F>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, I...>, F&& f) {
    (f(std::integral_constant<int, I>{}), ...);
}

// GW groups of 16 W rows per stage (every wave reads all of them). Four, one
// workgroup per CU: two groups in a 64 KB ring with two workgroups per CU
// ran the 4-request step 59 us slower. (The per-thread arrays below have
// the fixed size 4 >= GW: local arrays
// whose size depends on the template parameter, used inside the lambdas,
// make the host pass drop the launch stub.)
template <int GW>
struct WRingCfg {
    static constexpr int NST = kWRingStages;
    static constexpr int NT = 256, CH = kRS / 8;
    static constexpr int WR = 16 * GW;       // W rows per stage
    static constexpr int WL = WR * CH / NT;  // W loads per thread per stage: load j = group j
    static constexpr int XLD = kRS / 32;     // X fragment loads per lane per stage (4)
    static constexpr int L = WL + XLD;       // vector memory ops per thread per stage
    static constexpr int SE = WR * kRS;      // elements per stage
};

template <int EPI, int GW>
__global__ __launch_bounds__(256) void gemm_wring_kernel(GemmArgs a) {
    using Cf = WRingCfg<GW>;
    constexpr int NST = Cf::NST, NT = Cf::NT, CH = Cf::CH, WR = Cf::WR, WL = Cf::WL, XLD = Cf::XLD;
    constexpr int L = Cf::L, SE = Cf::SE;
    constexpr bool PAIR = (EPI == EPI_SWIGLU);
    static_assert(EPI == EPI_PARTIAL || EPI == EPI_SWIGLU, "projections");
    constexpr int TW = PAIR ? WR / 2 : WR;      // output columns per tile
    static_assert((NST - 2) * L <= 63, "the waits fit the vmcnt field");
    static_assert(WL == GW && WL <= 4 && XLD == 4 && NT / CH == 16, "load j of a thread is row tid / 16 of group j");
    static_assert(!PAIR || GW % 2 == 0, "gate and up groups in pairs");
    __shared__ __align__(16) uint16_t ring[Cf::NST * Cf::SE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // = the wave's X tile
    const int r16 = lane & 15, g4 = lane >> 4;
    const int m = 16 * wave + r16;   // this lane's output row

    const int ksteps = (a.K + kRS - 1) / kRS;
    const int per = (ksteps + a.splits - 1) / a.splits;
    const int ntn = (a.N + TW - 1) / TW;
    const int nitems = ntn * a.splits;
    const int item = blockIdx.x;   // the plan launches one workgroup per item
    if (item >= nitems) return;    // whole workgroup

    // This thread's W loads of every stage: load j copies row tid / 16 of
    // group j (staged row 16 j + tid / 16) at LDS chunk tid % 16, which holds
    // global chunk (tid % 16) ^ (tid / 16). SwiGLU: groups 0 .. GW/2 - 1 are
    // gate columns of the tile, the rest the up rows of the same columns.
    const int wrow = tid >> 4;
    const int wchb = (((tid & 15) ^ wrow) * 8) * 2;   // byte offset of the chunk within a row stage
    // this lane's X row, or none past M
    int xrow = -1;
    if (m < a.M) {
        int row = m;
        if (a.xrows) {
            row = a.xrows[m];
            if (row < 0 || row >= a.xrows_limit) {
                row = -1;
                flag(a.status, PD_STATUS_BAD_ROW);
            }
        }
        xrow = row;
    }
    const unsigned lds0 = ring_lds(ring);

    // Copies go through buffer descriptors: weights global -> LDS (the MUBUF
    // form: the compiler treats the global form as a FLAT access that may
    // touch LDS, and while one is in flight it turns every wait of its own
    // for the X registers into a full drain), X into registers. A whole
    // stage adds its K offset as the scalar soffset, so it costs 4 M0 moves
    // and 8 loads. The range check covers the per-lane offset only (not
    // soffset): a stage that reaches past K adds its K offset per lane
    // instead, so that reads past the last weight row come back as zeros;
    // weight chunks past K otherwise read the next row, which only meets X
    // chunks that are zero there. Offsets past the range (kOut) read zeros
    // and touch no memory: W rows past N, X rows past M or badly gathered,
    // X chunks past K, and every load of a stage past the last one. The
    // planner keeps N * K * 2 below 2^31.
    constexpr unsigned kOut = 0x80000000u;
    const __amdgpu_buffer_rsrc_t wrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.W, 0, a.N * a.K * 2, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t wrs2 =
        __builtin_amdgcn_make_buffer_rsrc((void*)(PAIR ? a.W2 : a.W), 0, a.N * a.K * 2, kBufferRsrcWord3);
    const int xrows_n = a.xrows ? a.xrows_limit : a.M;
    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.X, 0, xrows_n * a.ldx * 2, kBufferRsrcWord3);
    unsigned xvo[Cf::XLD];   // byte offset of this lane's X chunk j at k = 0
#pragma unroll
    for (int j = 0; j < XLD; ++j)
        xvo[j] = xrow >= 0 ? (unsigned)((xrow * a.ldx + 32 * j + 8 * g4) * 2) : kOut;

    // the item: column tile n0, K split sp = stages kb0 .. kb0 + kcnt - 1
    const int sp = item / ntn;
    const int n0 = (item % ntn) * TW;
    const int kb0 = sp * per;
    const int total = max(0, min(ksteps, (sp + 1) * per) - kb0);
    const int kcnt = max(1, total);
    unsigned wvo[4];   // byte offset of this thread's chunk j at k = 0, or kOut past N
#pragma unroll
    for (int j = 0; j < WL; ++j) {
        const int col = n0 + (PAIR ? (j % (GW / 2)) * 16 : 16 * j) + wrow;
        wvo[j] = col < a.N ? (unsigned)(col * a.K * 2 + wchb) : kOut;
    }
    // the stages start at a point set by the column tile, so that workgroups
    // sharing a K split read different X lines at any moment
    const int rot = (item % ntn) % kcnt;
    int iks = 0;   // stages issued
    // Loads of the next stage into LDS slot `slot` and register slot xd.
    // Every call issues the same L loads, also past the last stage (live
    // false), so the loads in flight behind a stage are the same on every
    // path; only their offsets depend on the case.
    auto issue = [&](int slot, bf16x8 (&xd)[Cf::XLD], bool live) __attribute__((always_inline)) {
        const int k0 = (kb0 + (iks + rot) % kcnt) * kRS;
        const unsigned sbase = lds0 + (unsigned)(slot * SE) * 2u;
        unsigned so = (unsigned)k0 * 2u;
        unsigned wv[4], xv[4];
#pragma unroll
        for (int j = 0; j < WL; ++j) wv[j] = wvo[j];
#pragma unroll
        for (int j = 0; j < XLD; ++j) xv[j] = xvo[j];
        if (!live || k0 + kRS > a.K) {
            so = 0;
#pragma unroll
            for (int j = 0; j < WL; ++j) wv[j] = (live && wvo[j] != kOut) ? wvo[j] + (unsigned)k0 * 2u : kOut;
#pragma unroll
            for (int j = 0; j < XLD; ++j)
                xv[j] = (live && k0 + 32 * j + 8 * g4 < a.K) ? xvo[j] + (unsigned)k0 * 2u : kOut;
        }
#pragma unroll
        for (int j = 0; j < WL; ++j)   // every weight is read once: non-temporal (cache policy 2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds((PAIR && j >= GW / 2) ? wrs2 : wrs,
                (__attribute__((address_space(3))) void*)(uintptr_t)(sbase + (unsigned)(wave * 64 + NT * j) * 16u),
                16, wv[j], so, 0, 2);
#pragma unroll
        for (int j = 0; j < XLD; ++j)
            xd[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xrs, xv[j], so, 0));
        if (live) ++iks;
    };

    bf16x8 xr[Cf::NST][Cf::XLD];
    ring_wait<0>();   // row gathers done before the ring starts counting
    // the ring's waits count whole stages: the compiler must not move the X
    // loads (plain reads) of one stage across another's, hence the fence
#pragma unroll
    for (int st = 0; st < NST - 1; ++st) {
        issue(st, xr[st], st < total);
        asm volatile("" ::: "memory");
    }

    f32x4 acc[4];
#pragma unroll
    for (int q = 0; q < GW; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One stage: qc = the stage, us = qc mod NST (a compile-time constant at
    // every call: the LDS slot and the register slot of the stage).
    auto step = [&](const int qc, auto usc) __attribute__((always_inline)) {
        constexpr int us = decltype(usc)::value;
        // loads of stage qc done (the NST - 2 stages after it may stay in
        // flight), then every wave's
        ring_wait<(NST - 2) * L>();
        ring_barrier();
        issue((us + NST - 1) % NST, xr[(us + NST - 1) % NST], qc + NST - 1 < total);
        const uint16_t* Ws = ring + us * SE;
#pragma unroll
        for (int j = 0; j < kRS / 32; ++j) {
            const int pos = ((4 * j + g4) ^ r16) * 8;
#pragma unroll
            for (int q = 0; q < GW; ++q) {
                const bf16x8 wf = *reinterpret_cast<const bf16x8*>(Ws + (16 * q + r16) * kRS + pos);
                acc[q] = mfma_16x16x32(wf, xr[us][j], acc[q]);
            }
        }
    };
    // Whole passes of NST stages, then the last < NST stages in straight
    // code, so that no edge leads from inside a pass back to its start.
    int q0 = 0;
    for (; q0 + NST <= total; q0 += NST)
        for_each_index(std::make_integer_sequence<int, NST>{}, [&](auto i) __attribute__((always_inline)) {
            step(q0 + decltype(i)::value, i);
        });
    for_each_index(std::make_integer_sequence<int, NST>{}, [&](auto i) __attribute__((always_inline)) {
        if (q0 + decltype(i)::value < total) step(q0 + decltype(i)::value, i);
    });
    ring_wait<0>();   // the zero-page loads past the last stage have landed

    if (total == 0) return;
    if constexpr (EPI == EPI_PARTIAL) {
        if (m < a.M) {
#pragma unroll
            for (int q = 0; q < GW; ++q) {
                const int n = n0 + 16 * q + 4 * g4;
                if (n < a.N) *reinterpret_cast<f32x4*>(a.ws + ((size_t)sp * a.M + m) * a.N + n) = acc[q];
            }
        }
    } else {
        if (m < a.M) {
#pragma unroll
            for (int q = 0; q < GW / 2; ++q) {
                const int n = n0 + 16 * q + 4 * g4;
                if (n >= a.N) continue;
                float h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = silu(acc[q][e]) * acc[q + GW / 2][e];
                uint2 pk;
                pk.x = uint32_t(f2bf(h[0])) | (uint32_t(f2bf(h[1])) << 16);
                pk.y = uint32_t(f2bf(h[2])) | (uint32_t(f2bf(h[3])) << 16);
                *reinterpret_cast<uint2*>(a.yb + (size_t)m * a.ldyb + n) = pk;
            }
        }
    }
}

// Persistent ring-fed tile kernel for many rows (M > 64). With BT = 256 a
// workgroup of 8 waves (two per SIMD: one wave per SIMD cannot keep the
// matrix core busy) owns a 256 (W rows = output columns) x 256 (X rows =
// output rows) tile; each wave computes 128 x 64 of it (8 x 4 MFMA tiles),
// which keeps the LDS fragment reads at 3 bytes per flop-pair lower than
// 64 x 64 wave tiles. With BT = 128 (for 64 < M < 384) four waves of 64 x 64
// share a 128 x 128 tile and two workgroups fit a CU. W and X tiles of 32
// reduction elements go straight from HBM/L2 into a 4-stage LDS ring
// (global_load_lds, 2 BT x 64 B per stage); each resident workgroup walks its
// work items (tile, K split) without restarting the ring. The copy sources
// are set once per item, so a stage only adds its K offset. Rows are 64 B in LDS
// with their 16-byte chunks XOR-permuted (big_sw): a fragment read (rows
// r..r+15, one chunk) meets no bank conflict, counting the banks as 64 or
// as 32 four-byte banks. Items are dealt so that in
// every round each XCD takes a contiguous run of tiles (M blocks innermost):
// tiles sharing a W tile and K range meet in one L2. For SwiGLU a tile's W
// rows are 128 gate rows then the same 128 up rows; a wave takes 64 of each.
// X rows are read directly (no row gather). The MFMA operands of the next
// stage are read from LDS while the current stage's MFMAs run (X fragments
// double-buffered, each W fragment register refilled right after its last
// MFMA), so a wave never stalls on LDS between MFMAs.
constexpr int kBT = 256;                 // tile rows of W and of X
// Chunk permutation of a 64-byte staged row. Rows r..r+15 at one chunk land
// in 16 distinct 16-byte slots of a 256-byte line set (r & 3 picks the
// quarter, the permuted chunk differs among rows with equal r & 3), and rows
// 8t..8t+7 in 8 distinct slots of a 128-byte one (r & 1 picks the half, the
// permuted chunk differs among rows with equal parity). With the
// permutation (r >> 2) & 3 alone the 128-byte view saw 2-way conflicts on
// half of the LDS cycles (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE = 0.5).
__device__ __forceinline__ int big_sw(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }
constexpr int kBS = 32;                  // reduction elements per stage (64 B of each row)
constexpr int kBNST = 4;                 // ring stages (max/argmax epilogue: its LDS tables fit beside 4)
constexpr int kBNSTP = 4;                // ring stages of the other epilogues

template <int EPI, int BT>
__global__ __launch_bounds__(2 * BT, 2) void gemm_big_kernel(GemmArgs a) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    constexpr int L = 4;                      // 16-byte loads per thread per stage: 2 of W, 2 of X
    constexpr int NT = 2 * BT;                // threads: BT / 32 waves
    constexpr int NA = BT / 32;               // W fragments (16 output columns each) per wave
    constexpr int SE = 2 * BT * kBS;          // elements per stage: W tile rows, then X tile rows
    constexpr int COLS = DUAL ? BT / 2 : BT;  // output columns per tile
    constexpr int NST = EPI == EPI_ARGMAX ? kBNST : kBNSTP;
    __shared__ __align__(16) uint16_t ring[NST * SE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = lane >> 4;
    const int wn = wave & 1, wm = wave >> 1;   // 2 column halves x (BT / 64) groups of 64 rows

    // rows present (a device count when given): only their row blocks are
    // tiled, and the K split count is chosen here for that many tiles
    const int meff = a.m_dev ? min(a.M, max(0, *a.m_dev)) : a.M;
    const int mblocks = (meff + BT - 1) / BT;
    const int ntn = (a.N + COLS - 1) / COLS;
    const int tiles = ntn * mblocks;
    const int ksteps = (a.K + kBS - 1) / kBS;
    const int G = gridDim.x;
    int splits = a.splits;
    if constexpr (EPI == EPI_PARTIAL) {
        if (a.m_dev) splits = big_splits(tiles, ksteps, G, a.splits);
        if (a.splits_out && blockIdx.x == 0 && threadIdx.x == 0) a.splits_out[0] = splits;
    }
    const int per = (ksteps + splits - 1) / splits;
    const int nitems = tiles * splits;
    // workgroups go round-robin to the 8 XCDs: XCD x holds blocks x, x+8, ...;
    // give it a contiguous run of item positions (any G: the first G % 8
    // XCDs hold one block more)
    const int xcd = blockIdx.x & 7, q8 = G >> 3, r8 = G & 7;
    const int rpos = xcd * q8 + min(xcd, r8) + (blockIdx.x >> 3);

    // this thread's fixed share of every stage: units u = tid + NT j; j = 0, 1
    // are W rows u / 4, j = 2, 3 are X rows (u - 2 NT) / 4; chunk u % 4
    int rowrel[4], ch[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int u = tid + NT * j;
        const int r = (j < 2 ? u : u - 2 * NT) >> 2;
        rowrel[j] = r;
        ch[j] = ((u & 3) ^ big_sw(r)) * 8;
    }
    const uint16_t* zp = g_gemm_zero;
    const unsigned lds0 = ring_lds(ring);

    int total = 0;
    for (int it = rpos; it < nitems; it += G) {
        const int sp = it / tiles;
        total += max(0, min(ksteps, (sp + 1) * per) - sp * per);
    }
    // The copy sources of the item being issued: row pointers (at the row's
    // chunk) set once per item, so a stage only adds its K offset. Rows past
    // N / M point at the zero buffer with a zero K mask; chunks past K (only
    // in a last, partial stage) also come from the zero buffer.
    int iitem = rpos, iks = 0, ike = 0;
    const uint16_t* rsrc[4];
    unsigned kmask[4];
    auto set_item = [&]() {
        const int sp = iitem / tiles;
        iks = sp * per;
        ike = min(ksteps, (sp + 1) * per);
        const int tile = iitem % tiles;
        const int m0 = (tile % mblocks) * BT;
        const int n0 = (tile / mblocks) * COLS;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < 2) {
                const int r = rowrel[j];
                const int n = n0 + (DUAL ? (r & (COLS - 1)) : r);
                const uint16_t* base = (DUAL && r >= COLS) ? a.W2 : a.W;
                const bool ok = n < a.N;
                kmask[j] = ok ? ~0u : 0u;
                rsrc[j] = ok ? base + (size_t)n * a.K + ch[j] : zp;
            } else {
                const int m = m0 + rowrel[j];
                const bool ok = m < meff;
                kmask[j] = ok ? ~0u : 0u;
                rsrc[j] = ok ? a.X + (size_t)m * a.ldx + ch[j] : zp;
            }
        }
    };
    if (iitem < nitems) set_item();
    auto issue = [&](int slot) {
        while (iitem < nitems && iks >= ike) {
            iitem += G;
            if (iitem < nitems) set_item();
        }
        const int k0 = iks * kBS;
        const unsigned sbase = lds0 + (unsigned)(slot * SE) * 2u;
        const uint16_t* src[4];
        if (k0 + kBS <= a.K) {   // the whole stage inside K
#pragma unroll
            for (int j = 0; j < 4; ++j) src[j] = rsrc[j] + ((unsigned)k0 & kmask[j]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) src[j] = (kmask[j] && k0 + ch[j] < a.K) ? rsrc[j] + k0 : zp;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds((void*)src[j],
                (__attribute__((address_space(3))) void*)(uintptr_t)(sbase + (unsigned)(wave * 64 + NT * j) * 16u),
                16, 0, 0);
        ++iks;
    };

    // LDS element offsets of this lane's first W and X fragment rows; W
    // fragment i lies arow(i) rows further (gate rows, then the matching up
    // rows COLS further for SwiGLU), X fragment j 16 j rows further: both
    // compile-time, so every fragment read is one base plus an immediate
    const int rsw = big_sw(r16);
    const int pos = (g4 ^ rsw) * 8;
    const int la = ((DUAL ? BT / 4 : BT / 2) * wn + r16) * kBS + pos;
    const int lb = (BT + 64 * wm + r16) * kBS + pos;
    auto arow = [](int i) { return DUAL ? (i < NA / 2 ? 16 * i : COLS + 16 * (i - NA / 2)) : 16 * i; };

    // one stage's MFMA operands: W fragments a[NA] are overwritten with the
    // next stage's one by one, each right after its last MFMA has been issued;
    // X fragments are double-buffered (read at the start of the previous stage)
    auto read_a = [&](int q, int i) {
        const uint16_t* Ws = ring + ((unsigned)q % NST) * SE + la;
        return *reinterpret_cast<const bf16x8*>(Ws + arow(i) * kBS);
    };
    auto read_b = [&](bf16x8 (&b)[4], int q) {
        const uint16_t* Xs = ring + ((unsigned)q % NST) * SE + lb;
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8*>(Xs + 16 * j * kBS);
    };

    f32x4 acc[NA][4];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // lane holds rows m = m0 + 64*wm + 16*j + r16 and 4 consecutive columns per group i
    auto epilogue = [&](int it) {
        const int sp = it / tiles;
        const int tile = it % tiles;
        const int m0 = (tile % mblocks) * BT;
        const int ntile = tile / mblocks;
        const int n0 = ntile * COLS;
        if constexpr (EPI == EPI_ARGMAX) {
            __shared__ float s_v[2][BT];
            __shared__ int s_i[2][BT];
            ring_barrier();   // the previous item's readers of s_v / s_i are done
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ml = 64 * wm + 16 * j + r16;
                const int m = m0 + ml;
                float bv = -FLT_MAX;
                int bi = INT_MAX;
#pragma unroll
                for (int i = 0; i < NA; ++i) {
                    const int n = n0 + (BT / 2) * wn + 16 * i + 4 * g4;
                    if (n >= a.N) continue;
#pragma unroll
                    for (int e = 0; e < 4; ++e) better(bv, bi, acc[i][j][e], a.n_base + n + e);
                    if (a.logits && m < a.M)
                        *reinterpret_cast<f32x4*>(a.logits + (size_t)m * a.ldlog + n) = acc[i][j];
                }
#pragma unroll
                for (int off = 16; off <= 32; off <<= 1) {
                    const float ov = __shfl_xor(bv, off, kWave);
                    const int oi = __shfl_xor(bi, off, kWave);
                    better(bv, bi, ov, oi);
                }
                if (g4 == 0) {
                    s_v[wn][ml] = bv;
                    s_i[wn][ml] = bi;
                }
            }
            ring_barrier();   // (no wait on the ring's copies in flight)
            if (tid < BT) {
                const int m = m0 + tid;
                float bv = s_v[0][tid];
                int bi = s_i[0][tid];
                better(bv, bi, s_v[1][tid], s_i[1][tid]);
                const int ld = a.amax_ld ? a.amax_ld : a.ntiles;
                if (m < a.M) {
                    a.amax_v[(size_t)m * ld + ntile] = bv;
                    a.amax_i[(size_t)m * ld + ntile] = bi;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = m0 + 64 * wm + 16 * j + r16;
                if (m >= meff) continue;
                if constexpr (EPI == EPI_PARTIAL) {
#pragma unroll
                    for (int i = 0; i < NA; ++i) {
                        const int n = n0 + (BT / 2) * wn + 16 * i + 4 * g4;
                        if (n < a.N)
                            *reinterpret_cast<f32x4*>(a.ws + ((size_t)sp * a.M + m) * a.N + n) = acc[i][j];
                    }
                } else {  // SwiGLU: groups 0..NA/2-1 = gate, the rest the matching up columns
#pragma unroll
                    for (int i = 0; i < NA / 2; ++i) {
                        const int n = n0 + (BT / 4) * wn + 16 * i + 4 * g4;
                        if (n >= a.N) continue;
                        float h[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) h[e] = silu(acc[i][j][e]) * acc[i + NA / 2][j][e];
                        uint2 pk;
                        pk.x = uint32_t(f2bf(h[0])) | (uint32_t(f2bf(h[1])) << 16);
                        pk.y = uint32_t(f2bf(h[2])) | (uint32_t(f2bf(h[3])) << 16);
                        *reinterpret_cast<uint2*>(a.yb + (size_t)m * a.ldyb + n) = pk;
                    }
                }
            }
        }
    };

    // all ring slots filled up front; stage q lives in slot q % NST
    for (int st = 0; st < NST && st < total; ++st) issue(st);
    bf16x8 af[NA], bc[4], bn[4];
    if (total > 0) {
        ring_wait_later<L, NST - 1>(min(NST - 1, total - 1));
        ring_barrier();
#pragma unroll
        for (int i = 0; i < NA; ++i) af[i] = read_a(0, i);
        read_b(bc, 0);
    }
    int qc = 0;
    // one stage: wait for the next stage's copies, refill the slot everyone
    // has read, then this stage's MFMAs interleaved with the reads of the
    // next stage's operands. After the last stage the reads fetch a stale
    // (in-bounds) slot whose values are never used; the waits and barriers
    // are uniform over the workgroup.
    auto stage = [&](bf16x8 (&bc)[4], bf16x8 (&bn)[4]) {
        // the next stage's copies done, the ones issued after it still in
        // flight (near the end: all done)
        if (qc + NST - 1 < total) ring_wait<L * (NST - 2)>();
        else ring_wait<0>();
        ring_barrier();
        if (qc + NST < total) issue((unsigned)(qc + NST) % NST);
        read_b(bn, qc + 1);
#pragma unroll
        for (int i = 0; i < NA; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(af[i], bc[j], acc[i][j]);
            af[i] = read_a(qc + 1, i);
            __builtin_amdgcn_sched_barrier(0);   // each read after its register's last MFMA
        }
        ++qc;
    };
    for (int it = rpos; it < nitems; it += G) {
        const int sp = it / tiles;
        const int kb = sp * per, ke = min(ksteps, (sp + 1) * per);
        if (kb >= ke) continue;
        zero_acc();
        for (int ks = kb; ks < ke; ks += 2) {
            stage(bc, bn);
            if (ks + 1 < ke) {
                stage(bn, bc);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) bc[j] = bn[j];
            }
        }
        epilogue(it);
    }
}

template <int EPI>
int launch_big(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
    if (a.xrows) return PD_EINVAL;   // many-row GEMMs read X rows directly
    if (p.wn == 8)
        hipLaunchKernelGGL((gemm_big_kernel<EPI, 256>), dim3(p.grid), dim3(512), 0, s, a);
    else if (p.wn == 4)
        hipLaunchKernelGGL((gemm_big_kernel<EPI, 128>), dim3(p.grid), dim3(256), 0, s, a);
    else
        return PD_EINVAL;
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

template <int EPI, int NM>
int launch_ring_nm(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
    constexpr int WN = EPI == EPI_SWIGLU ? 2 : 4;
    if (p.wn != WN) return PD_EINVAL;
    // row splits: the LM head on 8 or 2 X tiles, two waves per column group
    if (p.rs != 1 && !(EPI == EPI_ARGMAX && (p.mt == 8 || p.mt == 2) && p.rs == 2)) return PD_EINVAL;
    switch (p.mt) {
        case 1: hipLaunchKernelGGL((gemm_ring_kernel<WN, NM, 1, EPI>), dim3(p.grid), dim3(64 * WN), 0, s, a); break;
        case 2:
            if (p.rs == 2) {
                if constexpr (EPI == EPI_ARGMAX)
                    hipLaunchKernelGGL((gemm_ring_kernel<WN, NM, 2, EPI, kRS, 2>), dim3(p.grid), dim3(128 * WN), 0, s, a);
                else
                    return PD_EINVAL;
            } else {
                hipLaunchKernelGGL((gemm_ring_kernel<WN, NM, 2, EPI>), dim3(p.grid), dim3(64 * WN), 0, s, a);
            }
            break;
        case 4: hipLaunchKernelGGL((gemm_ring_kernel<WN, NM, 4, EPI>), dim3(p.grid), dim3(64 * WN), 0, s, a); break;
        case 8:
            if constexpr (EPI == EPI_ARGMAX && NM == 2) {
                if (p.krs != 64) return PD_EINVAL;
                if (p.rs == 2)
                    hipLaunchKernelGGL((gemm_ring_kernel<WN, 2, 8, EPI_ARGMAX, 64, 2>), dim3(p.grid), dim3(128 * WN), 0,
                                       s, a);
                else
                    hipLaunchKernelGGL((gemm_ring_kernel<WN, 2, 8, EPI_ARGMAX, 64>), dim3(p.grid), dim3(64 * WN), 0, s, a);
                break;
            } else {
                return PD_EINVAL;
            }
        default: return PD_EINVAL;
    }
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

template <int EPI>
int launch_ring(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
    if constexpr (EPI == EPI_SWIGLU) {
        return p.nm == 2 ? launch_ring_nm<EPI, 2>(p, a, s) : PD_EINVAL;
    } else {
        if (p.nm == 1) return launch_ring_nm<EPI, 1>(p, a, s);
        if (p.nm == 2) return launch_ring_nm<EPI, 2>(p, a, s);
        return PD_EINVAL;
    }
}

// weight-only ring (17..64 rows, projections)
template <int EPI>
int launch_wring(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
    if constexpr (EPI == EPI_ARGMAX) {
        return PD_EINVAL;
    } else {
        if (p.mt != 4 || p.nm != 4 || p.grid < p.ntiles * p.splits) return PD_EINVAL;   // one item per workgroup
        hipLaunchKernelGGL((gemm_wring_kernel<EPI, 4>), dim3(p.grid), dim3(256), 0, s, a);
        return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
    }
}

template <int EPI>
int launch_epi(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
    switch (p.kind) {
        case GEMM_RING: return launch_ring<EPI>(p, a, s);
        case GEMM_WRING: return launch_wring<EPI>(p, a, s);
        case GEMM_BIG: return launch_big<EPI>(p, a, s);
        default: return PD_EINVAL;
    }
}

}  // namespace

GemmPlan plan_gemm_nm(int M, int N, int K, int epi, int ring_nm) {
    GemmPlan p;
    p.nm = 1;
    // M <= 64: weight-streaming ring (the LM head up to 128 rows, below).
    // More rows: the ring-fed tile kernel, 128-row tiles below 384 rows,
    // 256-row tiles from there, and for the LM head from 129 rows (measured
    // on the C = 64 step: 192 rows 372 us on 256-row tiles against 432 on
    // 128 x 128 register-staged tiles and 427 on 128-row ones; 320 rows 551
    // against 564 on 128-row tiles).
    p.kind = M <= 64 ? GEMM_RING : GEMM_BIG;
    p.splits = 1;
    p.grid = 0;
    p.krs = kRS;
    if (epi == EPI_ARGMAX && M > 64 && M <= 128) {
        // the LM head at 65..128 rows is still a weight stream (~128 flop per
        // weight byte, below the ridge): the ring with all 8 X tiles, two
        // column groups per wave and 64-element stages (the X rows would
        // otherwise fill the ring); every weight is read once
        p.kind = GEMM_RING;
        p.mt = 8;
        p.mblocks = 1;
        p.wn = 4;
        p.nm = 2;
        p.krs = 64;
        p.rs = kRingLmRowSplit;
        const long items = (N + 127) / 128;
        const long rounds = (items + 255) / 256;
        p.grid = (int)((items + rounds - 1) / rounds);
        p.ntiles = p.grid * p.wn;
        return p;
    }
    if (p.kind == GEMM_BIG) {
        // persistent tiles of bt x bt: 256 (8 waves, one workgroup per CU) from
        // 384 rows on, 128 (4 waves, two workgroups per CU) below; K splits
        // (partial planes, summed by the consumer) chosen to minimise the
        // stages of the busiest of the resident workgroups
        const int bt = (M >= 384 || (epi == EPI_ARGMAX && M > 128)) ? kBT : kBT / 2;
        const long cap = bt == kBT ? 256 : 512;
        p.mt = 0;
        p.wn = bt / 32;
        p.mblocks = (M + bt - 1) / bt;
        const int cols = (epi == EPI_SWIGLU) ? bt / 2 : bt;
        const int ntn = (N + cols - 1) / cols;
        const long tiles = (long)ntn * p.mblocks;
        const int ksteps = (K + kBS - 1) / kBS;
        if (epi == EPI_PARTIAL) p.splits = big_splits(tiles, ksteps, cap, 8);
        p.ntiles = ntn;
        const long items = tiles * p.splits;
        p.grid = (int)(items < cap ? items : cap);
        return p;
    }
    // persistent LDS ring: nm groups of 16 output columns per wave, 4 waves
    // (2 for the gate/up pair, whose two groups are the two matrices); K
    // splits (partial planes) chosen to minimise the stages the busiest of
    // the <= 256 workgroups streams
    p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.mblocks = 1;
    p.wn = (epi == EPI_SWIGLU) ? 2 : 4;
    p.nm = (epi == EPI_SWIGLU) ? 2 : ring_nm;
    const int tw = 16 * p.wn * (epi == EPI_SWIGLU ? 1 : p.nm);
    const int ntn = (N + tw - 1) / tw;
    const int ksteps = (K + kRS - 1) / kRS;
    if (epi == EPI_PARTIAL) {
        long best = -1;
        for (int sp = 1; sp <= 8 && sp <= ksteps; ++sp) {
            const int per = (ksteps + sp - 1) / sp;
            if ((sp - 1) * per >= ksteps) continue;   // no empty split
            const long items = (long)ntn * sp;
            const long span = ((items + 255) / 256) * per;
            if (best < 0 || span < best) { best = span; p.splits = sp; }
        }
    }
    // as few workgroups as keep every round full: the stream is HBM-bound, so
    // a last round with few workgroups runs far below the HBM rate (LM head
    // at C = 1: 3,142 column tiles are 13 rounds of 242, not 12.3 of 256)
    const long items = (long)ntn * p.splits;
    const long rounds = (items + 255) / 256;
    p.grid = (int)((items + rounds - 1) / rounds);
    // LM head: one max/argmax partial per row per wave
    p.ntiles = (epi == EPI_ARGMAX) ? p.grid * p.wn : ntn;
    return p;
}

// Projections of 17..64 rows take two column groups per wave whenever that
// plan still spreads over >= 220 of the 256 CUs: with two or four 16-row X
// tiles the X bytes staged per stage are a large share, and the wider tile
// halves them per weight byte (LM head at 28 rows in the drafting step, 225
// workgroups in 7 full rounds: 175 vs 182 us with the narrow tile). With one
// X tile the deeper ring of the narrow tile is faster (LM head at 7 rows:
// 207 vs 210 us), and so is the narrow tile where the wide one leaves CUs
// idle (the d-wide outputs, whose K splits are capped at 8: 184 workgroups,
// g_c4 step 632 vs 623 us).
// Weight-only ring for the projections of 17..64 rows (see
// gemm_wring_kernel), always with its four X tiles (padding rows read zeros;
// their MFMAs cost nothing in a stream this far below the ridge), one
// workgroup per (column tile, K split) item; K splits chosen as for the ring
// kernel.
static GemmPlan plan_wring(int N, int K, int epi) {
    GemmPlan p;
    p.kind = GEMM_WRING;
    p.mt = 4;
    p.mblocks = 1;
    p.wn = 4;
    p.nm = 4;
    p.krs = kRS;
    p.splits = 1;
    const int tw = epi == EPI_SWIGLU ? 8 * p.nm : 16 * p.nm;
    const int ntn = (N + tw - 1) / tw;
    const int ksteps = (K + kRS - 1) / kRS;
    if (epi == EPI_PARTIAL) {
        long best = -1;
        for (int sp = 1; sp <= 8 && sp <= ksteps; ++sp) {
            const int per = (ksteps + sp - 1) / sp;
            if ((sp - 1) * per >= ksteps) continue;
            const long items = (long)ntn * sp;
            const long span = ((items + 255) / 256) * per;
            if (best < 0 || span < best) { best = span; p.splits = sp; }
        }
    }
    p.grid = ntn * p.splits;
    p.ntiles = ntn;
    return p;
}

GemmPlan plan_gemm(int M, int N, int K, int epi, bool rows_on_device) {
    if (rows_on_device) {
        // the many-row kernel picks its K splits on the device (at most 8
        // planes, or one per K step); the grid covers every resident slot
        GemmPlan p = plan_gemm_nm(M, N, K, epi, 1);
        if (p.kind != GEMM_BIG || epi == EPI_ARGMAX) { p.kind = -1; return p; }
        const int bt = p.wn * 32;
        const long cap = bt == kBT ? 256 : 512;
        const int ksteps = (K + kBS - 1) / kBS;
        p.splits = epi == EPI_PARTIAL ? (ksteps < 8 ? ksteps : 8) : 1;
        const long items = (long)p.ntiles * p.mblocks * p.splits;
        p.grid = (int)(items < cap ? items : cap);
        return p;
    }
    // (the weight-only ring addresses a matrix with 32-bit byte offsets)
    if (M > 16 && M <= 64 && epi != EPI_ARGMAX && (long long)N * K * 2 < (1LL << 31)) return plan_wring(N, K, epi);
    const GemmPlan p = plan_gemm_nm(M, N, K, epi, 1);
    if (p.kind == GEMM_RING && p.mt >= 2 && p.mt <= 4 && epi != EPI_SWIGLU) {
        GemmPlan w = plan_gemm_nm(M, N, K, epi, 2);
        if (w.mt == 2 && epi == EPI_ARGMAX) w.rs = kRingLm2RowSplit;
        if (w.grid >= 220) return w;
    }
    return p;
}

LmHeadPlan plan_lm_head(int M, int N, int K) {
    LmHeadPlan lp;
    lp.main = plan_gemm(M, N, K, EPI_ARGMAX);
    lp.tail = lp.main;
    lp.tail.kind = -1;
    lp.n_main = N;
    lp.ntiles = lp.main.ntiles;
    if (lp.main.kind != GEMM_BIG || lp.main.wn != 8) return lp;
    // one workgroup per CU on 256-row tiles: rounds of 256 tiles (row blocks
    // innermost). With less than half a round left over, the main launch
    // keeps the largest column count whose tiles fill whole rounds (C = 64,
    // K = 7: 1,572 tiles are 6 rounds + 36; the 36 tiles' columns, 4,480 of
    // 201,088, run as 128 x 128 tiles, about a quarter of a round)
    const int mb = lp.main.mblocks, ntn = lp.main.ntiles;
    const long tiles = (long)ntn * mb;
    int g = 256, b = mb;
    while (b) { const int t = g % b; g = b; b = t; }   // gcd(256, mb)
    const int step = 256 / g;                           // column tiles per whole round set
    const int ntn_main = ntn / step * step;
    if (tiles % 256 == 0 || (tiles % 256) * 2 > 256 || ntn_main == 0 || ntn_main >= ntn) return lp;
    lp.n_main = ntn_main * kBT;
    lp.main = plan_gemm(M, lp.n_main, K, EPI_ARGMAX);
    GemmPlan t = lp.main;
    t.kind = GEMM_BIG;
    t.wn = 4;                                           // 128-row tiles, two workgroups per CU
    t.mblocks = (M + kBT / 2 - 1) / (kBT / 2);
    t.ntiles = (N - lp.n_main + kBT / 2 - 1) / (kBT / 2);
    t.splits = 1;
    const long tt = (long)t.ntiles * t.mblocks;
    t.grid = (int)(tt < 512 ? tt : 512);
    lp.tail = t;
    lp.ntiles = lp.main.ntiles + t.ntiles;
    return lp;
}

size_t gemm_ws_floats(const GemmPlan& p, int M, int N, int epi) {
    return epi == EPI_PARTIAL ? (size_t)p.splits * M * N : 0;
}

int launch_gemm(int epi, const GemmPlan& p, GemmArgs a, hipStream_t s) {
    // device row counts: many-row kernel only, not with the max/argmax epilogue
    if ((a.m_dev || a.splits_out) && (p.kind != GEMM_BIG || epi == EPI_ARGMAX)) return PD_EINVAL;
    // column offset / partial stride of a split LM head: many-row kernel only
    if ((a.n_base || a.amax_ld) && (p.kind != GEMM_BIG || epi != EPI_ARGMAX)) return PD_EINVAL;
    if (a.amax_ld && a.amax_ld < p.ntiles) return PD_EINVAL;
    a.splits = p.splits;
    a.ntiles = p.ntiles;
    switch (epi) {
        case EPI_PARTIAL: return launch_epi<EPI_PARTIAL>(p, a, s);
        case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(p, a, s);
        case EPI_ARGMAX: return launch_epi<EPI_ARGMAX>(p, a, s);
        default: return PD_EINVAL;
    }
}

}  // namespace pd
