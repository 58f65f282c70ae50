// bf16 GEMMs of the drafter, Y = X W^T with fp32 accumulation on CDNA4 MFMA.
//
// The drafter's projections (fc 3d->d, QKV, O, gate/up, down, LM head;
// [Paper] = "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training" summary
// page, sec. 2 architecture; [arXiv] = its ScienceStack page, Figure 2) see
// few rows per step: the draft batch has v_r + K - 1 computed rows per
// request and the LM head C*K rows. At low concurrency every projection is a
// stream of its weight matrix, so this kernel is built to stream W at HBM
// speed:
//
//  * a wave owns RG groups of 16 W rows (the A operand of
//    v_mfma_f32_16x16x32_bf16) and up to 64 X rows (the B operand), so each
//    lane ends with 4 consecutive output columns of one row;
//  * in every 128-wide K step, lane group g (lanes 16g..16g+15) takes
//    k = 32j + 8g .. +7 for j = 0..3: each load instruction reads 64
//    contiguous bytes of each of the 16 rows, and 4 such loads per row group
//    are in flight; the next step's W loads are issued before the current
//    step's MFMAs (register double buffering);
//  * a workgroup has WK waves that split its K range; their partial tiles are
//    summed through LDS inside the workgroup;
//  * projections with few output columns are further split over S
//    workgroups along K. Those splits never meet inside this kernel: each
//    writes an fp32 partial plane, and the row kernel that consumes the
//    projection (layer-0 input, RoPE + KV write, residual + RMSNorm) sums the
//    planes in split order. No workgroup ever waits on another, so no
//    device-wide fence is needed, and the result is deterministic.
//  * epilogues: fp32 partial plane, SwiGLU on a pair of matrices (gate and up
//    rows streamed side by side, one bf16 rounding), and LM-head max/argmax per
//    column tile (lowest index on ties) with optional fp32 logits.
#include <float.h>
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pd {

namespace {

constexpr int kU = 4;             // 16-byte loads per lane per row group per K step
constexpr int kKStep = 32 * kU;   // 128 reduction elements per K step

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ void better(float& bv, int& bi, float ov, int oi) {
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

template <int MT, int RG, int WK, int EPI>
__global__ __launch_bounds__(64 * WK) void gemm_stream_kernel(GemmArgs a) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    constexpr int NM = DUAL ? 2 : 1;  // matrices streamed side by side
    const int lane = threadIdx.x & 63, wk = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16 * RG;
    const int m0 = blockIdx.z * 16 * MT;

    // K range of this wave: part (split * WK + wave) of S*WK equal parts, in K steps
    const int ksteps = (a.K + kKStep - 1) / kKStep;
    const int parts = a.splits * WK;
    const int per = (ksteps + parts - 1) / parts;
    const int part = blockIdx.y * WK + wk;
    const int kb = min(a.K, part * per * kKStep);
    const int ke = min(a.K, (part + 1) * per * kKStep);

    f32x4 acc[NM][MT][RG];
#pragma unroll
    for (int q = 0; q < NM; ++q)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < RG; ++r) acc[q][t][r] = f32x4{0.f, 0.f, 0.f, 0.f};

    // operand rows of this lane
    const uint16_t* wp[NM][RG];
    bool rok[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        rok[r] = n0 + 16 * r < a.N;
        const size_t row = (size_t)(rok[r] ? n0 + 16 * r + r16 : 0) * a.K;
        wp[0][r] = a.W + row;
        if constexpr (DUAL) wp[NM - 1][r] = a.W2 + row;
    }
    const uint16_t* xp[MT];
    bool xok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int m = m0 + 16 * t + r16;
        xok[t] = m < a.M;
        int row = m;
        if (xok[t] && a.xrows) {
            row = a.xrows[m];
            if (row < 0 || row >= a.xrows_limit) {
                xok[t] = false;
                flag(a.status, PD_STATUS_BAD_ROW);
            }
        }
        xp[t] = a.X + (size_t)(xok[t] ? row : 0) * a.ldx;
    }

    if (kb < ke) {
        bf16x8 w[NM][RG][kU];
#pragma unroll
        for (int q = 0; q < NM; ++q)
#pragma unroll
            for (int r = 0; r < RG; ++r)
#pragma unroll
                for (int j = 0; j < kU; ++j) {
                    const int k = kb + 32 * j + 8 * g;
                    w[q][r][j] = (rok[r] && k < ke) ? ld_bf16x8(wp[q][r] + k) : zero_bf16x8();
                }
        for (int kk = kb; kk < ke; kk += kKStep) {
            const bool more = kk + kKStep < ke;
            bf16x8 nx[NM][RG][kU];
            if (more) {
#pragma unroll
                for (int q = 0; q < NM; ++q)
#pragma unroll
                    for (int r = 0; r < RG; ++r)
#pragma unroll
                        for (int j = 0; j < kU; ++j) {
                            const int k = kk + kKStep + 32 * j + 8 * g;
                            nx[q][r][j] = (rok[r] && k < ke) ? ld_bf16x8(wp[q][r] + k) : zero_bf16x8();
                        }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                bf16x8 x[kU];
#pragma unroll
                for (int j = 0; j < kU; ++j) {
                    const int k = kk + 32 * j + 8 * g;
                    x[j] = (xok[t] && k < ke) ? ld_bf16x8(xp[t] + k) : zero_bf16x8();
                }
#pragma unroll
                for (int q = 0; q < NM; ++q)
#pragma unroll
                    for (int r = 0; r < RG; ++r)
#pragma unroll
                        for (int j = 0; j < kU; ++j) acc[q][t][r] = mfma_16x16x32(w[q][r][j], x[j], acc[q][t][r]);
            }
            if (more) {
#pragma unroll
                for (int q = 0; q < NM; ++q)
#pragma unroll
                    for (int r = 0; r < RG; ++r)
#pragma unroll
                        for (int j = 0; j < kU; ++j) w[q][r][j] = nx[q][r][j];
            }
        }
    }

    // sum the WK waves' partial tiles through LDS (wave 0 keeps the result)
    if constexpr (WK > 1) {
        __shared__ f32x4 red[WK - 1][NM * MT * RG][64];
        if (wk > 0) {
#pragma unroll
            for (int q = 0; q < NM; ++q)
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int r = 0; r < RG; ++r) red[wk - 1][(q * MT + t) * RG + r][lane] = acc[q][t][r];
        }
        __syncthreads();
        if (wk > 0) return;
        for (int w = 0; w < WK - 1; ++w)
#pragma unroll
            for (int q = 0; q < NM; ++q)
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int r = 0; r < RG; ++r) acc[q][t][r] = acc[q][t][r] + red[w][(q * MT + t) * RG + r][lane];
    }

    // wave 0: lane holds rows m0+16t+r16, columns n0+16r+4g .. +3
    if constexpr (EPI == EPI_ARGMAX) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int m = m0 + 16 * t + r16;
            float bv = -FLT_MAX;
            int bi = INT_MAX;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                if (!rok[r]) continue;
                const int n = n0 + 16 * r + 4 * g;
#pragma unroll
                for (int i = 0; i < 4; ++i) better(bv, bi, acc[0][t][r][i], n + i);
                if (a.logits && m < a.M)
                    *reinterpret_cast<f32x4*>(a.logits + (size_t)m * a.ldlog + n) = acc[0][t][r];
            }
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float ov = __shfl_xor(bv, off, kWave);
                const int oi = __shfl_xor(bi, off, kWave);
                better(bv, bi, ov, oi);
            }
            if (g == 0 && m < a.M) {
                a.amax_v[(size_t)m * a.ntiles + blockIdx.x] = bv;
                a.amax_i[(size_t)m * a.ntiles + blockIdx.x] = bi;
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int m = m0 + 16 * t + r16;
            if (m >= a.M) continue;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                if (!rok[r]) continue;
                const int n = n0 + 16 * r + 4 * g;
                if constexpr (EPI == EPI_PARTIAL) {
                    *reinterpret_cast<f32x4*>(a.ws + ((size_t)blockIdx.y * a.M + m) * a.N + n) = acc[0][t][r];
                } else if constexpr (EPI == EPI_SWIGLU) {
                    float h[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) h[i] = silu(acc[0][t][r][i]) * acc[NM - 1][t][r][i];
                    uint2 pk;
                    pk.x = uint32_t(f2bf(h[0])) | (uint32_t(f2bf(h[1])) << 16);
                    pk.y = uint32_t(f2bf(h[2])) | (uint32_t(f2bf(h[3])) << 16);
                    *reinterpret_cast<uint2*>(a.yb + (size_t)m * a.ldyb + n) = pk;
                }
            }
        }
    }
}

// Row groups of W per wave: fewer when more X rows share the registers.
// ---------------------------------------------------------------------------
// Tiled kernel for many rows (M > 64): a 128 x 128 output tile per workgroup,
// K in steps of 64 staged through LDS (double buffered: the next step's
// global loads are in registers while the current step's MFMAs run), four
// waves each owning a 64 x 64 quarter (4 x 4 MFMA tiles). W is the A operand
// and X the B operand, as in the streaming kernel, so the epilogues are the
// same. For SwiGLU the tile's 128 W rows are 64 gate rows then the same 64 up
// rows, and each wave takes 32 of each: a lane holds matching gate and up
// columns.
constexpr int kTM = 128, kTN = 128, kTK = 64;
constexpr int kTRow = kTK + 8;   // padded LDS row (elements): 144 B stride, conflict-free 16-byte reads

template <int EPI>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmArgs a) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    __shared__ __align__(16) uint16_t ws_[2][kTN * kTRow];
    __shared__ __align__(16) uint16_t xs_[2][kTM * kTRow];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs,
    // so XCD x takes the contiguous tile range [x*chunk, (x+1)*chunk) with the
    // M blocks innermost: the workgroups sharing a W tile run back to back on
    // one XCD and find it in that XCD's L2.
    const int mblocks = (a.M + kTM - 1) / kTM;
    const int total = a.ntiles * mblocks;
    const int chunk = (total + 7) / 8;
    const int tile = (blockIdx.x & 7) * chunk + (blockIdx.x >> 3);
    if (tile >= total) return;
    const int m0 = (tile % mblocks) * kTM;
    // column base of the tile: 128 W rows, or 64 gate + 64 up rows for SwiGLU
    const int ntile = tile / mblocks;
    const int n0 = ntile * (DUAL ? kTN / 2 : kTN);

    // K range of this split (multiples of kTK)
    const int ksteps = (a.K + kTK - 1) / kTK;
    const int per = (ksteps + a.splits - 1) / a.splits;
    const int kb = min(a.K, blockIdx.z * per * kTK);
    const int ke = min(a.K, (blockIdx.z + 1) * per * kTK);

    // staging: each thread moves 4 W and 4 X 16-byte units per K step
    const uint16_t* wsrc[4];
    const uint16_t* xsrc[4];
    bool wok[4], xok[4];
    int soff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int u = tid + 256 * j;
        const int row = u >> 3, c8 = u & 7;
        soff[j] = row * kTRow + c8 * 8;
        int wrow;
        if constexpr (DUAL) {
            wrow = n0 + (row & 63);
            wok[j] = wrow < a.N;
            wsrc[j] = (row < 64 ? a.W : a.W2) + (size_t)(wok[j] ? wrow : 0) * a.K + c8 * 8;
        } else {
            wrow = n0 + row;
            wok[j] = wrow < a.N;
            wsrc[j] = a.W + (size_t)(wok[j] ? wrow : 0) * a.K + c8 * 8;
        }
        const int m = m0 + row;
        xok[j] = m < a.M;
        int xr = m;
        if (xok[j] && a.xrows) {
            xr = a.xrows[m];
            if (xr < 0 || xr >= a.xrows_limit) {
                xok[j] = false;
                flag(a.status, PD_STATUS_BAD_ROW);
            }
        }
        xsrc[j] = a.X + (size_t)(xok[j] ? xr : 0) * a.ldx + c8 * 8;
    }
    uint4 wreg[4], xreg[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = k0 + ((tid + 256 * j) & 7) * 8;
            wreg[j] = (wok[j] && k < ke) ? *reinterpret_cast<const uint4*>(wsrc[j] + k0) : make_uint4(0, 0, 0, 0);
            xreg[j] = (xok[j] && k < ke) ? *reinterpret_cast<const uint4*>(xsrc[j] + k0) : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<uint4*>(&ws_[b][soff[j]]) = wreg[j];
            *reinterpret_cast<uint4*>(&xs_[b][soff[j]]) = xreg[j];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS rows of this wave's A (W) and B (X) fragments
    int wrow_l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        wrow_l[i] = DUAL ? (i < 2 ? 32 * wn + 16 * i : 64 + 32 * wn + 16 * (i - 2)) : 64 * wn + 16 * i;

    if (kb < ke) {
        gload(kb);
        sstore(0);
    }
    __syncthreads();
    int b = 0;
    for (int k0 = kb; k0 < ke; k0 += kTK) {
        const bool more = k0 + kTK < ke;
        if (more) gload(k0 + kTK);
#pragma unroll
        for (int kk = 0; kk < kTK / 32; ++kk) {
            bf16x8 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(&ws_[b][(wrow_l[i] + r16) * kTRow + 32 * kk + 8 * g4]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const bf16x8*>(&xs_[b][(64 * wm + 16 * j + r16) * kTRow + 32 * kk + 8 * g4]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(af[i], bf[j], acc[i][j]);
        }
        if (more) sstore(b ^ 1);
        __syncthreads();
        b ^= 1;
    }

    // lane holds rows m = m0 + 64*wm + 16*j + r16 and 4 consecutive columns per fragment i
    if constexpr (EPI == EPI_ARGMAX) {
        __shared__ float s_v[2][kTM];
        __shared__ int s_i[2][kTM];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ml = 64 * wm + 16 * j + r16;
            const int m = m0 + ml;
            float bv = -FLT_MAX;
            int bi = INT_MAX;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = n0 + 64 * wn + 16 * i + 4 * g4;
                if (n >= a.N) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) better(bv, bi, acc[i][j][e], n + e);
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
        __syncthreads();
        if (tid < kTM) {
            const int m = m0 + tid;
            float bv = s_v[0][tid];
            int bi = s_i[0][tid];
            better(bv, bi, s_v[1][tid], s_i[1][tid]);
            if (m < a.M) {
                a.amax_v[(size_t)m * a.ntiles + ntile] = bv;
                a.amax_i[(size_t)m * a.ntiles + ntile] = bi;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + 64 * wm + 16 * j + r16;
            if (m >= a.M) continue;
            if constexpr (EPI == EPI_PARTIAL) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = n0 + 64 * wn + 16 * i + 4 * g4;
                    if (n < a.N)
                        *reinterpret_cast<f32x4*>(a.ws + ((size_t)blockIdx.z * a.M + m) * a.N + n) = acc[i][j];
                }
            } else {  // SwiGLU: fragments 0,1 = gate, 2,3 = the matching up columns
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int n = n0 + 32 * wn + 16 * i + 4 * g4;
                    if (n >= a.N) continue;
                    float h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[e] = silu(acc[i][j][e]) * acc[i + 2][j][e];
                    uint2 pk;
                    pk.x = uint32_t(f2bf(h[0])) | (uint32_t(f2bf(h[1])) << 16);
                    pk.y = uint32_t(f2bf(h[2])) | (uint32_t(f2bf(h[3])) << 16);
                    *reinterpret_cast<uint2*>(a.yb + (size_t)m * a.ldyb + n) = pk;
                }
            }
        }
    }
}

template <int EPI>
int launch_tiled(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
    const int chunk = (p.ntiles * p.mblocks + 7) / 8;
    hipLaunchKernelGGL(gemm_tiled_kernel<EPI>, dim3(8 * chunk, 1, p.splits), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

template <int MT, int EPI>
constexpr int rows_groups() {
    return EPI == EPI_ARGMAX ? (MT == 1 ? 4 : (MT == 2 ? 2 : 1))
                             : (EPI == EPI_SWIGLU ? (MT == 1 ? 2 : 1) : 1);
}

template <int MT, int EPI>
int launch_cfg(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
    constexpr int RG = rows_groups<MT, EPI>();
    dim3 grid(p.ntiles, p.splits, p.mblocks);
    if (p.rg != RG) return PD_EINVAL;
    if constexpr (EPI == EPI_PARTIAL) {
        if (p.wk == 8) {
            hipLaunchKernelGGL((gemm_stream_kernel<MT, RG, 8, EPI>), grid, dim3(512), 0, s, a);
            return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
        }
    }
    hipLaunchKernelGGL((gemm_stream_kernel<MT, RG, 4, EPI>), grid, dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

template <int EPI>
int launch_epi(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
    if (p.tiled) return launch_tiled<EPI>(p, a, s);
    switch (p.mt) {
        case 1: return launch_cfg<1, EPI>(p, a, s);
        case 2: return launch_cfg<2, EPI>(p, a, s);
        default: return launch_cfg<4, EPI>(p, a, s);
    }
}

}  // namespace

GemmPlan plan_gemm(int M, int N, int K, int epi) {
    GemmPlan p;
    p.tiled = M > 64;
    if (p.tiled) {
        // 128 x 128 tiles; K splits (partial planes, summed by the consumer)
        // only when the tile count leaves most of the 256 CUs idle
        p.mt = 0;
        p.rg = 0;
        p.wk = 4;
        p.mblocks = (M + kTM - 1) / kTM;
        const int cols = (epi == EPI_SWIGLU) ? kTN / 2 : kTN;
        p.ntiles = (N + cols - 1) / cols;
        p.splits = 1;
        if (epi == EPI_PARTIAL) {
            const long tiles = (long)p.ntiles * p.mblocks;
            const int ksteps = (K + kTK - 1) / kTK;
            int s = (int)((512 + tiles - 1) / tiles);
            if (s > 4) s = 4;
            while (s > 1 && s * 4 > ksteps) --s;
            p.splits = s < 1 ? 1 : s;
        }
        return p;
    }
    p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.mblocks = (M + 16 * p.mt - 1) / (16 * p.mt);
    p.rg = p.mt == 1 ? (epi == EPI_ARGMAX ? rows_groups<1, EPI_ARGMAX>() : rows_groups<1, EPI_SWIGLU>())
         : p.mt == 2 ? (epi == EPI_ARGMAX ? rows_groups<2, EPI_ARGMAX>() : rows_groups<2, EPI_SWIGLU>())
                     : (epi == EPI_ARGMAX ? rows_groups<4, EPI_ARGMAX>() : rows_groups<4, EPI_SWIGLU>());
    if (epi == EPI_PARTIAL) p.rg = 1;
    p.wk = 4;
    p.ntiles = (N + 16 * p.rg - 1) / (16 * p.rg);
    p.splits = 1;
    if (epi == EPI_PARTIAL) {
        // 8 waves per workgroup along K, and enough K splits across
        // workgroups for ~6000 waves (short projections are latency-bound)
        p.wk = 8;
        const int ksteps = (K + kKStep - 1) / kKStep;
        const long base = (long)p.ntiles * p.mblocks * p.wk;
        int s = (int)((6000 + base - 1) / base);
        if (s > 8) s = 8;
        while (s > 1 && s * p.wk > ksteps) --s;
        p.splits = s < 1 ? 1 : s;
    }
    return p;
}

size_t gemm_ws_floats(const GemmPlan& p, int M, int N, int epi) {
    return epi == EPI_PARTIAL ? (size_t)p.splits * M * N : 0;
}

int launch_gemm(int epi, const GemmPlan& p, GemmArgs a, hipStream_t s) {
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
