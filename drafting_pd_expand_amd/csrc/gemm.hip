// bf16 GEMMs of the drafter, Y = X W^T with fp32 accumulation on CDNA4 MFMA.
//
// The drafter's projections (fc 3d->d, QKV, O, gate/up, down, LM head;
// [Paper] sec. 2 architecture, [arXiv] Figure 2) run with few rows per step:
// the expanded batch has only v_r + K - 1 computed rows per request and the
// LM head sees C*K rows. At low concurrency every projection is a stream of
// its weight matrix, so this kernel is built around streaming W from HBM:
//
//  * a workgroup is 4 waves; each wave owns 16 rows of W (16 output columns)
//    and multiplies them with up to 64 rows of X using
//    v_mfma_f32_16x16x32_bf16 (W is the A operand, X the B operand, so each
//    lane ends up with 4 consecutive output columns of one row: vector
//    epilogue stores);
//  * the reduction index is permuted per lane: in one 256-wide K step, lane
//    group g (lanes 16g..16g+15) owns k in [64g, 64g+64) and feeds it to the
//    8 MFMAs in 8-element pieces. Both operands use the same permutation, so
//    the sum is unchanged while each lane reads 128 contiguous bytes of its W
//    row -- whole cache lines, 8 x 16-byte loads in flight per lane;
//  * small-N projections split K across workgroups to put >= ~1000
//    workgroups on 256 CUs; partial tiles go to a workspace and the last
//    workgroup to arrive (per-tile counter, agent-scope fences) sums them in
//    split order -- deterministic, and no extra launch;
//  * epilogues: fp32 store, fp32 residual add, bf16 store, SwiGLU on a pair
//    of matrices (gate and up rows read side by side), and LM-head max/argmax
//    per 64-column tile (lowest index on ties) with optional fp32 logits.
#include <float.h>
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pd {

namespace {

constexpr int kU = 8;                 // 16-byte loads per lane per operand per K step
constexpr int kKStep = 32 * kU;       // 256 reduction elements per K step
constexpr int kTileN = 64;            // output columns per workgroup (4 waves x 16)

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

template <int EPI>
__device__ __forceinline__ void epi_apply(const GemmArgs& a, int m, int n, f32x4 v, f32x4 v2) {
    if constexpr (EPI == EPI_STORE_F32) {
        *reinterpret_cast<f32x4*>(a.yf + (size_t)m * a.ldyf + n) = v;
    } else if constexpr (EPI == EPI_RESID_F32) {
        f32x4* p = reinterpret_cast<f32x4*>(a.yf + (size_t)m * a.ldyf + n);
        *p = *p + v;
    } else if constexpr (EPI == EPI_STORE_BF16 || EPI == EPI_SWIGLU) {
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (EPI == EPI_SWIGLU) ? silu(v[i]) * v2[i] : v[i];
        uint2 pk;
        pk.x = uint32_t(f2bf(r[0])) | (uint32_t(f2bf(r[1])) << 16);
        pk.y = uint32_t(f2bf(r[2])) | (uint32_t(f2bf(r[3])) << 16);
        *reinterpret_cast<uint2*>(a.yb + (size_t)m * a.ldyb + n) = pk;
    }
}

__device__ __forceinline__ void better(float& bv, int& bi, float ov, int oi) {
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

template <int MT, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs a) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * kTileN + wave * 16;
    const int m0 = blockIdx.z * (16 * MT);
    const int kbeg = blockIdx.y * a.kper;
    const int kend = min(a.K, kbeg + a.kper);
    const bool wact = n0 < a.N;

    f32x4 acc[MT], acc2[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc2[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // X rows of this lane (B operand column = r16 of each 16-row tile)
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

    if (wact) {
        const uint16_t* wp = a.W + (size_t)(n0 + r16) * a.K;
        const uint16_t* wp2 = DUAL ? a.W2 + (size_t)(n0 + r16) * a.K : nullptr;
        for (int kk = kbeg; kk < kend; kk += kKStep) {
            const int k0 = kk + g * (8 * kU);
            bf16x8 w[kU], w2[DUAL ? kU : 1];
#pragma unroll
            for (int j = 0; j < kU; ++j) {
                const int k = k0 + 8 * j;
                w[j] = k < kend ? ld_bf16x8(wp + k) : zero_bf16x8();
                if constexpr (DUAL) w2[j] = k < kend ? ld_bf16x8(wp2 + k) : zero_bf16x8();
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                bf16x8 x[kU];
#pragma unroll
                for (int j = 0; j < kU; ++j) {
                    const int k = k0 + 8 * j;
                    x[j] = (xok[t] && k < kend) ? ld_bf16x8(xp[t] + k) : zero_bf16x8();
                }
#pragma unroll
                for (int j = 0; j < kU; ++j) {
                    acc[t] = mfma_16x16x32(w[j], x[j], acc[t]);
                    if constexpr (DUAL) acc2[t] = mfma_16x16x32(w2[j], x[j], acc2[t]);
                }
            }
        }
    }

    if constexpr (EPI == EPI_ARGMAX) {
        // one K split only: lane holds logits of row m0+16t+r16, columns n0+4g .. +3
        __shared__ float s_v[4][16 * MT];
        __shared__ int s_i[4][16 * MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int m = m0 + 16 * t + r16;
            float bv = -FLT_MAX;
            int bi = INT_MAX;
            if (wact) {
#pragma unroll
                for (int i = 0; i < 4; ++i) better(bv, bi, acc[t][i], n0 + 4 * g + i);
                if (a.logits && m < a.M)
                    *reinterpret_cast<f32x4*>(a.logits + (size_t)m * a.ldlog + n0 + 4 * g) = acc[t];
            }
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float ov = __shfl_xor(bv, off, kWave);
                const int oi = __shfl_xor(bi, off, kWave);
                better(bv, bi, ov, oi);
            }
            if (g == 0) {
                s_v[wave][16 * t + r16] = bv;
                s_i[wave][16 * t + r16] = bi;
            }
        }
        __syncthreads();
        if (threadIdx.x < 16 * MT) {
            const int m = m0 + threadIdx.x;
            float bv = s_v[0][threadIdx.x];
            int bi = s_i[0][threadIdx.x];
#pragma unroll
            for (int w = 1; w < 4; ++w) better(bv, bi, s_v[w][threadIdx.x], s_i[w][threadIdx.x]);
            if (m < a.M) {
                a.amax_v[(size_t)m * a.ntiles + blockIdx.x] = bv;
                a.amax_i[(size_t)m * a.ntiles + blockIdx.x] = bi;
            }
        }
        return;
    } else {
        if (a.splits == 1) {
            if (wact) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const int m = m0 + 16 * t + r16;
                    if (m < a.M) epi_apply<EPI>(a, m, n0 + 4 * g, acc[t], acc2[t]);
                }
            }
            return;
        }
        // split-K: publish this split's partial tile
        const size_t plane = (size_t)a.splits * a.M * a.N;
        if (wact) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int m = m0 + 16 * t + r16;
                if (m < a.M) {
                    const size_t off = ((size_t)blockIdx.y * a.M + m) * a.N + n0 + 4 * g;
                    *reinterpret_cast<f32x4*>(a.ws + off) = acc[t];
                    if constexpr (DUAL) *reinterpret_cast<f32x4*>(a.ws + plane + off) = acc2[t];
                }
            }
        }
        __shared__ int s_last;
        __threadfence();
        __syncthreads();
        const int tile = blockIdx.z * gridDim.x + blockIdx.x;
        if (threadIdx.x == 0) {
            const int prev = atomicAdd(&a.counters[tile], 1);
            s_last = (prev == a.splits - 1);
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        // last arrival: sum the splits in order, then the epilogue
        const int n = blockIdx.x * kTileN + 4 * (threadIdx.x & 15);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int m = m0 + 16 * t + (threadIdx.x >> 4);
            if (m < a.M && n < a.N) {
                f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f}, s2 = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int sp = 0; sp < a.splits; ++sp) {
                    const size_t off = ((size_t)sp * a.M + m) * a.N + n;
                    s = s + *reinterpret_cast<const f32x4*>(a.ws + off);
                    if constexpr (DUAL) s2 = s2 + *reinterpret_cast<const f32x4*>(a.ws + plane + off);
                }
                epi_apply<EPI>(a, m, n, s, s2);
            }
        }
        if (threadIdx.x == 0) atomicExch(&a.counters[tile], 0);
    }
}

template <int EPI>
int launch_mt(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
    dim3 grid(p.ntiles, p.splits, p.mblocks), block(256);
    switch (p.mt) {
        case 1: hipLaunchKernelGGL((gemm_skinny_kernel<1, EPI>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((gemm_skinny_kernel<2, EPI>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((gemm_skinny_kernel<4, EPI>), grid, block, 0, s, a); break;
    }
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

}  // namespace

GemmPlan plan_gemm(int M, int N, int K, int epi) {
    GemmPlan p;
    p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.mblocks = (M + 16 * p.mt - 1) / (16 * p.mt);
    p.ntiles = (N + kTileN - 1) / kTileN;
    const int tiles = p.ntiles * p.mblocks;
    int splits = 1;
    if (epi != EPI_ARGMAX && tiles < 512) splits = (1024 + tiles - 1) / tiles;
    int ksteps = (K + kKStep - 1) / kKStep;
    if (splits > ksteps) splits = ksteps;
    if (splits < 1) splits = 1;
    const int steps_per = (ksteps + splits - 1) / splits;
    p.kper = steps_per * kKStep;
    p.splits = (K + p.kper - 1) / p.kper;
    if (p.splits < 1) p.splits = 1;
    return p;
}

size_t gemm_ws_floats(const GemmPlan& p, int M, int N, int epi) {
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * M * N * (epi == EPI_SWIGLU ? 2 : 1);
}

int launch_gemm(int epi, const GemmPlan& p, GemmArgs a, hipStream_t s) {
    a.splits = p.splits;
    a.kper = p.kper;
    a.ntiles = p.ntiles;
    switch (epi) {
        case EPI_STORE_F32: return launch_mt<EPI_STORE_F32>(p, a, s);
        case EPI_RESID_F32: return launch_mt<EPI_RESID_F32>(p, a, s);
        case EPI_STORE_BF16: return launch_mt<EPI_STORE_BF16>(p, a, s);
        case EPI_SWIGLU: return launch_mt<EPI_SWIGLU>(p, a, s);
        case EPI_ARGMAX: return launch_mt<EPI_ARGMAX>(p, a, s);
        default: return PD_EINVAL;
    }
}

}  // namespace pd
