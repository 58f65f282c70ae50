// Row-wise kernels of the drafter: RMSNorm, the layer-0 input, RoPE with the
// paged KV write, and the final argmax reduction.
//
// [Blog] = "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding
// in vLLM" (summary page); [Paper] = "P-EAGLE: Parallel-Drafting EAGLE with
// Scalable Training" (summary page); [arXiv] = its ScienceStack page.
//
// One workgroup (256 threads, 4 waves) per row; a row is at most a few tens
// of KB, read once with 16-byte vector loads, reduced in fp32 across the
// block, and written once.
#include <float.h>
#include <limits.h>
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pd {

namespace {

// y[i] = bf16(gamma * x / sqrt(mean(x^2) + eps)); x fp32 row `rows[o]` (or o).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, int ldx, const int32_t* rows,
                                                      int rows_limit, const uint16_t* gamma,
                                                      uint16_t* y, int ldy, int d, float eps,
                                                      int32_t* status) {
    __shared__ float red[4];
    const int o = blockIdx.x;
    int src = o;
    if (rows) {
        src = rows[o];
        if (src < 0 || src >= rows_limit) {
            if (threadIdx.x == 0) flag(status, PD_STATUS_BAD_ROW);
            src = -1;
        }
    }
    uint16_t* yr = y + (size_t)o * ldy;
    if (src < 0) {
        for (int c = threadIdx.x; c < d; c += 256) yr[c] = 0;
        return;
    }
    const float* xr = x + (size_t)src * ldx;
    float ss = 0.f;
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        const float4 v = *reinterpret_cast<const float4*>(xr + c);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = block_sum_256(ss, red);
    const float rs = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        const float4 v = *reinterpret_cast<const float4*>(xr + c);
        const uint2 gb = *reinterpret_cast<const uint2*>(gamma + c);
        uint2 pk;
        pk.x = uint32_t(f2bf(v.x * rs * bf2f(gb.x & 0xffff))) |
               (uint32_t(f2bf(v.y * rs * bf2f(gb.x >> 16))) << 16);
        pk.y = uint32_t(f2bf(v.z * rs * bf2f(gb.y & 0xffff))) |
               (uint32_t(f2bf(v.w * rs * bf2f(gb.y >> 16))) << 16);
        *reinterpret_cast<uint2*>(yr + c) = pk;
    }
}

// Layer-0 input of the drafter ([Blog] Input_i equation, emb (+) hidden):
// u = [RMSNorm(E[id]; g_emb) || RMSNorm(x; g_hid)] with x = fc(hidden) (fp32).
__global__ __launch_bounds__(256) void layer0_input_kernel(const int32_t* ids, const uint16_t* embed,
                                                           int V, const float* x,
                                                           const uint16_t* g_emb,
                                                           const uint16_t* g_hid, uint16_t* u,
                                                           int d, float eps, int32_t* status) {
    __shared__ float red[4];
    const int o = blockIdx.x;
    int id = ids[o];
    if (id < 0 || id >= V) {
        if (threadIdx.x == 0) flag(status, PD_STATUS_BAD_TOKEN);
        id = 0;
    }
    const uint16_t* er = embed + (size_t)id * d;
    const float* xr = x + (size_t)o * d;
    float se = 0.f, sx = 0.f;
    for (int c = threadIdx.x; c < d; c += 256) {
        const float e = bf2f(er[c]);
        const float h = xr[c];
        se += e * e;
        sx += h * h;
    }
    se = block_sum_256(se, red);
    sx = block_sum_256(sx, red);
    const float re = 1.0f / sqrtf(se / (float)d + eps);
    const float rx = 1.0f / sqrtf(sx / (float)d + eps);
    uint16_t* ur = u + (size_t)o * 2 * d;
    for (int c = threadIdx.x; c < d; c += 256) {
        ur[c] = f2bf(bf2f(er[c]) * re * bf2f(g_emb[c]));
        ur[d + c] = f2bf(xr[c] * rx * bf2f(g_hid[c]));
    }
}

// Rotate-half RoPE of q and k at the row's position, then the paged KV write
// at slot_mapping ([Blog] KV-cache paragraph: -1 = rejected, nothing
// written). K pages are token-major [16][dh], V pages dim-major [dh][16].
// The angle pos * theta^(-2i/dh) is formed and reduced in double precision,
// so positions up to 20k keep full fp32 accuracy in cos/sin.
__global__ __launch_bounds__(256) void rope_cache_kernel(const uint16_t* qkv, const int32_t* positions,
                                                         const int32_t* slots, int Hq, int Hkv, int dh,
                                                         float theta, uint16_t* q_out, uint16_t* kplane,
                                                         uint16_t* vplane, int num_blocks,
                                                         int32_t* status) {
    const int o = blockIdx.x;
    const int half = dh / 2;
    const int i = threadIdx.x % half;
    const int grp = threadIdx.x / half;
    const int ngrp = 256 / half;
    const int W = (Hq + 2 * Hkv) * dh;
    const uint16_t* row = qkv + (size_t)o * W;
    const int pos = positions[o];
    const double inv = exp(-(2.0 * i / dh) * log((double)theta));
    double sd, cd;
    sincos((double)pos * inv, &sd, &cd);
    const float c = (float)cd, s = (float)sd;

    for (int h = grp; h < Hq; h += ngrp) {
        const float a = bf2f(row[h * dh + i]);
        const float b = bf2f(row[h * dh + i + half]);
        q_out[(size_t)o * Hq * dh + h * dh + i] = f2bf(a * c - b * s);
        q_out[(size_t)o * Hq * dh + h * dh + i + half] = f2bf(b * c + a * s);
    }
    const int slot = slots[o];
    if (slot < 0) return;  // rejected: no KV write
    if (slot >= num_blocks * PD_PAGE) {
        if (threadIdx.x == 0) flag(status, PD_STATUS_BAD_PAGE);
        return;
    }
    const int blk = slot / PD_PAGE, off = slot % PD_PAGE;
    for (int g = grp; g < Hkv; g += ngrp) {
        const float a = bf2f(row[(Hq + g) * dh + i]);
        const float b = bf2f(row[(Hq + g) * dh + i + half]);
        uint16_t* kp = kplane + ((size_t)blk * Hkv + g) * PD_PAGE * dh + off * dh;
        kp[i] = f2bf(a * c - b * s);
        kp[i + half] = f2bf(b * c + a * s);
    }
    for (int idx = threadIdx.x; idx < Hkv * dh; idx += 256) {
        const int g = idx / dh, cc = idx % dh;
        uint16_t* vp = vplane + ((size_t)blk * Hkv + g) * PD_PAGE * dh;
        vp[cc * PD_PAGE + off] = row[(Hq + Hkv) * dh + idx];
    }
}

__device__ __forceinline__ void better(float& bv, int& bi, float ov, int oi) {
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

// Greedy draft token: argmax over the per-tile (max, index) pairs of one
// row, lowest index on exact ties.
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float* amax_v, const int* amax_i,
                                                            int ntiles, int32_t* out,
                                                            int32_t* status) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int m = blockIdx.x;
    float bv = -FLT_MAX;
    int bi = INT_MAX;
    for (int t = threadIdx.x; t < ntiles; t += 256)
        better(bv, bi, amax_v[(size_t)m * ntiles + t], amax_i[(size_t)m * ntiles + t]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        better(bv, bi, ov, oi);
    }
    if ((threadIdx.x & 63) == 0) {
        sv[threadIdx.x >> 6] = bv;
        si[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float v = sv[0];
        int ix = si[0];
        for (int w = 1; w < 4; ++w) better(v, ix, sv[w], si[w]);
        if (ix == INT_MAX) {
            flag(status, PD_STATUS_BAD_ROW);
            ix = 0;
        }
        out[m] = ix;
    }
}

}  // namespace

int launch_rmsnorm(const float* x, int ldx, const int32_t* rows, int rows_limit, int nrows,
                   const uint16_t* gamma, uint16_t* y, int ldy, int d, float eps,
                   int32_t* status, hipStream_t s) {
    if (nrows <= 0) return PD_OK;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(nrows), dim3(256), 0, s, x, ldx, rows, rows_limit,
                       gamma, y, ldy, d, eps, status);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_layer0_input(const int32_t* ids, const uint16_t* embed, int V, const float* x,
                        const uint16_t* g_emb, const uint16_t* g_hid, uint16_t* u, int T, int d,
                        float eps, int32_t* status, hipStream_t s) {
    if (T <= 0) return PD_OK;
    hipLaunchKernelGGL(layer0_input_kernel, dim3(T), dim3(256), 0, s, ids, embed, V, x, g_emb,
                       g_hid, u, d, eps, status);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_rope_cache(const uint16_t* qkv, const int32_t* positions, const int32_t* slots, int T,
                      int Hq, int Hkv, int dh, float theta, uint16_t* q_out, uint16_t* kplane,
                      uint16_t* vplane, int num_blocks, int32_t* status, hipStream_t s) {
    if (T <= 0) return PD_OK;
    hipLaunchKernelGGL(rope_cache_kernel, dim3(T), dim3(256), 0, s, qkv, positions, slots, Hq,
                       Hkv, dh, theta, q_out, kplane, vplane, num_blocks, status);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_argmax_reduce(const float* amax_v, const int* amax_i, int M, int ntiles, int32_t* out,
                         int32_t* status, hipStream_t s) {
    if (M <= 0) return PD_OK;
    hipLaunchKernelGGL(argmax_reduce_kernel, dim3(M), dim3(256), 0, s, amax_v, amax_i, ntiles,
                       out, status);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

}  // namespace pd
