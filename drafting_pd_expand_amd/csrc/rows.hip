// Row-wise kernels of the drafter: residual + RMSNorm, the layer-0 input, RoPE
// with the paged KV write, and the final argmax reduction. Each one also
// finishes the projection that feeds it by summing its split-K planes.
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

#include <cstring>

#include "attn_plan.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace pd {

namespace {

constexpr int kMaxSplits = 8;   // split-K planes a projection may leave behind

__device__ __forceinline__ void add4(float4& a, const float4& b) {
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    uint2 pk;
    pk.x = uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16);
    pk.y = uint32_t(f2bf(c)) | (uint32_t(f2bf(d)) << 16);
    return pk;
}

// Row chunks of 4 floats per thread: NC = ceil(d / 1024) <= 4 (d <= 4096).
// All loads of a row (x and every split plane) are issued before any is used.
template <int NC>
__device__ __forceinline__ void load_row_sum(float4 (&v)[NC], const float* xr, const float* ws,
                                             int S, size_t plane, size_t rowoff, int d, bool from_x) {
    float4 p[kMaxSplits][NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = threadIdx.x * 4 + 1024 * n;
        v[n] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < d && from_x) v[n] = *reinterpret_cast<const float4*>(xr + c);
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
            if (sp < S && c < d) p[sp][n] = *reinterpret_cast<const float4*>(ws + sp * plane + rowoff + c);
    }
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp)
#pragma unroll
        for (int n = 0; n < NC; ++n)
            if (sp < S) add4(v[n], p[sp][n]);
}

// Residual stream update and the next RMSNorm, one row per workgroup:
// x += sum_s ws[s] (the projection's split planes, in order), then
// y = bf16(gamma * x / sqrt(mean(x^2) + eps)). With a row list, output row o
// is the norm of row rows[o] (the rows the LM head samples, packed) and x is
// left as it is; a list entry outside [0, T) is flagged and gives a zero row.
// xout (row-list mode): also the row's residual itself, bf16 (the drafter's
// final hidden state, fed back by autoregressive passes).
template <int NC>
__global__ __launch_bounds__(256) void resid_norm_kernel(const float* ws, int S, float* x,
                                                         const uint16_t* gamma, uint16_t* y, int T,
                                                         int d, float eps, const int32_t* rows,
                                                         int32_t* status, uint16_t* xout, const int32_t* t_dev,
                                                         const int32_t* s_dev) {
    __shared__ float red[4];
    const int o = blockIdx.x;
    if (!rows && t_dev && o >= *t_dev) return;   // past the rows present (whole workgroup)
    if (s_dev) S = *s_dev;                       // planes the projection chose on the device
    int i = o;
    bool ok = true;
    if (rows) {
        i = rows[o];
        if (i < 0 || i >= T) {
            if (threadIdx.x == 0) flag(status, PD_STATUS_BAD_ROW);
            ok = false;
            i = 0;
        }
    }
    float* xr = x + (size_t)i * d;
    float4 v[NC];
    load_row_sum<NC>(v, xr, ws, S, (size_t)T * d, (size_t)i * d, d, true);
    uint2 gb[NC];
    float ss = 0.f;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = threadIdx.x * 4 + 1024 * n;
        if (c < d) {
            gb[n] = *reinterpret_cast<const uint2*>(gamma + c);
            if (S > 0 && !rows) *reinterpret_cast<float4*>(xr + c) = v[n];
            if (xout)   // the row's residual itself (bf16), before the norm
                *reinterpret_cast<uint2*>(xout + (size_t)o * d + c) =
                    pack4(ok ? v[n].x : 0.f, ok ? v[n].y : 0.f, ok ? v[n].z : 0.f, ok ? v[n].w : 0.f);
            ss += v[n].x * v[n].x + v[n].y * v[n].y + v[n].z * v[n].z + v[n].w * v[n].w;
        }
    }
    ss = block_sum_256(ss, red);
    const float rs = ok ? 1.0f / sqrtf(ss / (float)d + eps) : 0.f;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = threadIdx.x * 4 + 1024 * n;
        if (c < d)
            *reinterpret_cast<uint2*>(y + (size_t)o * d + c) =
                pack4(v[n].x * rs * bf2f(gb[n].x & 0xffff), v[n].y * rs * bf2f(gb[n].x >> 16),
                      v[n].z * rs * bf2f(gb[n].y & 0xffff), v[n].w * rs * bf2f(gb[n].y >> 16));
    }
}

// Layer-0 input of the drafter ([Blog] Input_i equation, emb (+) hidden):
// x = fc(hidden) = sum of the fc projection's split planes (starts the
// residual stream), u = [RMSNorm(E[id]; g_emb) || RMSNorm(x; g_hid)].
template <int NC>
__global__ __launch_bounds__(256) void layer0_input_kernel(const float* ws, int S, const int32_t* ids,
                                                           const uint16_t* embed, int V, float* x,
                                                           const uint16_t* g_emb,
                                                           const uint16_t* g_hid, uint16_t* u, int T,
                                                           int d, float eps, int32_t* status,
                                                           const uint16_t* xin, AttnArgs plan, int with_plan,
                                                           const int32_t* t_dev, const int32_t* s_dev) {
    __shared__ float red[4];
    if (with_plan && blockIdx.x == 0) {   // the attention split plan, beside the rows
        attn_plan_block(plan);
        return;
    }
    const int o = blockIdx.x - with_plan;
    if (t_dev && o >= *t_dev) return;   // past the rows present (whole workgroup)
    if (s_dev) S = *s_dev;
    int id = ids[o];
    if (id < 0 || id >= V) {
        if (threadIdx.x == 0) flag(status, PD_STATUS_BAD_TOKEN);
        id = 0;
    }
    const uint16_t* er = embed + (size_t)id * d;
    float* xr = x + (size_t)o * d;
    float4 v[NC];
    uint2 eb[NC], ge[NC], gh[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = threadIdx.x * 4 + 1024 * n;
        if (c < d) {
            eb[n] = *reinterpret_cast<const uint2*>(er + c);
            ge[n] = *reinterpret_cast<const uint2*>(g_emb + c);
            gh[n] = *reinterpret_cast<const uint2*>(g_hid + c);
        }
    }
    if (xin) {   // the projected hidden row given directly (bf16, d wide)
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const int c = threadIdx.x * 4 + 1024 * n;
            v[n] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < d) {
                const uint2 hb = *reinterpret_cast<const uint2*>(xin + (size_t)o * d + c);
                v[n] = make_float4(bf2f(hb.x & 0xffff), bf2f(hb.x >> 16), bf2f(hb.y & 0xffff), bf2f(hb.y >> 16));
            }
        }
    } else {
        load_row_sum<NC>(v, xr, ws, S, (size_t)T * d, (size_t)o * d, d, false);
    }
    float se = 0.f, sx = 0.f;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = threadIdx.x * 4 + 1024 * n;
        if (c < d) {
            *reinterpret_cast<float4*>(xr + c) = v[n];
            const float e0 = bf2f(eb[n].x & 0xffff), e1 = bf2f(eb[n].x >> 16);
            const float e2 = bf2f(eb[n].y & 0xffff), e3 = bf2f(eb[n].y >> 16);
            se += e0 * e0 + e1 * e1 + e2 * e2 + e3 * e3;
            sx += v[n].x * v[n].x + v[n].y * v[n].y + v[n].z * v[n].z + v[n].w * v[n].w;
        }
    }
    se = block_sum_256(se, red);
    sx = block_sum_256(sx, red);
    const float re = 1.0f / sqrtf(se / (float)d + eps);
    const float rx = 1.0f / sqrtf(sx / (float)d + eps);
    uint16_t* ur = u + (size_t)o * 2 * d;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = threadIdx.x * 4 + 1024 * n;
        if (c < d) {
            *reinterpret_cast<uint2*>(ur + c) =
                pack4(bf2f(eb[n].x & 0xffff) * re * bf2f(ge[n].x & 0xffff),
                      bf2f(eb[n].x >> 16) * re * bf2f(ge[n].x >> 16),
                      bf2f(eb[n].y & 0xffff) * re * bf2f(ge[n].y & 0xffff),
                      bf2f(eb[n].y >> 16) * re * bf2f(ge[n].y >> 16));
            *reinterpret_cast<uint2*>(ur + d + c) =
                pack4(v[n].x * rx * bf2f(gh[n].x & 0xffff), v[n].y * rx * bf2f(gh[n].x >> 16),
                      v[n].z * rx * bf2f(gh[n].y & 0xffff), v[n].w * rx * bf2f(gh[n].y >> 16));
        }
    }
}

// Rotate-half RoPE of q and k at the row's position, then the paged KV write
// at slot_mapping ([Blog] KV-cache paragraph: -1 = rejected, nothing
// written). The QKV projection arrives as fp32 split planes and is rounded to
// bf16 once, after the rotation. One thread per rotation pair (or V element),
// so every thread's loads go out together. K pages are token-major [16][dh],
// V pages dim-major [dh][16]. The angle pos * theta^(-2i/dh) is formed and
// reduced to [-pi, pi] in double precision (theta^(-2/dh) comes from the
// host, its i-th power by repeated squaring: <= 12 double products, ~1e-15
// relative; the reduction subtracts k * 2pi in two parts, Cody and Waite's
// method), so positions up to 20k keep full fp32 accuracy in cos/sin, which
// are then taken in fp32 on the reduced angle.
// fp8 cache: the E4M3 code of x / scale, nearest with ties to even (the
// hardware conversion), saturated to +-448
__device__ __forceinline__ uint8_t to_e4m3(float x, float scale) {
    const float y = fminf(fmaxf(x / scale, -448.0f), 448.0f);
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xff);
}

__global__ __launch_bounds__(256) void rope_cache_kernel(const float* ws, int S, const int32_t* positions,
                                                         const int32_t* slots, int T, int Hq, int Hkv,
                                                         int dh, double inv_step, uint16_t* q_out,
                                                         void* kplane, void* vplane,
                                                         int num_blocks, int32_t* status, int fp8,
                                                         float k_scale, float v_scale, const int32_t* t_dev,
                                                         const int32_t* s_dev) {
    const int o = blockIdx.y;
    if (t_dev && o >= *t_dev) return;   // past the rows present (whole workgroup)
    if (s_dev) S = *s_dev;
    const int half = dh / 2;
    const int npairs = (Hq + Hkv) * half;          // rotated pairs (q heads, then k heads)
    const int item = blockIdx.x * 256 + threadIdx.x;
    if (item >= npairs + Hkv * dh) return;
    const int W = (Hq + 2 * Hkv) * dh;
    const size_t plane = (size_t)T * W;
    const float* row = ws + (size_t)o * W;
    const int slot = slots[o];
    const bool write = slot >= 0 && slot < num_blocks * PD_PAGE;
    if (slot >= num_blocks * PD_PAGE && item == 0) flag(status, PD_STATUS_BAD_PAGE);
    const int blk = slot / PD_PAGE, off = slot % PD_PAGE;
    if (item < npairs) {
        const int h = item / half, i = item % half;   // h < Hq: q head, else k head h - Hq
        const int c0 = h * dh + i;
        float a = 0.f, b = 0.f, pa[kMaxSplits], pb[kMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
            if (sp < S) {
                pa[sp] = row[sp * plane + c0];
                pb[sp] = row[sp * plane + c0 + half];
            }
        const int pos = positions[o];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
            if (sp < S) { a += pa[sp]; b += pb[sp]; }
        double inv = 1.0, pw = inv_step;   // inv_step^i = theta^(-2i/dh)
        for (int e = i; e != 0; e >>= 1) {
            if (e & 1) inv *= pw;
            pw *= pw;
        }
        const double ang = (double)pos * inv;
        const double kq = rint(ang * 0.15915494309189535);             // 1 / (2 pi)
        double red = fma(-kq, 6.283185307179586, ang);                  // 2 pi, leading part
        red = fma(-kq, 2.4492935982947064e-16, red);                     // 2 pi, remainder
        float s, c;
        sincosf((float)red, &s, &c);
        const float x0 = a * c - b * s, x1 = b * c + a * s;
        if (h < Hq) {
            q_out[(size_t)o * Hq * dh + c0] = f2bf(x0);
            q_out[(size_t)o * Hq * dh + c0 + half] = f2bf(x1);
        } else if (write) {
            const size_t e = ((size_t)blk * Hkv + (h - Hq)) * PD_PAGE * dh + off * dh;
            if (fp8) {
                uint8_t* kp = static_cast<uint8_t*>(kplane) + e;
                kp[i] = to_e4m3(x0, k_scale);
                kp[i + half] = to_e4m3(x1, k_scale);
            } else {
                uint16_t* kp = static_cast<uint16_t*>(kplane) + e;
                kp[i] = f2bf(x0);
                kp[i + half] = f2bf(x1);
            }
        }
    } else if (write) {
        const int idx = item - npairs;                 // V element: head idx / dh, dim idx % dh
        float v = 0.f, pv[kMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
            if (sp < S) pv[sp] = row[sp * plane + (Hq + Hkv) * dh + idx];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
            if (sp < S) v += pv[sp];
        const int g = idx / dh, cc = idx % dh;
        const size_t e = ((size_t)blk * Hkv + g) * PD_PAGE * dh + cc * PD_PAGE + off;
        if (fp8) static_cast<uint8_t*>(vplane)[e] = to_e4m3(v, v_scale);
        else static_cast<uint16_t*>(vplane)[e] = f2bf(v);
    }
}

__device__ __forceinline__ void better(float& bv, int& bi, float ov, int oi) {
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

// Greedy draft token: argmax over the per-tile (max, index) pairs of one
// row, lowest index on exact ties.
__global__ __launch_bounds__(1024) void argmax_reduce_kernel(const float* amax_v, const int* amax_i,
                                                             int ntiles, int32_t* out,
                                                             int32_t* status) {
    __shared__ float sv[16];
    __shared__ int si[16];
    const int m = blockIdx.x;
    float bv = -FLT_MAX;
    int bi = INT_MAX;
    // a row's partials (a few thousand at most) in one round of independent loads per thread
#pragma unroll 16
    for (int t = threadIdx.x; t < ntiles; t += 1024)
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
        for (int w = 1; w < 16; ++w) better(v, ix, sv[w], si[w]);
        if (ix == INT_MAX) {
            flag(status, PD_STATUS_BAD_ROW);
            ix = 0;
        }
        out[m] = ix;
    }
}

// Row compaction (see launch_compact_rows). Workgroup 0: the kept-row
// prefix over all T rows (each thread a run of ceil(T / 256) rows, one block
// scan), then the compacted request starts, sampled-row indices and the kept
// count. Workgroup 1 + i: row i, if kept: its index (the kept rows before it,
// counted by the whole block), metadata and hidden-row copy (16-byte loads).
__global__ __launch_bounds__(256) void compact_rows_kernel(
    const uint8_t* is_rejected, const int32_t* ids, const int32_t* positions, const int32_t* slots,
    const int32_t* cu_out, const int32_t* nti, const uint16_t* hidden, int T, int C, int R, int h3,
    uint16_t* hid_c, int32_t* ids_c, int32_t* pos_c, int32_t* slot_c, int32_t* cu_c, int32_t* nti_c,
    int32_t* rowmap, int32_t* t_eff, int32_t* status) {
    __shared__ int s_pre[kCompactMaxRows + 1];
    __shared__ int s_w[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (blockIdx.x == 0) {
        const int per = (T + 255) / 256;   // <= 16 rows per thread
        const int r0 = min(T, tid * per), r1 = min(T, r0 + per);
        int cnt = 0;
        unsigned keep = 0;   // bit i - r0: row i kept
        for (int i = r0; i < r1; ++i) {
            const unsigned k = is_rejected[i] == 0;
            keep |= k << (i - r0);
            cnt += (int)k;
        }
        // exclusive prefix of the per-thread counts over the block
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += t;
        }
        if (lane == 63) s_w[w] = incl;
        __syncthreads();
        int run = incl - cnt;
        for (int k = 0; k < w; ++k) run += s_w[k];
        for (int i = r0; i < r1; ++i) {
            s_pre[i] = run;
            run += (int)((keep >> (i - r0)) & 1u);
        }
        if (tid == 255) s_pre[T] = run;   // (the last thread's run ends at T: per * 256 >= T)
        __syncthreads();
        if (tid == 0) t_eff[0] = s_pre[T];
        for (int r = tid; r <= C; r += 256) {
            const int c0 = cu_out[r];
            // request starts as the attention plan checks them: 0 <= start <= T, non-decreasing
            if (c0 < 0 || c0 > T || (r < C && cu_out[r + 1] < c0)) flag(status, PD_STATUS_BAD_ROW);
            cu_c[r] = s_pre[min(max(c0, 0), T)];
        }
        for (int j = tid; j < R; j += 256) {
            const int row = nti[j];
            const bool ok = row >= 0 && row < T;
            if (!ok) flag(status, PD_STATUS_BAD_ROW);
            // a rejected sampled row (a padding request's) has no defined
            // draft: it takes compacted row 0 (kept rows: s_pre steps there)
            nti_c[j] = (ok && s_pre[row + 1] != s_pre[row]) ? s_pre[row] : 0;
        }
        return;
    }
    const int i = blockIdx.x - 1;
    if (is_rejected[i] != 0) return;   // whole workgroup
    // the row's loads go out first (they do not depend on its index c), then
    // the count of kept rows before it, then the stores (a load-store loop
    // would wait out one memory round trip per iteration: the compiler cannot
    // tell the two rows apart); h3 <= 16384: at most 8 chunks per thread
    const uint4* src = reinterpret_cast<const uint4*>(hidden + (size_t)i * h3);
    constexpr int kMaxChunks = 8;
    uint4 buf[kMaxChunks];
#pragma unroll
    for (int j = 0; j < kMaxChunks; ++j)
        if (j * 256 + tid < h3 / 8) buf[j] = src[j * 256 + tid];
    int meta[3] = {0, 0, 0};
    if (tid == 0) {
        meta[0] = ids[i];
        meta[1] = positions[i];
        meta[2] = slots[i];
    }
    int cnt = 0;
    for (int j = tid; j < i; j += 256) cnt += is_rejected[j] == 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, kWave);
    if (lane == 0) s_w[w] = cnt;
    __syncthreads();
    const int c = s_w[0] + s_w[1] + s_w[2] + s_w[3];
    if (tid == 0) {
        rowmap[c] = i;
        ids_c[c] = meta[0];
        pos_c[c] = meta[1];
        slot_c[c] = meta[2];
    }
    uint4* dst = reinterpret_cast<uint4*>(hid_c + (size_t)c * h3);
#pragma unroll
    for (int j = 0; j < kMaxChunks; ++j)
        if (j * 256 + tid < h3 / 8) dst[j * 256 + tid] = buf[j];
}

// dst[rowmap[c]] = src[c], c < t_eff (one workgroup per compacted row)
__global__ __launch_bounds__(256) void scatter_rows_kernel(const float* src, float* dst, const int32_t* rowmap,
                                                           const int32_t* t_eff, int T, int d) {
    const int c = blockIdx.x;
    if (c >= t_eff[0]) return;
    const int i = rowmap[c];
    if (i < 0 || i >= T) return;
    for (int k = threadIdx.x; k < d; k += 256) dst[(size_t)i * d + k] = src[(size_t)c * d + k];
}

}  // namespace

#define PD_ROW_NC(d, launch) \
    switch (((d) + 1023) / 1024) {      \
        case 1: launch(1); break;       \
        case 2: launch(2); break;       \
        case 3: launch(3); break;       \
        case 4: launch(4); break;       \
        default: return PD_EINVAL;      \
    }

int launch_resid_norm(const float* ws, int S, float* x, const uint16_t* gamma, uint16_t* y, int T,
                      int d, float eps, hipStream_t s, const int32_t* rows, int nrows, int32_t* status,
                      uint16_t* xout, const int32_t* t_dev, const int32_t* s_dev) {
    const int nout = rows ? nrows : T;
    if (nout <= 0) return PD_OK;
    if (S > kMaxSplits) return PD_EINVAL;
#define L_(NC) hipLaunchKernelGGL(resid_norm_kernel<NC>, dim3(nout), dim3(256), 0, s, ws, S, x, gamma, y, T, d, \
                                  eps, rows, status, xout, t_dev, s_dev)
    PD_ROW_NC(d, L_)
#undef L_
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_layer0_input(const uint16_t* xin, const float* ws, int S, const int32_t* ids, const uint16_t* embed, int V,
                        float* x, const uint16_t* g_emb, const uint16_t* g_hid, uint16_t* u, int T,
                        int d, float eps, int32_t* status, hipStream_t s, const AttnArgs* plan,
                        const int32_t* t_dev, const int32_t* s_dev) {
    if (T <= 0) return PD_OK;
    if (S > kMaxSplits) return PD_EINVAL;
    AttnArgs pa;
    if (plan) pa = *plan;
    else std::memset(&pa, 0, sizeof(pa));
    const int wp = (plan && plan->C > 0) ? 1 : 0;
#define L_(NC) hipLaunchKernelGGL(layer0_input_kernel<NC>, dim3(T + wp), dim3(256), 0, s, ws, S, ids, embed, V, \
                                  x, g_emb, g_hid, u, T, d, eps, status, xin, pa, wp, t_dev, s_dev)
    PD_ROW_NC(d, L_)
#undef L_
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_rope_cache(const float* ws, int S, const int32_t* positions, const int32_t* slots, int T,
                      int Hq, int Hkv, int dh, float theta, uint16_t* q_out, void* kplane,
                      void* vplane, int num_blocks, int32_t* status, hipStream_t s, int fp8,
                      float k_scale, float v_scale, const int32_t* t_dev, const int32_t* s_dev) {
    if (T <= 0) return PD_OK;
    if (S > kMaxSplits) return PD_EINVAL;
    const int items = (Hq + Hkv) * (dh / 2) + Hkv * dh;
    const double inv_step = std::pow((double)theta, -2.0 / dh);
    hipLaunchKernelGGL(rope_cache_kernel, dim3((items + 255) / 256, T), dim3(256), 0, s, ws, S,
                       positions, slots, T, Hq, Hkv, dh, inv_step, q_out, kplane, vplane, num_blocks,
                       status, fp8, k_scale, v_scale, t_dev, s_dev);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_compact_rows(const uint8_t* is_rejected, const int32_t* ids, const int32_t* positions,
                        const int32_t* slots, const int32_t* cu_out, const int32_t* nti,
                        const uint16_t* hidden, int T, int C, int R, int h3, uint16_t* hid_c,
                        int32_t* ids_c, int32_t* pos_c, int32_t* slot_c, int32_t* cu_c, int32_t* nti_c,
                        int32_t* rowmap, int32_t* t_eff, int32_t* status, hipStream_t s) {
    if (T <= 0 || T > kCompactMaxRows || h3 % 8 || h3 > 8 * 256 * 8 || C < 0 || R < 0) return PD_EINVAL;
    if (((uintptr_t)hidden | (uintptr_t)hid_c) & 15) return PD_EINVAL;   // 16-byte row copies
    hipLaunchKernelGGL(compact_rows_kernel, dim3(T + 1), dim3(256), 0, s, is_rejected, ids, positions, slots,
                       cu_out, nti, hidden, T, C, R, h3, hid_c, ids_c, pos_c, slot_c, cu_c, nti_c, rowmap,
                       t_eff, status);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_scatter_rows(const float* src, float* dst, const int32_t* rowmap, const int32_t* t_eff, int T, int d,
                        hipStream_t s) {
    if (T <= 0) return PD_OK;
    hipLaunchKernelGGL(scatter_rows_kernel, dim3(T), dim3(256), 0, s, src, dst, rowmap, t_eff, T, d);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_argmax_reduce(const float* amax_v, const int* amax_i, int M, int ntiles, int32_t* out,
                         int32_t* status, hipStream_t s) {
    if (M <= 0) return PD_OK;
    hipLaunchKernelGGL(argmax_reduce_kernel, dim3(M), dim3(1024), 0, s, amax_v, amax_i, ntiles,
                       out, status);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

}  // namespace pd
