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
// into 16-wide MFMA tiles; each wave carries two such tiles. Per 16-token
// page:
//   S^T(16 keys x 16 queries) = K_page (16 x dh) * Q^T  -- 16x16x32 MFMA,
//       the K page is token-major so a lane's 16-byte load is one key's
//       8 consecutive dims;
//   online softmax per query column (fp32, exp2 domain; the four lane groups
//       of a column are combined with two xor shuffles);
//   O^T(dh x 16 queries) += V^T_page (dh x 16 keys) * P^T -- 16x16x16 MFMA,
//       the S^T accumulator layout is exactly the B-operand layout of this
//       MFMA, and the V page is dim-major so a lane's 8-byte load is one
//       dim's 4 consecutive keys.
// Nothing is transposed through LDS. Each split writes an unnormalized
// partial (O, running max, running sum) per query; a merge kernel combines
// the splits in order (deterministic) and writes bf16 output.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pd {

namespace {

constexpr int kTilesPerWave = 2;
constexpr float kNegInf = -INFINITY;

__device__ __forceinline__ int num_splits(int seq, int nsmax, int min_split) {
    const int ns = (seq + min_split - 1) / min_split;
    return ns < nsmax ? ns : nsmax;
}

__device__ __forceinline__ int split_len(int seq, int ns) {
    const int l = (seq + ns - 1) / ns;
    return (l + PD_PAGE - 1) & ~(PD_PAGE - 1);
}

template <int DH>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
    constexpr int KB = DH / 32;  // 16x16x32 steps over dh for the scores
    constexpr int OT = DH / 16;  // 16-dim output tiles
    const int r = blockIdx.z, g = blockIdx.y, s = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;

    const int row0 = a.cu_out[r], row1 = a.cu_out[r + 1];
    const int seq = a.seq_lens[r];
    if (row0 < 0 || row1 > a.T || row1 < row0 || seq < 1 || seq > a.max_blocks * PD_PAGE) {
        if (s == 0 && g == 0 && threadIdx.x == 0) flag(a.status, PD_STATUS_BAD_ROW);
        return;
    }
    const int ns = num_splits(seq, a.nsmax, a.min_split);
    if (s >= ns) return;
    const int sl = split_len(seq, ns);
    const int kb = s * sl;
    const int ke = min(seq, kb + sl);
    const int G = a.Hq / a.Hkv;
    const int nq = (row1 - row0) * G;
    const int32_t* bt = a.block_table + (size_t)r * a.max_blocks;

    for (int qbase = 0; qbase < nq; qbase += 4 * kTilesPerWave * 16) {
        if (qbase + wave * 16 >= nq) continue;  // this wave has no query here (wave-uniform)
        bf16x8 qv[kTilesPerWave][KB];
        int qpos[kTilesPerWave], qrow[kTilesPerWave], qh[kTilesPerWave];
        bool qok[kTilesPerWave];
        f32x4 o[kTilesPerWave][OT];
        float mrun[kTilesPerWave], lrun[kTilesPerWave];
#pragma unroll
        for (int tt = 0; tt < kTilesPerWave; ++tt) {
            const int qi = qbase + (wave + 4 * tt) * 16 + r16;
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

        for (int p0 = kb; p0 < ke; p0 += PD_PAGE) {
            const int blk = bt[p0 / PD_PAGE];
            if (blk < 0 || blk >= a.num_blocks) {  // uniform across the workgroup
                if (threadIdx.x == 0) flag(a.status, PD_STATUS_BAD_PAGE);
                continue;
            }
            const uint16_t* kp = a.kplane + ((size_t)blk * a.Hkv + g) * PD_PAGE * DH;
            const uint16_t* vp = a.vplane + ((size_t)blk * a.Hkv + g) * PD_PAGE * DH;
            bf16x8 kf[KB];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) kf[kk] = ld_bf16x8(kp + r16 * DH + 32 * kk + 8 * g4);
            s16x4 vf[OT];
#pragma unroll
            for (int j = 0; j < OT; ++j)
                vf[j] = *reinterpret_cast<const s16x4*>(vp + (16 * j + r16) * PD_PAGE + 4 * g4);

#pragma unroll
            for (int tt = 0; tt < kTilesPerWave; ++tt) {
                f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) sc = mfma_16x16x32(kf[kk], qv[tt][kk], sc);
                // lane holds scores of keys p0+4*g4+i for query column r16
                float sv[4];
                float mx = kNegInf;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = p0 + 4 * g4 + i;
                    sv[i] = (t < ke && t <= qpos[tt]) ? sc[i] * a.scale_log2 : kNegInf;
                    mx = fmaxf(mx, sv[i]);
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
                mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
                const float mnew = fmaxf(mrun[tt], mx);
                const float muse = (mnew == kNegInf) ? 0.f : mnew;
                const float alpha = exp2f(mrun[tt] - muse);
                float p[4], ls = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = exp2f(sv[i] - muse);
                    ls += p[i];
                }
                ls += __shfl_xor(ls, 16, kWave);
                ls += __shfl_xor(ls, 32, kWave);
                lrun[tt] = lrun[tt] * alpha + ls;
                mrun[tt] = mnew;
                s16x4 pb;
#pragma unroll
                for (int i = 0; i < 4; ++i) pb[i] = (short)f2bf(p[i]);
#pragma unroll
                for (int j = 0; j < OT; ++j) {
                    o[tt][j] = o[tt][j] * alpha;
                    o[tt][j] = mfma_16x16x16(vf[j], pb, o[tt][j]);
                }
            }
        }

#pragma unroll
        for (int tt = 0; tt < kTilesPerWave; ++tt) {
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

// out[row][h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, splits in order.
template <int DH>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
    const int row = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // request of this row
    int lo = 0, hi = a.C - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu_out[mid] <= row) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int seq = a.seq_lens[r];
    const bool ok = !a.is_rejected[row] && seq >= 1 && seq <= a.max_blocks * PD_PAGE &&
                    a.cu_out[r] <= row && row < a.cu_out[r + 1];
    const int ns = ok ? num_splits(seq, a.nsmax, a.min_split) : 0;
    constexpr int PER = DH / 64;
    for (int h = wave; h < a.Hq; h += 4) {
        float M = kNegInf;
        for (int sp = 0; sp < ns; ++sp)
            M = fmaxf(M, a.part_ml[(((size_t)sp * a.T + row) * a.Hq + h) * 2]);
        float L = 0.f, acc[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = 0.f;
        if (M != kNegInf) {
            for (int sp = 0; sp < ns; ++sp) {
                const size_t base = ((size_t)sp * a.T + row) * a.Hq + h;
                const float w = exp2f(a.part_ml[base * 2] - M);
                L += w * a.part_ml[base * 2 + 1];
#pragma unroll
                for (int i = 0; i < PER; ++i) acc[i] += w * a.part_o[base * DH + lane + 64 * i];
            }
        }
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        uint16_t* op = a.out + ((size_t)row * a.Hq + h) * DH;
#pragma unroll
        for (int i = 0; i < PER; ++i) op[lane + 64 * i] = f2bf(acc[i] * inv);
    }
}

template <int DH>
int launch_dh(const AttnArgs& a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (e0) (void)hipEventRecord(e0, s);
    hipLaunchKernelGGL(attn_split_kernel<DH>, dim3(a.nsmax, a.Hkv, a.C), dim3(256), 0, s, a);
    if (e1) (void)hipEventRecord(e1, s);
    if (hipGetLastError() != hipSuccess) return PD_EHIP;
    hipLaunchKernelGGL(attn_merge_kernel<DH>, dim3(a.T), dim3(256), 0, s, a);
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
