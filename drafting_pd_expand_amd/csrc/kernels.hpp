// Internal launchers shared between the kernel files and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pd.h"

namespace pd {

// ---------------------------------------------------------------- expansion
int launch_expand(const pd_batch_dims& d, const pd_expand_in& in, const pd_batch& out,
                  hipStream_t s);

// ---------------------------------------------------------------- GEMM
enum Epi : int {
    EPI_STORE_F32 = 0,  // y_f32 = acc
    EPI_RESID_F32 = 1,  // y_f32 += acc (residual stream)
    EPI_STORE_BF16 = 2, // y_bf16 = acc
    EPI_SWIGLU = 3,     // y_bf16 = silu(X W^T) * (X W2^T)
    EPI_ARGMAX = 4,     // per (row, 64-column tile) max / argmax (+ optional fp32 logits)
};

struct GemmArgs {
    const uint16_t* X;       // bf16 [rows][ldx]
    int ldx;
    const int32_t* xrows;    // optional gather: GEMM row m reads X row xrows[m]
    int xrows_limit;         // rows of X (bound for xrows entries)
    const uint16_t* W;       // bf16 [N][K]
    const uint16_t* W2;      // second matrix for EPI_SWIGLU
    int M, N, K;
    int splits, kper;        // split-K: split s covers k in [s*kper, min(K, (s+1)*kper))
    float* ws;               // split-K partials [splits][M][N] (x2 planes for SWIGLU)
    int* counters;           // per output tile arrival counters (all zero between launches)
    float* yf; int ldyf;
    uint16_t* yb; int ldyb;
    float* logits; int ldlog;
    float* amax_v; int* amax_i; int ntiles;
    int32_t* status;
};

struct GemmPlan {
    int mt;        // 16-row MFMA tiles per workgroup (1, 2 or 4)
    int mblocks;   // workgroups along M
    int ntiles;    // 64-column tiles along N
    int splits;
    int kper;
};

GemmPlan plan_gemm(int M, int N, int K, int epi);
size_t gemm_ws_floats(const GemmPlan& p, int M, int N, int epi);
int launch_gemm(int epi, const GemmPlan& p, GemmArgs a, hipStream_t s);

// ---------------------------------------------------------------- row kernels
int launch_rmsnorm(const float* x, int ldx, const int32_t* rows, int rows_limit, int nrows,
                   const uint16_t* gamma, uint16_t* y, int ldy, int d, float eps,
                   int32_t* status, hipStream_t s);
int launch_layer0_input(const int32_t* ids, const uint16_t* embed, int V, const float* x,
                        const uint16_t* g_emb, const uint16_t* g_hid, uint16_t* u, int T, int d,
                        float eps, int32_t* status, hipStream_t s);
int launch_rope_cache(const uint16_t* qkv, const int32_t* positions, const int32_t* slots, int T,
                      int Hq, int Hkv, int dh, float theta, uint16_t* q_out, uint16_t* kplane,
                      uint16_t* vplane, int num_blocks, int32_t* status, hipStream_t s);
int launch_argmax_reduce(const float* amax_v, const int* amax_i, int M, int ntiles, int32_t* out,
                         int32_t* status, hipStream_t s);

// ---------------------------------------------------------------- attention
struct AttnArgs {
    const uint16_t* q;            // bf16 [T][Hq][dh] (rotated)
    const uint16_t* kplane;       // this layer's K plane [num_blocks][Hkv][16][dh]
    const uint16_t* vplane;       // this layer's V plane [num_blocks][Hkv][dh][16]
    const int32_t* positions;
    const uint8_t* is_rejected;
    const int32_t* cu_out;        // [C+1]
    const int32_t* seq_lens;      // [C]
    const int32_t* block_table;   // [C][max_blocks]
    int C, T, Hq, Hkv, max_blocks, num_blocks;
    int nsmax, min_split;         // split-KV: ns_r = min(nsmax, ceil(seq_r / min_split))
    float scale_log2;             // log2(e) / sqrt(dh)
    float* part_o;                // [nsmax][T][Hq][dh]
    float* part_ml;               // [nsmax][T][Hq][2]  (running max in log2 units, sum)
    uint16_t* out;                // bf16 [T][Hq][dh] (merge output)
    int32_t* status;
};

int launch_attention(int dh, const AttnArgs& a, hipStream_t s, hipEvent_t split_begin,
                     hipEvent_t split_end);

}  // namespace pd
