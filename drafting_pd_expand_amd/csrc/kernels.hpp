// Internal launchers shared between the kernel files and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pd.h"

namespace pd {

// ---------------------------------------------------------------- expansion
int launch_expand(const pd_batch_dims& d, const pd_expand_in& in, const pd_batch& out,
                  hipStream_t s);
int launch_seq_partition(const pd_partition_dims& d, const uint8_t* keep, const int32_t* boundaries,
                         int32_t* seg, int32_t* seg_offsets, int32_t* rows, int32_t* status,
                         hipStream_t s);
int launch_verify_stub(const pd_batch_dims& d, const pd_batch& prev, const int32_t* draft_ids,
                       const int32_t* next_prev, const int32_t* accepted, int32_t* num_tokens,
                       int32_t* num_rejected, int32_t* target_ids, int32_t* target_pos,
                       int32_t* status, hipStream_t s);
int launch_ar_advance(const pd_batch_dims& d, const pd_batch& prev, const int32_t* draft_ids,
                      const int32_t* block_table, const pd_batch& next, hipStream_t s);

// ---------------------------------------------------------------- GEMM
enum Epi : int {
    EPI_PARTIAL = 0,  // fp32 partial plane per K split: ws[split][M][N] (the consumer sums)
    EPI_SWIGLU = 1,   // y_bf16 = silu(X W^T) * (X W2^T)
    EPI_ARGMAX = 2,   // max / argmax partials per row (+ optional fp32 logits): one per
                      // (row, column tile), or per (row, wave) in the few-row kernel
};

struct GemmArgs {
    const uint16_t* X;       // bf16 [rows][ldx]
    int ldx;
    const int32_t* xrows;    // optional gather: GEMM row m reads X row xrows[m]
    int xrows_limit;         // rows of X (bound for xrows entries)
    const uint16_t* W;       // bf16 [N][K]
    const uint16_t* W2;      // second matrix for EPI_SWIGLU
    int M, N, K;
    int splits;              // K splits across workgroups (EPI_PARTIAL only)
    float* ws;               // partial planes [splits][M][N]
    uint16_t* yb; int ldyb;
    float* logits; int ldlog;
    float* amax_v; int* amax_i; int ntiles;
    int32_t* status;
};

enum GemmKind : int {
    GEMM_RING = 0,    // M <= 64: persistent LDS-ring weight streaming
    GEMM_TILED = 1,   // LM head at 64 < M < 256: 128 x 128 register-staged tiles, two workgroups per CU
    GEMM_BIG = 2,     // other M > 64: persistent ring-fed tiles, 256 x 256 (8 waves) from 384 rows, else 128 x 128
};

struct GemmPlan {
    int kind;      // GemmKind
    int mt;        // ring: 16-row X tiles (1, 2 or 4)
    int mblocks;   // tiled / big: workgroups along M
    int wn;        // waves per workgroup (ring-fed tiles: 8 = 256-row, 4 = 128-row)
    int nm;        // ring: groups of 16 output columns per wave
    int ntiles;    // column tiles (ARGMAX: groups of the max/argmax partial results per row)
    int splits;    // K splits (EPI_PARTIAL: one fp32 plane each)
    int grid;      // ring / big: persistent workgroups
};

GemmPlan plan_gemm(int M, int N, int K, int epi);
GemmPlan plan_gemm_nm(int M, int N, int K, int epi, int ring_nm);
size_t gemm_ws_floats(const GemmPlan& p, int M, int N, int epi);
int launch_gemm(int epi, const GemmPlan& p, GemmArgs a, hipStream_t s);

// ---------------------------------------------------------------- row kernels
// Every consumer of a projection sums its fp32 partial planes
// (ws[s][T][width], s < S) in split order.
// xin != nullptr: the projected hidden rows given directly (bf16 [T][d]); ws / S unused.
// plan != nullptr: the attention split plan (launch_attn_plan's work) runs as
// one more workgroup of the same launch.
struct AttnArgs;
int launch_layer0_input(const uint16_t* xin, const float* ws, int S, const int32_t* ids,
                        const uint16_t* embed, int V, float* x, const uint16_t* g_emb,
                        const uint16_t* g_hid, uint16_t* u, int T, int d, float eps,
                        int32_t* status, hipStream_t s, const AttnArgs* plan = nullptr);
// rows != nullptr: output row o = norm of row rows[o] (o < nrows), x untouched;
// xout (row-list mode) also gets the bf16 residual row itself.
int launch_resid_norm(const float* ws, int S, float* x, const uint16_t* gamma, uint16_t* y, int T,
                      int d, float eps, hipStream_t s, const int32_t* rows = nullptr, int nrows = 0,
                      int32_t* status = nullptr, uint16_t* xout = nullptr);
// fp8: the planes hold E4M3 codes of value / k_scale (K) and value / v_scale (V)
int launch_rope_cache(const float* ws, int S, const int32_t* positions, const int32_t* slots, int T,
                      int Hq, int Hkv, int dh, float theta, uint16_t* q_out, void* kplane,
                      void* vplane, int num_blocks, int32_t* status, hipStream_t s, int fp8 = 0,
                      float k_scale = 1.0f, float v_scale = 1.0f);
int launch_argmax_reduce(const float* amax_v, const int* amax_i, int M, int ntiles, int32_t* out,
                         int32_t* status, hipStream_t s);

// ---------------------------------------------------------------- attention
// Split-KV plan, computed on the device once per forward from seq_lens:
// split_len = max(min_split, ceil(sum_r seq_r * Hkv / target_wg),
// ceil(max_r seq_r / scap)) rounded up to a page -- or, where a split of at
// most 512 keys puts every workgroup into one round of 512 resident ones, the
// shortest such split (if longer); request r gets
// ns_r = ceil(seq_r / split_len) units of work (one workgroup per unit and kv
// head). The host sizes everything from bounds it knows without a sync.
struct AttnSplit {
    int min_split;   // keys per split at least (multiple of 16)
    int target_wg;   // workgroups the split length aims at
    int scap;        // splits per request at most (partial planes allocated)
    int max_units;   // capacity of the unit list = grid x of the split kernel
};
AttnSplit plan_attn_split(int C, int T, int Hq, int Hkv, int dh, int max_blocks);
// the fewest splits per request (scap) that cover max_blocks pages of keys
int attn_min_splits(int max_blocks);
// int32 words of the plan: [units, split_len, -, -, ns[PD_MAX_C],
// unit records[max_units][kPlanRec]]
constexpr int kPlanNs = 4;
constexpr int kPlanUnits = 4 + PD_MAX_C;
constexpr int kPlanRec = 8;
inline size_t attn_plan_ints(const AttnSplit& p) {
    return (size_t)kPlanUnits + (size_t)p.max_units * kPlanRec;
}

struct AttnArgs {
    const uint16_t* q;            // bf16 [T][Hq][dh] (rotated)
    const void* kplane;           // this layer's K plane [num_blocks][Hkv][16][dh] (bf16 or fp8 codes)
    const void* vplane;           // this layer's V plane [num_blocks][Hkv][dh][16]
    const int32_t* positions;
    const uint8_t* is_rejected;
    const int32_t* cu_out;        // [C+1]
    const int32_t* seq_lens;      // [C]
    const int32_t* block_table;   // [C][max_blocks]
    int C, T, Hq, Hkv, max_blocks, num_blocks;
    AttnSplit sp;
    int32_t* plan;                // attn_plan_ints(sp) words, written by launch_attn_plan
    float scale_log2;             // log2(e) / sqrt(dh)
    bool fp8;                     // planes hold E4M3 codes: value = code * k_scale (K), * v_scale (V)
    float k_scale, v_scale;
    float* part_o;                // [scap][T][Hq][dh]
    float* part_ml;               // [scap][T][Hq][2]  (running max in log2 units, sum)
    uint16_t* out;                // bf16 [T][Hq][dh]
    int32_t* status;
};

// Once per forward (the plan only depends on cu_out / seq_lens).
int launch_attn_plan(const AttnArgs& a, hipStream_t s);
// Optional events around the split kernel and around the merge kernel.
int launch_attention(int dh, const AttnArgs& a, hipStream_t s, hipEvent_t split_begin,
                     hipEvent_t split_end, hipEvent_t merge_begin = nullptr,
                     hipEvent_t merge_end = nullptr);

}  // namespace pd
