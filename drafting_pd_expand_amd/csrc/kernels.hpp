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
    // Optional, many-row kernel only (plan_gemm with rows_on_device): m_dev[0]
    // = rows present (<= M), read on the device; only their row blocks are
    // computed, and (EPI_PARTIAL) the K split count is chosen there for
    // those blocks, at most `splits`, and written to splits_out[0] for the
    // consumer of the planes.
    const int32_t* m_dev;
    int32_t* splits_out;
    // max/argmax epilogue, many-row kernel only: index of this launch's first
    // output column in the whole row (the argmax reports n_base + column) and
    // the partials per row of amax_v / amax_i (0: this launch's own count)
    int n_base;
    int amax_ld;
};

enum GemmKind : int {
    GEMM_RING = 0,    // M <= 64 (LM head: <= 128): persistent LDS-ring weight streaming
    GEMM_BIG = 2,     // M > 64 (LM head: > 128): persistent ring-fed tiles, 256 x 256 (8 waves) from 384
                      // rows (LM head: 129), else 128 x 128
    GEMM_WRING = 3,   // M <= 64: weight-only LDS ring, X fragments loaded into registers
};

struct GemmPlan {
    int kind;      // GemmKind
    int mt;        // ring: 16-row X tiles (1, 2, 4, or 8 for the LM head at 65..128 rows)
    int mblocks;   // big: row blocks (workgroup tiles along M)
    int wn;        // waves per workgroup (ring-fed tiles: 8 = 256-row, 4 = 128-row)
    int nm;        // ring / weight-only ring: groups of 16 output columns (W rows) per wave
    int ntiles;    // column tiles (ARGMAX: groups of the max/argmax partial results per row)
    int splits;    // K splits (EPI_PARTIAL: one fp32 plane each)
    int grid;      // ring / big: persistent workgroups
    int krs;       // ring: reduction elements per stage (128, or 64 with 8 X tiles)
    int rs = 1;    // ring, LM head on 8 or 2 X tiles: waves per column group (each takes mt / rs tiles)
};

// rows_on_device: the rows present are counted on the device (GemmArgs::m_dev,
// M > 64, not EPI_ARGMAX); `splits` is then the most planes the kernel may
// write and `grid` covers that many.
GemmPlan plan_gemm(int M, int N, int K, int epi, bool rows_on_device = false);
// K splits of the many-row kernel: the count (<= smax) that minimises the K
// steps of the busiest of `slots` resident workgroups over `tiles` tiles
__host__ __device__ inline int big_splits(long tiles, int ksteps, long slots, int smax) {
    int best_sp = 1;
    long best = -1;
    for (int sp = 1; sp <= smax && sp <= ksteps; ++sp) {
        const int per = (ksteps + sp - 1) / sp;
        if ((sp - 1) * per >= ksteps) continue;   // no empty split
        const long span = ((tiles * sp + slots - 1) / slots) * per;
        if (best < 0 || span < best) { best = span; best_sp = sp; }
    }
    return best_sp;
}
GemmPlan plan_gemm_nm(int M, int N, int K, int epi, int ring_nm);
// The LM head (max/argmax epilogue) as one or two launches: on 256-row tiles
// a last round of the persistent grid that is less than half full goes to a
// second launch on 128-row tiles over the last columns (n_main onwards), so
// that the first runs whole rounds only. ntiles: argmax partials per row of
// the two together (the first launch's first).
struct LmHeadPlan {
    GemmPlan main, tail;   // tail.kind < 0: one launch
    int n_main;            // columns of the first launch
    int ntiles;
};
LmHeadPlan plan_lm_head(int M, int N, int K);
size_t gemm_ws_floats(const GemmPlan& p, int M, int N, int epi);
int launch_gemm(int epi, const GemmPlan& p, GemmArgs a, hipStream_t s);

// ---------------------------------------------------------------- row kernels
// Every consumer of a projection sums its fp32 partial planes
// (ws[s][T][width], s < S) in split order.
// xin != nullptr: the projected hidden rows given directly (bf16 [T][d]); ws / S unused.
// plan != nullptr: the attention split plan (launch_attn_plan's work) runs as
// one more workgroup of the same launch.
struct AttnArgs;
// t_dev (all row kernels, optional): rows present, on the device (<= T); rows
// at or past it are skipped. s_dev (optional): the split-plane count, on the
// device (written by a projection that chose it there), in place of S.
int launch_layer0_input(const uint16_t* xin, const float* ws, int S, const int32_t* ids,
                        const uint16_t* embed, int V, float* x, const uint16_t* g_emb,
                        const uint16_t* g_hid, uint16_t* u, int T, int d, float eps,
                        int32_t* status, hipStream_t s, const AttnArgs* plan = nullptr,
                        const int32_t* t_dev = nullptr, const int32_t* s_dev = nullptr);
// rows != nullptr: output row o = norm of row rows[o] (o < nrows), x untouched;
// xout (row-list mode) also gets the bf16 residual row itself.
int launch_resid_norm(const float* ws, int S, float* x, const uint16_t* gamma, uint16_t* y, int T,
                      int d, float eps, hipStream_t s, const int32_t* rows = nullptr, int nrows = 0,
                      int32_t* status = nullptr, uint16_t* xout = nullptr, const int32_t* t_dev = nullptr,
                      const int32_t* s_dev = nullptr);
// fp8: the planes hold E4M3 codes of value / k_scale (K) and value / v_scale (V)
int launch_rope_cache(const float* ws, int S, const int32_t* positions, const int32_t* slots, int T,
                      int Hq, int Hkv, int dh, float theta, uint16_t* q_out, void* kplane,
                      void* vplane, int num_blocks, int32_t* status, hipStream_t s, int fp8 = 0,
                      float k_scale = 1.0f, float v_scale = 1.0f, const int32_t* t_dev = nullptr,
                      const int32_t* s_dev = nullptr);

// Row compaction of a many-row pass: the rows that are not rejected, in
// order, get consecutive indices c = (kept rows before them). Gathers their
// hidden rows (bf16 [T][h3] -> hid_c), token ids, positions and slots, and
// writes rowmap[c] = original row, the compacted request starts cu_c[0..C],
// the compacted indices of the sampled rows nti_c[0..R) and the kept count
// t_eff[0]. A sampled row outside [0, T), and request starts outside
// [0, T] or decreasing, are flagged (PD_STATUS_BAD_ROW); a sampled row that
// is outside [0, T) or rejected (a padding request's) maps to 0.
// T <= kCompactMaxRows.
constexpr int kCompactMaxRows = 4096;
int launch_compact_rows(const uint8_t* is_rejected, const int32_t* ids, const int32_t* positions,
                        const int32_t* slots, const int32_t* cu_out, const int32_t* nti,
                        const uint16_t* hidden, int T, int C, int R, int h3, uint16_t* hid_c,
                        int32_t* ids_c, int32_t* pos_c, int32_t* slot_c, int32_t* cu_c, int32_t* nti_c,
                        int32_t* rowmap, int32_t* t_eff, int32_t* status, hipStream_t s);
// dst[rowmap[c]] = src[c] for c < t_eff[0] (fp32 rows of d; residual snapshots)
int launch_scatter_rows(const float* src, float* dst, const int32_t* rowmap, const int32_t* t_eff, int T, int d,
                        hipStream_t s);
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
    int round_slots; // split workgroups resident at once (the one-round rule)
};
AttnSplit plan_attn_split(int C, int T, int Hq, int Hkv, int dh, int max_blocks);
// The same plan for a fixed grid of `grid` workgroups, one item each at most
// when the keys allow (the persistent decode kernel).
AttnSplit plan_attn_split_grid(int C, int T, int Hq, int Hkv, int dh, int max_blocks, int grid);
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
    const uint8_t* is_rejected;   // may be null: no row rejected (compacted rows)
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

// Everything one decode launch needs (by value, in the kernel arguments).
struct DecodeArgs {
    // model (bf16 [out][in])
    const uint16_t *embed, *fc, *norm_emb, *norm_hid, *norm_final, *lm_head;
    const uint16_t* norm_in[PD_MAX_LAYERS];
    const uint16_t* w_qkv[PD_MAX_LAYERS];
    const uint16_t* w_o[PD_MAX_LAYERS];
    const uint16_t* norm_post[PD_MAX_LAYERS];
    const uint16_t* w_gate[PD_MAX_LAYERS];
    const uint16_t* w_up[PD_MAX_LAYERS];
    const uint16_t* w_down[PD_MAX_LAYERS];
    int d, Hq, Hkv, dh, F, NL, V, hidden3;
    float eps;
    double inv_step;                  // theta^(-2/dh)
    // the expanded batch (written by pd_expand_batch, an earlier launch)
    const int32_t *ids, *positions, *slots, *new_idx;
    const uint16_t* hidden;           // [T][hidden3] or null with hidden_d
    const uint16_t* hidden_d;         // [T][d] projected rows given directly, or null
    uint16_t* hidden_out;             // [R][d] final residual of the sampled rows, or null
    int T, R;
    char* kv;                         // bf16 cache base
    size_t plane_bytes;               // bytes of one K or V plane
    int num_blocks;
    int32_t* draft_ids;
    float* logits;                    // [R][V] or null
    // scratch. Activations that a projection reads as its X operand are
    // written once per launch, each into a slot of its own (plain loads may
    // then be served from L2: no XCD holds a stale copy of a slot):
    // u slot 0 = layer-0 input [T][2d], slot 2l + 1 = layer l's post-attention
    // norm, slot 2l + 2 = layer l + 1's input norm; ao and act one slot per layer
    float* x;                         // fp32 residual [T][d]
    uint16_t *u, *q, *ao, *act, *xg;
    size_t u_slot, ao_slot, act_slot; // elements per slot
    int rows0;                        // workgroups rows0 .. rows0 + T - 1 do the row phases
    int lm_in_kernel;                 // the LM head and argmax run as the last phases
    float* ws;                        // split-K planes
    float* amax_v;
    int* amax_i;
    float* dbg;                       // [N+1][T][d] residual snapshots, or null
    unsigned* sync;                   // barrier words: [0] release, [64 + i] arrival of workgroup i
    int32_t* status;
    uint64_t* timeline;               // or null: [phase][workgroup] end of the phase's work, then
                                      // [phase] barrier release, then the start (100 MHz clock)
    // projections: K splits and workgroups taking part
    int sp_fc, sp_qkv0, sp_qkv, sp_o, sp_down;
    int g_fc, g_qkv0, g_qkv, g_o, g_gu, g_down, g_lm;
    AttnArgs at;                      // plan, partials, split sizes; q / planes set per layer
};

// Plan of the persistent decode kernel: K splits and workgroups taking part
// in each projection (grid = the device's CUs, one workgroup each).
struct DecodePlan {
    bool ok;         // the pass fits the kernel (rows, head size, cache type, device)
    int mt;          // 16-row activation tiles (1, 2 or 4)
    int grid;        // workgroups of the launch
    int rows0;       // first row workgroup (= grid - T); projections use workgroups below it
    int lm_in_kernel;
    int sp_fc, sp_qkv0, sp_qkv, sp_o, sp_down;
    int g_fc, g_qkv0, g_qkv, g_o, g_gu, g_down, g_lm;
    size_t ws_floats;   // split-K planes the pass needs
    int lm_ntiles;      // argmax partials per sampled row
};
// T expanded rows, R sampled rows; fp8: the cache holds E4M3 codes.
DecodePlan plan_decode(const pd_model& m, int T, int R, bool fp8);
// Sync words the decode kernel keeps in scratch (zero before the first launch).
constexpr size_t kDecodeSyncWords = 64 + 256;
int launch_decode(const DecodePlan& p, const DecodeArgs& a, hipStream_t s);

}  // namespace pd
