/*
 * pd.h -- C ABI of the P-EAGLE parallel-drafting step on AMD MI355X (gfx950).
 *
 * Pages cited (titles; sections are those printed on the pages):
 *   [Blog]  "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding
 *           in vLLM" (summary page of the vLLM blog post)
 *   [Paper] "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training"
 *           (summary page)
 *   [arXiv] ScienceStack page for arXiv 2602.01469 (the same paper)
 *
 * One draft step = pd_expand_batch + pd_draft_forward on one stream.
 *
 * Conventions for every entry point:
 *   - Pointers marked [dev] are device pointers (hipMalloc / torch CUDA
 *     tensors on the current device); pointers to the structs themselves are
 *     host pointers. bf16 values travel as uint16_t bit patterns.
 *   - The caller owns every buffer it passes; the library never frees or
 *     keeps caller memory beyond the call. Work is enqueued asynchronously on
 *     `stream` (a hipStream_t; NULL = the null stream) and nothing waits for
 *     it, except where a call says it may synchronize.
 *   - Return codes: PD_OK, or PD_EINVAL for bad host arguments (nothing is
 *     enqueued), PD_ENOMEM when a library scratch allocation fails, PD_EHIP
 *     when a launch reports a HIP error, PD_ESCRATCH when a call of the
 *     allocation-free forward needs more than its static scratch.
 *   - Device data is never trusted for addressing: an index that would fall
 *     outside a buffer is skipped and a bit is set in a device status word
 *     (PD_STATUS_*), which the caller reads after the stream is done.
 */
#ifndef PD_H
#define PD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PD_OK      0
#define PD_EINVAL (-1)
#define PD_ENOMEM (-2)
#define PD_EHIP   (-3)
#define PD_ESCRATCH (-4)  /* pd_draft_forward_noalloc: the call needs more than its static scratch */

#define PD_MAX_C      1024  /* requests per step (the blog's serving runs allow 1024 sequences) */
#define PD_MAX_K      16    /* draft depth; the blog's drafter predicts up to 10 tokens */
#define PD_MAX_LAYERS 16
#define PD_PAGE       16    /* KV page size (tokens) the forward's cache layout uses */
#define PD_MAX_BLOCKS 65536 /* block-table columns pd_draft_forward accepts (1,048,576 keys) */

/* Device status bits (ORed into a caller- or handle-owned int32). */
#define PD_STATUS_BAD_COUNTS   1  /* n_r < 1, rho_r outside [0, n_r), or sum(n_r) != T_in   */
#define PD_STATUS_BAD_POSITION 2  /* a position < 0 or past the block table's reach         */
#define PD_STATUS_BAD_PAGE     4  /* a block-table entry outside [0, num_blocks)            */
#define PD_STATUS_BAD_TOKEN    8  /* a token id outside [0, V)                              */
#define PD_STATUS_BAD_ROW     16  /* row bookkeeping (cu_out / new-token index) inconsistent */
#define PD_STATUS_BAD_CHAIN   32  /* pd_seq_partition: a kept position whose dependency is not placeable */
#define PD_STATUS_BAD_BOUNDS  64  /* pd_seq_partition: segment boundaries not 0 = b_0 <= ... <= b_S = n */
#define PD_STATUS_SYNC_TIMEOUT 128 /* pd_draft_forward: a grid-wide wait of the persistent decode pass gave up */

/* Sizes of one draft step. [host]
 *   C             requests, 0..PD_MAX_C (0 = nothing to do)
 *   K             draft depth, 1..PD_MAX_K (K = 1 is autoregressive EAGLE's single pass)
 *   T_in          rows of the verify batch = sum of num_tokens
 *   mask_token_id the MASK placeholder's token id ([Blog] fused-kernel paragraph)
 *   hidden3       width of a target hidden row (3d; [arXiv] Figure 2), multiple of 8
 *   block_size    KV page size in tokens (pd_draft_forward needs PD_PAGE)
 *   max_blocks    columns of the block table
 *   num_blocks    pages in the KV pool; valid block-table entries are < num_blocks
 * The expanded batch has T_out = T_in + C*(K-1) rows. */
typedef struct {
    int32_t C, K, T_in, mask_token_id, hidden3, block_size, max_blocks, num_blocks;
} pd_batch_dims;

/* The verify batch the expansion reads. All [dev]. */
typedef struct {
    const int32_t*  num_tokens;     /* [C]  n_r >= 1 verify tokens of request r                 */
    const int32_t*  num_rejected;   /* [C]  rho_r in [0, n_r): the last rho_r were rejected      */
    const int32_t*  target_ids;     /* [T_in] token ids, request-major                          */
    const int32_t*  target_pos;     /* [T_in] positions (consecutive within a request)           */
    const uint16_t* target_hidden;  /* [T_in][hidden3] bf16 target hidden rows                   */
    const int32_t*  next_token_ids; /* [C]  the token the target sampled for request r          */
    const int32_t*  block_table;    /* [C][max_blocks] page numbers                              */
    const uint16_t* h_shared;       /* [hidden3] bf16 learned shared hidden state                */
    const int32_t*  live_counts;    /* [2] {C, T_in} of the live batch, or NULL (= dims); see below */
} pd_expand_in;

/* The expanded (draft) batch: written by pd_expand_batch, read by
 * pd_draft_forward. All [dev], sized by the caller. */
typedef struct {
    int32_t*  input_ids;            /* [T_out] */
    int32_t*  positions;            /* [T_out] */
    int32_t*  slot_mapping;         /* [T_out] page*block_size + offset; -1 = rejected, no KV write */
    uint8_t*  is_rejected;          /* [T_out] 1 for a rejected verify token                    */
    uint8_t*  is_masked;            /* [T_out] 1 for a MASK (parallel-drafting) slot             */
    int32_t*  hidden_state_mapping; /* [T_in]  target row j -> expanded row                     */
    int32_t*  new_token_indices;    /* [C*K]   request-major: the NTP row, then the K-1 MASK rows */
    int32_t*  cu_out;               /* [C+1]   first expanded row of each request; cu_out[C] = T_out */
    int32_t*  seq_lens;             /* [C]     keys visible to the request's last row (p_ntp + K) */
    uint16_t* hidden;               /* [T_out][hidden3] bf16 expanded hidden rows                */
    int32_t*  status;               /* [1] or NULL: PD_STATUS_* bits ORed in on bad device data  */
} pd_batch;

/*
 * pd_expand_batch -- build the draft batch from the verify batch.
 *
 * Follows [Blog] "vLLM engineering details": the draft batch appends MASK
 * slots after each request's tokens, so ids, hidden rows and positions are
 * expanded, positions grow, and the slot mapping and per-request starts are
 * rebuilt; one fused launch copies ids/positions into their new slots,
 * inserts the sampled token, fills the MASK ids and emits the rejected-token
 * mask, the MASK-slot mask, the new-token indices and the hidden-state map;
 * target hidden rows are scattered through that map and MASK rows take
 * h_shared; rejected tokens get slot -1 so no KV entry is written for them.
 * The pairing is the one-position shift of [Blog] "P-EAGLE core method"
 * (slot i: token i+1 with hidden i; the last accepted slot: the sampled token).
 *
 * For request r with n_r tokens, rho_r rejected, v_r = n_r - rho_r, starting
 * at input row a_r and output row b_r = a_r + r*(K-1):
 *   row b_r+i (i < n_r): id = next_r if i == v_r-1 or i == n_r-1, else
 *     target_ids[a_r+i+1]; position = target_pos[a_r+i]; rejected iff
 *     i >= v_r; hidden = target_hidden[a_r+i].
 *   row b_r+n_r+m-1 (m = 1..K-1): id = mask_token_id, position = p_ntp + m
 *     with p_ntp = target_pos[a_r+v_r-1]; hidden = h_shared.
 *   seq_lens[r] = p_ntp + K.
 * The hidden rows are copied bit-for-bit.
 *
 * Bucketed batches (live_counts != NULL): dims give the capacity a captured
 * graph was sized for ([Blog] "vLLM engineering details": the draft step runs
 * under graph capture, its range extended to hold the larger draft batch), and
 * the device words live_counts = {C, T_in} the batch actually present, 0 <= C
 * <= dims->C, C <= T_in <= dims->T_in; the inputs hold that batch in their
 * first C requests / T_in rows. The live rows come out exactly as for a call
 * with those sizes. Requests C .. dims->C-1 are padding: cu_out = the live
 * T_out (also cu_out[dims->C]), seq_lens = 1, their K new-token indices =
 * the last expanded row. Rows from the live T_out to dims' T_out are padding:
 * mask_token_id, position 0, rejected, slot -1, zero hidden rows. Padding
 * input rows map to -1. pd_draft_forward then runs at the capacity's sizes:
 * padding rows write no KV and change no live row's result, and the draft ids
 * of padding requests are meaningless. Bad live counts set
 * PD_STATUS_BAD_COUNTS and write nothing.
 *
 * Errors: PD_EINVAL if dims/in/out or a required pointer is NULL, C outside
 * [0, PD_MAX_C], K outside [1, PD_MAX_K], T_in < C, hidden3 <= 0 or not a
 * multiple of 8, block_size < 1, max_blocks < 1 or num_blocks < 1. C = 0 is a
 * no-op. Bad device data sets out->status bits (if given) and never makes the
 * kernel read or write outside the buffers sized above.
 */
int pd_expand_batch(const pd_batch_dims* dims, const pd_expand_in* in,
                    const pd_batch* out, void* stream);

/* Drafter weights. [host] struct of [dev] bf16 pointers, row-major [out][in].
 * Layer 0 takes [RMSNorm(emb; norm_emb) || RMSNorm(fc(h); norm_hid)] (2d wide)
 * into its QKV projection and starts the residual stream at fc(h); layers
 * 1..N-1 are pre-norm LLaMA layers ([Paper] sec. 2 architecture and experiment
 * setup; [Blog] Input_i equation; [arXiv] Figure 2). */
typedef struct {
    int32_t d, Hq, Hkv, dh, F, N, V, hidden3;
    float   rms_eps, rope_theta;
    const uint16_t* embed;                    /* [V][d]                                    */
    const uint16_t* fc;                       /* [d][hidden3]                              */
    const uint16_t* norm_emb;                 /* [d]                                       */
    const uint16_t* norm_hid;                 /* [d]                                       */
    const uint16_t* norm_in[PD_MAX_LAYERS];   /* [d] (layers >= 1)                         */
    const uint16_t* w_qkv[PD_MAX_LAYERS];     /* [(Hq+2*Hkv)*dh][2d at layer 0, else d]; q, k, v row blocks */
    const uint16_t* w_o[PD_MAX_LAYERS];       /* [d][Hq*dh]                                */
    const uint16_t* norm_post[PD_MAX_LAYERS]; /* [d]                                       */
    const uint16_t* w_gate[PD_MAX_LAYERS];    /* [F][d]                                    */
    const uint16_t* w_up[PD_MAX_LAYERS];      /* [F][d]                                    */
    const uint16_t* w_down[PD_MAX_LAYERS];    /* [d][F]                                    */
    const uint16_t* norm_final;               /* [d]                                       */
    const uint16_t* lm_head;                  /* [V][d]                                    */
} pd_model;

typedef struct pd_handle pd_handle;

/*
 * pd_draft_forward -- the one drafter pass that yields all K draft tokens of
 * every request ([Blog] "P-EAGLE core method": all positions go through the
 * N layers and the LM head together).
 *
 * Computes, for every non-rejected row of the expanded batch: fc projection
 * (hidden3 -> d), the layer-0 input above, N layers of [RMSNorm] -> QKV ->
 * rotate-half RoPE at the row's position (base rope_theta) -> K/V written to
 * the cache at slot_mapping (rows with slot -1 write nothing; [Blog] KV-cache
 * paragraph) -> causal GQA attention over positions 0..p of the row's own
 * request, read through block_table -> O projection + residual -> RMSNorm ->
 * SwiGLU MLP + residual; then the final RMSNorm and LM head on the K rows
 * named by new_token_indices, and the greedy argmax (lowest index on ties).
 * Within a layer every K/V write lands before any row attends. Rejected
 * rows influence nothing: passes of more than 64 rows (at most 4096) gather
 * the other rows to the front on the device and compute only those; smaller
 * passes compute rejected rows as don't-care values. A sampled row
 * (new_token_indices) that is rejected, as a padding request's is, yields an
 * unspecified draft; one outside [0, T_out) sets PD_STATUS_BAD_ROW.
 *
 * Arguments:
 *   h          [host] handle slot: *h == NULL creates the handle (scratch is
 *              allocated then, and again, after a stream synchronize, when a
 *              later call needs more). One handle serves one stream at a time.
 *   m          [host] model; requires d, F, V multiples of 16, d <= 4096, hidden3 = 3d,
 *              Hq % Hkv == 0, dh in {64, 128}, 1 <= N <= PD_MAX_LAYERS,
 *              every weight pointer non-NULL.
 *   dims       [host] the same sizes given to pd_expand_batch; block_size must
 *              be PD_PAGE and max_blocks <= PD_MAX_BLOCKS.
 *   batch      [host] struct of [dev] pointers written by pd_expand_batch
 *              (status may be NULL).
 *   block_table[dev] [C][max_blocks].
 *   kv_cache   [dev] bf16, N layers x {K plane, V plane}; each plane is
 *              [num_blocks][Hkv][PD_PAGE*dh]: a K page is token-major
 *              [16][dh], a V page is dim-major [dh][16]. Element (layer l,
 *              plane t, page b, head g, token s, dim c) sits at
 *              ((l*2+t)*num_blocks + b)*Hkv*16*dh + g*16*dh + (t ? c*16+s : s*dh+c).
 *   draft_ids  [dev] int32 [C*K] out, request-major like new_token_indices.
 *   logits     [dev] float [C*K][V] out, or NULL.
 * Errors: PD_EINVAL on bad host arguments (nothing enqueued), PD_ENOMEM,
 * PD_EHIP. Bad device data sets bits in the handle's status word
 * (pd_status) and never leads to an out-of-bounds access.
 */
int pd_draft_forward(pd_handle** h, const pd_model* m, const pd_batch_dims* dims,
                     const pd_batch* batch, const int32_t* block_table,
                     uint16_t* kv_cache, int32_t* draft_ids, float* logits, void* stream);

/* Free a handle and its scratch (NULL-safe; waits for the handle's device
 * work to finish). Never frees caller memory. */
void pd_free(pd_handle* h);

/* ---- autoregressive baseline ------------------------------------------------
 *
 * [Blog] "background and motivation": autoregressive EAGLE drafts K tokens
 * with K serial drafter passes, which parallel drafting replaces by one pass.
 * [Blog] "P-EAGLE core method" / [arXiv] Figure 2 caption: the NTP position
 * works exactly like the autoregressive case. These two calls run that
 * baseline on the same kernels: pass 1 = pd_expand_batch with K = 1 +
 * pd_draft_forward_ex; pass k >= 2 = pd_ar_advance + pd_draft_forward_ex on
 * one row per request whose hidden input is the drafter's own final hidden
 * state of the previous pass (d wide, so fc is skipped). The pages leave that
 * fed-back state open; this is the reading taken.
 */

/* Options of pd_draft_forward_ex. [host] struct, [dev] pointers. */
typedef struct {
    const uint16_t* hidden_d;   /* bf16 [T_out][d]: every row's projected hidden input given
                                   directly (fc is skipped, batch->hidden is not read and may be
                                   NULL), or NULL for fc(batch->hidden)                        */
    uint16_t*       hidden_out; /* bf16 [C*K][d] out: the final residual (before the final norm)
                                   of every sampled row, request-major, or NULL                */
    int32_t         kv_fp8;     /* nonzero: kv_cache holds fp8 E4M3 codes ([Blog] "vLLM engineering
                                   details": the serving setup keeps the KV cache in fp8), one byte
                                   per element, same layout and index formula as the bf16 cache;
                                   a stored code is value / scale, nearest with ties to even,
                                   saturated to +-448, and reads back as code value * scale    */
    const float*    kv_scales;  /* [host] [N][2] (K scale, V scale) per layer, each > 0 and finite;
                                   NULL = 1.0. Read only when kv_fp8                            */
} pd_forward_opts;

/* pd_draft_forward with options (opts NULL = pd_draft_forward). Same
 * arguments, ownership and errors; hidden_d / hidden_out must be 16-byte
 * aligned. With opts->kv_fp8 the kv_cache pointer addresses uint8 codes (pass
 * it cast to uint16_t*); PD_EINVAL for a scale that is not > 0 and finite. */
int pd_draft_forward_ex(pd_handle** h, const pd_model* m, const pd_batch_dims* dims,
                        const pd_batch* batch, const int32_t* block_table,
                        uint16_t* kv_cache, int32_t* draft_ids, float* logits,
                        const pd_forward_opts* opts, void* stream);

/* Build the next autoregressive pass's batch, one row per request, from the
 * previous pass (dims_prev: its C, K, T_in and the block table sizes; prev:
 * its batch; draft_ids [dev] [C*K]: the tokens it sampled). Row r of `next`
 * is request r: input_ids = the token sampled at the previous pass's last
 * sampled row, positions = that row's position + 1, slot_mapping through
 * block_table (-1 and PD_STATUS_BAD_POSITION / _BAD_PAGE if outside it),
 * is_rejected = is_masked = 0, new_token_indices = hidden_state_mapping = r,
 * cu_out = 0..C, seq_lens = position + 1. next->hidden is not written (the
 * next pass reads pd_forward_opts.hidden_d). The next pass's dims are
 * {C, K = 1, T_in = C}. Errors: PD_EINVAL for bad dims or NULL pointers,
 * PD_EHIP; a bad new-token index of `prev` sets PD_STATUS_BAD_ROW in
 * next->status (if given) and gives a row with slot -1. */
int pd_ar_advance(const pd_batch_dims* dims_prev, const pd_batch* prev, const int32_t* draft_ids,
                  const int32_t* block_table, const pd_batch* next, void* stream);

/* ---- allocation-free forward -------------------------------------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * pd_draft_forward_noalloc is pd_draft_forward_ex without a handle: its
 * scratch (activations, split-K partials, attention partials and plan, LM-head
 * partials) lives in one static device array of PD_NOALLOC_SCRATCH_BYTES per
 * GPU, which the library holds from its first use on that GPU until the
 * process ends. The call allocates nothing: no hipMalloc, hipFree or
 * allocating library routine. Arguments, layouts, kernels and results are
 * those of pd_draft_forward_ex (opts may be NULL); bad device data sets
 * PD_STATUS_* bits in batch->status when it is non-NULL.
 *
 * Every call on a GPU shares that GPU's array and leaves its contents behind;
 * calls that overlap on one GPU (other streams, other threads) race and give
 * undefined results: serialize them. Nothing in the array has to start at
 * zero. A batch whose workspace does not fit returns PD_ESCRATCH and enqueues
 * nothing (the attention partials take fewer, longer splits per request before
 * that: same results up to the order of rounding). With 64 MiB the
 * GPT-OSS-20B-scale drafter fits up to a few hundred expanded rows.
 */
#define PD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int pd_draft_forward_noalloc(const pd_model* m, const pd_batch_dims* dims, const pd_batch* batch,
                             const int32_t* block_table, uint16_t* kv_cache, int32_t* draft_ids,
                             float* logits, const pd_forward_opts* opts, void* stream);

/* ---- extras ---------------------------------------------------------------- */

/* Text for a PD_* return code. */
const char* pd_strerror(int code);

/* Synchronize `stream`, copy the handle's PD_STATUS_* word to *out [host] and
 * clear it. PD_EINVAL if h or out is NULL. */
int pd_status(pd_handle* h, int32_t* out, void* stream);

/* Optional copy of the residual stream: when dst [dev] is non-NULL, later
 * pd_draft_forward calls write float [N+1][T_out][d] (after fc, then after
 * each layer). Rows of rejected tokens are not computed in passes of more
 * than 64 rows, and there they are left as they are. Pass NULL to stop. */
int pd_set_debug_resid(pd_handle* h, float* dst);

/* Optional phase timestamps of the persistent decode kernel (the pass of up
 * to 64 rows in one launch): when dst [dev] is non-NULL, later
 * pd_draft_forward calls that take that kernel write uint64 readings of the
 * device's constant 100 MHz clock: [p][w] = when workgroup w finished the work
 * of phase p (p < P - 1, P = 4 + 9 N phases, w < the device's CU count G),
 * then [P - 1][p] = when phase p's grid barrier released, and
 * [P - 1][P - 1] = the start of the launch. dst holds P * G words. Pass NULL
 * to stop. For profiling only. */
int pd_set_decode_timeline(pd_handle* h, uint64_t* dst);

/* Per-kernel timing with HIP events on the launch stream. Kernel classes: */
#define PD_KERNEL_LMHEAD  0   /* LM-head GEMM with the fused argmax partials     */
#define PD_KERNEL_GEMM    1   /* every other GEMM (fc, QKV, O, gate/up, down)    */
#define PD_KERNEL_ATTN    2   /* split-KV paged attention (not the merge)         */
#define PD_KERNEL_OTHER   3   /* norms, RoPE+cache, split plan, merge, argmax reduce */
#define PD_KERNEL_DECODE  4   /* the persistent decode kernel: a whole pass of up to 64 rows */
#define PD_KERNEL_CLASSES 5
/* class_mask != 0 starts recording an event pair around every launch of the
 * kernel classes whose bit (1 << PD_KERNEL_*) is set, for later
 * pd_draft_forward calls with this handle; 0 stops. Either way the records
 * collected so far are dropped (after a device synchronize). */
int pd_profile(pd_handle* h, int class_mask);
/* Wait for the recorded events and return the summed duration (ms) and the
 * launch count of one kernel class since profiling was enabled. */
int pd_profile_read(pd_handle* h, int kernel_class, double* total_ms, int64_t* launches);

/* ---- multi-round runs --------------------------------------------------------
 *
 * [Blog] "vLLM engineering details": for EAGLE the window the drafter
 * consumes is the window the verifier checks next (the K drafts plus one
 * token the target sampled), and the draft step runs under graph capture.
 * pd_verify_stub stands in for the verifier so that rounds of
 * verify -> pd_expand_batch -> pd_draft_forward can run back to back on the
 * device (and be captured as one graph): how many drafts the target accepts,
 * the token it samples and its hidden rows are the caller's inputs.
 */

/* Build round t+1's verify batch from round t. dims_prev: round t's sizes;
 * prev: round t's expanded batch (positions and new_token_indices are read);
 * prev_draft_ids [dev] [C*K]: round t's drafts; prev_next_token_ids [dev] [C]:
 * the token the target sampled in round t (round t's next_token_ids);
 * accepted [dev] [C]: drafts of round t the target accepts, 0..K.
 * Out [dev]: num_tokens [C] (= K+1), num_rejected [C] (= K - accepted),
 * target_ids and target_pos [C*(K+1)]: per request the sampled token at
 * p_ntp + 1 (p_ntp = round t's NTP slot position), then the K drafts at
 * p_ntp + 2 ... p_ntp + K + 1. Round t+1's dims are {C, K, T_in = C*(K+1)};
 * its target_hidden and next_token_ids come from the caller.
 * status [dev] [1] or NULL: PD_STATUS_BAD_ROW for a bad NTP index of prev,
 * PD_STATUS_BAD_COUNTS for accepted outside [0, K] (clamped).
 * Errors: PD_EINVAL for bad dims or NULL pointers; PD_EHIP. */
int pd_verify_stub(const pd_batch_dims* dims_prev, const pd_batch* prev, const int32_t* prev_draft_ids,
                   const int32_t* prev_next_token_ids, const int32_t* accepted, int32_t* num_tokens,
                   int32_t* num_rejected, int32_t* target_ids, int32_t* target_pos, int32_t* status,
                   void* stream);

/* ---- sequence partitioning (training side) ----------------------------------
 *
 * [Paper] sec. 3.2 "Sequence Partitioning"; [arXiv] Figure 4 caption. A
 * training sequence of n tokens with K prediction depths holds position p
 * at depth d if COD sampling kept it; position p at depth d >= 1 depends on
 * position p-1 at depth d-1. The sequence is cut into S segments trained one
 * after another: depths 0 and 1 go to the segment their index falls in,
 * deeper positions go where their dependency went (so every dependency stays
 * inside one segment), and each segment also carries, as attention context,
 * the depth-0 positions before its first boundary (causal completion).
 */

#define PD_PART_MAX_K   16         /* prediction depths                      */
#define PD_PART_MAX_S   256        /* segments per sequence                  */
#define PD_PART_MAX_POS (1 << 19)  /* K * (n rounded up to 64) per sequence   */

/* Sizes of one pd_seq_partition call. [host]
 *   B  sequences (0 = nothing to do); K depths, 1..PD_PART_MAX_K;
 *   n  positions per sequence (padded length), a multiple of 8,
 *      K * (n rounded up to a multiple of 64) <= PD_PART_MAX_POS;
 *   S  segments, 1..PD_PART_MAX_S. */
typedef struct {
    int32_t B, K, n, S;
} pd_partition_dims;

/* Assign every kept position of B sequences to a segment.
 *   keep        [dev] uint8 [B][K][n], 8-byte aligned: nonzero = position p kept at depth d
 *               (depth 0 holds the real tokens; padding is 0 at every depth).
 *   boundaries  [dev] int32 [B][S+1]: 0 = b_0 <= b_1 <= ... <= b_S = n; segment s covers the
 *               depth-0 indices [b_s, b_{s+1}); empty segments are allowed.
 *   seg         [dev] int32 [B][K][n] out, 16-byte aligned: the segment of position (d, p), or -1
 *               if it is not kept or not placeable (a link of its chain down to depth 0 is
 *               missing).
 *   seg_offsets [dev] int32 [B][S+1] out: segment s's rows are rows[b][seg_offsets[b][s] ..
 *               seg_offsets[b][s+1]); seg_offsets[b][S] = placeable positions of sequence b.
 *   rows        [dev] int32 [B][K*n] out: per sequence, the placeable positions as d * n + p,
 *               segment by segment, then depth by depth, p ascending. Entries past
 *               seg_offsets[b][S] are not written. Segment s's context is the depth-0
 *               positions [0, b_s) (kept ones only), implied and not listed.
 *   status      [dev] int32 [1] or NULL: PD_STATUS_BAD_CHAIN if a kept position is not
 *               placeable, PD_STATUS_BAD_BOUNDS for a sequence with bad boundaries (its seg
 *               is all -1 and its offsets 0).
 * Errors: PD_EINVAL for bad dims, NULL or misaligned pointers (nothing enqueued); PD_EHIP.
 * Deterministic; no scratch memory; one workgroup per sequence. */
int pd_seq_partition(const pd_partition_dims* dims, const uint8_t* keep, const int32_t* boundaries,
                     int32_t* seg, int32_t* seg_offsets, int32_t* rows, int32_t* status,
                     void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PD_H */
