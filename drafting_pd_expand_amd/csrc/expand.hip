// Batch expansion for parallel drafting, one fused launch.
//
// [Blog] = "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding
// in vLLM" (summary page), section "vLLM engineering details": the draft batch
// no longer matches the verify batch because each request gains K-1 MASK
// slots; ids, positions and hidden rows are expanded, positions grow, the
// slot mapping and per-request starts are rebuilt, and the metadata (rejected
// mask, MASK-slot mask, new-token indices, hidden-state map) is produced in a
// single kernel; the hidden rows are scattered through the map and MASK rows
// take the learned shared hidden state; rejected tokens get slot -1.
// Section "P-EAGLE core method": slot i pairs the token of position i+1 with
// the hidden state of position i; the NTP slot takes the sampled token.
//
// Design for gfx950: every workgroup recomputes the per-request start
// indices with a block-wide prefix sum over <= 1024 counts (4 KB, L2
// resident), so no second launch or global scratch is needed; it then owns
// one (or two) output rows, writes their metadata and copies each 3d-wide bf16 row with
// 16-byte vector loads/stores (a full row is contiguous, so every wave issues
// fully coalesced 1 KB transactions).
#include "common.hpp"
#include "kernels.hpp"

namespace pd {

namespace {

struct ExpandArgs {
    pd_batch_dims d;
    pd_expand_in in;
    pd_batch out;
    int T_out;
    int rows_per_block;   // 1, or 2 for very long batches (fewer redundant prefix sums)
};

__device__ __forceinline__ int slot_of(const int32_t* bt_row, int pos, int bs, int max_blocks,
                                       int num_blocks, int32_t* status) {
    if (pos < 0) { flag(status, PD_STATUS_BAD_POSITION); return -1; }
    const int b = pos / bs;
    if (b >= max_blocks) { flag(status, PD_STATUS_BAD_POSITION); return -1; }
    const int page = bt_row[b];
    if (page < 0 || page >= num_blocks) { flag(status, PD_STATUS_BAD_PAGE); return -1; }
    return page * bs + pos % bs;
}

__global__ __launch_bounds__(256) void expand_kernel(ExpandArgs a) {
    __shared__ int s_in[PD_MAX_C + 1];  // first input row of each request
    __shared__ int s_n[PD_MAX_C];
    __shared__ int s_v[PD_MAX_C];
    __shared__ int s_wsum[4];
    __shared__ int s_bad;

    // capacity (the bucket the launch is sized for) and live sizes: with
    // live counts, requests C .. Cb-1 and rows T_out .. T_outb-1 are padding
    const int Cb = a.d.C, K = a.d.K, tid = threadIdx.x;
    int C = Cb, T_in = a.d.T_in;
    int32_t* status = a.out.status;
    if (a.in.live_counts) {
        C = a.in.live_counts[0];
        T_in = a.in.live_counts[1];
        if (C < 0 || C > Cb || T_in < C || T_in > a.d.T_in) {
            if (blockIdx.x == 0 && tid == 0) flag(status, PD_STATUS_BAD_COUNTS);
            return;
        }
    }
    const int T_out = T_in + C * (K - 1);   // live rows
    if (tid == 0) s_bad = 0;
    __syncthreads();

    // counts: thread t owns requests 4t .. 4t+3
    int cnt[4];
    int sum = 0, bad = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tid * 4 + i;
        int n = 0;
        if (r < C) {
            n = a.in.num_tokens[r];
            const int rho = a.in.num_rejected[r];
            if (n < 1 || n > T_in || rho < 0 || rho >= n) {
                bad = 1;
                n = 1;
            }
            s_n[r] = n;
            s_v[r] = n - ((rho >= 0 && rho < n) ? rho : 0);
        }
        cnt[i] = n;
        sum += n;
    }
    if (bad) atomicOr(&s_bad, 1);
    // inclusive scan of the per-thread sums: within each wave by lane
    // shifts, then across the 4 waves through LDS
    const int lane = tid & 63, wv = tid >> 6;
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += t;
    }
    if (lane == 63) s_wsum[wv] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) before += w < wv ? s_wsum[w] : 0;
    int run = before + incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tid * 4 + i;
        if (r < C) s_in[r] = run;
        run += cnt[i];
    }
    if (tid == 0) s_in[C] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    __syncthreads();
    if (s_in[C] != T_in) s_bad = 1;  // benign race: every writer stores 1
    __syncthreads();
    if (s_bad) {
        if (blockIdx.x == 0 && tid == 0) flag(status, PD_STATUS_BAD_COUNTS);
        return;
    }

    const int H3 = a.d.hidden3;
    const int bs = a.d.block_size, maxb = a.d.max_blocks, nb = a.d.num_blocks;

    // per-request outputs: block 0 writes them. Padding requests own no rows
    // (cu_out = the live T_out, one visible key so that nothing reads as bad),
    // sample the last expanded row, and the padding input rows map nowhere.
    if (blockIdx.x == 0) {
        for (int r = tid; r < Cb; r += 256) {
            if (r < C) {
                const int in0 = s_in[r];
                const int p_ntp = a.in.target_pos[in0 + s_v[r] - 1];
                a.out.cu_out[r] = in0 + r * (K - 1);
                a.out.seq_lens[r] = p_ntp + K;
            } else {
                a.out.cu_out[r] = T_out;
                a.out.seq_lens[r] = 1;
                for (int m = 0; m < K; ++m) a.out.new_token_indices[r * K + m] = a.T_out - 1;
            }
        }
        for (int j = T_in + tid; j < a.d.T_in; j += 256) a.out.hidden_state_mapping[j] = -1;
        if (tid == 0) a.out.cu_out[Cb] = T_out;
    }

    for (int rr = 0; rr < a.rows_per_block; ++rr) {
        const int o = blockIdx.x * a.rows_per_block + rr;
        if (o >= a.T_out) break;
        if (o >= T_out) {
            // padding row: a rejected MASK-id row with zero hidden state (finite
            // everywhere, writes no KV, never sampled by a live request)
            if (tid == 0) {
                a.out.input_ids[o] = a.d.mask_token_id;
                a.out.positions[o] = 0;
                a.out.is_rejected[o] = 1;
                a.out.is_masked[o] = 0;
                a.out.slot_mapping[o] = -1;
            }
            uint4* d4 = reinterpret_cast<uint4*>(a.out.hidden + (size_t)o * a.d.hidden3);
            for (int c = tid; c < a.d.hidden3 / 8; c += 256) d4[c] = make_uint4(0, 0, 0, 0);
            continue;
        }
        // request of row o: the last r whose first output row is <= o
        int lo = 0, hi = C - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_in[mid] + mid * (K - 1) <= o) lo = mid; else hi = mid - 1;
        }
        const int r = lo;
        const int in0 = s_in[r];
        const int i = o - (in0 + r * (K - 1));
        const int n = s_n[r], v = s_v[r];
        const int32_t* bt_row = a.in.block_table + (size_t)r * maxb;
        // the row copy's loads go out first (the first 2048 16-byte chunks: a
        // 16384-wide row), so they overlap the metadata loads below
        const uint16_t* src = i < n ? a.in.target_hidden + (size_t)(in0 + i) * H3 : a.in.h_shared;
        const uint4* s4 = reinterpret_cast<const uint4*>(src);
        uint4* d4 = reinterpret_cast<uint4*>(a.out.hidden + (size_t)o * H3);
        const int n16 = H3 / 8;
        uint4 buf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = j * 256 + tid;
            if (c < n16) buf[j] = s4[c];
        }
        if (i < n) {
            const int j = in0 + i;
            if (tid == 0) {
                const int next = a.in.next_token_ids[r];
                const int id = (i == v - 1 || i + 1 >= n) ? next : a.in.target_ids[j + 1];
                const int pos = a.in.target_pos[j];
                const bool rej = i >= v;
                a.out.input_ids[o] = id;
                a.out.positions[o] = pos;
                a.out.is_rejected[o] = rej ? 1 : 0;
                a.out.is_masked[o] = 0;
                a.out.slot_mapping[o] = rej ? -1 : slot_of(bt_row, pos, bs, maxb, nb, status);
                a.out.hidden_state_mapping[j] = o;
                if (i == v - 1) a.out.new_token_indices[r * K] = o;
            }
        } else {
            const int m = i - n + 1;  // 1 .. K-1
            if (tid == 0) {
                const int pos = a.in.target_pos[in0 + v - 1] + m;
                a.out.input_ids[o] = a.d.mask_token_id;
                a.out.positions[o] = pos;
                a.out.is_rejected[o] = 0;
                a.out.is_masked[o] = 1;
                a.out.slot_mapping[o] = slot_of(bt_row, pos, bs, maxb, nb, status);
                a.out.new_token_indices[r * K + m] = o;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = j * 256 + tid;
            if (c < n16) d4[c] = buf[j];
        }
        // wider rows: the rest, loads before stores
        for (int c0 = 256 * 8; c0 < n16; c0 += 256 * 8) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = c0 + j * 256 + tid;
                if (c < n16) buf[j] = s4[c];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = c0 + j * 256 + tid;
                if (c < n16) d4[c] = buf[j];
            }
        }
    }
}

// Next pass of autoregressive (EAGLE-style) drafting, one row per request
// ([Blog] "background and motivation": K serial drafter passes): the token
// the previous pass sampled at its last sampled row, at that row's position
// + 1, with its slot through the block table. One thread per request.
struct AdvanceArgs {
    pd_batch_dims d;   // the previous pass's sizes
    pd_batch prev;
    const int32_t* draft;
    const int32_t* bt;
    pd_batch next;
};

__global__ __launch_bounds__(256) void ar_advance_kernel(AdvanceArgs a) {
    const int C = a.d.C, K = a.d.K;
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r > C) return;
    if (r == C) {
        a.next.cu_out[C] = C;
        return;
    }
    int32_t* status = a.next.status;
    const int T_prev = a.d.T_in + C * (K - 1);
    const int i = r * K + K - 1;
    const int row = a.prev.new_token_indices[i];
    int pos = -1, slot = -1;
    if (row < 0 || row >= T_prev) {
        flag(status, PD_STATUS_BAD_ROW);
    } else {
        pos = a.prev.positions[row] + 1;
        const int bs = a.d.block_size;
        if (pos < 1 || pos / bs >= a.d.max_blocks) {
            flag(status, PD_STATUS_BAD_POSITION);
            pos = -1;
        } else {
            const int page = a.bt[(size_t)r * a.d.max_blocks + pos / bs];
            if (page < 0 || page >= a.d.num_blocks) flag(status, PD_STATUS_BAD_PAGE);
            else slot = page * bs + pos % bs;
        }
    }
    a.next.input_ids[r] = a.draft[i];
    a.next.positions[r] = pos < 0 ? 0 : pos;
    a.next.slot_mapping[r] = slot;
    a.next.is_rejected[r] = pos < 0 ? 1 : 0;   // an unusable row is computed as rejected
    a.next.is_masked[r] = 0;
    a.next.new_token_indices[r] = r;
    a.next.hidden_state_mapping[r] = r;
    a.next.cu_out[r] = r;
    a.next.seq_lens[r] = pos < 0 ? 1 : pos + 1;
}

// Stand-in verifier of a multi-round run ([Blog] "vLLM engineering
// details": the drafter's window is the window the verifier checks next --
// the K drafts plus the token the target sampled). Request r's next verify
// window: that sampled token at p_ntp + 1 (p_ntp = the previous round's NTP
// slot position: the slot pairs the sampled token with the hidden state at
// p_ntp), then its K drafts at p_ntp + 2 ...; a_r of the drafts accepted.
// One thread per window row.
struct StubArgs {
    pd_batch_dims d;   // the previous round's sizes
    pd_batch prev;
    const int32_t* draft;
    const int32_t* next_prev;
    const int32_t* accepted;
    int32_t* num_tokens;
    int32_t* num_rejected;
    int32_t* target_ids;
    int32_t* target_pos;
    int32_t* status;
};

__global__ __launch_bounds__(256) void verify_stub_kernel(StubArgs a) {
    const int C = a.d.C, K = a.d.K;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= C * (K + 1)) return;
    const int r = i / (K + 1), j = i - r * (K + 1);
    const int T_prev = a.d.T_in + C * (K - 1);
    const int row = a.prev.new_token_indices[r * K];
    int p_ntp = 0;
    if (row < 0 || row >= T_prev) {
        if (j == 0) flag(a.status, PD_STATUS_BAD_ROW);
    } else {
        p_ntp = a.prev.positions[row];
    }
    a.target_ids[i] = j == 0 ? a.next_prev[r] : a.draft[r * K + j - 1];
    a.target_pos[i] = p_ntp + 1 + j;
    if (j == 0) {
        int acc = a.accepted[r];
        if (acc < 0 || acc > K) {
            flag(a.status, PD_STATUS_BAD_COUNTS);
            acc = acc < 0 ? 0 : K;
        }
        a.num_tokens[r] = K + 1;
        a.num_rejected[r] = K - acc;
    }
}

}  // namespace

int launch_ar_advance(const pd_batch_dims& d, const pd_batch& prev, const int32_t* draft_ids,
                      const int32_t* block_table, const pd_batch& next, hipStream_t s) {
    AdvanceArgs a;
    a.d = d;
    a.prev = prev;
    a.draft = draft_ids;
    a.bt = block_table;
    a.next = next;
    hipLaunchKernelGGL(ar_advance_kernel, dim3((d.C + 1 + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_verify_stub(const pd_batch_dims& d, const pd_batch& prev, const int32_t* draft_ids,
                       const int32_t* next_prev, const int32_t* accepted, int32_t* num_tokens,
                       int32_t* num_rejected, int32_t* target_ids, int32_t* target_pos,
                       int32_t* status, hipStream_t s) {
    StubArgs a;
    a.d = d;
    a.prev = prev;
    a.draft = draft_ids;
    a.next_prev = next_prev;
    a.accepted = accepted;
    a.num_tokens = num_tokens;
    a.num_rejected = num_rejected;
    a.target_ids = target_ids;
    a.target_pos = target_pos;
    a.status = status;
    const int n = d.C * (d.K + 1);
    hipLaunchKernelGGL(verify_stub_kernel, dim3((n + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_expand(const pd_batch_dims& d, const pd_expand_in& in, const pd_batch& out,
                  hipStream_t s) {
    ExpandArgs a;
    a.d = d;
    a.in = in;
    a.out = out;
    a.T_out = d.T_in + d.C * (d.K - 1);
    // one output row per workgroup (their dependent load chains run side by
    // side); two for very long batches, where each workgroup's prefix sum
    // over the counts is the larger cost
    a.rows_per_block = a.T_out <= 8192 ? 1 : 2;
    const int grid = (a.T_out + a.rows_per_block - 1) / a.rows_per_block;
    hipLaunchKernelGGL(expand_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

}  // namespace pd
