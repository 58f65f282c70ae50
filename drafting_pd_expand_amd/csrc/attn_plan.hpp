// Split-KV plan of the paged attention, as a block-level device routine for
// one 256-thread workgroup: run by its own launch or as workgroup 0 of the
// layer-0 input kernel (the plan depends only on cu_out / seq_lens, so it
// runs beside that kernel's rows and costs no launch of its own).
//
// [Blog] = "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding
// in vLLM" (summary page), "P-EAGLE core method": every position of a
// request attends through the request's KV pages in the same pass; the plan
// only decides how that work is cut into workgroups.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace pd {

constexpr int kAttnBtMax = 512;                          // block-table entries of one split cached in LDS
constexpr int kAttnMaxSplitKeys = kAttnBtMax * PD_PAGE;  // keys of one split at most
// split-kernel workgroups one round holds (two per CU). At dh 64 over a bf16
// cache three fit, but counting 768 lets short batches take shorter splits
// whose extra merge work costs more than it saves (4 x 17.7k keys: 8 us more
// per step)
constexpr int kAttnRoundSlots = 512;
constexpr int kAttnOneRoundMaxKeys = 512;
constexpr int kAttnPlanThreads = 256;

// Reads cu_out / seq_lens of every request (requests 4t .. 4t+3 on thread
// t), validates them, picks the split length and writes the per-request
// split counts and the unit records {r, s, ns, row0, row1, kb, ke, 0}.
// CG: other workgroups of the same launch read the plan (coherent stores).
// MAXC: requests the caller guarantees at most (sizes the LDS tables).
template <bool CG = false, int MAXC = PD_MAX_C>
__device__ __forceinline__ void attn_plan_block(const AttnArgs& a) {
    __shared__ long long s_sum[4];
    __shared__ int s_max[4];
    __shared__ int s_cnt[4];
    __shared__ int s_incl[MAXC];   // inclusive prefix of the split counts
    __shared__ int4 s_req[MAXC];   // validated {row0, row1, seq} of every request
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int seq[4];
    long long sv = 0;
    int mv = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * tid + i;
        seq[i] = 0;
        if (r < a.C && r < MAXC) {
            const int row0 = a.cu_out[r], row1 = a.cu_out[r + 1];
            int sq = a.seq_lens[r];
            const bool ok = row0 >= 0 && row1 <= a.T && row1 >= row0 && sq >= 1 &&
                            sq <= a.max_blocks * PD_PAGE;
            if (!ok) flag(a.status, PD_STATUS_BAD_ROW);
            if (!ok || row1 == row0) sq = 0;   // no work
            seq[i] = sq;
            s_req[r] = make_int4(row0, row1, sq, 0);
            sv += sq;
            mv = max(mv, sq);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        sv += __shfl_xor(sv, o, kWave);
        mv = max(mv, __shfl_xor(mv, o, kWave));
    }
    if (lane == 0) {
        s_sum[w] = sv;
        s_max[w] = mv;
    }
    __syncthreads();
    long long total = 0;
    int mx = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        total += s_sum[i];
        mx = max(mx, s_max[i]);
    }
    const long long tw = a.sp.target_wg;
    long long sl = (total * a.Hkv + tw - 1) / tw;
    // Few keys in all: the shortest split whose (unit, kv head) workgroups
    // all fit in one round of kAttnRoundSlots (units <= total / sl + C per
    // head), as long as that split stays short. A second round costs more
    // than the longer splits: C = 4 with 17.7k keys, 22 us at 304 keys / 472
    // workgroups vs 27 us at 128 keys / 1120 and at 256 keys / 568 (26 us
    // at 512 keys / 288); with 13k keys, 19 us at 224 keys vs 22 at 128.
    const long long free_slots = (long long)a.sp.round_slots - (long long)a.Hkv * a.C;
    if (free_slots > 0) {
        const long long one = (total * a.Hkv + free_slots - 1) / free_slots;
        if (one <= kAttnOneRoundMaxKeys) sl = max(sl, one);
    }
    sl = max(sl, (long long)a.sp.min_split);
    sl = max(sl, (long long)((mx + a.sp.scap - 1) / a.sp.scap));
    sl = (sl + PD_PAGE - 1) / PD_PAGE * PD_PAGE;
    const int split_len = (int)min(sl, (long long)kAttnMaxSplitKeys);
    int ns[4], nsum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ns[i] = seq[i] > 0 ? (seq[i] + split_len - 1) / split_len : 0;
        if (ns[i] > a.sp.scap) {   // excluded by the host's choice of scap; never write past it
            flag(a.status, PD_STATUS_BAD_ROW);
            ns[i] = 0;
        }
        nsum += ns[i];
    }
    // exclusive prefix of the split counts over the block
    int incl = nsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_cnt[w] = incl;
    __syncthreads();
    int before = 0, units = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        before += i < w ? s_cnt[i] : 0;
        units += s_cnt[i];
    }
    int run = before + incl - nsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * tid + i;
        run += ns[i];
        if (r < a.C && r < MAXC) {
            stc<CG>(a.plan + kPlanNs + r, ns[i]);
            s_incl[r] = run;
        }
    }
    if (tid == 0) {
        if (units > a.sp.max_units) flag(a.status, PD_STATUS_BAD_ROW);   // excluded by the host's bound
        stc<CG>(a.plan, min(units, a.sp.max_units));
        stc<CG>(a.plan + 1, split_len);
    }
    __syncthreads();
    // unit records, spread over the block: unit u belongs to the first
    // request whose inclusive split count exceeds u (never one without splits)
    const int nu = min(units, a.sp.max_units);
    for (int u = tid; u < nu; u += kAttnPlanThreads) {
        int lo = 0, hi = a.C - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_incl[mid] > u) hi = mid; else lo = mid + 1;
        }
        const int q = lo;
        const int nsq = s_incl[q] - (q > 0 ? s_incl[q - 1] : 0);
        const int sq = u - (s_incl[q] - nsq);
        const int4 rq = s_req[q];
        const int kb = sq * split_len;
        const int ke = min(rq.z, kb + split_len);
        int4* rec = reinterpret_cast<int4*>(a.plan + kPlanUnits + (size_t)u * kPlanRec);
        stc<CG>(rec, make_int4(q, sq, nsq, rq.x));
        stc<CG>(rec + 1, make_int4(rq.y, kb, ke, 0));
    }
}

}  // namespace pd
