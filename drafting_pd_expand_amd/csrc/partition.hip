// Sequence partitioning for within-sequence gradient accumulation
// ([Paper] sec. 3.2 "Sequence Partitioning"; [arXiv] Figure 4 caption).
//
// Position p at depth d (d >= 1) depends on position p-1 at depth d-1. A kept
// position is placeable when its whole chain down to depth 0 is kept:
// valid(d, p) = keep(d, p) AND keep(d-1, p-1) AND ... AND keep(0, p-d).
// Depths 0 and 1 go to the segment their index falls in, deeper positions
// follow their dependency; following the chain d-1 steps lands on depth-1
// index p-d+1, so position (d, p) belongs to the segment whose depth-0 range
// holds q = p - max(d-1, 0). The segment's causal-completion context (the
// depth-0 positions before its first boundary) follows from the boundaries.
//
// One workgroup (512 threads) per sequence. Positions are handled in groups
// of 64 (one 64-bit mask per depth and group, in LDS):
//   A  the keep bytes are read once (several 8-byte loads in flight per
//      thread) and packed to bits;
//   B  one thread per group: validity at all depths at once from the keep
//      masks of the group and the one before it (a chain reaches back at most
//      15 positions), a block scan over the groups of all depths together
//      gives every group's row prefix (kept in LDS), the thread whose group
//      holds a segment range start records the prefix there, and the valid
//      masks replace the keep masks;
//   C  the output base of every (segment, depth) run, then per (depth, group)
//      the group's output base when all its positions fall in one segment;
//      each wave then takes 4 such groups at a time, lane = 4 consecutive
//      positions: one 16-byte store of segment ids per lane; row-list slot =
//      group base + rank in the mask, staged in LDS by rank so that the
//      group's entries go out as runs of 16 consecutive slots. The few groups
//      that straddle a boundary are done last, one wave per group, lane =
//      position.
// Within a row the segment id is non-decreasing in p, so a (segment, depth)
// run is a contiguous range of p: no sorting or atomics are needed and the
// row list comes out segment by segment, depth by depth, p ascending.

#include "common.hpp"
#include "kernels.hpp"

namespace pd {
namespace {

constexpr int kPT = 512;           // threads per workgroup
constexpr int kNW = kPT / 64;      // waves
constexpr int kLoadBatch = 8;      // keep loads in flight per thread (8 bytes each)
constexpr int kMaxGroups = PD_PART_MAX_POS / 64;   // 64-position groups over all depths
// packed per-item word of the output phase: bits 0-19 output base (or the
// group prefix), 20-27 segment, bit 28 set when the group spans a boundary
constexpr int kBaseMask = (1 << 20) - 1;
constexpr int kSegShift = 20;
constexpr int kMixed = 1 << 28;
static_assert(PD_PART_MAX_POS <= kBaseMask + 1 && PD_PART_MAX_S <= 256, "packed item word");

struct PartArgs {
    int B, K, n, S;
    const uint8_t* keep;
    const int32_t* bnd;
    int32_t* seg;
    int32_t* offsets;
    int32_t* rows;
    int32_t* status;
};

// workgroup barrier that waits for this wave's LDS traffic only: global
// stores stay in flight across it (__syncthreads would drain them every row)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// exclusive scans over the workgroup of KM values per thread at once (one
// per depth; entries d >= K are zero): x[d] in = this thread's count, out =
// carry[d] + the counts of all threads before it; carry[d] += the total.
// `ws` holds KM x kNW ints and must not be rewritten by the next call before
// every thread has passed this call's barrier (callers alternate two buffers).
template <int KM>
__device__ __forceinline__ void block_scan_carry(int (&x)[KM], int (&carry)[KM], int* ws) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
        for (int d = 0; d < KM; ++d) {
            const int y = __shfl_up(x[d], o, 64);
            if (lane >= o) x[d] += y;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int d = 0; d < KM; ++d) ws[d * kNW + w] = x[d];
    }
#pragma unroll
    for (int d = 0; d < KM; ++d) {   // inclusive -> exclusive within the wave
        const int y = __shfl_up(x[d], 1, 64);
        x[d] = lane ? y : 0;
    }
    lds_barrier();
#pragma unroll
    for (int d = 0; d < KM; ++d) {
        int base = 0, t = 0;
#pragma unroll
        for (int i = 0; i < kNW; i += 4) {
            const int4 q = *reinterpret_cast<const int4*>(ws + d * kNW + i);
            base += (i + 0 < w ? q.x : 0) + (i + 1 < w ? q.y : 0) + (i + 2 < w ? q.z : 0) + (i + 3 < w ? q.w : 0);
            t += q.x + q.y + q.z + q.w;
        }
        x[d] += base + carry[d];
        carry[d] += t;
    }
}

// exclusive block scan of one value per thread (same buffer rule)
__device__ __forceinline__ int block_excl_scan(int v, int* ws, int& total) {
    int x[1] = {v}, c[1] = {0};
    block_scan_carry<1>(x, c, ws);
    total = c[0];
    return x[0];
}

// number of boundaries b[0..S] that are <= q, minus one: the segment whose
// range [b_s, b_{s+1}) holds q (for 0 <= q < n), -1 for q < 0
__device__ __forceinline__ int seg_of(const int* bnd, int S, int q) {
    int lo = 0, hi = S + 1;   // first index with bnd > q lies in [lo, hi]
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (bnd[mid] <= q) lo = mid + 1;
        else hi = mid;
    }
    return lo - 1;
}

// first boundary index whose value is >= v
__device__ __forceinline__ int first_bnd_ge(const int* bnd, int S, int v) {
    int lo = 0, hi = S + 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (bnd[mid] < v) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ uint32_t pack_bits(uint2 x) {
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r |= (((x.x >> (8 * i)) & 0xffu) != 0u ? 1u : 0u) << i;
        r |= (((x.y >> (8 * i)) & 0xffu) != 0u ? 1u : 0u) << (i + 4);
    }
    return r;
}

template <int KM>
__global__ __launch_bounds__(kPT) void seq_partition_kernel(PartArgs a) {
    __shared__ uint64_t s_mask[kMaxGroups];                      // [d][g]: keep, then valid
    __shared__ int s_gpre[kMaxGroups];                           // [d][g]: row prefix at the group start
    __shared__ int16_t s_gseg[kMaxGroups];                       // [g]: segment of q = 64 g - offq_max
    __shared__ int s_bnd[PD_PART_MAX_S + 1];
    __shared__ int s_pre[(PD_PART_MAX_S + 1) * PD_PART_MAX_K];   // row prefix at range starts, [s][d]
    __shared__ int s_adj[PD_PART_MAX_S * PD_PART_MAX_K];         // run base - row prefix, [s][d]
    __shared__ __align__(16) int s_ws[2][KM * kNW];
    __shared__ int s_stage[kNW][256];   // a wave's row-list entries of its 4 groups, by rank

    const int b = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int K = a.K, n = a.n, S = a.S;
    const int nc = n / 8;               // bytes of one depth's keep bits
    const int ng = (n + 63) / 64;       // groups per depth
    const int offq_max = K > 2 ? K - 2 : 0;   // q = p - offq(d), offq(d) = max(d-1, 0)
    const size_t KN = (size_t)K * n;
    int32_t* seg = a.seg + (size_t)b * KN;
    int32_t* off_out = a.offsets + (size_t)b * (S + 1);
    int32_t* rows = a.rows + (size_t)b * KN;
    uint8_t* bytes = reinterpret_cast<uint8_t*>(s_mask);

    // the boundaries, checked (0 = b_0 <= ... <= b_S = n)
    int badb = 0;
    for (int i = tid; i <= S; i += kPT) {
        const int v = a.bnd[(size_t)b * (S + 1) + i];
        s_bnd[i] = v;
        if ((i == 0 && v != 0) || (i == S && v != n)) badb = 1;
    }
    __syncthreads();
    for (int i = tid; i < S; i += kPT)
        if (s_bnd[i] > s_bnd[i + 1]) badb = 1;
    if (__syncthreads_or(badb)) {
        if (tid == 0) flag(a.status, PD_STATUS_BAD_BOUNDS);
        const int4 m1 = make_int4(-1, -1, -1, -1);
        for (size_t i = tid; i < KN / 4; i += kPT) reinterpret_cast<int4*>(seg)[i] = m1;
        for (int i = tid; i <= S; i += kPT) off_out[i] = 0;
        return;
    }

    // phase A: keep bytes -> bits (byte c of depth d at bytes[d * 8 ng + c];
    // bit i of a byte = position 8c + i; the last group's tail bytes are 0)
    const int nct = (nc + kPT - 1) / kPT;   // byte tiles per depth
    const int items = K * nct;
    for (int it0 = 0; it0 < items; it0 += kLoadBatch) {
        uint2 v[kLoadBatch];
#pragma unroll
        for (int j = 0; j < kLoadBatch; ++j) {
            const int it = it0 + j;
            const int d = it / nct, c = (it - d * nct) * kPT + tid;
            v[j] = make_uint2(0u, 0u);
            if (it < items && c < nc)
                v[j] = *reinterpret_cast<const uint2*>(a.keep + (size_t)b * KN + (size_t)d * n + (size_t)c * 8);
        }
#pragma unroll
        for (int j = 0; j < kLoadBatch; ++j) {
            const int it = it0 + j;
            const int d = it / nct, c = (it - d * nct) * kPT + tid;
            if (it < items && c < nc) bytes[d * 8 * ng + c] = (uint8_t)pack_bits(v[j]);
        }
    }
    {
        const int pad = 8 * ng - nc;   // 0..7 tail bytes per depth
        for (int i = tid; i < K * pad; i += kPT) bytes[(i / pad) * 8 * ng + nc + i % pad] = 0;
    }
    for (int i = tid; i < (S + 1) * K; i += kPT) s_pre[i] = -1;
    lds_barrier();

    // phase B: one thread per group, all depths
    int badc = 0, wb = 0;
    int carry[KM];
#pragma unroll
    for (int d = 0; d < KM; ++d) carry[d] = 0;
    const int ngt = (ng + kPT - 1) / kPT;   // group tiles
    for (int t = 0; t < ngt; ++t) {
        const int g = t * kPT + tid;
        const bool in = g < ng;
        // vm[d] starts as the keep mask; computed from the deepest depth down,
        // so every depth still reads the keep masks of the depths below it.
        // kp: the top half of the group before (a chain reaches back <= 15)
        uint64_t vm[KM];
        uint32_t kp[KM];
#pragma unroll
        for (int d = 0; d < KM; ++d) {
            vm[d] = (in && d < K) ? s_mask[d * ng + g] : 0ull;
            kp[d] = (in && d < K && g > 0) ? (uint32_t)(s_mask[d * ng + g - 1] >> 32) : 0u;
        }
#pragma unroll
        for (int d = KM - 1; d > 0; --d) {
            uint64_t v = vm[d];
#pragma unroll
            for (int j = 1; j <= d; ++j)   // keep(d-j, p-j)
                v &= (vm[d - j] << j) | (uint64_t)(kp[d - j] >> (32 - j));
            if (vm[d] & ~v) badc = 1;
            vm[d] = v;
        }
        int pre[KM];
#pragma unroll
        for (int d = 0; d < KM; ++d) pre[d] = __popcll(vm[d]);
        block_scan_carry<KM>(pre, carry, s_ws[wb]);   // pre: row prefix at the group start
        wb ^= 1;
        if (in) {
            const int p0 = g * 64;
#pragma unroll
            for (int d = 0; d < KM; ++d)
                if (d < K) s_gpre[d * ng + g] = pre[d];
            const int s0 = seg_of(s_bnd, S, p0 - offq_max);
            s_gseg[g] = (int16_t)s0;
            // every range start x = b_s + offq(d) inside this group, at any depth
            // (start from the first boundary >= the group's lowest q: empty
            // segments repeat a boundary value and each needs its own record)
            for (int s = first_bnd_ge(s_bnd, S, p0 - offq_max); s <= S && s_bnd[s] < p0 + 64; ++s) {
                const int bs = s_bnd[s];
#pragma unroll
                for (int d = 0; d < KM; ++d) {
                    const int x = bs + (d > 0 ? d - 1 : 0);
                    if (d < K && x >= p0 && x < p0 + 64) {
                        const int r = x - p0;
                        const uint64_t below = r ? (vm[d] << (64 - r)) : 0ull;   // bits under r
                        s_pre[s * K + d] = pre[d] + __popcll(below);
                    }
                }
            }
        }
        lds_barrier();   // every read of this tile's keep masks is done
        if (in) {
#pragma unroll
            for (int d = 0; d < KM; ++d)
                if (d < K) s_mask[d * ng + g] = vm[d];
        }
    }
    lds_barrier();
    for (int i = tid; i < (S + 1) * K; i += kPT) {   // range starts at or past n: the row total
        if (s_pre[i] < 0) {
            const int d = i % K;
            int tot = 0;
#pragma unroll
            for (int e = 0; e < KM; ++e) tot = (e == d) ? carry[e] : tot;
            s_pre[i] = tot;
        }
    }
    if (__syncthreads_or(badc) && tid == 0) flag(a.status, PD_STATUS_BAD_CHAIN);

    // phase C1: run bases. cnt(s, d) = pre[s+1][d] - pre[s][d]; runs are laid
    // out segment-major, depth-minor; adj = run base - pre[s][d]
    {
        const int SK = S * K;
        constexpr int kPer = (PD_PART_MAX_S * PD_PART_MAX_K + kPT - 1) / kPT;
        int loc[kPer], sum = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = tid * kPer + j;
            loc[j] = 0;
            if (i < SK) {
                const int s = i / K, d = i - s * K;
                loc[j] = s_pre[(s + 1) * K + d] - s_pre[s * K + d];
            }
            sum += loc[j];
        }
        int total;
        int base = block_excl_scan(sum, s_ws[wb], total);
        wb ^= 1;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = tid * kPer + j;
            if (i < SK) {
                const int s = i / K, d = i - s * K;
                s_adj[i] = base - s_pre[s * K + d];
                if (d == 0) off_out[s] = base;
            }
            base += loc[j];
        }
        if (tid == 0) off_out[S] = total;
    }
    lds_barrier();

    // phase C2a: per (depth, group) item, its output base and segment when
    // the group's q range [64 g - offq, 64 g + 63 - offq] lies in one segment
    // (packed: base | segment << 20), else the group prefix | the segment of
    // its lowest q << 20 | kMixed
    for (int it = tid; it < K * ng; it += kPT) {
        const int d = it / ng, g = it - d * ng;
        const int qlo = g * 64 - (d > 0 ? d - 1 : 0);
        int s = s_gseg[g];   // segment of 64 g - offq_max <= qlo
        while (s + 1 < S && s_bnd[s + 1] <= qlo) ++s;
        const bool mixed = s < 0 || (s + 1 < S && s_bnd[s + 1] <= qlo + 63);
        const int gp = s_gpre[it];
        // (a group below q = 0 starts its walk at segment 0: its valid
        // positions all have q >= 0)
        s_gpre[it] = mixed ? (gp | ((s < 0 ? 0 : s) << kSegShift) | kMixed)
                           : ((s_adj[s * K + d] + gp) | (s << kSegShift));
    }
    lds_barrier();

    // phase C2b: each wave takes 4 groups (256 positions) of one depth at a
    // time; lane = 4 consecutive positions, so a wave writes 1 KB of segment
    // ids with one 16-byte store per lane and its row-list entries to
    // consecutive addresses
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int sub = (lane & 15) * 4;                     // the lane's first position in its group
    const uint64_t below = (1ull << sub) - 1ull;         // positions of the group before the lane's
    for (int d = 0; d < K; ++d) {
        const int offq = d > 0 ? d - 1 : 0;
        int32_t* segd = seg + (size_t)d * n;
        for (int g0 = wv * 4; g0 < ng; g0 += kNW * 4) {
            const int g = g0 + (lane >> 4);
            uint64_t m = 0ull;
            int w = 0;
            if (g < ng) {
                m = s_mask[d * ng + g];
                w = s_gpre[d * ng + g];
            }
            const uint32_t nib = (uint32_t)(m >> sub) & 0xfu;
            const int rank0 = __popcll(m & below);
            const int p = g * 64 + sub;
            // groups that straddle a boundary are left to phase C2c
            const bool live = g < ng && (w & kMixed) == 0;
            const int su = (w >> kSegShift) & 0xff;
            int* stage = s_stage[wv] + (lane >> 4) * 64;   // this lane's group, by rank
            int out[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                out[i] = -1;
                if (live && ((nib >> i) & 1u)) {
                    out[i] = su;
                    stage[rank0 + __popc(nib & ((1u << i) - 1u))] = d * n + p + i;
                }
            }
            if (live && p < n) *reinterpret_cast<int4*>(segd + p) = make_int4(out[0], out[1], out[2], out[3]);
            // the group's row-list entries (consecutive slots from its base)
            // go out from the stage, 16 consecutive slots per store and group:
            // whole cache lines instead of a slot every ~2 positions per lane.
            // A wave's LDS accesses complete in order, so the reads see every
            // lane's writes above and precede the next group's writes.
            const int cnt = live ? __popcll(m) : 0;
            const int gb = w & kBaseMask;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int k = (lane & 15) + 16 * t;
                const int r = gb + k;
                if (k < cnt && r >= 0 && (size_t)r < KN) rows[r] = stage[k];
            }
        }
    }

    // phase C2c: the groups that straddle a segment boundary (a few per
    // boundary and depth), one wave per group, lane = position
    const uint64_t below_lane = lane ? (~0ull >> (64 - lane)) : 0ull;
    for (int c0 = wv * 64; c0 < K * ng; c0 += kNW * 64) {
        const int it_l = c0 + lane;
        const bool mx = it_l < K * ng && (s_gpre[it_l] & kMixed);
        uint64_t todo = __ballot(mx);
        while (todo) {
            const int j = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int it = c0 + j;
            const int d = it / ng, g = it - d * ng;
            const uint64_t m = s_mask[it];
            const int w = s_gpre[it];
            const int p = g * 64 + lane;
            const bool v = (m >> lane) & 1ull;
            int sg = -1;
            if (v) {
                sg = seg_of(s_bnd, S, p - (d > 0 ? d - 1 : 0));
                const int r = s_adj[sg * K + d] + (w & kBaseMask) + __popcll(m & below_lane);
                if (r >= 0 && (size_t)r < KN) rows[r] = d * n + p;
            }
            if (p < n) seg[(size_t)d * n + p] = sg;
        }
    }
}

}  // namespace

int launch_seq_partition(const pd_partition_dims& d, const uint8_t* keep, const int32_t* boundaries,
                         int32_t* seg, int32_t* seg_offsets, int32_t* rows, int32_t* status,
                         hipStream_t s) {
    PartArgs a;
    a.B = d.B; a.K = d.K; a.n = d.n; a.S = d.S;
    a.keep = keep; a.bnd = boundaries; a.seg = seg; a.offsets = seg_offsets; a.rows = rows;
    a.status = status;
    if (d.K <= 4) hipLaunchKernelGGL(seq_partition_kernel<4>, dim3(d.B), dim3(kPT), 0, s, a);
    else if (d.K <= 8) hipLaunchKernelGGL(seq_partition_kernel<8>, dim3(d.B), dim3(kPT), 0, s, a);
    else hipLaunchKernelGGL(seq_partition_kernel<16>, dim3(d.B), dim3(kPT), 0, s, a);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

}  // namespace pd
