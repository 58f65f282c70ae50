// Paged split-KV attention kernels of the drafter and their launchers; the
// device code (work split, LDS layouts, softmax) is in attn_dev.hpp.
//
// [Blog] = "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding
// in vLLM" (summary page): every draft position of a request attends in the
// same pass through the request's KV pages.
#include "attn_dev.hpp"

namespace pd {

namespace {

// The split plan on its own (the forward runs it inside the layer-0 input
// kernel instead).
__global__ __launch_bounds__(kAttnPlanThreads) void attn_plan_kernel(AttnArgs a) { attn_plan_block(a); }


template <int DH, bool F8>
__global__ __launch_bounds__((64 * AttnCfg<DH, F8>::NW)) void attn_split_kernel(AttnArgs a) {
    __shared__ AttnSmem<DH, F8, 0> sm;
    attn_split_item<DH, F8, false, 0>(a, blockIdx.x, sm);
}

template <int DH, int HPW>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
    attn_merge_wave<DH, HPW, false>(a, (blockIdx.x * 4 + (threadIdx.x >> 6)) * HPW);   // HPW | Hq: one row per wave
}

template <int DH>
int launch_dh(const AttnArgs& a, hipStream_t s, hipEvent_t e0, hipEvent_t e1, hipEvent_t e2,
              hipEvent_t e3) {
    constexpr int NW = AttnCfg<DH>::NW;
    if (e0) (void)hipEventRecord(e0, s);
    if (a.fp8)
        hipLaunchKernelGGL((attn_split_kernel<DH, true>), dim3((unsigned)a.sp.max_units * a.Hkv), dim3(64 * NW),
                           0, s, a);
    else
        hipLaunchKernelGGL((attn_split_kernel<DH, false>), dim3((unsigned)a.sp.max_units * a.Hkv), dim3(64 * NW),
                           0, s, a);
    if (e1) (void)hipEventRecord(e1, s);
    if (hipGetLastError() != hipSuccess) return PD_EHIP;
    if (e2) (void)hipEventRecord(e2, s);
    // heads per wave: one while a wave per (row, head) fits one round of
    // resident workgroups (every wave's load chain then runs side by side);
    // four (or two) for more rows, which cuts the rounds (C = 64: 34.5 ->
    // 24.9 us; at C = 1 four heads per wave would take 10.9 instead of 4.7)
    const int hpw = (a.T * a.Hq + 3) / 4 <= kMergeRoundWgs ? 1 : (a.Hq % 4 == 0 ? 4 : (a.Hq % 2 == 0 ? 2 : 1));
    const unsigned mgrid = (unsigned)((a.T * a.Hq / hpw + 3) / 4);
    if (hpw == 4) hipLaunchKernelGGL((attn_merge_kernel<DH, 4>), dim3(mgrid), dim3(256), 0, s, a);
    else if (hpw == 2) hipLaunchKernelGGL((attn_merge_kernel<DH, 2>), dim3(mgrid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_merge_kernel<DH, 1>), dim3(mgrid), dim3(256), 0, s, a);
    if (e3) (void)hipEventRecord(e3, s);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

}  // namespace

AttnSplit plan_attn_split(int C, int T, int Hq, int Hkv, int dh, int max_blocks) {
    AttnSplit p;
    p.min_split = 128;
    // workgroups the split length aims at: dh 128 moves twice the bytes per
    // key and per partial, and runs best with ~4x fewer, longer splits
    // (measured on the 16 x 20000-key batch: 142 us at 512 vs 177 us at 2048)
    p.target_wg = dh == 64 ? 2048 : 512;
    const long long reach = (long long)max_blocks * PD_PAGE;
    // a split never exceeds the LDS block-table cache: enough workgroups for
    // the longest batch the block table can describe
    const long long need = ((long long)C * reach * Hkv + kMaxSplitKeys - 1) / kMaxSplitKeys;
    if (need > p.target_wg) p.target_wg = (int)std::min<long long>(need, 1LL << 30);
    // partial planes: about 1 GiB at most, but enough splits that the longest
    // request fits kMaxSplitKeys per split
    const long long plane = (long long)T * Hq * (dh + 2) * 4;
    long long scap = plane > 0 ? (1LL << 30) / plane : kMaxSplits;
    scap = std::max(scap, (reach + kMaxSplitKeys - 1) / kMaxSplitKeys);
    p.scap = (int)std::max(1LL, std::min(scap, (long long)kMaxSplits));
    p.max_units = (p.target_wg + Hkv - 1) / Hkv + C;
    // every split holds >= min_split keys of a request of <= reach keys:
    // short batches launch only the workgroups they can use
    const long long most = (long long)C * ((reach + p.min_split - 1) / p.min_split);
    if (most < p.max_units) p.max_units = (int)std::max(1LL, most);
    p.round_slots = kAttnRoundSlots;
    return p;
}

AttnSplit plan_attn_split_grid(int C, int T, int Hq, int Hkv, int dh, int max_blocks, int grid) {
    AttnSplit p = plan_attn_split(C, T, Hq, Hkv, dh, max_blocks);
    const long long reach = (long long)max_blocks * PD_PAGE;
    // the split length aims at one item per workgroup; units per head are at
    // most total / split + C, so the unit list needs grid / Hkv + C entries,
    // more only where the block-table cache caps the split length
    const long long need = ((long long)C * reach * Hkv + kMaxSplitKeys - 1) / kMaxSplitKeys;
    p.target_wg = (int)std::max<long long>(grid, need);
    p.round_slots = grid;
    p.max_units = (p.target_wg + Hkv - 1) / Hkv + C;
    const long long most = (long long)C * ((reach + p.min_split - 1) / p.min_split);
    if (most < p.max_units) p.max_units = (int)std::max(1LL, most);
    return p;
}

int attn_min_splits(int max_blocks) {
    const long long reach = (long long)max_blocks * PD_PAGE;
    return (int)std::max(1LL, (reach + kMaxSplitKeys - 1) / kMaxSplitKeys);
}

int launch_attn_plan(const AttnArgs& a, hipStream_t s) {
    if (a.C <= 0) return PD_OK;
    hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kAttnPlanThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

int launch_attention(int dh, const AttnArgs& a, hipStream_t s, hipEvent_t split_begin,
                     hipEvent_t split_end, hipEvent_t merge_begin, hipEvent_t merge_end) {
    if (a.C <= 0 || a.T <= 0) return PD_OK;
    if (dh == 64) return launch_dh<64>(a, s, split_begin, split_end, merge_begin, merge_end);
    if (dh == 128) return launch_dh<128>(a, s, split_begin, split_end, merge_begin, merge_end);
    return PD_EINVAL;
}

}  // namespace pd
