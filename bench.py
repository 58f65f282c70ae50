"""Benchmark of the P-EAGLE parallel drafting step on one MI355X.

One step = pd_expand_batch + pd_draft_forward for the whole batch (every row
of the hot path), on synthetic inputs already resident in HBM. Headline
workload: the GPT-OSS-20B-scale drafter at C=1, context 4096, K=7; then the
same drafter at C=4 and C=64 (K=7, and K=3 / 5 for the one-pass cost against
K) and the Qwen3-Coder-30B-scale drafter at C=16, each timed the same way.

    python bench.py [--steps K] [--warmup W] [--workload g_c1] [--configs g_c4,...|none]

Prints ONE JSON line on stdout (progress goes to stderr):
  value      draft steps/s of the headline workload (drafted tokens/s =
             value * C * K is reported too)
  roofline   the headline's dominant kernel: achieved bandwidth or flop rate
             (algorithmic bytes or flops per launch / average launch time
             from HIP events on the launch stream during the timed region)
             against the 8 TB/s HBM or 2.5 PFLOP/s bf16 peak
  cpu_baseline  the fp64 oracle (expand + forward) timed on the host cores on
             a bounded sample of the same workload
  configs    per workload: us/step, steps/s, drafted tok/s, the step's share
             of the HBM roofline, the dominant kernel's roofline, the GEMMs'
             MFMA roofline (flops of the non-rejected rows / summed GEMM
             launch time, from events around the GEMM launches only, in a
             second timed region) and the oracle on request 0
  yardsticks measured-peak references: a streaming read, a device copy and
             the installed vendor bf16 GEMM (torch.matmul) on two shapes
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

DESCR = {
    "tiny": "tiny drafter prefill (d 256, 4 layers, vocab 4096), 128-token prompt, K=4",
    "g_c1": "GPT-OSS-20B-scale drafter (d 2880, 64q/8kv x 64, SwiGLU 7680, 4 layers, vocab 201088), C=1, context 4096, K=7",
    "g_c4": "GPT-OSS-20B-scale drafter, C=4, lognormal contexts (median 3891, P90 10800, 128..20000), K=7",
    "g_c64": "GPT-OSS-20B-scale drafter, C=64, lognormal contexts, K=7",
    "g_c64_k3": "GPT-OSS-20B-scale drafter, C=64, lognormal contexts, K=3",
    "g_c64_k5": "GPT-OSS-20B-scale drafter, C=64, lognormal contexts, K=5",
    "q_c16": "Qwen3-Coder-30B-scale drafter (d 2048, 32q/4kv x 128, SwiGLU 6144, 4 layers, vocab 151936), C=16, context 20000, K=7",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def lm_head_bytes(dm, R: int) -> int:
    """Algorithmic bytes of one LM-head launch: the bf16 weight matrix, the R
    normalized bf16 input rows, and the R int32 draft ids."""
    return dm.V * dm.d * 2 + R * dm.d * 2 + R * 4


def attn_bytes(dm, b, K: int) -> int:
    """Algorithmic bytes of one attention launch (one layer): every visible
    cached K and V row once per kv head, the rotated queries in and the bf16
    outputs out."""
    v = b["num_tokens"] - b["num_rejected"]
    seq = b["context_lens"] + v + K - 1
    T_out = b["T_in"] + b["C"] * (K - 1)
    return int(seq.sum()) * dm.Hkv * dm.dh * 2 * 2 + 2 * T_out * dm.Hq * dm.dh * 2


def gemm_flops(dm, b, K: int) -> int:
    """GEMM flops of one step on the T_eff computed rows (rejected rows earn
    no credit) plus the LM head on C*K rows."""
    v = b["num_tokens"] - b["num_rejected"]
    T_eff = int((v + K - 1).sum())
    per_row = dm.d * dm.hidden3
    for l in range(dm.N):
        per_row += dm.qkv_out * dm.qkv_in(l) + dm.d * dm.Hq * dm.dh + 3 * dm.F * dm.d
    return 2 * T_eff * per_row + 2 * b["C"] * K * dm.V * dm.d


def forward_bytes(dm, b, K: int) -> int:
    """Algorithmic bytes of the drafter pass alone (pd_draft_forward): the
    step's bytes without the expansion's own traffic (the verify rows it reads
    and writes out; the pass reads the expanded rows once)."""
    T_in = b["T_in"]
    return step_bytes(dm, b, K) - (T_in + 1) * dm.hidden3 * 2


def step_bytes(dm, b, K: int) -> int:
    """Algorithmic bytes of one whole step (weights once, visible KV once per
    layer and kv head, KV writes, hidden rows in and out, ids)."""
    w = dm.V * dm.d * 2 + dm.d * dm.hidden3 * 2          # LM head + fc (embedding rows: gathered, below)
    for l in range(dm.N):
        w += dm.qkv_out * dm.qkv_in(l) * 2 + dm.d * dm.Hq * dm.dh * 2 + 3 * dm.F * dm.d * 2 + 4 * dm.d * 2
    C = b["C"]
    v = b["num_tokens"] - b["num_rejected"]
    seq = b["context_lens"] + v + K - 1
    kv_read = int(seq.sum()) * dm.Hkv * dm.dh * 2 * 2 * dm.N
    T_eff = int((v + K - 1).sum())
    kv_write = T_eff * dm.Hkv * dm.dh * 2 * 2 * dm.N
    T_in = b["T_in"]
    T_out = T_in + C * (K - 1)
    hid = (T_in + T_out) * dm.hidden3 * 2 + dm.hidden3 * 2
    emb = T_eff * dm.d * 2
    return w + kv_read + kv_write + hid + emb + C * K * 4


def cpu_baseline(w, model_np, b, pool, min_s: float = 10.0, max_runs: int = 64) -> dict:
    """Time the oracle (as it stands) on a bounded sample: the first request
    of the workload (the whole step at C = 1), expand + forward in fp64 on the
    host cores, repeated until about min_s seconds of CPU work have run."""
    import oracle  # CPU baseline leg only

    threads = len(os.sched_getaffinity(0))
    reqs = [0] if w.C > 1 else None
    runs = 0
    t0 = time.perf_counter()
    while True:
        exp = oracle.expand(b["num_tokens"], b["num_rejected"], b["target_ids"], b["target_pos"],
                            b["target_hidden"], b["next_token_ids"], b["block_table"], model_np["h_shared"],
                            w.K, b["mask_id"], b["block_size"])
        oracle.draft_forward(model_np, exp, b["block_table"], pool, w.K, requests=reqs,
                             block_size=b["block_size"])
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or runs >= max_runs:
            break
    n_req = 1 if reqs else w.C
    # one sampled request of C: scale to whole steps of the workload
    steps_per_s = runs * (n_req / w.C) / dt
    return {"value": steps_per_s, "unit": "draft steps/s", "cores": threads, "kind": "oracle",
            "sample": (f"{'request 0 of ' + str(w.C) if reqs else 'the whole step'}: fp64 NumPy oracle "
                       f"expand + forward, {runs} runs in {dt:.1f} s, scaled to whole steps"),
            "seconds": dt}


def copy_calibration(mib: int = 512, reps: int = 4):
    """A plain device-to-device copy of known size: reads and writes
    `mib` MiB per launch. Its FETCH_SIZE / WRITE_SIZE counter readings give
    the factor that turns those counters into HBM bytes."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} x {mib} MiB device copies")
    print(json.dumps({"copy_calibration_bytes_per_launch": mib * (1 << 20), "launches": reps}))


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_g_c1_q_c16_traffic.md")


def recorded_traffic(workload: str):
    """HBM bytes per LM-head launch recorded by the FETCH_SIZE / WRITE_SIZE
    counter passes (profiles/lmhead_g_c1_q_c16_traffic.md) for this
    workload, or None when none were taken on it or they were taken on a
    different GEMM source than the one built now."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("    ") and ":" in line:
            k, v = line.strip().split(":", 1)
            vals[k.strip()] = v.strip()
    src = os.path.join(ROOT, "drafting_pd_expand_amd", "csrc", "gemm.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    key = f"traffic_bytes_per_launch_{workload}"
    if vals.get("gemm_source_sha256_16") != digest or key not in vals:
        return None
    return float(vals[key])


def ar_baseline(pdx, mdev, b, w, inp, cache, par_draft, stream, steps: int) -> dict:
    """The autoregressive K-pass baseline on the same kernels and inputs
    ([Blog] "background and motivation"): expand with K = 1, then K drafter
    passes, pass k >= 2 on one row per request (pd_ar_advance +
    pd_draft_forward_ex fed the previous pass's final hidden state). One
    "step" drafts the same K tokens per request as one parallel step. Every
    pass writes its KV rows, which the next pass (and step) overwrites."""
    import torch
    dev = torch.device("cuda:0")
    dm, C, K = w.model, b["C"], w.K
    dims1 = pdx.batch_dims(C, 1, b["T_in"], b["mask_id"], dm.hidden3, b["max_blocks"], b["num_blocks"])
    nd = dict(dims1, K=1, T_in=C)
    out1 = pdx.alloc_batch(dims1, dev)
    nxt = [pdx.alloc_batch(nd, dev) for _ in range(K - 1)]
    draft = [torch.empty(C, dtype=torch.int32, device=dev) for _ in range(K)]
    hid = [torch.empty((C, dm.d), dtype=torch.bfloat16, device=dev) for _ in range(K)]
    ha = pdx.Handle()
    bt = inp["block_table"]

    def ar_step():
        pdx.pd_expand_batch(dims1, inp, out1, stream)
        pdx.pd_draft_forward(ha, mdev, dims1, out1, bt, cache, draft[0], None, stream, hidden_out=hid[0])
        prev, pd = out1, dims1
        for k in range(1, K):
            pdx.pd_ar_advance(pd, prev, draft[k - 1], bt, nxt[k - 1], stream)
            pdx.pd_draft_forward(ha, mdev, nd, nxt[k - 1], bt, cache, draft[k], None, stream,
                                 hidden_d=hid[k - 1], hidden_out=hid[k])
            prev, pd = nxt[k - 1], nd

    for _ in range(3):
        ar_step()
    torch.cuda.synchronize()
    st = ha.status() | int(out1["status"].item())
    for t in nxt:
        st |= int(t["status"].item())
    if st:
        raise SystemExit(f"device status {st} in the autoregressive baseline")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(1, steps // 2)
    e0.record(stream)
    for _ in range(n):
        ar_step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    # pass 1 computes the parallel step's NTP rows; near-ties may round either way
    ntp = par_draft.view(C, K)[:, 0]
    agree = float((ntp == draft[0]).float().mean().item())
    ha.free()
    log(f"[bench] autoregressive baseline: {ms * 1000:.1f} us per {K}-token step")
    return {"ms_per_step": ms, "steps_per_s": 1000.0 / ms, "drafted_tok_per_s": 1000.0 / ms * C * K,
            "passes": K, "steps_timed": n, "pass1_equals_parallel_ntp_frac": agree}


def rounds_leg(pdx, mdev, w, stream, R: int = 8, reps: int = 5) -> dict:
    """R draft/verify rounds back to back on the device (NEXT-3): per round
    the stand-in verifier (pd_verify_stub) builds the verify window from the
    previous round's drafts, then pd_expand_batch + pd_draft_forward; the KV
    cache carries over and each round's verify rows rewrite the previous
    round's MASK-row entries. Timed eagerly and as one captured graph; every
    graph replay must reproduce the eager drafts of every round."""
    import torch
    import synth
    dev = torch.device("cuda:0")
    dm, K = w.model, w.K
    b = synth.make_batch(w, extra_positions=(R - 1) * (K + 1))
    rounds = synth.make_rounds(w, R)
    pool = synth.make_kv_pool(dm, b["num_blocks"], w.seed)
    C = b["C"]

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(dev).view(torch.bfloat16)

    cache = pdx.pack_kv_cache(bf16(pool["k"]), bf16(pool["v"]))
    d1 = pdx.batch_dims(C, K, b["T_in"], b["mask_id"], dm.hidden3, b["max_blocks"], b["num_blocks"])
    dims = [d1] + [dict(d1, T_in=C * (K + 1)) for _ in range(R - 1)]
    bt = i32(b["block_table"])
    inp = [{"num_tokens": i32(b["num_tokens"]), "num_rejected": i32(b["num_rejected"]),
            "target_ids": i32(b["target_ids"]), "target_pos": i32(b["target_pos"]),
            "target_hidden": bf16(b["target_hidden"]), "next_token_ids": i32(b["next_token_ids"]),
            "block_table": bt, "h_shared": mdev["h_shared"]}]
    acc = []
    for rd in rounds:
        inp.append({"num_tokens": torch.empty(C, dtype=torch.int32, device=dev),
                    "num_rejected": torch.empty(C, dtype=torch.int32, device=dev),
                    "target_ids": torch.empty(C * (K + 1), dtype=torch.int32, device=dev),
                    "target_pos": torch.empty(C * (K + 1), dtype=torch.int32, device=dev),
                    "target_hidden": bf16(rd["target_hidden"]), "next_token_ids": i32(rd["next_token_ids"]),
                    "block_table": bt, "h_shared": mdev["h_shared"]})
        acc.append(i32(rd["accepted"]))
    out = [pdx.alloc_batch(d, dev) for d in dims]
    draft = [torch.empty(C * K, dtype=torch.int32, device=dev) for _ in range(R)]
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    h = pdx.Handle()

    def run(s):
        for t in range(R):
            if t:
                pdx.pd_verify_stub(dims[t - 1], out[t - 1], draft[t - 1], inp[t - 1]["next_token_ids"], acc[t - 1],
                                   inp[t], st, s)
            pdx.pd_expand_batch(dims[t], inp[t], out[t], s)
            pdx.pd_draft_forward(h, mdev, dims[t], out[t], bt, cache, draft[t], None, s)

    run(stream)
    torch.cuda.synchronize()
    status = h.status() | int(st.item()) | int(sum(int(o["status"].item()) for o in out))
    if status:
        raise SystemExit(f"multi-round run: device status {status}")
    eager = [d.clone() for d in draft]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1000.0 / (reps * R)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        run(cap)
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            run(cap)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    ok = True
    for _ in range(3):
        for d in draft:
            d.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        ok = ok and all(bool(torch.equal(a, x)) for a, x in zip(draft, eager))
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1000.0 / (reps * R)
    del g
    h.free()
    log(f"[bench] {R} rounds: {eager_us:.1f} us per round eager, {graph_us:.1f} us per round as one graph, "
        f"replays match eager: {ok}")
    return {"rounds": R, "us_per_round_eager": eager_us, "us_per_round_graph": graph_us,
            "graph_replays_match_eager": ok,
            "accepted_mean": float(np.mean([rd["accepted"].mean() for rd in rounds]))}


def fp8_leg(pdx, mdev, w, b, dims, inp, cache, stream, steps: int, bf16_ids, bf16_attn_us: float) -> dict:
    """The same step over an fp8 (E4M3) KV cache (NEXT-2): the prior cache is
    the bf16 one rounded to E4M3 codes (per-layer scales from synth), new
    K/V are written as codes. Timed like the main leg, with HIP events
    around the attention kernel; its roofline counts one byte per cached K/V
    element."""
    import torch
    import synth
    dm, K = w.model, w.K
    sc = synth.kv_fp8_scales(dm, w.seed)
    pairs = np.stack([sc["k_scale"], sc["v_scale"]], axis=1)
    # codes of the prior cache: value / scale rounded by the library's E4M3 type (saturated first)
    N = dm.N
    src = cache.view(torch.bfloat16).view(N, 2, -1)
    cache8 = torch.empty(src.shape, dtype=torch.uint8, device=cache.device)
    for l in range(N):
        for t, s in ((0, float(sc["k_scale"][l])), (1, float(sc["v_scale"][l]))):
            cache8[l, t] = (src[l, t].float() / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    cache8 = cache8.view(cache.shape)
    out = pdx.alloc_batch(dims, cache.device)
    draft = torch.empty(b["C"] * K, dtype=torch.int32, device=cache.device)
    h = pdx.Handle()

    def step():
        pdx.pd_expand_batch(dims, inp, out, stream)
        pdx.pd_draft_forward(h, mdev, dims, out, inp["block_table"], cache8, draft, None, stream, kv_scales=pairs)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    st = h.status() | int(out["status"].item())
    if st:
        raise SystemExit(f"fp8 leg: device status {st}")
    h.profile(1 << pdx.KERNEL_ATTN)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    a_ms, a_n = h.profile_read(pdx.KERNEL_ATTN)
    h.profile(0)
    a_us = a_ms * 1000.0 / max(a_n, 1)
    v = b["num_tokens"] - b["num_rejected"]
    seq = b["context_lens"] + v + K - 1
    T_out = b["T_in"] + b["C"] * (K - 1)
    abytes = int(seq.sum()) * dm.Hkv * dm.dh * 2 + 2 * T_out * dm.Hq * dm.dh * 2
    agree = float((draft == bf16_ids).float().mean().item())
    h.free()
    log(f"[bench] fp8 KV cache: {ms * 1000:.1f} us/step, attention {a_us:.1f} us/launch "
        f"({abytes / (a_us * 1e-6) / 1e9:.0f} GB/s; bf16 cache {bf16_attn_us:.1f} us)")
    return {"ms_per_step": ms, "steps_per_s": 1000.0 / ms, "attention_us_per_launch": a_us,
            "attention_us_per_launch_bf16_cache": bf16_attn_us,
            "attention_roofline": {"bound": "hbm", "kernel": f"attn_split_kernel<{dm.dh}, fp8>",
                                   "achieved": abytes / (a_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": abytes / (a_us * 1e-6) / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": abytes},
            "draft_ids_equal_bf16_cache_frac": agree}


def partition_leg(pdx, stream, reps: int = 200, warmup: int = 50) -> dict:
    """Sequence partitioning ([Paper] sec. 3.2) on a training batch: 256
    sequences of 8192 tokens, K = 8 depths kept with COD decay r = 0.8 (the
    pages' 8192 / K = 8 / r = 0.8 example, ~34K positions each), 4 segments.
    HBM-bound: algorithmic bytes = keep bytes read + segment ids written +
    row lists written + boundaries and offsets."""
    import torch
    import synth
    dev = torch.device("cuda:0")
    B, n, K, S = 256, 8192, 8, 4
    keep_np = synth.make_cod_keep(B, n, K, 0.8, 7)
    placed = int(keep_np.sum())
    keep = torch.from_numpy(keep_np).to(dev)
    bnd = torch.tensor([[(s * n) // S for s in range(S + 1)]] * B, dtype=torch.int32, device=dev)
    seg = torch.empty((B, K, n), dtype=torch.int32, device=dev)
    off = torch.empty((B, S + 1), dtype=torch.int32, device=dev)
    rows = torch.empty((B, K * n), dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    # (the first few dozen calls run slower while the clocks settle)
    for _ in range(warmup):
        pdx.pd_seq_partition(keep, bnd, seg, off, rows, st, stream)
    torch.cuda.synchronize()
    if int(st.item()) != 0 or int(off[:, S].sum().item()) != placed:
        raise SystemExit("sequence partitioning: unexpected status or row count")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        pdx.pd_seq_partition(keep, bnd, seg, off, rows, st, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    alg = B * K * n + 4 * B * K * n + 4 * placed + 2 * 4 * B * (S + 1)
    gbs = alg / (us * 1e-6) / 1e9
    log(f"[bench] sequence partitioning: {us:.1f} us per call, {gbs:.0f} GB/s algorithmic")
    return {"workload": f"{B} sequences x {n} tokens, K={K}, COD r=0.8, S={S} ({placed} positions)",
            "us_per_call": us, "positions_per_s": placed / (us * 1e-6),
            "roofline": {"bound": "hbm", "kernel": "seq_partition_kernel", "achieved": gbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "bytes_per_call": alg}}


def yardsticks() -> dict:
    """Measured-peak yardsticks beside the spec peaks (not targets): a plain
    streaming read (sum of a 2 GiB bf16 tensor, fp32 accumulation in torch),
    a device-to-device copy of 1 GiB, and torch.matmul in bf16 (the installed
    vendor GEMM) at the C = 64, K = 7 LM-head shape (448 x 2880 by
    2880 x 201088), at the two largest projection shapes of that step (the
    rows its projections compute, the non-rejected ones: gate and up
    together, and down) and at a large square shape."""
    import torch
    import synth
    dev = torch.device("cuda:0")
    out = {}
    w = synth.get_workload("g_c64")
    bb = synth.make_batch(w)
    rows = int((bb["num_tokens"] - bb["num_rejected"] + w.K - 1).sum())

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1000.0

    x = torch.ones(1 << 30, dtype=torch.bfloat16, device=dev)          # 2 GiB
    t = timed(lambda: x.sum(dtype=torch.float32), 10)
    out["stream_read_GBps"] = x.numel() * 2 / t / 1e9
    del x
    a = torch.ones(1 << 28, dtype=torch.float32, device=dev)           # 1 GiB
    b = torch.empty_like(a)
    t = timed(lambda: b.copy_(a), 10)
    out["copy_GBps_read_plus_write"] = 2 * a.numel() * 4 / t / 1e9
    del a, b
    # the drafter's layout: weights row-major [N][K] (out x in), Y = X W^T
    # (a 2-D product with a transposed-view right operand: one library call,
    # no copy)
    for name, (M, K, N) in (("lm_head_c64_k7", (448, 2880, 201088)), ("gate_up_c64_k7", (rows, 2880, 15360)),
                            ("down_c64_k7", (rows, 7680, 2880)), ("square_8192", (8192, 8192, 8192))):
        A = torch.randn(M, K, dtype=torch.bfloat16, device=dev)
        W = torch.randn(N, K, dtype=torch.bfloat16, device=dev)
        t = timed(lambda: torch.matmul(A, W.t()), 10)
        out[f"matmul_bf16_{name}"] = {"shape_MKN": [M, K, N], "layout": "X[M][K] @ W[N][K]^T", "us": t * 1e6,
                                      "TFLOPs": 2.0 * M * N * K / t / 1e12,
                                      "frac_of_2500": 2.0 * M * N * K / t / 1e12 / BF16_PEAK_TFLOPS}
        del A, W
    torch.cuda.empty_cache()
    log(f"[bench] yardsticks: read {out['stream_read_GBps']:.0f} GB/s, copy {out['copy_GBps_read_plus_write']:.0f} "
        f"GB/s, matmul LM head {out['matmul_bf16_lm_head_c64_k7']['TFLOPs']:.0f} TFLOP/s, "
        f"gate/up {out['matmul_bf16_gate_up_c64_k7']['TFLOPs']:.0f}, down {out['matmul_bf16_down_c64_k7']['TFLOPs']:.0f}, "
        f"8192^3 {out['matmul_bf16_square_8192']['TFLOPs']:.0f} TFLOP/s")
    return out


def run_leg(workload: str, steps: int, warmup: int, extras: bool, cpu: bool, cpu_s: float = 10.0) -> dict:
    """One workload: warm-up, a timed region of plain launches (HIP events on
    the launch stream around each step and around the dominant kernel's
    launches), a second timed region with events around every GEMM launch
    (projections + LM head) for the GEMM roofline, and optionally the report
    extras (hipGraph replay, autoregressive baseline, sequence partitioning,
    fp8 cache, multi-round loop) and the CPU oracle baseline."""
    import torch
    import synth
    import drafting_pd_expand_amd as pdx

    def i32(a, dev):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    def bf16(a, dev):
        a = np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)
        return torch.from_numpy(a).to(dev).view(torch.bfloat16)

    dev = torch.device("cuda:0")
    w = synth.get_workload(workload)
    dm = w.model
    log(f"[bench] {workload}: generating model + inputs")
    t0 = time.perf_counter()
    model_np = synth.make_model(dm, seed=1234)
    b = synth.make_batch(w)
    pool = synth.make_kv_pool(dm, b["num_blocks"], w.seed)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
    mdev = pdx.device_model(model_np, dev)
    dims = pdx.batch_dims(b["C"], w.K, b["T_in"], b["mask_id"], dm.hidden3, b["max_blocks"], b["num_blocks"])
    inp = {
        "num_tokens": i32(b["num_tokens"], dev), "num_rejected": i32(b["num_rejected"], dev),
        "target_ids": i32(b["target_ids"], dev), "target_pos": i32(b["target_pos"], dev),
        "target_hidden": bf16(b["target_hidden"], dev), "next_token_ids": i32(b["next_token_ids"], dev),
        "block_table": i32(b["block_table"], dev), "h_shared": mdev["h_shared"],
    }
    out = pdx.alloc_batch(dims, dev)
    cache = pdx.pack_kv_cache(bf16(pool["k"], dev), bf16(pool["v"], dev))
    if not cpu:
        del pool
        pool = None
    R = b["C"] * w.K
    draft = torch.empty(R, dtype=torch.int32, device=dev)
    h = pdx.Handle()
    stream = torch.cuda.current_stream()

    def step(strm):
        pdx.pd_expand_batch(dims, inp, out, strm)
        pdx.pd_draft_forward(h, mdev, dims, out, inp["block_table"], cache, draft, None, strm)

    log(f"[bench] warmup {warmup}")
    for _ in range(max(1, warmup)):
        step(stream)
    torch.cuda.synchronize()
    st = h.status() | int(out["status"].item())
    if st:
        raise SystemExit(f"{workload}: device status {st} after warmup")
    eager_ids = draft.clone()

    # which kernel dominates: the persistent decode kernel (the whole pass in
    # one launch, at few rows), else the LM head (once per step: one launch,
    # or two when its last round of tiles goes to a second launch) or the
    # attention kernel (one launch per layer), from one step with events
    # around those classes
    h.profile((1 << pdx.KERNEL_LMHEAD) | (1 << pdx.KERNEL_ATTN) | (1 << pdx.KERNEL_DECODE))
    step(stream)
    torch.cuda.synchronize()
    lm_ms, lm_n = h.profile_read(pdx.KERNEL_LMHEAD)
    at_ms, at_n = h.profile_read(pdx.KERNEL_ATTN)
    de_ms, de_n = h.profile_read(pdx.KERNEL_DECODE)
    h.profile(0)
    if de_n > 0:
        dom = "decode"
    else:
        dom = "lm_head" if lm_ms >= at_ms / max(at_n, 1) else "attention"
    dom_cls = {"decode": pdx.KERNEL_DECODE, "lm_head": pdx.KERNEL_LMHEAD, "attention": pdx.KERNEL_ATTN}[dom]

    def timed_region(class_mask):
        h.profile(class_mask)
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(stream)
        for i in range(steps):
            step(stream)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
        return evs[0].elapsed_time(evs[-1]) / steps, per

    # timed region: plain launches; events around the dominant kernel only
    log(f"[bench] {workload}: timing {steps} steps (plain launches)")
    w0 = time.perf_counter()
    ms_step, per = timed_region(1 << dom_cls)
    wall = time.perf_counter() - w0
    k_ms, k_n = h.profile_read(dom_cls)
    h.profile(0)
    lm_launches = k_n // steps if dom == "lm_head" else 1
    if dom == "lm_head":   # the LM head's time per step (both launches when split)
        k_n = steps
    steps_s = 1000.0 / ms_step
    k_avg_s = k_ms / max(k_n, 1) / 1000.0

    # second timed region: events around every GEMM launch (and nothing else);
    # the decode kernel runs its GEMMs inside one launch, so there are none
    ms_g, _ = timed_region((1 << pdx.KERNEL_LMHEAD) | (1 << pdx.KERNEL_GEMM))
    g_ms, g_n = h.profile_read(pdx.KERNEL_GEMM)
    l_ms, l_n = h.profile_read(pdx.KERNEL_LMHEAD)
    h.profile(0)
    gemm_us = (g_ms + l_ms) * 1000.0 / steps
    proj_us = g_ms * 1000.0 / steps
    lm_us = l_ms * 1000.0 / steps
    gf = gemm_flops(dm, b, w.K)
    lm_flops = 2.0 * R * dm.V * dm.d

    if dom == "decode":
        fb = forward_bytes(dm, b, w.K)
        roof = {"bound": "hbm", "kernel": "decode_kernel (persistent: the whole drafter pass in one launch)",
                "achieved": fb / k_avg_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes_per_launch": fb}
    elif dom == "lm_head":
        kname = ("gemm_ring_kernel<ARGMAX>" if R <= 64 else "gemm_ring_kernel<ARGMAX, 8 X tiles>" if R <= 128
                 else "gemm_big_kernel<ARGMAX, 256-row tiles>" if lm_launches == 1
                 else "gemm_big_kernel<ARGMAX>, 256-row tiles + a last-round launch on 128-row tiles")
        # R flop per weight byte: below the ridge (peak flops / peak bytes) the
        # weight stream bounds it, above it the matrix cores
        if R < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            roof = {"bound": "hbm", "kernel": f"{kname} (LM head + fused argmax)",
                    "achieved": lm_head_bytes(dm, R) / k_avg_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        else:
            roof = {"bound": "mfma", "kernel": f"{kname} (LM head + fused argmax)",
                    "achieved": lm_flops / k_avg_s / 1e12, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "kernel": f"attn_split_kernel<{dm.dh}> (paged split-KV attention)",
                "achieved": attn_bytes(dm, b, w.K) / k_avg_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = recorded_traffic(workload) if dom == "lm_head" else None
    roof["us_per_launch"] = k_avg_s * 1e6   # (the LM head: per step, over its launches)
    if dom == "lm_head":
        roof["launches_per_step"] = lm_launches
    sb = step_bytes(dm, b, w.K)
    v = b["num_tokens"] - b["num_rejected"]
    T_eff = int((v + w.K - 1).sum())
    log(f"[bench] {workload}: {ms_step * 1000:.1f} us/step ({steps_s:.1f} steps/s, {steps_s * R:.0f} drafted tok/s); "
        f"dominant {dom} {k_avg_s * 1e6:.1f} us = {roof['achieved']:.0f} {roof['unit']} ({roof['frac']:.2f}); "
        f"step {sb / 1e9:.3f} GB = {sb / (ms_step / 1000) / 1e9 / HBM_PEAK_GBS:.2f} of HBM; GEMMs {gemm_us:.0f} us "
        f"(in a {ms_g * 1000:.0f} us step) = {gf / max(gemm_us * 1e-6, 1e-12) / 1e12:.0f} TFLOP/s on {T_eff} rows")
    leg = {
        "workload": f"{workload}: {DESCR[workload]}",
        "C": w.C, "K": w.K, "T_in": b["T_in"], "T_out": b["T_in"] + w.C * (w.K - 1), "T_eff": T_eff,
        "us_per_step": ms_step * 1000.0,
        "steps_per_s": steps_s,
        "drafted_tok_per_s": steps_s * R,
        "ms_per_step_p10_p50_p90": [float(np.percentile(per, q)) for q in (10, 50, 90)],
        "wall_us_per_step": wall * 1e6 / steps,
        "step_algorithmic_bytes": sb,
        "step_hbm_frac": sb / (ms_step / 1000) / 1e9 / HBM_PEAK_GBS,
        "roofline": roof,
        "gemm_roofline": None if (g_n + l_n) == 0 or gemm_us < 1.0 else {
            "bound": "mfma", "kernels": "every projection GEMM + the LM head",
            "flops_per_step": gf, "rows_credited": T_eff,
            "us_per_step": gemm_us, "projections_us": proj_us, "lm_head_us": lm_us,
            "launches_per_step": (g_n + l_n) // steps,
            "achieved": gf / max(gemm_us * 1e-6, 1e-12) / 1e12, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": gf / max(gemm_us * 1e-6, 1e-12) / 1e12 / BF16_PEAK_TFLOPS,
            "step_us_in_this_region": ms_g * 1000.0,
        },
    }
    if extras:
        leg["hipgraph"] = graph_leg(step, draft, eager_ids, stream, steps)
        ar = ar_baseline(pdx, mdev, b, w, inp, cache, draft, stream, steps)
        ar["parallel_speedup"] = ar["ms_per_step"] / ms_step
        leg["ar_baseline"] = ar
        leg["seq_partition"] = partition_leg(pdx, stream)
        leg["kv_fp8"] = fp8_leg(pdx, mdev, w, b, dims, inp, cache, stream, max(5, steps // 2), eager_ids,
                                at_ms * 1000.0 / max(at_n, 1))
        leg["multi_round"] = rounds_leg(pdx, mdev, w, stream)
    h.free()
    del cache, mdev, inp, out
    torch.cuda.empty_cache()
    if cpu:
        log(f"[bench] {workload}: timing the CPU oracle on a bounded sample")
        c = cpu_baseline(w, model_np, b, pool, min_s=cpu_s)
        log(f"[bench] oracle {c['seconds']:.2f} s on {c['cores']} cores")
        c.pop("seconds")
        leg["cpu_baseline"] = c
    return leg


def graph_leg(step, draft, eager_ids, stream, steps: int) -> dict:
    """The same step captured once as a hipGraph and replayed; every
    replay's draft ids must equal the eager ones."""
    import torch
    try:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            step(cap)   # warm the capture stream (no allocation happens: the handle is sized)
            cap.synchronize()
            with torch.cuda.graph(g, stream=cap):
                step(cap)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        ok = True
        for _ in range(3):
            draft.zero_()
            g.replay()
            torch.cuda.synchronize()
            ok = ok and bool(torch.equal(draft, eager_ids))
        ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ge0.record(stream)
        for _ in range(steps):
            g.replay()
        ge1.record(stream)
        torch.cuda.synchronize()
        g_ms = ge0.elapsed_time(ge1) / steps
        log(f"[bench] hipGraph replay {g_ms * 1000:.1f} us/step, draft ids match eager: {ok}")
        del g
        return {"steps_per_s": 1000.0 / g_ms, "ms_per_step": g_ms, "replays_match_eager": ok}
    except Exception as ex:  # graph capture is a report extra; the plain-launch number stands
        log(f"[bench] hipGraph replay skipped: {ex}")
        return {"error": str(ex)[:200]}


CONFIG_LEGS = ["g_c4", "g_c64", "g_c64_k3", "g_c64_k5", "q_c16"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="g_c1", choices=sorted(DESCR),
                    help="the headline workload (value, roofline, cpu_baseline and the report extras)")
    ap.add_argument("--configs", default=",".join(CONFIG_LEGS),
                    help="comma-separated further workloads timed after the headline one ('none' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the headline leg's report extras")
    ap.add_argument("--no-yardsticks", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the drafting step runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import drafting_pd_expand_amd as pdx
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pdx.load()
    legs = [c for c in args.configs.split(",") if c and c != "none" and c != args.workload]
    for c in legs:
        if c not in DESCR:
            raise SystemExit(f"unknown workload {c}")
    head = run_leg(args.workload, args.steps, args.warmup, extras=not args.no_extras,
                   cpu=not args.no_cpu_baseline, cpu_s=10.0)
    configs = {args.workload: {k: head[k] for k in ("us_per_step", "steps_per_s", "drafted_tok_per_s",
                                                     "step_hbm_frac", "roofline", "gemm_roofline")}}
    for c in legs:
        leg = run_leg(c, args.steps, max(2, args.warmup // 2), extras=False, cpu=not args.no_cpu_baseline,
                      cpu_s=4.0)
        configs[c] = leg
    ys = None if args.no_yardsticks else yardsticks()

    res = {
        "metric": "draft steps/s & drafted tok/s (K=7) at C=1/4/64; % HBM / MFMA roofline",
        "value": head["steps_per_s"],
        "unit": "draft steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_step"] / 1000.0,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "C": head["C"], "K": head["K"], "T_in": head["T_in"],
                   "T_out": head["T_out"]},
        "drafted_tok_per_s": head["drafted_tok_per_s"],
        "ms_per_step_p10_p50_p90": head["ms_per_step_p10_p50_p90"],
        "step_hbm_frac": head["step_hbm_frac"],
        "step_algorithmic_bytes": head["step_algorithmic_bytes"],
        "gemm_mfma_frac": head["gemm_roofline"]["frac"] if head["gemm_roofline"] else None,
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "configs": configs,
        "yardsticks": ys,
    }
    for k in ("hipgraph", "ar_baseline", "seq_partition", "kv_fp8", "multi_round"):
        if k in head:
            res[k] = head[k]
    print(json.dumps(res))


if __name__ == "__main__":
    main()
