"""GPU parity of the whole drafting step (pd_expand_batch + pd_draft_forward,
through the C ABI) against the oracle.

Small models cover every row (and the residual stream layer by layer); the
full-size workloads are checked on every request when the oracle is quick
(C <= 4) and on sampled requests otherwise (requests are independent, so a
request's outputs can be computed alone). Also: K = 1, dh = 128, GQA groups
of 1, 4 and 8, causality and determinism (bit-identical), page relabelling
(bit-identical), request independence, and the status word on bad data.
"""
import numpy as np
import pytest
import torch

import synth
from harness import Case, check_case, check_logits, gpu_expand

pytestmark = pytest.mark.gpu

GQA64 = synth.ModelDims("gqa64", d=256, Hq=8, Hkv=2, dh=64, F=512, N=2, V=2048)
GQA128 = synth.ModelDims("gqa128", d=512, Hq=4, Hkv=1, dh=128, F=1024, N=2, V=1024)


def _say(msg):
    print(msg, flush=True)


def test_tiny_prefill_all_rows_and_layers():
    w = synth.get_workload("tiny")
    _say(f"[forward] tiny C={w.C} K={w.K}")
    c = Case(w, debug_resid=True).run()
    assert c.status() == 0
    res = check_case(c, check_layers=True)
    _say(f"  worst logit err/RMS {res['worst_logit_ratio']:.4g}")
    c.close()


@pytest.mark.parametrize("dims,C,K,ctx,L", [
    (GQA64, 5, 5, "lognormal", 0),
    (GQA64, 4, 1, "fixed", 777),
    (GQA64, 3, 16, "fixed", 40),
    (GQA128, 3, 7, "fixed", 1000),
    (GQA128, 2, 3, "lognormal", 0),
    # 65..128 sampled rows: the LM head on the 8-tile weight-streaming ring, every row checked
    (GQA64, 13, 7, "lognormal", 0),
    (GQA128, 16, 8, "fixed", 300),
], ids=["gqa64-c5k5", "gqa64-k1", "gqa64-k16", "gqa128-c3k7", "gqa128-c2k3", "gqa64-c13k7-lm",
        "gqa128-c16k8-lm"])
def test_small_models_all_rows(dims, C, K, ctx, L):
    w = synth.Workload(f"{dims.name}-c{C}k{K}", dims, C=C, K=K, context=ctx, L=L, seed=17 + C + K)
    _say(f"[forward] {w.name}")
    c = Case(w, debug_resid=True).run()
    assert c.status() == 0
    res = check_case(c, check_layers=True)
    _say(f"  worst logit err/RMS {res['worst_logit_ratio']:.4g}")
    c.close()


# Widths that are multiples of 16 but not of 32, 128 or 256 (d 208, 3d 624,
# F 688, V 1008): every GEMM kernel meets a partial last K stage and partial
# column and row tiles. The batch shapes pick the kernel by row count: 768
# expanded rows and 384 sampled rows (256-row ring-fed tiles), 576 expanded
# and 288 sampled rows (the LM head on 128-row ring-fed tiles), 128 rows
# (the projections on 128-row ring-fed tiles), 96 sampled rows (the LM head on
# the 8-tile weight-streaming ring with 64-element stages: a partial last
# column tile and a partial last stage), 64 and 10 sampled rows and 20
# expanded rows (weight-streaming kernel).
RAGGED = synth.ModelDims("ragged", d=208, Hq=4, Hkv=2, dh=64, F=688, N=2, V=1008)


@pytest.mark.parametrize("C,K,L", [(48, 8, 90), (36, 8, 60), (12, 8, 40), (8, 8, 300), (2, 5, 33)],
                         ids=["rows768", "rows576", "rows192-lm96", "rows128", "rows16"])
def test_ragged_widths_all_rows(C, K, L):
    w = synth.Workload(f"ragged-c{C}k{K}", RAGGED, C=C, K=K, context="fixed", L=L, seed=5 + C)
    _say(f"[forward] {w.name}")
    c = Case(w, debug_resid=True).run()
    assert c.status() == 0
    res = check_case(c, check_layers=True)
    _say(f"  worst logit err/RMS {res['worst_logit_ratio']:.4g}")
    c.close()


# An LM head of 288 sampled rows over V = 33040 columns: on 256-row tiles
# 130 column tiles x 2 row blocks = 260 tiles, 4 past one round of 256, so it
# runs as two launches, columns 0..32767 on 256-row tiles and the last 272
# (a partial last tile) on 128-row tiles; every row's logits and argmax are
# checked across the seam.
LMSPLIT = synth.ModelDims("lmsplit", d=208, Hq=4, Hkv=2, dh=64, F=688, N=1, V=33040)


def test_lm_head_in_two_launches():
    w = synth.Workload("lmsplit-c36k8", LMSPLIT, C=36, K=8, context="fixed", L=60, seed=41)
    _say(f"[forward] {w.name}")
    c = Case(w).run()
    assert c.status() == 0
    res = check_case(c, check_cache=False)
    assert res["rows"] == 36 * 8
    # the fused argmax of every row equals the argmax of the logits the same
    # launches wrote (lowest index on ties), whichever launch holds it: the
    # second launch reports its columns with their offset (with this seed the
    # oracle's maximum of one row lies past column 32768)
    lg = c.logits.cpu().numpy()
    got = c.draft.cpu().numpy()
    assert np.array_equal(got, np.argmax(lg, axis=1))
    _say(f"  worst logit err/RMS {res['worst_logit_ratio']:.4g}, argmax checked {res['argmax_checked']}, "
         f"argmax past the seam in {int((got >= 32768).sum())} rows")
    c.close()


@pytest.mark.parametrize("C,K,L", [(48, 8, 90), (8, 8, 300)], ids=["rows768", "rows128"])
def test_every_row_computed(C, K, L, monkeypatch):
    """Passes of more than 64 rows normally compute only the rows that are
    not rejected (gathered to the front on the device); with PD_COMPACT=0
    every row is computed in place. Both are checked against the oracle, and
    the sampled rows' logits of the two agree."""
    w = synth.Workload(f"ragged-c{C}k{K}", RAGGED, C=C, K=K, context="fixed", L=L, seed=5 + C)
    _say(f"[forward] {w.name} every row computed")
    monkeypatch.setenv("PD_COMPACT", "0")
    full = Case(w, debug_resid=True).run()
    assert full.status() == 0
    check_case(full, check_layers=True)
    monkeypatch.setenv("PD_COMPACT", "1")
    comp = Case(w, debug_resid=True).run()
    assert comp.status() == 0
    check_case(comp, check_layers=True)
    a, b = full.logits.cpu().numpy(), comp.logits.cpu().numpy()
    rms = np.sqrt(np.mean(a.astype(np.float64) ** 2, axis=1, keepdims=True))
    assert np.max(np.abs(a - b) / rms) < 0.03
    full.close()
    comp.close()


@pytest.mark.parametrize("C,K,n,accept,L", [(1, 2, 64, "uniform", 40), (9, 8, 0, "all", 50), (8, 4, 0, "uniform", 70)],
                         ids=["rows65-two-kept", "rows144-none-rejected", "rows64"])
def test_compaction_edges(C, K, n, accept, L):
    """Row compaction at its edges: 65 expanded rows (the first size that is
    compacted; 63 of them rejected), a batch with no rejected row (every row
    kept) and 64 rows (the last size computed in place); all rows and the
    residual stream layer by layer against the oracle."""
    w = synth.Workload(f"ragged-c{C}k{K}-{accept}", RAGGED, C=C, K=K, context="fixed", L=L, n_verify=n,
                       accept=accept, seed=11 + C)
    b = synth.make_batch(w)
    T_out = int(b["num_tokens"].sum()) + C * (K - 1)
    _say(f"[forward] {w.name}: {T_out} expanded rows")
    c = Case(w, debug_resid=True, batch=b).run()
    assert c.status() == 0
    res = check_case(c, check_layers=True)
    _say(f"  worst logit err/RMS {res['worst_logit_ratio']:.4g}")
    c.close()


def _sample(b, K, k=3):
    """Requests to check at large C: the longest context, the most rejections, the first."""
    L = b["context_lens"]
    picks = [int(np.argmax(L)), int(np.argmax(b["num_rejected"])), 0]
    out = []
    for p in picks:
        if p not in out:
            out.append(p)
    return out[:k]


@pytest.mark.parametrize("C,K,L", [(300, 3, 200), (1024, 2, 40)], ids=["c300", "c1024-max"])
def test_many_requests_sampled(C, K, L):
    """Large batches up to the 1024-request limit (plan, expansion and merge
    over many requests): the whole expansion bit-exact, logits and argmax on
    a spread of sampled requests (requests are independent)."""
    w = synth.Workload(f"gqa64-c{C}", GQA64, C=C, K=K, context="fixed", L=L, seed=C + K)
    _say(f"[forward] {w.name} K={K}")
    c = Case(w).run()
    assert c.status() == 0
    reqs = sorted(set([0, C - 1, C // 2] + list(np.random.default_rng(C).choice(C, 5, replace=False))))
    res = check_case(c, requests=reqs, check_cache=False)
    _say(f"  worst logit err/RMS {res['worst_logit_ratio']:.4g} over {len(reqs)} requests")
    c.close()


@pytest.mark.parametrize("dims", [GQA64, GQA128], ids=["dh64", "dh128"])
def test_merge_many_rows_many_splits(dims):
    """64 requests x 16 draft positions (over 1000 rows: the merge takes
    several heads per wave) with lognormal contexts, so the longest requests
    have 30-60 splits and the merge walks several chunks of partials per
    head. The longest requests and request 0 are checked."""
    w = synth.Workload(f"{dims.name}-c64k16", dims, C=64, K=16, context="lognormal", seed=47)
    _say(f"[forward] {w.name}")
    c = Case(w).run()
    assert c.status() == 0
    L = c.b["context_lens"]
    reqs = sorted(set([0] + [int(i) for i in np.argsort(L)[-2:]]))
    res = check_case(c, requests=reqs, check_cache=False)
    _say(f"  contexts {[int(L[r]) for r in reqs]}: worst logit err/RMS {res['worst_logit_ratio']:.4g}")
    c.close()


@pytest.mark.parametrize("name", ["g_c1", "g_c4", "g_c64", "g_c64_k3", "g_c64_k5", "q_c16"])
def test_full_size_workloads(name):
    w = synth.get_workload(name)
    _say(f"[forward] {name} C={w.C} K={w.K}")
    c = Case(w).run()
    assert c.status() == 0
    reqs = None if w.C <= 4 else _sample(c.b, w.K, 3 if w.C >= 64 else 2)
    res = check_case(c, requests=reqs)
    _say(f"  requests {reqs or 'all'}: worst logit err/RMS {res['worst_logit_ratio']:.4g}, "
         f"argmax checked {res['argmax_checked']}/{res['rows']}")
    c.close()


def test_causality_and_determinism_bit_identical():
    """(c) perturbing the last MASK row of every request changes nothing before
    it; a repeated step is bit-identical."""
    w = synth.Workload("gqa64-causal", GQA64, C=4, K=6, context="lognormal", seed=23)
    c = Case(w).run()
    base = c.logits.clone()
    base_ids = c.draft.clone()
    c.run()
    assert torch.equal(c.logits, base) and torch.equal(c.draft, base_ids)
    nti = c.out["new_token_indices"].cpu().numpy().reshape(w.C, w.K)
    last = torch.from_numpy(nti[:, -1].astype(np.int64)).to(c.dev)
    g = torch.Generator(device="cpu").manual_seed(3)
    noise = torch.randn((w.C, w.model.hidden3), generator=g).to(torch.bfloat16).to(c.dev)
    c.out["hidden"][last] = noise
    c.out["input_ids"][last] = 7
    c.run()
    keep = np.array([r * w.K + m for r in range(w.C) for m in range(w.K - 1)])
    keep_t = torch.from_numpy(keep).to(c.dev)
    assert torch.equal(c.logits[keep_t], base[keep_t])
    lastrows = torch.arange(w.K - 1, w.C * w.K, w.K, device=c.dev)
    assert not torch.equal(c.logits[lastrows], base[lastrows])
    c.close()


def test_page_relabelling_is_bit_identical():
    w = synth.Workload("gqa64-pages", GQA64, C=3, K=5, context="lognormal", seed=29)
    c1 = Case(w).run()
    b = dict(c1.b)
    nb = b["num_blocks"]
    perm = np.random.default_rng(1).permutation(nb)          # old page -> new page
    bt = b["block_table"]
    b["block_table"] = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    c2 = Case(w, batch=b)
    src = np.argsort(perm)
    sl = (src[:, None] * 16 + np.arange(16)).reshape(-1)
    import drafting_pd_expand_amd as pdx
    from harness import bf16
    k = bf16(c1.pool["k"][:, sl], c2.dev)
    v = bf16(c1.pool["v"][:, sl], c2.dev)
    c2.cache = pdx.pack_kv_cache(k, v)
    c2.run()
    assert torch.equal(c1.logits, c2.logits)
    assert torch.equal(c1.draft, c2.draft)
    c1.close(); c2.close()


def test_request_alone_matches_batch():
    w = synth.Workload("gqa64-indep", GQA64, C=4, K=5, context="lognormal", seed=31)
    c = Case(w).run()
    r = 2
    b = c.b
    lo = int(b["num_tokens"][:r].sum())
    hi = lo + int(b["num_tokens"][r])
    one = dict(b)
    one.update(C=1, T_in=hi - lo, num_tokens=b["num_tokens"][r:r + 1], num_rejected=b["num_rejected"][r:r + 1],
               target_ids=b["target_ids"][lo:hi], target_pos=b["target_pos"][lo:hi],
               target_hidden=b["target_hidden"][lo:hi], next_token_ids=b["next_token_ids"][r:r + 1],
               block_table=b["block_table"][r:r + 1], context_lens=b["context_lens"][r:r + 1])
    c1 = Case(w, batch=one).run()
    got = c1.logits.cpu().numpy()
    want = c.logits[r * w.K:(r + 1) * w.K].cpu().numpy().astype(np.float64)
    check_logits(got, want, tol=0.01)
    c.close(); c1.close()


def test_bad_token_and_page_flagged_in_forward():
    """Bad ids / slots reaching the forward are flagged and skipped (no fault)."""
    w = synth.Workload("gqa64-bad", GQA64, C=2, K=3, context="fixed", L=50, seed=37)
    c = Case(w)
    c.out["input_ids"][0] = GQA64.V + 5
    c.out["slot_mapping"][1] = 10 ** 8
    c.run()
    st = c.handle.status()
    assert st & 8 and st & 4
    c.close()


@pytest.mark.parametrize("dims,C,K,ctx,L", [(GQA64, 5, 5, "lognormal", 0), (GQA128, 3, 7, "fixed", 1001)],
                         ids=["gqa64", "gqa128"])
def test_nonfinite_cache_tails_do_not_leak(dims, C, K, ctx, L):
    """Slots past a request's last key inside its last page are not context:
    filled with NaN / +-Inf bf16 codes they must not reach any output."""
    import drafting_pd_expand_amd as pdx
    from harness import bf16, poison_slots, tail_slots
    w = synth.Workload(f"{dims.name}-nan-tail-c{C}k{K}", dims, C=C, K=K, context=ctx, L=L, seed=61 + C)
    _say(f"[forward] {w.name}")
    c = Case(w)
    sl = tail_slots(c.b, c.mnp["h_shared"], K)
    assert len(sl) > 0
    poison_slots(c.pool, sl, [0x7FC0, 0x7F80, 0xFF80, 0xFFC1])
    c.cache = pdx.pack_kv_cache(bf16(c.pool["k"], c.dev), bf16(c.pool["v"], c.dev))
    c.run()
    assert c.status() == 0
    res = check_case(c)
    _say(f"  {len(sl)} poisoned slots; worst logit err/RMS {res['worst_logit_ratio']:.4g}")
    c.close()
