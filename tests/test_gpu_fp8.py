"""GPU parity of the drafting step over an fp8 (E4M3) KV cache
(pd_draft_forward_ex with kv_fp8, through the C ABI) against the oracle's
fp8 mode.

The prior cache holds E4M3 codes (synth), read as code value * per-layer
scale on both sides; the new K/V rows are stored as codes of value / scale.
Bar: logits within 0.03 x RMS of the oracle row, argmax where the oracle's
top-2 margin > 0.05; every code written this step decodes to within
0.03 x RMS of its oracle row plus one code step of the oracle value (the
GPU quantizes fp32 values, the oracle fp64 ones, so a value near a rounding
boundary may land on the neighbouring code); every other byte of the cache
unchanged. Small models on every row (dh 64 and 128), the full-size drafters
on sampled requests, a multi-round run (stale MASK-row codes overwritten),
and the bf16 path unaffected.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import (LOGIT_TOL, assert_expansion_equal, bits, check_argmax, check_logits, expansion_to_np,
                     gpu_expand, model_dev, model_np, oracle_expand)

pytestmark = pytest.mark.gpu

GQA64 = synth.ModelDims("gqa64", d=256, Hq=8, Hkv=2, dh=64, F=512, N=2, V=2048)
GQA128 = synth.ModelDims("gqa128", d=512, Hq=4, Hkv=1, dh=128, F=1024, N=2, V=1024)


def _say(msg):
    print(msg, flush=True)


def _codes(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)


class Fp8Case:
    def __init__(self, w: synth.Workload, model_seed: int = 1234):
        import drafting_pd_expand_amd as pdx
        self.w, self.dm, self.K = w, w.model, w.K
        dev = self.dev = torch.device("cuda:0")
        self.mnp = model_np(self.dm, model_seed)
        self.mdev = model_dev(self.dm, model_seed)
        self.b = synth.make_batch(w)
        self.pool = synth.make_kv_pool(self.dm, self.b["num_blocks"], w.seed, fp8=True)
        self.scales = synth.kv_fp8_scales(self.dm, w.seed)
        self.kv8 = {"k_scale": self.scales["k_scale"].astype(np.float64),
                    "v_scale": self.scales["v_scale"].astype(np.float64)}
        self.dims, self.inp, self.out = gpu_expand(self.b, self.mnp["h_shared"], self.K, dev)
        self.cache = pdx.pack_kv_cache_fp8(_codes(self.pool["k"], dev), _codes(self.pool["v"], dev))
        R = self.b["C"] * self.K
        self.draft = torch.empty(R, dtype=torch.int32, device=dev)
        self.logits = torch.empty((R, self.dm.V), dtype=torch.float32, device=dev)
        self.handle = pdx.Handle()

    def scale_pairs(self):
        return np.stack([self.scales["k_scale"], self.scales["v_scale"]], axis=1)

    def run(self):
        import drafting_pd_expand_amd as pdx
        pdx.pd_draft_forward(self.handle, self.mdev, self.dims, self.out, self.inp["block_table"], self.cache,
                             self.draft, self.logits, kv_scales=self.scale_pairs())
        torch.cuda.synchronize()
        return self

    def status(self):
        return self.handle.status() | int(self.out["status"].cpu().item())


def check_fp8_kv(dm, cache, pool, kv8, written_list):
    """written_list: the oracle's kv_written of every pass, in order (later wins)."""
    import drafting_pd_expand_amd as pdx
    gk, gv = pdx.unpack_kv_cache(cache, dm.Hkv, dm.dh)
    gk, gv = gk.cpu().numpy(), gv.cpu().numpy()
    final = {}
    for written in written_list:
        for l, (sl, kk, vv) in enumerate(written):
            for j, s in enumerate(sl):
                final[(l, int(s))] = (kk[j], vv[j])
    keep = np.ones(gk.shape[1], bool)
    keep[np.unique([s for (_, s) in final])] = False
    assert np.array_equal(gk[:, keep], pool["k"][:, keep]), "K codes changed outside the written slots"
    assert np.array_equal(gv[:, keep], pool["v"][:, keep]), "V codes changed outside the written slots"
    worst = 0.0
    for (l, s), (kk, vv) in final.items():
        for name, gc, o, sc in (("k", gk, kk, kv8["k_scale"][l]), ("v", gv, vv, kv8["v_scale"][l])):
            gg = oracle.fp8.e4m3_decode(gc[l][s]).reshape(-1) * sc
            oo = np.asarray(o).reshape(-1)
            rms = np.sqrt(np.mean(oo * oo))
            step = np.maximum(2.0 ** -3 * np.abs(oo), 2.0 ** -9 * sc)   # one code step at the oracle value
            lim = LOGIT_TOL * rms + step
            err = np.abs(gg - oo)
            assert np.all(err <= lim), f"layer {l} slot {s} {name}: fp8 cache off by {np.max(err - lim):.4g}"
            worst = max(worst, float(np.max(err / rms)))
    return worst


def check_fp8_case(c: Fp8Case, requests=None):
    exp = oracle_expand(c.b, c.mnp["h_shared"], c.K)
    assert_expansion_equal(expansion_to_np(c.out, c.dims), exp)
    ora = oracle.draft_forward(c.mnp, exp, c.b["block_table"], c.pool, c.K, requests=requests,
                               block_size=c.b["block_size"], kv_fp8=c.kv8)
    reqs = ora["requests"]
    sel = np.concatenate([np.arange(r * c.K, (r + 1) * c.K) for r in reqs])
    gl = c.logits.cpu().numpy()[sel]
    worst = check_logits(gl, ora["logits"])
    n = check_argmax(c.draft.cpu().numpy()[sel], ora["logits"])
    kvw = None
    if requests is None:
        kvw = check_fp8_kv(c.dm, c.cache, c.pool, c.kv8, [ora["kv_written"]])
    _say(f"[parity] fp8 {c.w.name}: rows {len(sel)}, worst logit err/RMS {worst:.4f}, argmax checked {n}"
         + (f", worst cache err/RMS {kvw:.4f}" if kvw is not None else ""))


@pytest.mark.parametrize("dims,C,K,ctx,L", [
    (GQA64, 5, 5, "lognormal", 0),
    (GQA64, 3, 16, "fixed", 40),
    (GQA128, 3, 7, "fixed", 1000),
    (GQA128, 2, 1, "lognormal", 0),
], ids=["gqa64-c5k5", "gqa64-k16", "gqa128-c3k7", "gqa128-k1"])
def test_fp8_small_models_all_rows(dims, C, K, ctx, L):
    w = synth.Workload(f"{dims.name}-fp8-c{C}k{K}", dims, C=C, K=K, context=ctx, L=L, seed=91 + C + K)
    _say(f"[fp8] {w.name}")
    c = Fp8Case(w).run()
    assert c.status() == 0
    check_fp8_case(c)
    c.handle.free()


@pytest.mark.parametrize("name", ["g_c4", "q_c16", "g_c64"])
def test_fp8_full_size_sampled(name):
    w = synth.get_workload(name)
    _say(f"[fp8] {name}")
    c = Fp8Case(w).run()
    assert c.status() == 0
    b = c.b
    L = b["context_lens"]
    reqs = sorted({int(np.argmax(L)), int(np.argmax(b["num_rejected"])), 0}) if w.C > 4 else None
    check_fp8_case(c, requests=reqs)
    c.handle.free()


def test_fp8_multi_round_overwrites_stale_codes():
    """Three rounds over an fp8 cache: each round's verify rows rewrite the
    previous round's MASK-row codes before anything reads them."""
    import drafting_pd_expand_amd as pdx
    from test_gpu_rounds import Rounds
    w = synth.Workload("gqa64-fp8-rounds", GQA64, C=3, K=3, context="lognormal", seed=97)
    R = 3
    _say(f"[fp8] rounds {w.name} R={R}")
    rr = Rounds(w, R)
    dev = rr.dev
    pool8 = synth.make_kv_pool(rr.dm, rr.b["num_blocks"], w.seed, fp8=True)
    sc = synth.kv_fp8_scales(rr.dm, w.seed)
    pairs = np.stack([sc["k_scale"], sc["v_scale"]], axis=1)
    rr.cache = pdx.pack_kv_cache_fp8(_codes(pool8["k"], dev), _codes(pool8["v"], dev))
    for t in range(R):
        if t > 0:
            pdx.pd_verify_stub(rr.dims[t - 1], rr.out[t - 1], rr.draft[t - 1], rr.inp[t - 1]["next_token_ids"],
                               rr.accepted[t - 1], rr.inp[t], rr.stub_status)
        pdx.pd_expand_batch(rr.dims[t], rr.inp[t], rr.out[t])
        pdx.pd_draft_forward(rr.handle, rr.mdev, rr.dims[t], rr.out[t], rr.inp[t]["block_table"], rr.cache,
                             rr.draft[t], rr.logits[t], kv_scales=pairs)
    torch.cuda.synchronize()
    assert rr.status() == 0
    b = rr.b
    args1 = {k: b[k] for k in ("num_tokens", "num_rejected", "target_ids", "target_pos", "target_hidden",
                               "next_token_ids")}
    gd = rr.drafts()
    kv8 = {"k_scale": sc["k_scale"].astype(np.float64), "v_scale": sc["v_scale"].astype(np.float64)}
    ora = oracle.draft_rounds(rr.mnp, args1, rr.rounds, b["block_table"], pool8, w.K, b["mask_id"],
                              block_size=b["block_size"], tokens=gd[:-1], kv_fp8=kv8)
    worst = 0.0
    for t in range(R):
        assert_expansion_equal(expansion_to_np(rr.out[t], rr.dims[t]), ora[t]["exp"])
        worst = max(worst, check_logits(rr.logits[t].cpu().numpy(), ora[t]["logits"]))
        check_argmax(gd[t], ora[t]["logits"])
    check_fp8_kv(rr.dm, rr.cache, pool8, kv8, [o["kv_written"] for o in ora])
    _say(f"[parity] fp8 rounds: worst logit err/RMS {worst:.4f}")
    rr.handle.free()


def test_fp8_rejects_bad_scales():
    import drafting_pd_expand_amd as pdx
    w = synth.Workload("gqa64-fp8-bad", GQA64, C=2, K=2, context="fixed", L=20, seed=5)
    c = Fp8Case(w)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        pairs = c.scale_pairs().copy()
        pairs[1, 0] = bad
        with pytest.raises(pdx.PdError):
            pdx.pd_draft_forward(c.handle, c.mdev, c.dims, c.out, c.inp["block_table"], c.cache, c.draft,
                                 c.logits, kv_scales=pairs)
    c.handle.free()


def test_fp8_nan_codes_in_cache_tails_do_not_leak():
    """E4M3 NaN codes (0x7F, 0xFF) in the slots past each request's last key
    (inside its last page) must not reach any output."""
    import drafting_pd_expand_amd as pdx
    from harness import poison_slots, tail_slots
    w = synth.Workload("gqa64-fp8-nan-tail", GQA64, C=5, K=5, context="lognormal", seed=71)
    _say(f"[fp8] {w.name}")
    c = Fp8Case(w)
    sl = tail_slots(c.b, c.mnp["h_shared"], w.K)
    assert len(sl) > 0
    poison_slots(c.pool, sl, [0x7F, 0xFF])
    c.cache = pdx.pack_kv_cache_fp8(_codes(c.pool["k"], c.dev), _codes(c.pool["v"], c.dev))
    c.run()
    assert c.status() == 0
    check_fp8_case(c)
    c.handle.free()
