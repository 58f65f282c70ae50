"""GPU parity of the autoregressive (EAGLE-style) K-pass baseline, through the
C ABI (pd_expand_batch with K = 1, then pd_draft_forward_ex and pd_ar_advance
per pass), against the oracle's ``ar_draft``.

[Blog] "background and motivation": autoregressive drafting runs K serial
drafter passes; [Blog] "P-EAGLE core method": pass 1 is the NTP position.
Every pass is compared: the advance metadata bit-exact, logits and the fed
hidden state within the forward's bar, argmax where the oracle's margin is
clear, and the KV cache after the last pass at every slot any pass wrote
(every other slot bit-unchanged). The oracle is fed the GPU's sampled tokens,
so both sides take the same path through near-ties, and the GPU's fed-back
hidden states (bf16), so each pass is held to one forward pass's error budget:
left to itself the fed state's error compounds over the passes (the full-size
drafter's logits went past 0.03 x RMS within seven passes that way).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import (KV_ROUNDINGS, LOGIT_TOL, bf16, bits, check_argmax, check_logits, expansion_to_np,
                     gpu_expand, model_dev, model_np, oracle_expand, assert_expansion_equal)

pytestmark = pytest.mark.gpu

GQA64 = synth.ModelDims("gqa64", d=256, Hq=8, Hkv=2, dh=64, F=512, N=2, V=2048)
GQA128 = synth.ModelDims("gqa128", d=512, Hq=4, Hkv=1, dh=128, F=1024, N=2, V=1024)

ADV_KEYS = ["input_ids", "positions", "slot_mapping", "is_rejected", "is_masked", "new_token_indices",
            "cu_out", "seq_lens"]


def _say(msg):
    print(msg, flush=True)


def run_ar_gpu(w: synth.Workload, K: int, model_seed: int = 1234):
    """K autoregressive passes on the device. Returns the per-pass outputs."""
    import drafting_pd_expand_amd as pdx
    dev = torch.device("cuda:0")
    dm = w.model
    mnp = model_np(dm, model_seed)
    mdev = model_dev(dm, model_seed)
    b = synth.make_batch(w)
    pool = synth.make_kv_pool(dm, b["num_blocks"], w.seed)
    C = b["C"]
    dims1, inp, out1 = gpu_expand(b, mnp["h_shared"], 1, dev)
    cache = pdx.pack_kv_cache(bf16(pool["k"], dev), bf16(pool["v"], dev))
    nd = dict(dims1, K=1, T_in=C)
    draft = [torch.empty(C, dtype=torch.int32, device=dev) for _ in range(K)]
    logits = [torch.empty((C, dm.V), dtype=torch.float32, device=dev) for _ in range(K)]
    hid = [torch.empty((C, dm.d), dtype=torch.bfloat16, device=dev) for _ in range(K)]
    h = pdx.Handle()
    batches, dims = [out1], [dims1]
    bt = inp["block_table"]
    pdx.pd_draft_forward(h, mdev, dims1, out1, bt, cache, draft[0], logits[0], hidden_out=hid[0])
    for k in range(1, K):
        nb = pdx.alloc_batch(nd, dev)
        pdx.pd_ar_advance(dims[-1], batches[-1], draft[k - 1], bt, nb)
        pdx.pd_draft_forward(h, mdev, nd, nb, bt, cache, draft[k], logits[k], hidden_d=hid[k - 1],
                             hidden_out=hid[k])
        batches.append(nb)
        dims.append(nd)
    torch.cuda.synchronize()
    status = h.status()
    for nb in batches:
        status |= int(nb["status"].cpu().item())
    h.free()
    return {
        "b": b, "pool": pool, "mnp": mnp, "dims": dims, "batches": batches, "status": status,
        "draft": [t.cpu().numpy() for t in draft], "logits": [t.cpu().numpy() for t in logits],
        "hidden_out": [oracle.bf16_to_f64(bits(t)) for t in hid], "cache": cache,
    }


def check_ar(w: synth.Workload, K: int):
    import drafting_pd_expand_amd as pdx
    g = run_ar_gpu(w, K)
    assert g["status"] == 0, f"status {g['status']}"
    b, mnp, C = g["b"], g["mnp"], g["b"]["C"]
    exp1 = oracle_expand(b, mnp["h_shared"], 1)
    assert_expansion_equal(expansion_to_np(g["batches"][0], g["dims"][0]), exp1)
    ora = oracle.ar_draft(mnp, exp1, b["block_table"], g["pool"], K, block_size=b["block_size"],
                          tokens=g["draft"][:-1], hidden=g["hidden_out"][:-1])
    worst, checked = 0.0, 0
    for k in range(K):
        if k:
            got = {n: g["batches"][k][n][: len(ora[k]["batch"][n])].cpu().numpy() for n in ADV_KEYS}
            for n in ADV_KEYS:
                assert np.array_equal(got[n].astype(np.int64), np.asarray(ora[k]["batch"][n], np.int64)), \
                    (k, n, got[n][:8], ora[k]["batch"][n][:8])
            hsm = g["batches"][k]["hidden_state_mapping"][:C].cpu().numpy()
            assert np.array_equal(hsm, np.arange(C)), (k, hsm[:8])
        worst = max(worst, check_logits(g["logits"][k], ora[k]["logits"]))
        checked += check_argmax(g["draft"][k], ora[k]["logits"])
        ho = ora[k]["hidden_out"]
        rms = np.sqrt(np.mean(ho * ho, axis=1))
        err = np.max(np.abs(g["hidden_out"][k] - ho), axis=1)
        assert np.all(err <= LOGIT_TOL * rms), f"pass {k + 1} hidden_out error/RMS {np.max(err / rms):.4f}"
    # the cache after the last pass: every slot some pass wrote, and nothing else
    dm = w.model
    k_c, v_c = pdx.unpack_kv_cache(g["cache"], dm.Hkv, dm.dh)
    gk, gv = bits(k_c), bits(v_c)
    final = {}
    for p in ora:
        for l, (sl, kk, vv) in enumerate(p["kv_written"]):
            for j, s in enumerate(sl):
                final[(l, int(s))] = (kk[j], vv[j])
    written = np.unique([s for (_, s) in final])
    keep = np.ones(gk.shape[1], bool)
    keep[written] = False
    assert np.array_equal(gk[:, keep], g["pool"]["k"][:, keep]), "K cache changed outside the written slots"
    assert np.array_equal(gv[:, keep], g["pool"]["v"][:, keep]), "V cache changed outside the written slots"
    for (l, s), (kk, vv) in final.items():
        for name, gc, o in (("k", gk, kk), ("v", gv, vv)):
            gg = oracle.bf16_to_f64(gc[l][s]).reshape(-1)
            oo = np.asarray(o).reshape(-1)
            rms = np.sqrt(np.mean(oo * oo))
            lim = LOGIT_TOL * rms + KV_ROUNDINGS * 2.0 ** -9 * np.abs(oo)
            assert np.all(np.abs(gg - oo) <= lim), f"layer {l} slot {s} {name} cache off"
    _say(f"[parity] ar {w.name} K={K}: passes {K}, worst logit err/RMS {worst:.4f}, argmax checked {checked}")


@pytest.mark.parametrize("dims,C,K,ctx,L", [
    (GQA64, 3, 4, "lognormal", 0),
    (GQA64, 5, 6, "fixed", 37),
    (GQA128, 2, 3, "fixed", 500),
], ids=["gqa64-c3k4", "gqa64-c5k6", "gqa128-c2k3"])
def test_ar_small_models(dims, C, K, ctx, L):
    w = synth.Workload(f"{dims.name}-ar-c{C}k{K}", dims, C=C, K=K, context=ctx, L=L, seed=31 + C + K)
    _say(f"[ar] {w.name}")
    check_ar(w, K)


def test_ar_full_size_g_c1():
    w = synth.get_workload("g_c1")
    _say(f"[ar] {w.name} K={w.K}")
    check_ar(w, w.K)


def test_ar_advance_flags_bad_new_token_index():
    """A new-token index outside the previous batch is flagged, and the row is
    made harmless (slot -1, computed as rejected) rather than read out of bounds."""
    import drafting_pd_expand_amd as pdx
    dev = torch.device("cuda:0")
    w = synth.Workload("gqa64-ar-bad", GQA64, C=3, K=2, context="fixed", L=20, seed=5)
    b = synth.make_batch(w)
    mnp = model_np(GQA64)
    dims1, inp, out1 = gpu_expand(b, mnp["h_shared"], 1, dev)
    torch.cuda.synchronize()
    T_prev = dims1["T_in"]
    nti = out1["new_token_indices"].clone()
    out1["new_token_indices"][1] = T_prev + 5
    nd = dict(dims1, K=1, T_in=3)
    nb = pdx.alloc_batch(nd, dev)
    draft = torch.tensor([4, 5, 6], dtype=torch.int32, device=dev)
    pdx.pd_ar_advance(dims1, out1, draft, inp["block_table"], nb)
    torch.cuda.synchronize()
    assert int(nb["status"].cpu().item()) & 16
    assert nb["slot_mapping"][1].item() == -1 and nb["is_rejected"][1].item() == 1
    pos = out1["positions"].cpu().numpy()
    for r in (0, 2):
        assert nb["positions"][r].item() == pos[nti[r].item()] + 1
        assert nb["slot_mapping"][r].item() >= 0 and nb["is_rejected"][r].item() == 0
    assert nb["input_ids"].cpu().tolist()[:3] == [4, 5, 6]
    assert nb["cu_out"][:4].cpu().tolist() == [0, 1, 2, 3]
