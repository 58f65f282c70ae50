"""GPU parity of multi-round runs (pd_verify_stub -> pd_expand_batch ->
pd_draft_forward, round after round on the device, KV cache carried over)
against the oracle's ``draft_rounds``, eagerly and as one captured graph.

Per round: the expansion bit-exact, logits and argmax at the forward's bar;
after the last round the KV cache at every slot any round wrote (the last
writer's values: a round's MASK rows are overwritten by the next round's
verify rows) and every other slot bit-unchanged. The oracle is fed the GPU's
drafts so both sides take the same path through near-ties. Graph replays of
all rounds must reproduce the eager drafts bit for bit (every slot a round
reads is written earlier in the same run, so stale entries from earlier
replays cannot leak in).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import (KV_ROUNDINGS, LOGIT_TOL, assert_expansion_equal, bf16, bits, check_argmax, check_logits,
                     expansion_to_np, i32, model_dev, model_np)

pytestmark = pytest.mark.gpu

GQA64 = synth.ModelDims("gqa64", d=256, Hq=8, Hkv=2, dh=64, F=512, N=2, V=2048)
GQA128 = synth.ModelDims("gqa128", d=512, Hq=4, Hkv=1, dh=128, F=1024, N=2, V=1024)


def _say(msg):
    print(msg, flush=True)


class Rounds:
    """R rounds of one workload, every buffer allocated up front."""

    def __init__(self, w: synth.Workload, R: int, with_logits: bool = True, model_seed: int = 1234):
        import drafting_pd_expand_amd as pdx
        self.pdx = pdx
        self.w, self.R, self.K = w, R, w.K
        dev = self.dev = torch.device("cuda:0")
        dm = self.dm = w.model
        self.mnp = model_np(dm, model_seed)
        self.mdev = model_dev(dm, model_seed)
        K = w.K
        b = self.b = synth.make_batch(w, extra_positions=(R - 1) * (K + 1))
        self.rounds = synth.make_rounds(w, R)
        self.pool = synth.make_kv_pool(dm, b["num_blocks"], w.seed)
        C = self.C = b["C"]
        self.cache = pdx.pack_kv_cache(bf16(self.pool["k"], dev), bf16(self.pool["v"], dev))
        H3 = dm.hidden3
        self.dims = [pdx.batch_dims(C, K, b["T_in"], b["mask_id"], H3, b["max_blocks"], b["num_blocks"],
                                    b["block_size"])]
        self.dims += [dict(self.dims[0], T_in=C * (K + 1)) for _ in range(R - 1)]
        bt = i32(b["block_table"], dev)
        hs = bf16(self.mnp["h_shared"], dev)
        self.inp = [{"num_tokens": i32(b["num_tokens"], dev), "num_rejected": i32(b["num_rejected"], dev),
                     "target_ids": i32(b["target_ids"], dev), "target_pos": i32(b["target_pos"], dev),
                     "target_hidden": bf16(b["target_hidden"], dev),
                     "next_token_ids": i32(b["next_token_ids"], dev), "block_table": bt, "h_shared": hs}]
        self.accepted = []
        for rd in self.rounds:
            self.inp.append({"num_tokens": torch.empty(C, dtype=torch.int32, device=dev),
                             "num_rejected": torch.empty(C, dtype=torch.int32, device=dev),
                             "target_ids": torch.empty(C * (K + 1), dtype=torch.int32, device=dev),
                             "target_pos": torch.empty(C * (K + 1), dtype=torch.int32, device=dev),
                             "target_hidden": bf16(rd["target_hidden"], dev),
                             "next_token_ids": i32(rd["next_token_ids"], dev), "block_table": bt, "h_shared": hs})
            self.accepted.append(i32(rd["accepted"], dev))
        self.out = [pdx.alloc_batch(d, dev) for d in self.dims]
        self.draft = [torch.empty(C * K, dtype=torch.int32, device=dev) for _ in range(R)]
        self.logits = ([torch.empty((C * K, dm.V), dtype=torch.float32, device=dev) for _ in range(R)]
                       if with_logits else [None] * R)
        self.stub_status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.handle = pdx.Handle()

    def run(self, stream=None):
        pdx = self.pdx
        for t in range(self.R):
            if t > 0:
                pdx.pd_verify_stub(self.dims[t - 1], self.out[t - 1], self.draft[t - 1],
                                   self.inp[t - 1]["next_token_ids"], self.accepted[t - 1], self.inp[t],
                                   self.stub_status, stream)
            pdx.pd_expand_batch(self.dims[t], self.inp[t], self.out[t], stream)
            pdx.pd_draft_forward(self.handle, self.mdev, self.dims[t], self.out[t], self.inp[t]["block_table"],
                                 self.cache, self.draft[t], self.logits[t], stream)

    def status(self) -> int:
        st = self.handle.status() | int(self.stub_status.item())
        for o in self.out:
            st |= int(o["status"].item())
        return st

    def drafts(self):
        return [d.cpu().numpy().copy() for d in self.draft]


def check_rounds(rr: Rounds):
    import drafting_pd_expand_amd as pdx
    b, K = rr.b, rr.K
    args1 = {k: b[k] for k in ("num_tokens", "num_rejected", "target_ids", "target_pos", "target_hidden",
                               "next_token_ids")}
    gd = rr.drafts()
    ora = oracle.draft_rounds(rr.mnp, args1, rr.rounds, b["block_table"], rr.pool, K, b["mask_id"],
                              block_size=b["block_size"], tokens=gd[:-1])
    worst, checked = 0.0, 0
    for t in range(rr.R):
        assert_expansion_equal(expansion_to_np(rr.out[t], rr.dims[t]), ora[t]["exp"])
        if rr.logits[t] is not None:
            worst = max(worst, check_logits(rr.logits[t].cpu().numpy(), ora[t]["logits"]))
        checked += check_argmax(gd[t], ora[t]["logits"])
    k_c, v_c = pdx.unpack_kv_cache(rr.cache, rr.dm.Hkv, rr.dm.dh)
    gk, gv = bits(k_c), bits(v_c)
    final = {}
    for res in ora:
        for l, (sl, kk, vv) in enumerate(res["kv_written"]):
            for j, s in enumerate(sl):
                final[(l, int(s))] = (kk[j], vv[j])
    keep = np.ones(gk.shape[1], bool)
    keep[np.unique([s for (_, s) in final])] = False
    assert np.array_equal(gk[:, keep], rr.pool["k"][:, keep]), "K cache changed outside the written slots"
    assert np.array_equal(gv[:, keep], rr.pool["v"][:, keep]), "V cache changed outside the written slots"
    for (l, s), (kk, vv) in final.items():
        for name, gc, o in (("k", gk, kk), ("v", gv, vv)):
            gg = oracle.bf16_to_f64(gc[l][s]).reshape(-1)
            oo = np.asarray(o).reshape(-1)
            rms = np.sqrt(np.mean(oo * oo))
            lim = LOGIT_TOL * rms + KV_ROUNDINGS * 2.0 ** -9 * np.abs(oo)
            assert np.all(np.abs(gg - oo) <= lim), f"layer {l} slot {s} {name} cache off"
    _say(f"[parity] rounds {rr.w.name} R={rr.R}: worst logit err/RMS {worst:.4f}, argmax checked {checked}")


@pytest.mark.parametrize("dims,C,K,R,ctx,L", [
    (GQA64, 3, 4, 4, "lognormal", 0),
    (GQA64, 5, 2, 5, "fixed", 33),
    (GQA128, 2, 3, 3, "fixed", 300),
], ids=["gqa64-c3k4r4", "gqa64-c5k2r5", "gqa128-c2k3r3"])
def test_rounds_small_models(dims, C, K, R, ctx, L):
    w = synth.Workload(f"{dims.name}-rounds-c{C}k{K}", dims, C=C, K=K, context=ctx, L=L, seed=71 + C + K)
    _say(f"[rounds] {w.name} R={R}")
    rr = Rounds(w, R)
    rr.run()
    torch.cuda.synchronize()
    assert rr.status() == 0
    check_rounds(rr)
    rr.handle.free()


def test_rounds_full_size_g_c4():
    w = synth.get_workload("g_c4")
    _say(f"[rounds] {w.name} R=3")
    rr = Rounds(w, 3)
    rr.run()
    torch.cuda.synchronize()
    assert rr.status() == 0
    check_rounds(rr)
    rr.handle.free()


def test_rounds_graph_replays_match_eager():
    """All rounds captured as one graph on a side stream; three replays, with
    eager work and synchronizations between them, each reproduce the eager
    drafts of every round bit for bit."""
    w = synth.Workload("gqa64-rounds-graph", GQA64, C=6, K=3, context="lognormal", seed=79)
    R = 4
    _say(f"[rounds] graph {w.name} R={R}")
    rr = Rounds(w, R, with_logits=False)
    rr.run()
    torch.cuda.synchronize()
    assert rr.status() == 0
    eager = rr.drafts()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        rr.run(cap)
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            rr.run(cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        for d in rr.draft:
            d.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        got = rr.drafts()
        for t in range(R):
            assert np.array_equal(got[t], eager[t]), (rep, t)
        _ = torch.ones(8, device=rr.dev).sum().item()   # eager work between replays
    assert rr.status() == 0
    del g
    rr.handle.free()
