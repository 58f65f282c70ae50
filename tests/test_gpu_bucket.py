"""GPU: one graph captured at a bucket size serves smaller batches (bucketed
capture, [Blog] "vLLM engineering details": the draft step runs under graph
capture with its range extended to the larger draft batch).

The expansion reads the live request and row counts from device memory; the
forward runs at the bucket's sizes. A graph captured once at C = 64 replays a
37-request batch and then the full 64-request batch (new inputs copied into
the same buffers, new live counts): every replay must equal the same call run
eagerly, bit for bit, and the live rows must meet the oracle's bar (expansion
bit-exact, logits, argmax, KV cache). Padding requests and rows follow the
conventions of include/pd.h.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import (LOGIT_TOL, bf16, bits, check_argmax, check_logits, i32, model_dev, model_np, oracle_expand)

pytestmark = pytest.mark.gpu

GQA64 = synth.ModelDims("gqa64", d=256, Hq=8, Hkv=2, dh=64, F=512, N=2, V=2048)


def _say(msg):
    print(msg, flush=True)


def test_bucket_graph_serves_37_and_64_requests():
    import drafting_pd_expand_amd as pdx
    dev = torch.device("cuda:0")
    w = synth.Workload("gqa64-bucket64", GQA64, C=64, K=7, context="lognormal", seed=303)
    dm, K = w.model, w.K
    mnp, mdev = model_np(dm), model_dev(dm)
    b = synth.make_batch(w)
    pool = synth.make_kv_pool(dm, b["num_blocks"], w.seed)
    Cb, Tb = b["C"], b["T_in"]
    n = b["num_tokens"]
    dims = pdx.batch_dims(Cb, K, Tb, b["mask_id"], dm.hidden3, b["max_blocks"], b["num_blocks"])
    T_out_b = Tb + Cb * (K - 1)
    # bucket-sized inputs (the graph's buffers)
    inp = {"num_tokens": i32(b["num_tokens"], dev), "num_rejected": i32(b["num_rejected"], dev),
           "target_ids": i32(b["target_ids"], dev), "target_pos": i32(b["target_pos"], dev),
           "target_hidden": bf16(b["target_hidden"], dev), "next_token_ids": i32(b["next_token_ids"], dev),
           "block_table": i32(b["block_table"], dev), "h_shared": mdev["h_shared"],
           "live_counts": torch.zeros(2, dtype=torch.int32, device=dev)}
    out = pdx.alloc_batch(dims, dev)
    cache0 = pdx.pack_kv_cache(bf16(pool["k"], dev), bf16(pool["v"], dev))
    cache = cache0.clone()
    R = Cb * K
    draft = torch.empty(R, dtype=torch.int32, device=dev)
    logits = torch.empty((R, dm.V), dtype=torch.float32, device=dev)
    h = pdx.Handle()
    stream = torch.cuda.current_stream()

    def step(s):
        pdx.pd_expand_batch(dims, inp, out, s)
        pdx.pd_draft_forward(h, mdev, dims, out, inp["block_table"], cache, draft, logits, s)

    exp64 = oracle_expand(b, mnp["h_shared"], K)

    def set_live(C):
        T_in = int(n[:C].sum())
        inp["live_counts"].copy_(torch.tensor([C, T_in], dtype=torch.int32))
        # the rest of the buffers keep the 64-request data: padding must ignore it
        return T_in

    def snapshot():
        torch.cuda.synchronize()
        return draft.clone(), logits.clone(), cache.clone(), {k: v.clone() for k, v in out.items()}

    def eager(C):
        set_live(C)
        cache.copy_(cache0)
        out["status"].zero_()
        step(stream)
        return snapshot()

    def check_against_oracle(C, res):
        d_, lg, cc, o = res
        T_in = int(n[:C].sum())
        T_out = T_in + C * (K - 1)
        assert int(o["status"].item()) == 0 and h.status() == 0
        # live rows: exactly the oracle's (a prefix of the 64-request expansion)
        for key in ("input_ids", "positions", "slot_mapping", "is_rejected", "is_masked"):
            assert np.array_equal(o[key][:T_out].cpu().numpy().astype(np.int64),
                                  np.asarray(exp64[key][:T_out]).astype(np.int64)), key
        assert np.array_equal(bits(o["hidden"][:T_out]), np.asarray(exp64["hidden"][:T_out]))
        assert np.array_equal(o["hidden_state_mapping"][:T_in].cpu().numpy(), exp64["hidden_state_mapping"][:T_in])
        assert np.array_equal(o["new_token_indices"][:C * K].cpu().numpy(), exp64["new_token_indices"][:C * K])
        assert np.array_equal(o["cu_out"][:C].cpu().numpy(), exp64["cu_out"][:C])
        assert np.array_equal(o["seq_lens"][:C].cpu().numpy(), exp64["seq_lens"][:C])
        # padding conventions
        assert np.all(o["cu_out"][C:].cpu().numpy() == T_out)
        if C < Cb:
            assert np.all(o["seq_lens"][C:].cpu().numpy() == 1)
            assert np.all(o["new_token_indices"][C * K:].cpu().numpy() == T_out_b - 1)
            assert np.all(o["hidden_state_mapping"][T_in:].cpu().numpy() == -1)
            assert np.all(o["slot_mapping"][T_out:].cpu().numpy() == -1)
            assert np.all(o["is_rejected"][T_out:].cpu().numpy() == 1)
            assert not bits(o["hidden"][T_out:]).any()
        # logits and argmax of sampled live requests (first, last, longest)
        L = b["context_lens"][:C]
        reqs = sorted({0, C - 1, int(np.argmax(L))})
        ora = oracle.draft_forward(mnp, exp64, b["block_table"], pool, K, requests=reqs, block_size=b["block_size"])
        sel = np.concatenate([np.arange(r * K, (r + 1) * K) for r in reqs])
        worst = check_logits(lg.cpu().numpy()[sel], ora["logits"])
        check_argmax(d_.cpu().numpy()[sel], ora["logits"])
        # KV: every slot the live requests wrote matches the oracle; padding rows wrote nothing
        gk, gv = pdx.unpack_kv_cache(cc, dm.Hkv, dm.dh)
        gk, gv = bits(gk), bits(gv)
        written = np.asarray(exp64["slot_mapping"][:T_out])
        written = written[written >= 0]
        keep = np.ones(gk.shape[1], bool)
        keep[written] = False
        assert np.array_equal(gk[:, keep], pool["k"][:, keep]) and np.array_equal(gv[:, keep], pool["v"][:, keep])
        for l, (sl, kk, vv) in enumerate(ora["kv_written"]):
            for g_, oo in ((gk, kk), (gv, vv)):
                gg = oracle.bf16_to_f64(g_[l][sl]).reshape(len(sl), -1)
                oo = oo.reshape(len(sl), -1)
                rms = np.sqrt(np.mean(oo * oo, axis=1, keepdims=True))
                assert np.all(np.abs(gg - oo) <= LOGIT_TOL * rms + 2 * 2.0 ** -9 * np.abs(oo))
        return worst

    ref = {C: eager(C) for C in (37, 64)}
    for C in (37, 64):
        worst = check_against_oracle(C, ref[C])
        _say(f"[bucket] eager C={C}: worst logit err/RMS {worst:.4g}")

    # one graph at the bucket size, captured with the live counts of C = 64
    set_live(64)
    cache.copy_(cache0)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        step(cap)
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            step(cap)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    for C in (37, 64, 37):
        set_live(C)
        cache.copy_(cache0)
        out["status"].zero_()
        draft.fill_(-1)
        logits.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        want = ref[C]
        assert torch.equal(got[0], want[0]), f"C={C}: draft ids differ from eager"
        assert torch.equal(got[1].view(torch.int32), want[1].view(torch.int32)), f"C={C}: logits differ"
        assert torch.equal(got[2], want[2]), f"C={C}: KV cache differs"
        for k in ("input_ids", "positions", "slot_mapping", "new_token_indices", "cu_out", "seq_lens"):
            assert torch.equal(got[3][k], want[3][k]), f"C={C}: {k} differs"
        _say(f"[bucket] replay C={C}: bit-identical to eager")
    del g
    h.free()


def test_bucket_bad_live_counts_flagged():
    import drafting_pd_expand_amd as pdx
    dev = torch.device("cuda:0")
    w = synth.Workload("gqa64-bucket-bad", GQA64, C=4, K=3, context="fixed", L=40, seed=9)
    b = synth.make_batch(w)
    mdev = model_dev(w.model)
    dims = pdx.batch_dims(b["C"], w.K, b["T_in"], b["mask_id"], w.model.hidden3, b["max_blocks"], b["num_blocks"])
    inp = {"num_tokens": i32(b["num_tokens"], dev), "num_rejected": i32(b["num_rejected"], dev),
           "target_ids": i32(b["target_ids"], dev), "target_pos": i32(b["target_pos"], dev),
           "target_hidden": bf16(b["target_hidden"], dev), "next_token_ids": i32(b["next_token_ids"], dev),
           "block_table": i32(b["block_table"], dev), "h_shared": mdev["h_shared"]}
    for live in ([5, b["T_in"]], [2, b["T_in"] + 1], [3, 2], [-1, 0]):
        inp["live_counts"] = torch.tensor(live, dtype=torch.int32, device=dev)
        out = pdx.alloc_batch(dims, dev)
        pdx.pd_expand_batch(dims, inp, out)
        torch.cuda.synchronize()
        assert int(out["status"].item()) & 1, f"live counts {live} not flagged"
