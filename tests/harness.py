"""Test harness: build one seeded case, run it through the C ABI on the GPU,
run the oracle on the same inputs, and compare.

Comparison rules (the drafting step's stated bar):
  * expansion outputs and hidden rows: bit-exact;
  * logits: max_v |gpu - oracle| <= 0.03 * RMS_v(oracle row);
  * draft ids: equal wherever the oracle's top-1 minus top-2 margin > 0.05;
  * KV written this step: each value within 0.03 * RMS of its oracle slot row
    plus two bf16 roundings of the value itself (the cache is bf16 and k is
    rounded at the QKV output and again after RoPE); every other slot
    bit-unchanged.
"""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
import synth

LOGIT_TOL = 0.03
ARGMAX_MARGIN = 0.05
KV_ROUNDINGS = 2   # bf16 roundings a stored K/V value goes through


@functools.lru_cache(maxsize=2)
def model_np(dims: synth.ModelDims, seed: int = 1234):
    return synth.make_model(dims, seed=seed)


_DEV_MODELS = {}


def model_dev(dims: synth.ModelDims, seed: int = 1234):
    import drafting_pd_expand_amd as pdx
    key = (dims, seed)
    if key not in _DEV_MODELS:
        _DEV_MODELS.clear()
        torch.cuda.empty_cache()
        _DEV_MODELS[key] = pdx.device_model(model_np(dims, seed), torch.device("cuda:0"))
    return _DEV_MODELS[key]


def i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def bf16(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(dev).view(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_expand(b: dict, h_shared, K: int) -> dict:
    return oracle.expand(b["num_tokens"], b["num_rejected"], b["target_ids"], b["target_pos"],
                         b["target_hidden"], b["next_token_ids"], b["block_table"], h_shared, K,
                         b["mask_id"], b["block_size"])


def gpu_expand(b: dict, h_shared, K: int, dev=None):
    import drafting_pd_expand_amd as pdx
    dev = dev or torch.device("cuda:0")
    H3 = b["target_hidden"].shape[1]
    dims = pdx.batch_dims(b["C"], K, b["T_in"], b["mask_id"], H3, b["max_blocks"], b["num_blocks"],
                          b["block_size"])
    inp = {
        "num_tokens": i32(b["num_tokens"], dev), "num_rejected": i32(b["num_rejected"], dev),
        "target_ids": i32(b["target_ids"], dev), "target_pos": i32(b["target_pos"], dev),
        "target_hidden": bf16(b["target_hidden"], dev), "next_token_ids": i32(b["next_token_ids"], dev),
        "block_table": i32(b["block_table"], dev), "h_shared": bf16(h_shared, dev),
    }
    out = pdx.alloc_batch(dims, dev)
    pdx.pd_expand_batch(dims, inp, out)
    return dims, inp, out


def expansion_to_np(out: dict, dims: dict) -> dict:
    T_out = dims["T_in"] + dims["C"] * (dims["K"] - 1)
    C, K = dims["C"], dims["K"]
    g = lambda n, k: out[n][:k].cpu().numpy()
    return {
        "input_ids": g("input_ids", T_out), "positions": g("positions", T_out),
        "slot_mapping": g("slot_mapping", T_out), "is_rejected": g("is_rejected", T_out),
        "is_masked": g("is_masked", T_out), "hidden_state_mapping": g("hidden_state_mapping", dims["T_in"]),
        "new_token_indices": g("new_token_indices", C * K), "cu_out": g("cu_out", C + 1),
        "seq_lens": g("seq_lens", C), "hidden": bits(out["hidden"][:T_out]),
        "status": int(out["status"].cpu().item()),
    }


EXP_KEYS = ["input_ids", "positions", "slot_mapping", "is_rejected", "is_masked",
            "hidden_state_mapping", "new_token_indices", "cu_out", "seq_lens", "hidden"]


def assert_expansion_equal(got: dict, want: dict):
    for k in EXP_KEYS:
        a, b = np.asarray(got[k]), np.asarray(want[k])
        assert a.shape == b.shape, (k, a.shape, b.shape)
        if not np.array_equal(a.astype(np.int64), b.astype(np.int64)):
            bad = np.nonzero(a.reshape(len(a), -1).astype(np.int64) != b.reshape(len(b), -1).astype(np.int64))[0]
            raise AssertionError(f"{k} differs at rows {bad[:10]}: gpu {a[bad[:3]]} oracle {b[bad[:3]]}")


def check_logits(gpu: np.ndarray, ora: np.ndarray, tol: float = LOGIT_TOL):
    rms = np.sqrt(np.mean(ora * ora, axis=1))
    err = np.max(np.abs(gpu.astype(np.float64) - ora), axis=1)
    ratio = err / rms
    assert np.all(np.isfinite(gpu)), "non-finite GPU logits"
    assert np.all(ratio <= tol), f"logit error / RMS up to {ratio.max():.4f} (> {tol}) at rows {np.nonzero(ratio > tol)[0][:10]}"
    return float(ratio.max())


def check_argmax(gpu_ids: np.ndarray, ora: np.ndarray, margin: float = ARGMAX_MARGIN):
    top = np.sort(ora, axis=1)[:, -2:]
    m = top[:, 1] - top[:, 0]
    sel = m > margin
    want = np.argmax(ora, axis=1)
    bad = np.nonzero(sel & (gpu_ids != want))[0]
    assert len(bad) == 0, f"argmax mismatch at rows {bad[:10]}: gpu {gpu_ids[bad[:5]]} oracle {want[bad[:5]]}"
    return int(sel.sum())


class Case:
    """One seeded draft step on the device, plus the oracle's view of it."""

    def __init__(self, w: synth.Workload, model_seed: int = 1234, with_logits: bool = True,
                 debug_resid: bool = False, batch=None):
        import drafting_pd_expand_amd as pdx
        self.w = w
        self.dm = w.model
        self.dev = torch.device("cuda:0")
        self.mnp = model_np(self.dm, model_seed)
        self.mdev = model_dev(self.dm, model_seed)
        self.b = batch if batch is not None else synth.make_batch(w)
        self.pool = synth.make_kv_pool(self.dm, self.b["num_blocks"], w.seed)
        self.K = w.K
        self.dims, self.inp, self.out = gpu_expand(self.b, self.mnp["h_shared"], self.K, self.dev)
        k = bf16(self.pool["k"], self.dev)
        v = bf16(self.pool["v"], self.dev)
        self.cache = pdx.pack_kv_cache(k, v)
        del k, v
        R = self.b["C"] * self.K
        self.draft = torch.empty(max(R, 1), dtype=torch.int32, device=self.dev)
        self.logits = torch.empty((max(R, 1), self.dm.V), dtype=torch.float32, device=self.dev) if with_logits else None
        self.handle = pdx.Handle()
        self.resid = None
        if debug_resid:
            T_out = self.dims["T_in"] + self.dims["C"] * (self.K - 1)
            self.resid = torch.zeros((self.dm.N + 1, T_out, self.dm.d), dtype=torch.float32, device=self.dev)

    def run(self):
        import drafting_pd_expand_amd as pdx
        if self.resid is not None:
            if not self.handle.ptr.value:
                # first call creates the handle; run once to create, then register
                pdx.pd_draft_forward(self.handle, self.mdev, self.dims, self.out, self.inp["block_table"],
                                     self.cache, self.draft, self.logits)
                torch.cuda.synchronize()
            self.handle.set_debug_resid(self.resid)
        pdx.pd_draft_forward(self.handle, self.mdev, self.dims, self.out, self.inp["block_table"],
                             self.cache, self.draft, self.logits)
        torch.cuda.synchronize()
        return self

    def status(self) -> int:
        return self.handle.status() | int(self.out["status"].cpu().item())

    def gpu_cache_slots(self):
        import drafting_pd_expand_amd as pdx
        k, v = pdx.unpack_kv_cache(self.cache, self.dm.Hkv, self.dm.dh)
        return bits(k), bits(v)

    def oracle(self, requests=None, return_layers=False):
        exp = oracle_expand(self.b, self.mnp["h_shared"], self.K)
        return exp, oracle.draft_forward(self.mnp, exp, self.b["block_table"], self.pool, self.K,
                                         requests=requests, block_size=self.b["block_size"],
                                         return_layers=return_layers)

    def close(self):
        self.handle.free()


def check_case(case: Case, requests=None, check_cache=True, check_layers=False):
    """Full comparison of a run against the oracle (on `requests` or all)."""
    exp, ora = case.oracle(requests, return_layers=check_layers)
    got_exp = expansion_to_np(case.out, case.dims)
    assert_expansion_equal(got_exp, exp)
    K = case.K
    reqs = ora["requests"]
    sel = np.concatenate([np.arange(r * K, (r + 1) * K) for r in reqs])
    worst = None
    if case.logits is not None:
        gl = case.logits[torch.from_numpy(sel).to(case.dev)].cpu().numpy()
        worst = check_logits(gl, ora["logits"])
    gd = case.draft.cpu().numpy()[sel]
    n_checked = check_argmax(gd, ora["logits"])
    kv_use = kv_plain = None
    if check_cache:
        kv_use = kv_plain = 0.0
        gk, gv = case.gpu_cache_slots()
        # slots written on the GPU are exactly the valid slot_mapping entries
        written = exp["slot_mapping"][exp["slot_mapping"] >= 0]
        keep = np.ones(gk.shape[1], bool)
        keep[written] = False
        assert np.array_equal(gk[:, keep], case.pool["k"][:, keep]), "K cache changed outside the written slots"
        assert np.array_equal(gv[:, keep], case.pool["v"][:, keep]), "V cache changed outside the written slots"
        for l, (sl, k, v) in enumerate(ora["kv_written"]):
            for name, g, o in (("k", gk, k), ("v", gv, v)):
                gg = oracle.bf16_to_f64(g[l][sl]).reshape(len(sl), -1)
                oo = o.reshape(len(sl), -1)
                rms = np.sqrt(np.mean(oo * oo, axis=1, keepdims=True))
                # the cache is bf16: on top of the compute budget each stored
                # value may carry two roundings to bf16 (2^-9 relative each)
                lim = LOGIT_TOL * rms + KV_ROUNDINGS * 2.0 ** -9 * np.abs(oo)
                err = np.abs(gg - oo)
                if err.size:
                    # share of the limit used, and the error in units of the
                    # compute budget alone (0.03 RMS, without the storage roundings)
                    kv_use = max(kv_use, float(np.max(err / lim)))
                    kv_plain = max(kv_plain, float(np.max(err / (LOGIT_TOL * rms))))
                bad = err > lim
                assert not bad.any(), (f"layer {l} {name} cache error: worst "
                                       f"{np.max((np.abs(gg - oo) - lim) / rms):.4f} RMS over the limit")
    if check_layers and case.resid is not None:
        rows = ora["rows"]
        for l, xo in enumerate(ora["layers"]):
            xg = case.resid[l][torch.from_numpy(rows).to(case.dev)].cpu().numpy()
            rms = np.sqrt(np.mean(xo * xo, axis=1))
            err = np.max(np.abs(xg - xo), axis=1)
            assert np.all(err <= LOGIT_TOL * rms), f"residual after stage {l}: error/RMS {np.max(err / rms):.4f}"
    res = {"worst_logit_ratio": worst, "argmax_checked": n_checked, "rows": len(sel),
           "kv_limit_used": kv_use, "kv_err_over_compute_budget": kv_plain}
    # one line per checked case (visible with pytest -s): the observed error budget use
    kv_txt = "" if kv_use is None else (f", KV cache worst err {kv_use:.3f} of its limit "
                                        f"({kv_plain:.3f} of 0.03 RMS alone)")
    print(f"[parity] {case.w.name}: rows {len(sel)}, worst logit err/RMS "
          f"{'-' if worst is None else f'{worst:.4f}'}, argmax checked {n_checked}{kv_txt}", flush=True)
    return res


def tail_slots(b: dict, h_shared, K: int) -> np.ndarray:
    """Cache slots past each request's last visible key inside its last page
    (positions seq_len .. the page's end): never read as context and never
    written by the step, so they may hold anything."""
    exp = oracle_expand(b, h_shared, K)
    bs = b["block_size"]
    out = []
    for r, s in enumerate(np.asarray(exp["seq_lens"], np.int64)):
        end = -(-int(s) // bs) * bs
        t = np.arange(int(s), end)
        out.append(np.asarray(b["block_table"])[r][t // bs] * bs + t % bs)
    return np.concatenate(out).astype(np.int64)


def poison_slots(pool: dict, slots: np.ndarray, codes) -> None:
    """Fill K and V of `slots` (every layer, head and dim) with the given raw
    codes in turn (bf16 bits for a uint16 pool, E4M3 codes for a uint8 one)."""
    codes = np.asarray(codes, dtype=pool["k"].dtype)
    for i, s in enumerate(slots):
        pool["k"][:, s] = codes[i % len(codes)]
        pool["v"][:, s] = codes[(i + 1) % len(codes)]
