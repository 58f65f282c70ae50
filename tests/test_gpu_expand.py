"""GPU parity of the batch expansion (through the C ABI), bit-exact against the
oracle, on every workload and on the edge cases: one request, K=1, K=16, all
or none rejected, a 128-token prefill, C up to 1024 (several prefix-sum
chunks per thread), page sizes other than 16, and bad device data that must
be flagged without any out-of-bounds access."""
import numpy as np
import pytest
import torch

import synth
from harness import assert_expansion_equal, expansion_to_np, gpu_expand, oracle_expand

pytestmark = pytest.mark.gpu


def _hs(H3, seed=5):
    return synth.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(H3).astype(np.float32))


@pytest.mark.parametrize("name", ["tiny", "g_c1", "g_c4", "g_c64_k3", "g_c64_k5", "g_c64", "q_c16"])
def test_expand_workloads(name):
    w = synth.get_workload(name)
    b = synth.make_batch(w)
    hs = _hs(w.model.hidden3)
    print(f"[expand] {name} C={w.C} K={w.K} T_in={b['T_in']}", flush=True)
    dims, _, out = gpu_expand(b, hs, w.K)
    torch.cuda.synchronize()
    got = expansion_to_np(out, dims)
    assert got["status"] == 0
    assert_expansion_equal(got, oracle_expand(b, hs, w.K))


def _batch(C, K, n, accept, L=(0, 300), seed=0, H3=64, bs=16, spare=4):
    rng = np.random.default_rng(seed)
    Ls = rng.integers(L[0], L[1] + 1, size=C)
    ns = np.full(C, n) if np.isscalar(n) else np.asarray(n)
    if accept == "all":
        v = ns.copy()
    elif accept == "none":
        v = np.ones(C, np.int64)
    else:
        v = np.array([rng.integers(1, x + 1) for x in ns])
    pages = [-(-(Ls[r] + ns[r] + K) // bs) for r in range(C)]
    nb = sum(pages) + spare
    perm = rng.permutation(nb)
    bt = np.full((C, max(pages)), -1)
    u = 0
    for r in range(C):
        bt[r, :pages[r]] = perm[u:u + pages[r]]
        u += pages[r]
    T_in = int(ns.sum())
    return {
        "C": C, "K": K, "T_in": T_in, "mask_id": 50000, "block_size": bs, "max_blocks": max(pages),
        "num_blocks": nb, "num_tokens": ns.astype(np.int32), "num_rejected": (ns - v).astype(np.int32),
        "target_ids": rng.integers(0, 50000, T_in).astype(np.int32),
        "target_pos": np.concatenate([np.arange(Ls[r], Ls[r] + ns[r]) for r in range(C)]).astype(np.int32),
        "target_hidden": rng.integers(0, 65535, (T_in, H3)).astype(np.uint16),
        "next_token_ids": rng.integers(0, 50000, C).astype(np.int32),
        "block_table": bt.astype(np.int32),
    }


EDGE = [
    dict(C=1, K=1, n=1, accept="all"),
    dict(C=1, K=7, n=8, accept="none"),
    dict(C=3, K=16, n=17, accept="rand"),
    dict(C=4, K=7, n=8, accept="all"),
    dict(C=1, K=4, n=128, accept="all", L=(0, 0)),
    dict(C=65, K=5, n=6, accept="rand"),
    dict(C=257, K=3, n=[1 + (i % 9) for i in range(257)], accept="rand"),
    dict(C=1024, K=7, n=8, accept="rand", L=(0, 40)),
    dict(C=1024, K=2, n=[1 + (i % 3) for i in range(1024)], accept="rand", L=(0, 10)),
    dict(C=5, K=6, n=7, accept="rand", bs=1),
    dict(C=5, K=6, n=7, accept="rand", bs=4, H3=8),
    dict(C=2, K=3, n=[3, 2], accept="rand", bs=64, H3=8640),
]


@pytest.mark.parametrize("cfg", EDGE, ids=[str(i) for i in range(len(EDGE))])
def test_expand_edge_cases(cfg):
    cfg = dict(cfg)
    K = cfg.pop("K")
    b = _batch(K=K, **cfg)
    hs = _hs(b["target_hidden"].shape[1])
    print(f"[expand-edge] C={b['C']} K={K} T_in={b['T_in']} bs={b['block_size']}", flush=True)
    dims, _, out = gpu_expand(b, hs, K)
    torch.cuda.synchronize()
    got = expansion_to_np(out, dims)
    assert got["status"] == 0
    assert_expansion_equal(got, oracle_expand(b, hs, K))


def test_expand_C0_noop():
    import drafting_pd_expand_amd as pdx
    dims = pdx.batch_dims(0, 3, 0, 9, 16, 1, 1)
    pdx.pd_expand_batch(dims, {}, {})


def _run_bad(b, K):
    hs = _hs(b["target_hidden"].shape[1])
    dims, _, out = gpu_expand(b, hs, K)
    torch.cuda.synchronize()
    return int(out["status"].cpu().item())


def test_bad_counts_are_flagged():
    b = _batch(C=4, K=3, n=5, accept="rand", seed=3)
    b["num_rejected"] = b["num_rejected"].copy()
    b["num_rejected"][2] = 5            # rho == n: no valid token
    assert _run_bad(b, 3) & 1
    b = _batch(C=4, K=3, n=5, accept="rand", seed=3)
    b["num_tokens"] = b["num_tokens"].copy()
    b["num_tokens"][1] = 4              # sum(n) != T_in
    assert _run_bad(b, 3) & 1


def test_bad_pages_and_positions_are_flagged():
    import drafting_pd_expand_amd as pdx
    b = _batch(C=3, K=4, n=5, accept="all", seed=4)
    b["block_table"] = b["block_table"].copy()
    b["block_table"][1, :] = b["num_blocks"] + 7        # outside the pool
    st = _run_bad(b, 4)
    assert st & pdx_flag("BAD_PAGE")
    b = _batch(C=3, K=4, n=5, accept="all", seed=4)
    b["target_pos"] = b["target_pos"].copy()
    b["target_pos"][:5] += 10 ** 6                      # past the block table's reach
    st = _run_bad(b, 4)
    assert st & pdx_flag("BAD_POSITION")


def pdx_flag(name):
    return {"BAD_COUNTS": 1, "BAD_POSITION": 2, "BAD_PAGE": 4, "BAD_TOKEN": 8, "BAD_ROW": 16}[name]
