"""Pins for the oracle's drafter forward (CPU only).

Each pin ties the oracle to something other than itself:
  * RoPE: closed form on unit vectors; the relative-position identity of
    (R_p q)^T (R_p' k) = q^T R_(p'-p) k (Theorem 2.3 on the arXiv page,
    appendix B on the paper-summary page); norm preservation.
  * RMSNorm / SiLU: torch.nn.functional.rms_norm and scipy's expit.
  * Prefill from an empty cache: a dense torch-library forward (dense_ref.py)
    built straight from the Input_i rule, with GQA (8 q / 2 kv heads).
  * Decode over scattered pages with rejected tokens: the K/V the oracle
    wrote during a prefix prefill, then one decode step, must reproduce the
    dense prefill of the accepted prompt.
  * Invariants: (a) identical MASK inputs, (c) causality, NTP logits
    independent of K, (d) rejected rows change nothing, request independence,
    page-relabelling invariance.
"""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import synth
from dense_ref import dense_prefill_logits

MINI = synth.ModelDims("mini", d=64, Hq=8, Hkv=2, dh=16, F=96, N=2, V=512)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / (np.max(np.abs(b)) + 1e-300))


# ----------------------------------------------------------------------------- RoPE

@pytest.mark.parametrize("dh", [2, 16, 64])
def test_rope_closed_form_unit_vectors(dh):
    half, theta = dh // 2, 10000.0
    for p in [0, 1, 7, 4095, 19999]:
        for i in range(half):
            ang = p * theta ** (-2.0 * i / dh)
            e = np.zeros((1, dh)); e[0, i] = 1.0
            r = oracle.rope_rotate(e, p, theta)[0]
            want = np.zeros(dh); want[i] = np.cos(ang); want[i + half] = np.sin(ang)
            assert np.allclose(r, want, atol=1e-12)
            e = np.zeros((1, dh)); e[0, i + half] = 1.0
            r = oracle.rope_rotate(e, p, theta)[0]
            want = np.zeros(dh); want[i] = -np.sin(ang); want[i + half] = np.cos(ang)
            assert np.allclose(r, want, atol=1e-12)


def test_rope_relative_position_identity_and_norm():
    rng = np.random.default_rng(5)
    for dh in [16, 64, 128]:
        q = rng.standard_normal((1, dh)); k = rng.standard_normal((1, dh))
        for p, pp in [(0, 5), (3, 3), (100, 37), (4096, 4103), (19990, 20000)]:
            lhs = float(oracle.rope_rotate(q, p, 1e4)[0] @ oracle.rope_rotate(k, pp, 1e4)[0])
            rhs = float(q[0] @ oracle.rope_rotate(k, pp - p, 1e4)[0])
            assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))
            # a uniform shift of both positions leaves the score unchanged
            sh = float(oracle.rope_rotate(q, p + 1000, 1e4)[0] @ oracle.rope_rotate(k, pp + 1000, 1e4)[0])
            assert abs(sh - lhs) < 1e-9 * (1 + abs(lhs))
            assert abs(np.linalg.norm(oracle.rope_rotate(q, p, 1e4)) - np.linalg.norm(q)) < 1e-12


def test_rope_vectorised_positions():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 3, 16))
    pos = np.array([0, 1, 2, 50, 9999])
    full = oracle.rope_rotate(x, pos, 1e4)
    for i in range(5):
        assert np.allclose(full[i], oracle.rope_rotate(x[i], pos[i], 1e4), atol=1e-14)


# ----------------------------------------------------------------------------- norms, activations

def test_rms_norm_matches_library_and_closed_form():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, 37)) * 3
    g = rng.standard_normal(37)
    want = F.rms_norm(torch.from_numpy(x), (37,), torch.from_numpy(g), 1e-5).numpy()
    assert _rel(oracle.rms_norm(x, g, 1e-5), want) < 1e-14
    c = 0.7
    y = oracle.rms_norm(np.full((1, 8), c), np.ones(8), 1e-5)
    assert np.allclose(y, c / np.sqrt(c * c + 1e-5), rtol=1e-14)


def test_silu_matches_library():
    z = np.linspace(-80, 80, 1001)
    assert np.allclose(oracle.silu(z), z * scipy.special.expit(z), rtol=1e-13, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


# ----------------------------------------------------------------------------- full forward

def _prefill_case(dims, n, K, seed):
    model = synth.make_model(dims, seed=seed)
    rng = np.random.default_rng(seed + 1)
    ids = rng.integers(0, dims.V - 1, size=n)
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((n, dims.hidden3)).astype(np.float32))
    nxt = int(rng.integers(0, dims.V - 1))
    return model, ids, hidden, nxt


def _oracle_prefill(model, ids, hidden, nxt, K, bs=4, seed=0):
    dims = model["dims"]
    n = len(ids)
    pages = -(-(n + K) // bs)
    rng = np.random.default_rng(seed)
    nb = pages + 3
    bt = rng.permutation(nb)[:pages][None]
    pool = {"k": rng.standard_normal((dims.N, nb * bs, dims.Hkv, dims.dh)),
            "v": rng.standard_normal((dims.N, nb * bs, dims.Hkv, dims.dh))}
    exp = oracle.expand([n], [0], ids, np.arange(n), hidden, [nxt], bt, model["h_shared"],
                        K, dims.V - 1, bs)
    return oracle.draft_forward(model, exp, bt, pool, K, block_size=bs), exp, bt, pool


@pytest.mark.parametrize("dims,n,K", [(MINI, 21, 5), (MINI, 3, 1), (synth.MODELS["tiny"], 128, 4)])
def test_prefill_matches_dense_library_forward(dims, n, K):
    model, ids, hidden, nxt = _prefill_case(dims, n, K, seed=11)
    got, _, _, _ = _oracle_prefill(model, ids, hidden, nxt, K)
    want = dense_prefill_logits(model, ids, hidden, nxt, K, dims.V - 1)
    assert got["logits"].shape == want.shape
    assert _rel(got["logits"], want) < 1e-10


def _sum_model(model, seed):
    """The same weights with a d-wide layer-0 QKV (fresh N(0, 0.02) draws):
    the shape the combine="sum" reading needs."""
    dims = model["dims"]
    rng = np.random.default_rng(seed)
    w = synth.f32_to_bf16_bits((0.02 * rng.standard_normal((dims.qkv_out, dims.d))).astype(np.float32))
    out = dict(model)
    out["layers"] = [dict(model["layers"][0], w_qkv=w)] + list(model["layers"][1:])
    return out


@pytest.mark.parametrize("dims,n,K", [(MINI, 21, 5), (MINI, 4, 1)])
def test_prefill_combine_sum_matches_dense_library_forward(dims, n, K):
    """The other reading of how emb and h meet (emb + fc(h), [Paper] sec. 2
    architecture wording) against the dense library forward with the same
    reading; it differs from the concatenation reading."""
    model, ids, hidden, nxt = _prefill_case(dims, n, K, seed=12)
    ms = _sum_model(model, 99)
    n_ = len(ids)
    bs, pages = 4, -(-(n_ + K) // 4)
    rng = np.random.default_rng(3)
    nb = pages + 3
    bt = rng.permutation(nb)[:pages][None]
    pool = {"k": rng.standard_normal((dims.N, nb * bs, dims.Hkv, dims.dh)),
            "v": rng.standard_normal((dims.N, nb * bs, dims.Hkv, dims.dh))}
    exp = oracle.expand([n_], [0], ids, np.arange(n_), hidden, [nxt], bt, model["h_shared"], K, dims.V - 1, bs)
    got = oracle.draft_forward(ms, exp, bt, pool, K, block_size=bs, combine="sum")
    want = dense_prefill_logits(ms, ids, hidden, nxt, K, dims.V - 1, combine="sum")
    assert _rel(got["logits"], want) < 1e-10
    other = dense_prefill_logits(model, ids, hidden, nxt, K, dims.V - 1, combine="concat")
    assert _rel(got["logits"], other) > 1e-3
    with pytest.raises(ValueError):
        oracle.draft_forward(ms, exp, bt, pool, K, block_size=bs, combine="add")


@pytest.mark.parametrize("L,n,v,K", [(13, 6, 4, 5), (9, 4, 1, 3), (16, 8, 8, 7), (30, 2, 2, 1)])
def test_decode_over_written_cache_matches_dense_prefill(L, n, v, K):
    """Prefix prefill of L tokens writes K/V into scattered pages; a decode step
    with n verify tokens (v accepted) then reads them back through the block
    table. Its K sampled logits must equal a dense prefill of the L+v accepted
    tokens."""
    dims, bs = MINI, 4
    model = synth.make_model(dims, seed=21)
    rng = np.random.default_rng(22)
    P = L + n
    ids = rng.integers(0, dims.V - 1, size=P)
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((P, dims.hidden3)).astype(np.float32))
    nxt = int(rng.integers(0, dims.V - 1))
    pages = -(-(L + n + K) // bs)
    nb = pages + 5
    bt = rng.permutation(nb)[:pages][None]
    pool = {"k": rng.standard_normal((dims.N, nb * bs, dims.Hkv, dims.dh)),
            "v": rng.standard_normal((dims.N, nb * bs, dims.Hkv, dims.dh))}
    # 1) prefill of the first L tokens; its "sampled" token is the prompt token at position L
    e1 = oracle.expand([L], [0], ids[:L], np.arange(L), hidden[:L], [int(ids[L])], bt,
                       model["h_shared"], K, dims.V - 1, bs)
    f1 = oracle.draft_forward(model, e1, bt, pool, K, block_size=bs)
    for l, (sl, k, vv) in enumerate(f1["kv_written"]):
        pool["k"][l][sl] = k
        pool["v"][l][sl] = vv
    # 2) decode step over the verify segment at positions L..L+n-1 (last n-v rejected)
    e2 = oracle.expand([n], [n - v], ids[L:L + n], np.arange(L, L + n), hidden[L:L + n], [nxt], bt,
                       model["h_shared"], K, dims.V - 1, bs)
    f2 = oracle.draft_forward(model, e2, bt, pool, K, block_size=bs)
    want = dense_prefill_logits(model, ids[:L + v], hidden[:L + v], nxt, K, dims.V - 1)
    assert _rel(f2["logits"], want) < 1e-10


def _small_decode_case(C=3, K=5, seed=31, bs=4, Lmax=40):
    dims = MINI
    rng = np.random.default_rng(seed)
    L = rng.integers(1, Lmax, size=C)
    n = np.full(C, K + 1)
    rho = rng.integers(0, K + 1, size=C)
    pos = np.concatenate([np.arange(L[r], L[r] + n[r]) for r in range(C)])
    pages = [-(-(L[r] + n[r] + K) // bs) for r in range(C)]
    nb = sum(pages) + 4
    perm = rng.permutation(nb)
    bt = np.full((C, max(pages)), -1)
    u = 0
    for r in range(C):
        bt[r, :pages[r]] = perm[u:u + pages[r]]
        u += pages[r]
    T_in = int(n.sum())
    model = synth.make_model(dims, seed=seed)
    pool = synth.make_kv_pool(dims, nb, seed, block_size=bs)
    ids = rng.integers(0, dims.V - 1, size=T_in)
    nxt = rng.integers(0, dims.V - 1, size=C)
    hid = synth.f32_to_bf16_bits(rng.standard_normal((T_in, dims.hidden3)).astype(np.float32))
    args = dict(num_tokens=n, num_rejected=rho, target_ids=ids, target_pos=pos, target_hidden=hid,
                next_token_ids=nxt, block_table=bt)
    exp = oracle.expand(n, rho, ids, pos, hid, nxt, bt, model["h_shared"], K, dims.V - 1, bs)
    return model, args, pool, exp, bs


def test_mask_rows_identical_inputs_and_causality():
    """(a) every MASK row gets the same (id, hidden) input; (c) perturbing the
    last MASK row of a request leaves all of its earlier sampled logits
    unchanged (and changes its own)."""
    model, args, pool, exp, bs = _small_decode_case()
    K = 5
    base = oracle.draft_forward(model, exp, args["block_table"], pool, K, block_size=bs)
    mrows = np.nonzero(exp["is_masked"])[0]
    assert len({exp["input_ids"][o] for o in mrows}) == 1
    assert all((exp["hidden"][o] == exp["hidden"][mrows[0]]).all() for o in mrows)
    for r in range(3):
        last = exp["new_token_indices"][r * K + K - 1]
        pert = dict(exp)
        pert["hidden"] = exp["hidden"].copy()
        pert["hidden"][last] ^= np.uint16(0x5555)
        pert["input_ids"] = exp["input_ids"].copy()
        pert["input_ids"][last] = 3
        got = oracle.draft_forward(model, pert, args["block_table"], pool, K, block_size=bs)
        sel = slice(r * K, r * K + K - 1)
        assert np.array_equal(got["logits"][sel], base["logits"][sel])
        assert not np.allclose(got["logits"][r * K + K - 1], base["logits"][r * K + K - 1])


def test_ntp_logits_independent_of_K():
    model, args, pool, _, bs = _small_decode_case(K=7, seed=41)
    outs = {}
    for K in (1, 3, 7):
        exp = oracle.expand(args["num_tokens"], args["num_rejected"], args["target_ids"],
                            args["target_pos"], args["target_hidden"], args["next_token_ids"],
                            args["block_table"], model["h_shared"], K, MINI.V - 1, bs)
        outs[K] = oracle.draft_forward(model, exp, args["block_table"], pool, K, block_size=bs)["logits"]
    C = 3
    for r in range(C):
        assert _rel(outs[1][r], outs[7][r * 7]) < 1e-12
        assert _rel(outs[3][r * 3:r * 3 + 3], outs[7][r * 7:r * 7 + 3]) < 1e-12


def test_rejected_rows_change_nothing():
    """(d) a rejected row writes no K/V and influences no logit."""
    model, args, pool, exp, bs = _small_decode_case(seed=51)
    K = 5
    base = oracle.draft_forward(model, exp, args["block_table"], pool, K, block_size=bs)
    rej = np.nonzero(exp["is_rejected"])[0]
    assert len(rej) > 0
    assert (exp["slot_mapping"][rej] == -1).all()
    for sl, _, _ in base["kv_written"]:
        assert (sl >= 0).all()
        assert sorted(sl.tolist()) == sorted(exp["slot_mapping"][exp["is_rejected"] == 0].tolist())
    pert = dict(exp)
    pert["hidden"] = exp["hidden"].copy()
    pert["hidden"][rej] ^= np.uint16(0x00FF)
    pert["input_ids"] = exp["input_ids"].copy()
    pert["input_ids"][rej] = 1
    got = oracle.draft_forward(model, pert, args["block_table"], pool, K, block_size=bs)
    assert np.array_equal(got["logits"], base["logits"])


def test_request_independence():
    model, args, pool, exp, bs = _small_decode_case(C=4, seed=61)
    K = 5
    full = oracle.draft_forward(model, exp, args["block_table"], pool, K, block_size=bs)
    for r in range(4):
        one = oracle.draft_forward(model, exp, args["block_table"], pool, K, requests=[r], block_size=bs)
        assert _rel(one["logits"], full["logits"][r * K:(r + 1) * K]) < 1e-12


def test_page_relabelling_invariance():
    model, args, pool, exp, bs = _small_decode_case(seed=71)
    K = 5
    base = oracle.draft_forward(model, exp, args["block_table"], pool, K, block_size=bs)
    nb = pool["k"].shape[1] // bs
    perm = np.random.default_rng(3).permutation(nb)        # old page -> new page
    bt2 = np.where(args["block_table"] >= 0, perm[np.maximum(args["block_table"], 0)], -1)
    src = np.argsort(perm)                                   # new page -> old page
    sl_new = (src[:, None] * bs + np.arange(bs)).reshape(-1)
    pool2 = {k: pool[k][:, sl_new] for k in ("k", "v")}
    exp2 = oracle.expand(args["num_tokens"], args["num_rejected"], args["target_ids"], args["target_pos"],
                         args["target_hidden"], args["next_token_ids"], bt2, model["h_shared"], K,
                         MINI.V - 1, bs)
    got = oracle.draft_forward(model, exp2, bt2, pool2, K, block_size=bs)
    assert _rel(got["logits"], base["logits"]) < 1e-13
