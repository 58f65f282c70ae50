"""Pins for the oracle's batch expansion (CPU only).

Pinned against: a hand-worked example (tests/golden), the hidden-state fill
described on the vLLM blog page ("vLLM engineering details", hidden-state
paragraph) re-expressed with torch index ops, the K=1 reduction to the
autoregressive-EAGLE input, and brute-force invariants on many random batches.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "expand_hand_example.json")


def _gold():
    with open(GOLD) as f:
        return json.load(f)


def _run_gold(K):
    g = _gold()
    inp, p = g["inputs"], g["params"]
    H3 = 8
    T_in = sum(inp["num_tokens"])
    hidden = np.arange(T_in * H3, dtype=np.uint16).reshape(T_in, H3) + 1
    h_shared = np.full(H3, 0xBEEF, np.uint16)
    out = oracle.expand(inp["num_tokens"], inp["num_rejected"], inp["target_ids"],
                        inp["target_pos"], hidden, inp["next_token_ids"],
                        np.array(inp["block_table"]), h_shared, K, p["mask_id"], p["block_size"])
    return out, hidden, h_shared


@pytest.mark.parametrize("K,key", [(3, "expected"), (1, "expected_K1")])
def test_hand_worked_example(K, key):
    exp = _gold()[key]
    out, hidden, h_shared = _run_gold(K)
    for name in ["input_ids", "positions", "slot_mapping", "is_rejected", "is_masked",
                 "hidden_state_mapping", "new_token_indices", "cu_out", "seq_lens"]:
        assert out[name].tolist() == exp[name], name
    for o in range(out["T_out"]):
        if o in exp["mask_rows"]:
            assert (out["hidden"][o] == h_shared).all()
    for j, o in enumerate(exp["hidden_state_mapping"]):
        assert (out["hidden"][o] == hidden[j]).all()


def _fill_as_described(hmap, target_hidden, is_masked, h_shared, T_out):
    """Hidden fill as the blog page describes it, written with torch ops:
    scatter the target rows through the map, then select h_shared wherever
    the MASK-slot mask is set."""
    t = torch.from_numpy(target_hidden.astype(np.int32))
    buf = torch.zeros((T_out, t.shape[1]), dtype=torch.int32)
    buf.index_copy_(0, torch.from_numpy(hmap.astype(np.int64)), t)
    sel = torch.from_numpy(is_masked.astype(bool)).unsqueeze(1)
    shared = torch.from_numpy(h_shared.astype(np.int32)).unsqueeze(0).expand_as(buf)
    return torch.where(sel, shared, buf).numpy().astype(np.uint16)


@pytest.mark.parametrize("name", ["tiny", "g_c4", "g_c64"])
def test_hidden_fill_matches_page_description(name):
    w = synth.get_workload(name)
    b = synth.make_batch(w)
    H3 = 24  # narrow rows keep the test fast; the fill is width-agnostic
    hid = b["target_hidden"][:, :H3].copy()
    hs = np.arange(H3, dtype=np.uint16) + 7
    out = oracle.expand(b["num_tokens"], b["num_rejected"], b["target_ids"], b["target_pos"],
                        hid, b["next_token_ids"], b["block_table"], hs, w.K, b["mask_id"], 16)
    ref = _fill_as_described(out["hidden_state_mapping"], hid, out["is_masked"], hs, out["T_out"])
    assert np.array_equal(out["hidden"], ref)


def _random_batch(rng, C, K, bs):
    n = rng.integers(1, 2 * K + 3, size=C)
    rho = np.array([rng.integers(0, x) for x in n])
    L = rng.integers(0, 60, size=C)
    pos = np.concatenate([np.arange(L[r], L[r] + n[r]) for r in range(C)])
    pages = [-(-(L[r] + n[r] + K) // bs) for r in range(C)]
    nb = sum(pages) + 3
    perm = rng.permutation(nb)
    bt = np.full((C, max(pages)), -1)
    u = 0
    for r in range(C):
        bt[r, :pages[r]] = perm[u:u + pages[r]]
        u += pages[r]
    T_in = int(n.sum())
    ids = rng.integers(0, 1000, size=T_in)
    nxt = rng.integers(0, 1000, size=C)
    hid = rng.integers(0, 60000, size=(T_in, 4)).astype(np.uint16)
    hs = np.array([1, 2, 3, 4], np.uint16)
    return dict(n=n, rho=rho, L=L, pos=pos, bt=bt, ids=ids, nxt=nxt, hid=hid, hs=hs)


@pytest.mark.parametrize("seed", range(40))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    C = int(rng.integers(1, 9))
    K = int(rng.integers(1, 9))
    bs = int(rng.choice([1, 4, 16]))
    B = _random_batch(rng, C, K, bs)
    out = oracle.expand(B["n"], B["rho"], B["ids"], B["pos"], B["hid"], B["nxt"], B["bt"],
                        B["hs"], K, 4095, bs)
    T_in = int(B["n"].sum())
    assert out["T_out"] == T_in + C * (K - 1)
    # counts
    assert int(out["is_masked"].sum()) == C * (K - 1)
    assert int(out["is_rejected"].sum()) == int(B["rho"].sum())
    # (d) rejected rows get -1, everything else a distinct, non-negative slot
    sl = out["slot_mapping"]
    assert (sl[out["is_rejected"] == 1] == -1).all()
    good = sl[out["is_rejected"] == 0]
    assert (good >= 0).all() and len(np.unique(good)) == len(good)
    # (a) all MASK rows carry identical inputs (id and hidden row)
    mrows = np.nonzero(out["is_masked"])[0]
    assert (out["input_ids"][mrows] == 4095).all()
    assert (out["hidden"][mrows] == B["hs"]).all()
    # per request: one non-rejected row per position L_r .. p_ntp+K-1, slot = page address
    cu = out["cu_out"]
    for r in range(C):
        v = int(B["n"][r] - B["rho"][r])
        rows = [o for o in range(cu[r], cu[r + 1]) if not out["is_rejected"][o]]
        ps = sorted(out["positions"][rows].tolist())
        p_ntp = int(B["L"][r] + v - 1)
        assert ps == list(range(int(B["L"][r]), p_ntp + K))
        for o in rows:
            p = int(out["positions"][o])
            assert sl[o] == B["bt"][r][p // bs] * bs + p % bs
        assert out["seq_lens"][r] == p_ntp + K
        ni = out["new_token_indices"][r * K:(r + 1) * K]
        assert out["input_ids"][ni[0]] == B["nxt"][r] and out["positions"][ni[0]] == p_ntp
        assert (out["is_masked"][ni[1:]] == 1).all()
        assert out["positions"][ni].tolist() == list(range(p_ntp, p_ntp + K))
    # the hidden map is a bijection onto the non-MASK rows
    hm = out["hidden_state_mapping"]
    assert sorted(hm.tolist()) == sorted(np.nonzero(out["is_masked"] == 0)[0].tolist())
    assert np.array_equal(out["hidden"][hm], B["hid"])


@pytest.mark.parametrize("seed", range(10))
def test_K1_reduces_to_autoregressive_input(seed):
    """Invariant (b): at K=1 nothing is appended, and the K>1 expansion with its
    MASK rows removed is exactly the K=1 (autoregressive EAGLE) batch."""
    rng = np.random.default_rng(100 + seed)
    C, K, bs = int(rng.integers(1, 7)), int(rng.integers(2, 9)), 16
    B = _random_batch(rng, C, K, bs)
    args = (B["n"], B["rho"], B["ids"], B["pos"], B["hid"], B["nxt"], B["bt"], B["hs"])
    one = oracle.expand(*args, 1, 4095, bs)
    many = oracle.expand(*args, K, 4095, bs)
    assert one["T_out"] == int(B["n"].sum()) and one["is_masked"].sum() == 0
    keep = many["is_masked"] == 0
    for name in ["input_ids", "positions", "slot_mapping", "is_rejected"]:
        assert np.array_equal(many[name][keep], one[name]), name
    assert np.array_equal(many["hidden"][keep], one["hidden"])
    # the NTP row of every request is its only sampled row at K=1
    ntp_many = many["new_token_indices"].reshape(C, K)[:, 0]
    remap = np.cumsum(keep) - 1
    assert np.array_equal(remap[ntp_many], one["new_token_indices"])
    # autoregressive EAGLE pairing: token i+1 with hidden i; the sampled token at the last valid slot
    start = 0
    for r in range(C):
        n, v = int(B["n"][r]), int(B["n"][r] - B["rho"][r])
        for i in range(v - 1):
            assert one["input_ids"][start + i] == B["ids"][start + i + 1]
        assert one["input_ids"][start + v - 1] == B["nxt"][r]
        start += n
