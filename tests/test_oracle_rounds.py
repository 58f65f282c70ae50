"""Pins for the oracle's multi-round loop (verify stand-in -> expansion ->
drafter pass, KV carried over; CPU only).

  * the verify stand-in on a hand-worked example (tests/golden), built on the
    hand-worked expansion example;
  * R rounds from an empty cache == a dense library prefill over every
    position the rounds accepted: at each round, the K sampled rows' logits
    equal tests/dense_ref.py run on the whole accepted sequence (tokens and
    target hidden rows collected from the rounds' verify windows). A wrong
    verify position, a missing sampled token, a wrong rejected count or a
    KV cache that is not carried between rounds breaks it, and so would a
    stale MASK-row entry that a later round read before rewriting;
  * cache entries past each request's context (never written before round
    1) do not change any round;
  * the rounds' bookkeeping: each window starts right after the previous
    NTP slot, K + 1 tokens, K - a rejected.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from dense_ref import dense_prefill_logits
from test_oracle_forward import MINI, _rel

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "verify_stub_hand_example.json")


def test_verify_stub_hand_example():
    g = json.load(open(GOLD))
    got = oracle.verify_stub(g["prev"], g["K"], g["prev_draft_ids"], g["prev_next_token_ids"], g["accepted"])
    for k, v in g["expected"].items():
        assert list(got[k]) == v, k


def _prefill_rounds(C=2, n0=(7, 5), K=3, R=4, seed=61, bs=4):
    dims = MINI
    rng = np.random.default_rng(seed)
    model = synth.make_model(dims, seed=seed)
    n0 = np.asarray(n0[:C])
    total = [int(n0[r]) + R * (K + 1) + K for r in range(C)]
    pages = [-(-t // bs) for t in total]
    nb = sum(pages) + 3
    perm = rng.permutation(nb)
    bt = np.full((C, max(pages)), -1)
    u = 0
    for r in range(C):
        bt[r, :pages[r]] = perm[u:u + pages[r]]
        u += pages[r]
    pool = synth.make_kv_pool(dims, nb, seed, block_size=bs)
    T0 = int(n0.sum())
    args1 = dict(num_tokens=n0, num_rejected=np.zeros(C, np.int64),
                 target_ids=rng.integers(0, dims.V - 1, size=T0),
                 target_pos=np.concatenate([np.arange(int(x)) for x in n0]),
                 target_hidden=synth.f32_to_bf16_bits(rng.standard_normal((T0, dims.hidden3)).astype(np.float32)),
                 next_token_ids=rng.integers(0, dims.V - 1, size=C))
    rounds = []
    for t in range(R - 1):
        rounds.append({"accepted": rng.integers(0, K + 1, size=C),
                       "next_token_ids": rng.integers(0, dims.V - 1, size=C),
                       "target_hidden": synth.f32_to_bf16_bits(
                           rng.standard_normal((C * (K + 1), dims.hidden3)).astype(np.float32))})
    return model, args1, rounds, bt, pool, bs


@pytest.mark.parametrize("C,K,R,seed", [(2, 3, 4, 61), (1, 1, 3, 62), (2, 5, 3, 63)])
def test_rounds_equal_dense_prefill(C, K, R, seed):
    model, args1, rounds, bt, pool, bs = _prefill_rounds(C=C, K=K, R=R, seed=seed)
    res = oracle.draft_rounds(model, args1, rounds, bt, pool, K, MINI.V - 1, block_size=bs)
    assert len(res) == R
    # the sequence the rounds accepted: round 1's prompt, then per round the
    # previous sampled token and the accepted drafts, with the window's hidden rows
    for r in range(C):
        n0 = int(args1["num_tokens"][r])
        s0 = int(np.sum(args1["num_tokens"][:r]))
        toks = list(args1["target_ids"][s0:s0 + n0])
        hids = list(args1["target_hidden"][s0:s0 + n0])
        nxt = int(args1["next_token_ids"][r])
        for t in range(R):
            if t > 0:
                rd = rounds[t - 1]
                a = int(rd["accepted"][r])
                drafts = np.asarray(res[t - 1]["draft_ids"]).reshape(C, K)[r]
                window = [nxt] + list(drafts)
                toks += window[:a + 1]
                hids += list(rd["target_hidden"][r * (K + 1):r * (K + 1) + a + 1])
                nxt = int(rd["next_token_ids"][r])
            # tokens and hidden rows at 0..p_ntp; the sampled token sits at p_ntp + 1
            assert len(toks) == len(hids)
            want = dense_prefill_logits(model, np.asarray(toks), np.asarray(hids), nxt, K, MINI.V - 1)
            want = want.numpy() if hasattr(want, "numpy") else np.asarray(want)
            got = np.asarray(res[t]["logits"])[r * K:(r + 1) * K]
            assert _rel(got, want) < 1e-9, (r, t)


def test_unwritten_cache_entries_do_not_matter():
    model, args1, rounds, bt, pool, bs = _prefill_rounds(C=2, K=3, R=3, seed=64)
    a = oracle.draft_rounds(model, args1, rounds, bt, pool, 3, MINI.V - 1, block_size=bs)
    rng = np.random.default_rng(5)
    pool2 = {k: synth.f32_to_bf16_bits(rng.standard_normal(v.shape).astype(np.float32)) for k, v in pool.items()}
    b = oracle.draft_rounds(model, args1, rounds, bt, pool2, 3, MINI.V - 1, block_size=bs)
    for x, y in zip(a, b):
        assert np.array_equal(x["logits"], y["logits"])


def test_round_bookkeeping():
    model, args1, rounds, bt, pool, bs = _prefill_rounds(C=2, K=3, R=4, seed=65)
    res = oracle.draft_rounds(model, args1, rounds, bt, pool, 3, MINI.V - 1, block_size=bs)
    for t in range(1, 4):
        prev, cur = res[t - 1]["exp"], res[t]["exp"]
        for r in range(2):
            p_ntp = int(prev["positions"][prev["new_token_indices"][r * 3]])
            lo, hi = int(cur["cu_out"][r]), int(cur["cu_out"][r + 1])
            a = int(rounds[t - 1]["accepted"][r])
            # the window: K + 1 copied rows from p_ntp + 1, then K - 1 MASK rows
            assert hi - lo == 3 + 1 + 2
            assert list(cur["positions"][lo:lo + 4]) == list(range(p_ntp + 1, p_ntp + 5))
            assert int(np.sum(cur["is_rejected"][lo:hi])) == 3 - a
            # this round's NTP slot is the last accepted row
            assert int(cur["positions"][cur["new_token_indices"][r * 3]]) == p_ntp + 1 + a
