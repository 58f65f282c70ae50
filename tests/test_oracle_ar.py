"""Pins for the oracle's autoregressive (EAGLE-style) K-pass drafting (CPU only).

The autoregressive baseline runs K serial drafter passes ([Blog] "background
and motivation"); pass 1 is the NTP position of the parallel drafter
([Blog] "P-EAGLE core method"). Pins, each against something other than the
multi-pass driver itself:
  * K serial passes == one causal forward over the same rows: the verify
    window, then each pass's row with the token and hidden state that pass
    was fed, all sampled together. Causal attention makes a row independent
    of later rows, so the two must agree; a missing KV carry-over between
    passes, a wrong position, slot or sequence length of a new row breaks it.
  * pass 1 == the parallel drafter's NTP logits (at any K).
  * feeding a chosen token sequence reaches the same path as the driver's own
    argmax when the choices agree, and a different one when they differ.
"""
import numpy as np

import oracle
from test_oracle_forward import MINI, _rel, _small_decode_case


def _ar_case(K=4, seed=51):
    model, args, pool, _, bs = _small_decode_case(C=3, K=K, seed=seed)
    exp1 = oracle.expand(args["num_tokens"], args["num_rejected"], args["target_ids"], args["target_pos"],
                         args["target_hidden"], args["next_token_ids"], args["block_table"],
                         model["h_shared"], 1, MINI.V - 1, bs)
    return model, args, pool, exp1, bs


def _combined_batch(exp1, passes, block_table, bs):
    """One batch holding, per request, the K=1 batch's rows and then one row
    per later pass (its fed token and hidden state), every pass's sampled row
    sampled together."""
    C = len(exp1["cu_out"]) - 1
    Kp = len(passes)
    bt = np.asarray(block_table)
    cols = {k: [] for k in ("input_ids", "positions", "slot_mapping", "is_rejected", "is_masked")}
    hidden, hidden_d, use_d, new_idx, cu, seq = [], [], [], [], [0], []
    d = passes[0]["hidden_out"].shape[1]
    for r in range(C):
        base = len(cols["input_ids"])
        for o in range(exp1["cu_out"][r], exp1["cu_out"][r + 1]):
            for k in cols:
                cols[k].append(exp1[k][o])
            hidden.append(exp1["hidden"][o])
            hidden_d.append(np.zeros(d))
            use_d.append(False)
        ntp = base + int(exp1["new_token_indices"][r]) - int(exp1["cu_out"][r])
        new_idx.append(ntp)
        p = int(exp1["positions"][exp1["new_token_indices"][r]])
        for k in range(1, Kp):
            p += 1
            cols["input_ids"].append(int(passes[k]["batch"]["input_ids"][r]))
            cols["positions"].append(p)
            cols["slot_mapping"].append(int(bt[r][p // bs]) * bs + p % bs)
            cols["is_rejected"].append(0)
            cols["is_masked"].append(0)
            hidden.append(np.zeros_like(exp1["hidden"][0]))
            hidden_d.append(passes[k - 1]["hidden_out"][r])
            use_d.append(True)
            new_idx.append(len(cols["input_ids"]) - 1)
        cu.append(len(cols["input_ids"]))
        seq.append(p + 1)
    out = {k: np.asarray(v) for k, v in cols.items()}
    out.update(hidden=np.asarray(hidden), hidden_d=np.asarray(hidden_d), use_hidden_d=np.asarray(use_d),
               new_token_indices=np.asarray(new_idx), cu_out=np.asarray(cu), seq_lens=np.asarray(seq))
    return out


def test_serial_passes_equal_one_causal_forward():
    K = 4
    model, args, pool, exp1, bs = _ar_case(K=K)
    passes = oracle.ar_draft(model, exp1, args["block_table"], pool, K, block_size=bs)
    assert len(passes) == K
    comb = _combined_batch(exp1, passes, args["block_table"], bs)
    one = oracle.draft_forward(model, comb, args["block_table"], pool, K, block_size=bs)
    C = 3
    for r in range(C):
        for k in range(K):
            assert _rel(one["logits"][r * K + k], passes[k]["logits"][r]) < 1e-9, (r, k)
    # the later passes really depend on the fed state: a different fed token changes them
    bad = [np.asarray(p["draft_ids"]) for p in passes[:-1]]
    bad[0] = (bad[0] + 1) % (MINI.V - 1)
    alt = oracle.ar_draft(model, exp1, args["block_table"], pool, K, block_size=bs, tokens=bad)
    assert _rel(alt[0]["logits"], passes[0]["logits"]) < 1e-12
    assert not np.allclose(alt[1]["logits"], passes[1]["logits"])


def test_pass1_equals_parallel_ntp_logits():
    model, args, pool, exp1, bs = _ar_case(K=7, seed=53)
    first = oracle.ar_draft(model, exp1, args["block_table"], pool, 1, block_size=bs)[0]
    for K in (1, 5):
        exp = oracle.expand(args["num_tokens"], args["num_rejected"], args["target_ids"], args["target_pos"],
                            args["target_hidden"], args["next_token_ids"], args["block_table"],
                            model["h_shared"], K, MINI.V - 1, bs)
        par = oracle.draft_forward(model, exp, args["block_table"], pool, K, block_size=bs)
        for r in range(3):
            assert _rel(par["logits"][r * K], first["logits"][r]) < 1e-12


def test_forced_tokens_equal_own_choice():
    K = 3
    model, args, pool, exp1, bs = _ar_case(K=K, seed=57)
    own = oracle.ar_draft(model, exp1, args["block_table"], pool, K, block_size=bs)
    forced = oracle.ar_draft(model, exp1, args["block_table"], pool, K, block_size=bs,
                             tokens=[p["draft_ids"] for p in own[:-1]])
    for a, b in zip(own, forced):
        assert np.array_equal(a["logits"], b["logits"])
    # feeding the run's own hidden states back reproduces it too; other states change the later passes
    fed = oracle.ar_draft(model, exp1, args["block_table"], pool, K, block_size=bs,
                          hidden=[p["hidden_out"] for p in own[:-1]])
    for a, b in zip(own, fed):
        assert np.array_equal(a["logits"], b["logits"])
    alt = oracle.ar_draft(model, exp1, args["block_table"], pool, K, block_size=bs,
                          hidden=[0.5 * p["hidden_out"] for p in own[:-1]])
    assert np.array_equal(alt[0]["logits"], own[0]["logits"])
    assert not np.allclose(alt[1]["logits"], own[1]["logits"])
    # pass k >= 2 rows sit right after the previous pass's sampled row, one row per request
    for k in range(1, K):
        bk = own[k]["batch"]
        prev = own[k - 1]["batch"]
        want = np.asarray(prev["positions"])[np.asarray(prev["new_token_indices"])] + 1
        assert np.array_equal(bk["positions"], want)
        assert np.array_equal(bk["seq_lens"], want + 1)
        assert np.array_equal(bk["input_ids"], own[k - 1]["draft_ids"])
