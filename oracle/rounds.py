"""Oracle: several draft/verify rounds in a row with a stand-in verifier
-- TEST INFRASTRUCTURE ONLY.

[Blog] "vLLM engineering details", batch-reshape paragraph: for EAGLE the
window the drafter consumes is the window the verifier checks next (the K
drafts plus one extra sampled token). One round here: the verifier stand-in
builds the verify batch from the previous round's drafts, then the expansion
and the drafter pass run on it. There is no target model: how many drafts
are accepted, the token the target samples after them and the target's
hidden rows are inputs of each round (seeded draws).

Readings (the pages give the loop, not its bookkeeping):
  * a round's verify window for request r is [the token the target sampled
    last round, the K drafts], at positions p_ntp + 1 .. p_ntp + 1 + K, where
    p_ntp is the previous round's NTP slot position (that slot paired the
    sampled token with the hidden state at p_ntp, so the token itself sits
    at p_ntp + 1);
  * the target accepts a_r of the K drafts (0..K): num_tokens = K + 1,
    num_rejected = K - a_r;
  * the drafter's KV cache carries over between rounds; a round's MASK rows
    wrote positions the next round's verify rows write again before any row
    reads them (stale entries are overwritten, never read).
"""
from __future__ import annotations

import numpy as np

from .expand import expand
from .forward import draft_forward, _cache_values


def verify_stub(prev_exp: dict, K: int, prev_draft_ids, prev_next_token_ids, accepted) -> dict:
    """The next round's verify batch (counts, ids, positions) from the
    previous round's expanded batch, its drafts [C*K] (request-major) and
    sampled tokens [C], and this round's accepted-draft counts [C]."""
    C = len(prev_exp["cu_out"]) - 1
    d = np.asarray(prev_draft_ids, np.int64).reshape(C, K)
    nxt = np.asarray(prev_next_token_ids, np.int64)
    a = np.asarray(accepted, np.int64)
    pos = np.asarray(prev_exp["positions"], np.int64)
    nti = np.asarray(prev_exp["new_token_indices"], np.int64)
    ids, tpos = [], []
    for r in range(C):
        p_ntp = int(pos[nti[r * K]])          # the previous round's NTP slot
        ids.append(int(nxt[r]))               # the token the target sampled, at p_ntp + 1
        tpos.append(p_ntp + 1)
        for j in range(K):                    # then the K drafts
            ids.append(int(d[r, j]))
            tpos.append(p_ntp + 2 + j)
    return {
        "num_tokens": np.full(C, K + 1, np.int32),
        "num_rejected": (K - a).astype(np.int32),
        "target_ids": np.asarray(ids, np.int32),
        "target_pos": np.asarray(tpos, np.int32),
    }


def draft_rounds(model: dict, args1: dict, rounds: list, block_table, kv: dict, K: int, mask_id: int,
                 block_size: int = 16, tokens=None, kv_fp8=None) -> list:
    """R = len(rounds) + 1 rounds of verify stand-in -> expansion -> drafter pass.

    args1: round 1's verify batch (num_tokens, num_rejected, target_ids,
    target_pos, target_hidden, next_token_ids). rounds[t]: the inputs of round
    t + 2 -- "accepted" [C], "next_token_ids" [C] (the token the target
    samples after that round's verification) and "target_hidden"
    [C*(K+1)][3d] bf16 bits. tokens: optional [R-1][C*K] drafts to feed the
    verifier instead of this function's own argmax.
    Returns per round: the expansion ("exp") and the drafter results
    (logits, draft_ids, kv_written, ...). The KV cache is carried in float64.
    """
    m = model["dims"]
    kvf = {"k": [_cache_values(kv["k"][l], kv_fp8, l, "k").copy() for l in range(m.N)],
           "v": [_cache_values(kv["v"][l], kv_fp8, l, "v").copy() for l in range(m.N)]}
    out = []
    args = args1
    for t in range(len(rounds) + 1):
        exp = expand(args["num_tokens"], args["num_rejected"], args["target_ids"], args["target_pos"],
                     args["target_hidden"], args["next_token_ids"], block_table, model["h_shared"], K,
                     mask_id, block_size)
        res = draft_forward(model, exp, block_table, kvf, K, block_size=block_size, kv_fp8=kv_fp8)
        res["exp"] = exp
        out.append(res)
        for l, (sl, kk, vv) in enumerate(res["kv_written"]):
            kvf["k"][l][sl] = kk
            kvf["v"][l][sl] = vv
        if t == len(rounds):
            break
        drafts = res["draft_ids"] if tokens is None else np.asarray(tokens[t])
        nxt_in = rounds[t]
        vb = verify_stub(exp, K, drafts, args["next_token_ids"], nxt_in["accepted"])
        vb["target_hidden"] = nxt_in["target_hidden"]
        vb["next_token_ids"] = np.asarray(nxt_in["next_token_ids"], np.int32)
        args = vb
    return out
