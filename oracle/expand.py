"""Oracle: batch expansion for parallel drafting (test infrastructure only).

What it follows:
  * [Blog] "vLLM engineering details", batch-reshape paragraph: the draft batch
    appends MASK placeholders after each request's token ([token, MASK, MASK,
    ...]); ids, hidden states and positions are expanded, each request's
    positions grow, and the slot mapping and per-request start indices are
    rebuilt from the new positions.
  * [Blog] same section, fused-kernel paragraph: previous ids and positions go
    to their new slots, the target-sampled token is inserted, the extra slots
    get the MASK id, and the kernel emits a rejected-token mask, a MASK-slot
    mask, the new-token indices used for sampling drafts, and a hidden-state
    map.
  * [Blog] same section, hidden-state paragraph (the printed code): target
    rows are scattered through the map, then MASK rows take the learned
    shared hidden state.
  * [Blog] same section, KV-cache paragraph: rejected tokens get slot -1 so
    nothing is written for them.
  * [Blog] "P-EAGLE core method", prompt-position rule: slot i pairs the token
    of position i+1 with the hidden state of position i (one-position shift,
    as in autoregressive EAGLE); the NTP slot pairs the newly sampled token
    with the last accepted hidden state.

Readings taken where the pages leave a step open (each also listed in the
design notes):
  * a request's verify segment has n_r tokens of which the last rho_r were
    rejected; v_r = n_r - rho_r >= 1 are valid, and the NTP slot is the last
    valid one (i = v_r - 1);
  * MASK slots sit right after the request's n_r copied slots, at positions
    p_ntp+1 .. p_ntp+K-1;
  * a rejected slot keeps the shifted id (or the sampled token when it is the
    segment's last slot) and its copied position; it is never written to the
    cache and never sampled, so these values are unobservable downstream;
  * new_token_indices is request-major: the NTP slot, then the K-1 MASK slots;
  * seq_len of a request = p_ntp + K (keys visible to its last MASK row + 1).
"""
from __future__ import annotations

import numpy as np


def _slot(block_table_row, pos: int, block_size: int) -> int:
    """Paged-KV address of a position: page number times page size plus offset."""
    return int(block_table_row[pos // block_size]) * block_size + pos % block_size


def expand(num_tokens, num_rejected, target_ids, target_pos, target_hidden,
           next_token_ids, block_table, h_shared, K: int, mask_id: int,
           block_size: int) -> dict:
    """Expand a verify batch into the parallel-drafting batch.

    Inputs are per-request counts (n_r, rho_r), flattened target rows
    (ids, positions, 3d-wide hidden rows as bf16 bits), the sampled token per
    request, the block table [C][max_blocks] and h_shared (bf16 bits).
    Returns int arrays and the expanded hidden rows (bf16 bits, copied
    bit-for-bit: the fill moves values, it computes none).
    """
    n = np.asarray(num_tokens, dtype=np.int64)
    rho = np.asarray(num_rejected, dtype=np.int64)
    tid = np.asarray(target_ids, dtype=np.int64)
    tpos = np.asarray(target_pos, dtype=np.int64)
    nxt = np.asarray(next_token_ids, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    C = len(n)
    T_in = int(n.sum())
    T_out = T_in + C * (K - 1)
    H3 = np.asarray(h_shared).shape[-1]

    ids = np.zeros(T_out, np.int64)
    pos = np.zeros(T_out, np.int64)
    slot = np.zeros(T_out, np.int64)
    is_rej = np.zeros(T_out, np.uint8)
    is_mask = np.zeros(T_out, np.uint8)
    hmap = np.zeros(T_in, np.int64)
    new_idx = np.zeros(C * K, np.int64)
    cu_out = np.zeros(C + 1, np.int64)
    seq_lens = np.zeros(C, np.int64)

    in_start = 0
    for r in range(C):
        v = int(n[r] - rho[r])
        out_start = in_start + r * (K - 1)
        cu_out[r] = out_start
        for i in range(int(n[r])):
            o, j = out_start + i, in_start + i
            if i == v - 1:
                ids[o] = nxt[r]                 # the target-sampled token
            elif i + 1 < n[r]:
                ids[o] = tid[j + 1]             # one-position shift
            else:
                ids[o] = nxt[r]                 # last slot, rejected
            pos[o] = tpos[j]
            is_rej[o] = 1 if i >= v else 0
            slot[o] = -1 if is_rej[o] else _slot(bt[r], int(pos[o]), block_size)
            hmap[j] = o
        p_ntp = int(tpos[in_start + v - 1])
        new_idx[r * K] = out_start + v - 1
        for mm in range(1, K):
            o = out_start + int(n[r]) + mm - 1
            ids[o] = mask_id
            pos[o] = p_ntp + mm
            is_mask[o] = 1
            slot[o] = _slot(bt[r], p_ntp + mm, block_size)
            new_idx[r * K + mm] = o
        seq_lens[r] = p_ntp + K
        in_start += int(n[r])
    cu_out[C] = T_out

    # hidden-state fill: scatter target rows through the map, then the MASK
    # rows take h_shared (every row is then defined: T_out = T_in + C(K-1)).
    hidden = np.zeros((T_out, H3), np.uint16)
    hidden[hmap] = np.asarray(target_hidden, dtype=np.uint16).reshape(T_in, H3)
    hidden[is_mask.astype(bool)] = np.asarray(h_shared, dtype=np.uint16)

    i32 = lambda a: a.astype(np.int32)
    return {
        "T_out": T_out,
        "input_ids": i32(ids), "positions": i32(pos), "slot_mapping": i32(slot),
        "is_rejected": is_rej, "is_masked": is_mask,
        "hidden_state_mapping": i32(hmap), "new_token_indices": i32(new_idx),
        "cu_out": i32(cu_out), "seq_lens": i32(seq_lens), "hidden": hidden,
    }


def ar_advance(prev: dict, K_prev: int, draft_ids, block_table, block_size: int) -> dict:
    """The next pass of autoregressive (EAGLE-style) drafting, one row per request.

    [Blog] "background and motivation": autoregressive EAGLE drafts K tokens
    with K serial forward passes of the drafter. [Blog] "P-EAGLE core method"
    and [arXiv] Figure 2 caption: the NTP position (pass 1) is exactly the
    autoregressive case; the later positions lack inputs in the parallel
    drafter because, autoregressively, they would come from the previous pass.

    Reading (the pages leave the fed-back state open): pass k >= 2 has one row
    per request, at the position after the previous pass's last sampled row;
    its token is the token that pass sampled, and its hidden input is the
    drafter's own final hidden state of that sampled row (d wide, so it does
    not go through fc; the forward's ``hidden_d`` rows). Rows are never
    rejected and every row is sampled.

    prev: the previous pass's batch (an ``expand`` result or an earlier
    ``ar_advance`` result); K_prev: its draft depth; draft_ids: the tokens it
    sampled, request-major [C * K_prev].
    """
    C = len(prev["cu_out"]) - 1
    new_idx = np.asarray(prev["new_token_indices"], np.int64)
    pos_prev = np.asarray(prev["positions"], np.int64)
    ids = np.asarray(draft_ids, np.int64)
    bt = np.asarray(block_table, np.int64)
    last = [r * K_prev + K_prev - 1 for r in range(C)]   # the last sampled row of each request
    positions = np.array([pos_prev[new_idx[i]] + 1 for i in last], np.int32)
    return {
        "input_ids": np.array([ids[i] for i in last], np.int32),
        "positions": positions,
        "slot_mapping": np.array([_slot(bt[r], int(positions[r]), block_size) for r in range(C)], np.int32),
        "is_rejected": np.zeros(C, np.uint8),
        "is_masked": np.zeros(C, np.uint8),
        "new_token_indices": np.arange(C, dtype=np.int32),
        "cu_out": np.arange(C + 1, dtype=np.int32),
        "seq_lens": (positions + 1).astype(np.int32),
    }
