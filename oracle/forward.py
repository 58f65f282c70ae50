"""Oracle: the parallel-drafting forward pass (test infrastructure only).

What it follows:
  * [Blog] "P-EAGLE core method", the input equation Input_i: position 1 (NTP)
    pairs emb(new) with h_context, positions 2..K (MTP) pair emb(mask) with
    h_shared; all positions go through the N transformer layers and the LM
    head together, giving all K draft tokens in one pass.
  * [Paper] sec. 2 "architecture" and [arXiv] Figure 2 caption: target hidden
    states are 3d wide, the drafter projects them and combines them with the
    token embeddings; N LLaMA-3-style layers with RoPE; LM head.
  * [Paper] "experiment setup": 4 decoder layers of LLaMA 3.1 structure.
  * [Blog] "vLLM engineering details", KV-cache paragraph: a row writes its
    K/V at its slot, rejected rows (slot -1) write nothing.
  * [arXiv] Theorem 2.1 / 2.3 and [Paper] appendix B: the attention score of a
    rotated query/key pair depends on the positions only through their
    difference (R_p q)^T (R_p' k) = q^T R_(p'-p) k.

Readings taken where the pages leave a step open:
  * combine = concatenation (the Input_i equation's direct-sum sign and the
    blog's "concatenated"): layer 0 consumes [RMSNorm(emb; g_e) || RMSNorm(
    fc(h); g_h)] (2d wide) in its QKV projection, and the residual stream
    starts at fc(h); layers 1..N-1 are plain pre-norm LLaMA layers. The other
    reading (the paper's "embedding + projected hidden state": the residual
    starts at emb + fc(h), layer 0 is a plain layer) is kept as
    combine="sum";
  * h_shared is 3d wide and goes through fc like any target row;
  * every non-rejected row is computed (the whole copied verify window plus
    the MASK rows), not only the K sampled rows;
  * within a layer all K/V writes happen before any row attends;
  * RoPE is rotate-half with base rope_theta; RMSNorm eps = rms_eps; no
    biases; attention scale 1/sqrt(dh); greedy argmax, lowest index on ties.

Everything is float64. Matrix products use numpy's matmul (a library
primitive); nothing is blocked, fused or reordered.
"""
from __future__ import annotations

import numpy as np

from .bf16 import bf16_to_f64
from .fp8 import e4m3_decode, fp8_roundtrip
from .expand import ar_advance as _ar_advance


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """gamma * x / sqrt(mean(x^2) + eps) over the last axis."""
    return gamma * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def rope_rotate(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE. x: [..., H, dh]; pos: integer array of shape x.shape[:-2]
    (or a scalar). For i < dh/2 the pair (x_i, x_{i+dh/2}) is rotated by the
    angle pos * theta^(-2i/dh)."""
    dh = x.shape[-1]
    half = dh // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / dh)
    ang = np.asarray(pos, dtype=np.float64)[..., None, None] * inv_freq  # [..., 1, half]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _as_f64(a) -> np.ndarray:
    """bf16 bit patterns (uint16) are widened exactly; float arrays are used as they are."""
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def _cache_values(a, kv_fp8, l: int, which: str) -> np.ndarray:
    """Cache contents of layer l as values: bf16 bits (uint16), E4M3 codes
    (uint8: the code's value times the layer's scale) or floats as they are."""
    a = np.asarray(a)
    if a.dtype == np.uint8:
        if kv_fp8 is None:
            raise ValueError("an fp8 cache needs kv_fp8 scales")
        return e4m3_decode(a) * float(kv_fp8[which + "_scale"][l])
    return _as_f64(a)


def _softmax(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def draft_forward(model: dict, exp: dict, block_table, kv: dict, K: int,
                  requests=None, block_size: int = 16, return_layers: bool = False, kv_fp8=None,
                  combine: str = "concat") -> dict:
    """Run the drafter over the expanded batch `exp` (the oracle's own expansion).

    model: bf16-bit weights as made by synth.make_model (row-major [out][in]).
    kv:    the prior cache, slot-addressed: kv["k"], kv["v"] have shape
           [N][slots][Hkv][dh] (slot = page * block_size + offset), either bf16
           bits (uint16) or float values.
    requests: subset of request indices to compute (requests are independent),
           default all.
    exp may carry "hidden_d" ([T_out][d] float) with "use_hidden_d" ([T_out]
    bool): those rows take hidden_d as their projected hidden input directly
    (no fc) -- the drafter's own hidden state fed back in autoregressive
    passes (see expand.ar_advance).
    kv_fp8: None for a bf16 cache, or {"k_scale": [N], "v_scale": [N]} for an
    fp8 E4M3 cache ([Blog] "vLLM engineering details": the serving
    configuration keeps the KV cache in fp8): every K/V value this pass writes
    is stored as the code of value / scale (oracle.fp8) and read back as
    code value * scale; kv then holds uint8 codes (or values already read
    back).
    combine: how the token embedding and the projected hidden state meet.
    "concat" (the reading taken everywhere else: the Input_i equation's
    direct-sum sign in [Blog] "P-EAGLE core method") -- layer 0's QKV reads
    [RMSNorm(emb; norm_emb) || RMSNorm(fc(h); norm_hid)], 2d wide, and the
    residual starts at fc(h). "sum" (the other reading, [Paper] sec. 2
    architecture: the embedding plus the projected hidden state) -- the
    residual starts at emb + fc(h) and layer 0 is a plain pre-norm layer
    (norm_in of layer 0, a d-wide QKV).
    Returns logits [R][V] and draft_ids [R] for the K sampled rows of each
    requested request (request-major, NTP row first), hidden_out [R][d] (their
    final residual, before the final norm), the K/V each layer wrote (slots,
    k, v), and optionally the residual stream after fc and after every layer.
    """
    m = model["dims"]
    if combine not in ("concat", "sum"):
        raise ValueError(f"combine must be 'concat' or 'sum', not {combine!r}")
    eps, theta = m.rms_eps, m.rope_theta
    G = m.Hq // m.Hkv
    cu = np.asarray(exp["cu_out"], np.int64)
    C = len(cu) - 1
    reqs = list(range(C)) if requests is None else [int(r) for r in requests]
    bt = np.asarray(block_table, np.int64)
    rej = np.asarray(exp["is_rejected"]).astype(bool)
    seq_lens = np.asarray(exp["seq_lens"], np.int64)

    rows, row_req = [], []
    for r in reqs:
        for o in range(cu[r], cu[r + 1]):
            if not rej[o]:
                rows.append(o)
                row_req.append(r)
    rows = np.asarray(rows, np.int64)
    row_req = np.asarray(row_req, np.int64)
    nrow = len(rows)
    ids = np.asarray(exp["input_ids"], np.int64)[rows]
    pos = np.asarray(exp["positions"], np.int64)[rows]
    slots = np.asarray(exp["slot_mapping"], np.int64)[rows]

    # slots every computed request may read: positions 0..seq_len-1 through its block table
    read_slots = {}
    for r in reqs:
        t = np.arange(seq_lens[r])
        read_slots[r] = bt[r][t // block_size] * block_size + t % block_size
    all_slots = np.unique(np.concatenate([read_slots[r] for r in reqs] + [slots]))
    local = lambda s: np.searchsorted(all_slots, s)

    # fc projection of the 3d-wide hidden rows (or the given d-wide rows), token embeddings
    use_d = (np.asarray(exp["use_hidden_d"], bool)[rows] if "use_hidden_d" in exp
             else np.zeros(nrow, bool))
    x = np.empty((nrow, m.d))
    if (~use_d).any():
        h = bf16_to_f64(np.asarray(exp["hidden"])[rows[~use_d]])
        x[~use_d] = h @ bf16_to_f64(model["fc"]).T
    if use_d.any():
        x[use_d] = np.asarray(exp["hidden_d"], np.float64)[rows[use_d]]
    e = bf16_to_f64(np.asarray(model["embed"])[ids])
    if combine == "sum":
        x = x + e
    layers_out = [x.copy()] if return_layers else None
    written = []

    for l, L in enumerate(model["layers"]):
        if l == 0 and combine == "concat":
            u = np.concatenate([rms_norm(e, bf16_to_f64(model["norm_emb"]), eps),
                                rms_norm(x, bf16_to_f64(model["norm_hid"]), eps)], axis=-1)
        else:
            u = rms_norm(x, bf16_to_f64(L["norm_in"]), eps)
        qkv = u @ bf16_to_f64(L["w_qkv"]).T
        q = qkv[:, : m.Hq * m.dh].reshape(nrow, m.Hq, m.dh)
        k = qkv[:, m.Hq * m.dh: (m.Hq + m.Hkv) * m.dh].reshape(nrow, m.Hkv, m.dh)
        v = qkv[:, (m.Hq + m.Hkv) * m.dh:].reshape(nrow, m.Hkv, m.dh)
        q = rope_rotate(q, pos, theta)
        k = rope_rotate(k, pos, theta)

        # cache: prior contents of the readable slots, then this layer's writes
        kc = _cache_values(kv["k"][l][all_slots], kv_fp8, l, "k")
        vc = _cache_values(kv["v"][l][all_slots], kv_fp8, l, "v")
        if kv_fp8 is not None:   # what an fp8 cache holds for the new rows
            k = fp8_roundtrip(k, float(kv_fp8["k_scale"][l]))
            v = fp8_roundtrip(v, float(kv_fp8["v_scale"][l]))
        kc[local(slots)] = k
        vc[local(slots)] = v
        written.append((slots.copy(), k.copy(), v.copy()))

        # causal attention of each row over positions 0..p of its own request
        o = np.empty((nrow, m.Hq, m.dh))
        for i in range(nrow):
            p = int(pos[i])
            idx = local(read_slots[int(row_req[i])][: p + 1])
            Kc, Vc = kc[idx], vc[idx]                         # [p+1][Hkv][dh]
            qg = q[i].reshape(m.Hkv, G, m.dh)
            s = np.einsum("tkd,kgd->kgt", Kc, qg) / np.sqrt(m.dh)
            a = _softmax(s)
            o[i] = np.einsum("kgt,tkd->kgd", a, Vc).reshape(m.Hq, m.dh)

        x = x + o.reshape(nrow, m.Hq * m.dh) @ bf16_to_f64(L["w_o"]).T
        y = rms_norm(x, bf16_to_f64(L["norm_post"]), eps)
        gate = y @ bf16_to_f64(L["w_gate"]).T
        up = y @ bf16_to_f64(L["w_up"]).T
        x = x + (silu(gate) * up) @ bf16_to_f64(L["w_down"]).T
        if return_layers:
            layers_out.append(x.copy())

    # LM head on the K sampled rows of each request (NTP row, then MASK rows)
    new_idx = np.asarray(exp["new_token_indices"], np.int64)
    sampled = np.concatenate([new_idx[r * K:(r + 1) * K] for r in reqs]) if reqs else np.zeros(0, np.int64)
    where = {int(o): i for i, o in enumerate(rows)}
    xs = x[[where[int(o)] for o in sampled]]
    z = rms_norm(xs, bf16_to_f64(model["norm_final"]), eps)
    logits = z @ bf16_to_f64(model["lm_head"]).T
    out = {
        "requests": reqs, "rows": rows, "sampled_rows": sampled,
        "logits": logits, "draft_ids": np.argmax(logits, axis=1).astype(np.int32),
        "hidden_out": xs, "kv_written": written,
    }
    if return_layers:
        out["layers"] = layers_out
    return out


def ar_draft(model: dict, exp1: dict, block_table, kv: dict, K: int, block_size: int = 16,
             tokens=None, hidden=None, kv_fp8=None) -> list:
    """Autoregressive EAGLE-style drafting of K tokens per request: K serial
    drafter passes ([Blog] "background and motivation"), the baseline that
    parallel drafting replaces.

    exp1 is the K = 1 expansion of the verify batch (pass 1 = the NTP
    position, [Blog] "P-EAGLE core method"). Pass k >= 2 runs the one-row batch
    of ``ar_advance``: the previous pass's sampled token with the drafter's own
    final hidden state of that row as the (already d-wide) hidden input. Every
    pass writes its K/V to the cache before the next reads it.

    tokens: optional [K][C] tokens to feed forward instead of this function's
    own argmax (a caller comparing against another implementation feeds its
    choices so both take the same path through near-ties).
    hidden: optional [K-1][C][d] fed-back hidden states to use instead of this
    function's own ``hidden_out`` (so such a caller can hold each pass to a
    single pass's error budget instead of letting the fed state's error
    compound over the passes).
    Returns the K pass results of ``draft_forward`` (logits, draft_ids,
    hidden_out, ...) and the batches they ran on ("batch").
    """
    m = model["dims"]
    kvf = {"k": [_cache_values(kv["k"][l], kv_fp8, l, "k").copy() for l in range(m.N)],
           "v": [_cache_values(kv["v"][l], kv_fp8, l, "v").copy() for l in range(m.N)]}
    out, batch = [], exp1
    for k in range(K):
        res = draft_forward(model, batch, block_table, kvf, 1, block_size=block_size, kv_fp8=kv_fp8)
        res["batch"] = batch
        out.append(res)
        for l, (sl, kk, vv) in enumerate(res["kv_written"]):
            kvf["k"][l][sl] = kk
            kvf["v"][l][sl] = vv
        if k + 1 == K:
            break
        ids = res["draft_ids"] if tokens is None else np.asarray(tokens[k])
        nxt = _ar_advance(batch, 1, ids, block_table, block_size)
        C = len(nxt["cu_out"]) - 1
        nxt["hidden_d"] = res["hidden_out"] if hidden is None else np.asarray(hidden[k], np.float64)
        nxt["use_hidden_d"] = np.ones(C, bool)
        batch = nxt
    return out
