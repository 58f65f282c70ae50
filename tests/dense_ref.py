"""Dense torch-library reference for prefill-shaped drafting (pins the oracle).

When the drafter runs on a prompt from an empty cache, positions are 0..T-1
in row order and paged causal attention reduces to dense causal attention.
This helper builds the drafter input from the pages' input rule directly
(slot i: token of position i+1 with target hidden i; the last prompt slot:
the sampled token; then K-1 MASK slots with h_shared -- the Input_i equation
on the vLLM blog page) and runs it with torch library routines in float64:
torch.nn.functional.rms_norm, silu and scaled_dot_product_attention
(is_causal=True), and RoPE as multiplication by a unit complex number
(RoFormer's rotation written in complex form). It shares no code with the
oracle.
"""
import numpy as np
import torch
import torch.nn.functional as F


def _w(bits):
    b = torch.from_numpy(np.asarray(bits, dtype=np.uint16).astype(np.int32))
    return (b << 16).view(torch.float32).to(torch.float64)


def _rope_complex(x, positions, theta):
    # x: [T, H, dh]; pair (x_i, x_{i+dh/2}) is the complex number x_i + 1j*x_{i+dh/2}
    T, H, dh = x.shape
    half = dh // 2
    freqs = 1.0 / (theta ** (torch.arange(0, dh, 2, dtype=torch.float64) / dh))
    ang = positions.to(torch.float64)[:, None] * freqs[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def _fp8_cache(t, scale):
    """What an fp8 (E4M3) cache returns for t: the library's float8_e4m3fn
    rounding of t / scale (saturated to +-448 first: the type itself does not
    saturate), times scale."""
    c = torch.clamp(t / scale, -448.0, 448.0).to(torch.float32).to(torch.float8_e4m3fn)
    return c.to(torch.float64) * scale


def dense_prefill_logits(model, prompt_ids, prompt_hidden, next_token, K, mask_id, kv_fp8=None,
                         combine="concat"):
    """Logits [K][V] of the K sampled rows (NTP, then MASK rows) for a prompt
    of n tokens at positions 0..n-1 with target hidden rows prompt_hidden.
    kv_fp8: {"k_scale": [N], "v_scale": [N]} to read K and V as an fp8
    cache holds them. combine="sum": the drafter input is emb + fc(h) (the
    paper's architecture wording) and layer 0 is a plain pre-norm layer;
    "concat": layer 0 reads the two RMSNorm'd halves side by side."""
    m = model["dims"]
    n = len(prompt_ids)
    toks = list(prompt_ids[1:]) + [int(next_token)] + [mask_id] * (K - 1)
    hid = np.concatenate([np.asarray(prompt_hidden, np.uint16),
                          np.repeat(np.asarray(model["h_shared"], np.uint16)[None], K - 1, 0)])
    T = n + K - 1
    positions = torch.arange(T)
    x = _w(hid) @ _w(model["fc"]).T
    e = _w(model["embed"])[torch.tensor(toks)]
    eps = m.rms_eps
    if combine == "sum":
        x = torch.add(x, e)
    for l, L in enumerate(model["layers"]):
        if l == 0 and combine == "concat":
            u = torch.cat([F.rms_norm(e, (m.d,), _w(model["norm_emb"]), eps),
                           F.rms_norm(x, (m.d,), _w(model["norm_hid"]), eps)], dim=-1)
        else:
            u = F.rms_norm(x, (m.d,), _w(L["norm_in"]), eps)
        qkv = u @ _w(L["w_qkv"]).T
        q, k, v = torch.split(qkv, [m.Hq * m.dh, m.Hkv * m.dh, m.Hkv * m.dh], dim=-1)
        q = _rope_complex(q.reshape(T, m.Hq, m.dh), positions, m.rope_theta)
        k = _rope_complex(k.reshape(T, m.Hkv, m.dh), positions, m.rope_theta)
        v = v.reshape(T, m.Hkv, m.dh)
        if kv_fp8 is not None:
            k = _fp8_cache(k, float(kv_fp8["k_scale"][l]))
            v = _fp8_cache(v, float(kv_fp8["v_scale"][l]))
        G = m.Hq // m.Hkv
        k = k.repeat_interleave(G, dim=1)
        v = v.repeat_interleave(G, dim=1)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                           is_causal=True)
        x = x + o.transpose(0, 1).reshape(T, m.Hq * m.dh) @ _w(L["w_o"]).T
        y = F.rms_norm(x, (m.d,), _w(L["norm_post"]), eps)
        x = x + (F.silu(y @ _w(L["w_gate"]).T) * (y @ _w(L["w_up"]).T)) @ _w(L["w_down"]).T
    z = F.rms_norm(x[n - 1: n + K - 1], (m.d,), _w(model["norm_final"]), eps)
    return (z @ _w(model["lm_head"]).T).numpy()
