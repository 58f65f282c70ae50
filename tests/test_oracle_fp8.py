"""Pins for the oracle's E4M3 codec (CPU only), against the library's
float8_e4m3fn type (torch) and the format's closed forms."""
import numpy as np
import torch

from oracle.fp8 import E4M3_MAX, e4m3_decode, e4m3_encode, fp8_roundtrip


def _torch_values(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().double().numpy()


def test_decode_every_code_matches_library():
    codes = np.arange(256, dtype=np.uint8)
    got, want = e4m3_decode(codes), _torch_values(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])


def test_closed_forms():
    assert e4m3_decode([0x7E])[0] == 448.0 == E4M3_MAX
    assert e4m3_decode([0x01])[0] == 2.0 ** -9          # smallest subnormal
    assert e4m3_decode([0x08])[0] == 2.0 ** -6          # smallest normal
    assert e4m3_decode([0x38])[0] == 1.0
    assert np.isnan(e4m3_decode([0x7F])[0]) and np.isnan(e4m3_decode([0xFF])[0])
    # saturation and ties to even
    assert list(e4m3_encode([1e9, -1e9, 464.0, 449.0])) == [0x7E, 0xFE, 0x7E, 0x7E]
    assert list(e4m3_encode([1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -10])) == [0x38, 0x3A, 0x00, 0x01]


def test_encode_matches_library_rounding():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-12, 10, 200000))
    pos = np.unique(_torch_values(np.arange(0x7F, dtype=np.uint8)))
    mids = (pos[1:] + pos[:-1]) / 2                     # every exact tie between neighbouring codes
    x = np.concatenate([x, mids, -mids, [0.0, -0.0, 2.0 ** -6, 0.9375 * 2.0 ** -6]])
    xc = np.clip(x, -E4M3_MAX, E4M3_MAX).astype(np.float32)   # the library type does not saturate
    want = torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3_encode(xc.astype(np.float64))
    assert np.array_equal(got, want)


def test_roundtrip_error_bound_and_scale():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(50000) * 3
    for s in (1.0, 0.25, 0.3):
        r = fp8_roundtrip(x, s)
        big = np.abs(x / s) >= 2.0 ** -6
        # normal range: within half a step (2^-4 relative); subnormal: within 2^-10 absolute (times s)
        assert np.all(np.abs(r - x)[big] <= 2.0 ** -4 * np.abs(x[big]) * (1 + 1e-12))
        assert np.all(np.abs(r - x)[~big] <= 2.0 ** -10 * s * (1 + 1e-12))


# ---- the forward with an fp8 cache -------------------------------------------

import pytest  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402
from dense_ref import dense_prefill_logits  # noqa: E402
from test_oracle_forward import MINI, _prefill_case, _rel  # noqa: E402


def _fp8_pool(dims, nb, bs, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((2, dims.N, nb * bs, dims.Hkv, dims.dh))
    c = torch.from_numpy(np.clip(x, -448, 448)).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return {"k": c[0], "v": c[1]}


@pytest.mark.parametrize("scales", [((1.0, 1.0), (1.0, 1.0)), ((0.5, 0.125), (0.25, 2.0)), ((0.3, 0.7), (1.3, 0.05))])
def test_fp8_prefill_matches_dense_library_forward(scales):
    """Prefill from an empty fp8 cache: the oracle's K/V rounding (its own
    E4M3 encoder) against the library type's, inside a dense causal forward."""
    dims, n, K, bs = MINI, 19, 4, 4
    model, ids, hidden, nxt = _prefill_case(dims, n, K, seed=13)
    kv8 = {"k_scale": np.asarray(scales[0]), "v_scale": np.asarray(scales[1])}
    pages = -(-(n + K) // bs)
    nb = pages + 2
    bt = np.random.default_rng(3).permutation(nb)[:pages][None]
    pool = _fp8_pool(dims, nb, bs, 4)
    exp = oracle.expand([n], [0], ids, np.arange(n), hidden, [nxt], bt, model["h_shared"], K, dims.V - 1, bs)
    got = oracle.draft_forward(model, exp, bt, pool, K, block_size=bs, kv_fp8=kv8)["logits"]
    want = dense_prefill_logits(model, ids, hidden, nxt, K, dims.V - 1, kv_fp8=kv8)
    assert _rel(got, want) < 1e-10
    plain = dense_prefill_logits(model, ids, hidden, nxt, K, dims.V - 1)
    assert _rel(plain, want) > 1e-4     # the rounding is really applied


def test_fp8_decode_over_written_codes_matches_dense():
    """A prefix prefill writes K/V into an fp8 cache (stored as codes); a
    decode step with rejections reads them back: equal to a dense prefill of
    the accepted tokens with the same fp8 rounding."""
    dims, bs, L, n, v, K = MINI, 4, 11, 5, 3, 4
    kv8 = {"k_scale": np.asarray([0.5, 0.25]), "v_scale": np.asarray([2.0, 0.125])}   # powers of two
    model = synth.make_model(dims, seed=23)
    rng = np.random.default_rng(24)
    P = L + n
    ids = rng.integers(0, dims.V - 1, size=P)
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((P, dims.hidden3)).astype(np.float32))
    nxt = int(rng.integers(0, dims.V - 1))
    pages = -(-(L + n + K) // bs)
    nb = pages + 3
    bt = rng.permutation(nb)[:pages][None]
    pool = _fp8_pool(dims, nb, bs, 25)
    e1 = oracle.expand([L], [0], ids[:L], np.arange(L), hidden[:L], [int(ids[L])], bt, model["h_shared"],
                       K, dims.V - 1, bs)
    f1 = oracle.draft_forward(model, e1, bt, pool, K, block_size=bs, kv_fp8=kv8)
    for l, (sl, k, vv) in enumerate(f1["kv_written"]):
        pool["k"][l][sl] = oracle.fp8.e4m3_encode(k / kv8["k_scale"][l])
        pool["v"][l][sl] = oracle.fp8.e4m3_encode(vv / kv8["v_scale"][l])
    e2 = oracle.expand([n], [n - v], ids[L:P], np.arange(L, P), hidden[L:P], [nxt], bt, model["h_shared"],
                       K, dims.V - 1, bs)
    got = oracle.draft_forward(model, e2, bt, pool, K, block_size=bs, kv_fp8=kv8)["logits"]
    want = dense_prefill_logits(model, ids[:L + v], hidden[:L + v], nxt, K, dims.V - 1, kv_fp8=kv8)
    assert _rel(got, want) < 1e-10
