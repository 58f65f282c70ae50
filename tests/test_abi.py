"""The C-ABI library loads, exports every symbol include/pd.h declares, and
rejects bad host arguments before touching a GPU (CPU only: no compute call
is made here)."""
import ctypes
import os
import re

import pytest
import torch

import drafting_pd_expand_amd as pdx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pdx.library_path()):
        from drafting_pd_expand_amd import build
        build.build()
    return pdx.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pd_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"pd_expand_batch", "pd_draft_forward", "pd_free"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pd.h but not exported"


def test_library_is_gfx950_build(lib):
    data = open(pdx.library_path(), "rb").read()
    assert b"gfx950" in data


def test_strerror(lib):
    assert lib.pd_strerror(0) == b"ok"
    assert lib.pd_strerror(-1) == b"invalid argument"
    assert lib.pd_strerror(-2) == b"device allocation failed"
    assert lib.pd_strerror(-3) == b"HIP launch error"


def _dims(**kw):
    d = dict(C=2, K=3, T_in=5, mask_token_id=99, hidden3=24, block_size=16, max_blocks=4, num_blocks=8)
    d.update(kw)
    return pdx.BatchDims(*[d[n] for n, _ in pdx.BatchDims._fields_])


FAKE = 0x1000  # never dereferenced: every call below fails (or returns) on host checks


def _fake_in():
    return pdx.ExpandIn(*([FAKE] * 8))


def _fake_batch():
    return pdx.Batch(*([FAKE] * 10 + [None]))


@pytest.mark.parametrize("kw", [dict(C=-1), dict(C=1025), dict(K=0), dict(K=17), dict(T_in=1, C=2),
                                dict(hidden3=12), dict(hidden3=0), dict(block_size=0),
                                dict(max_blocks=0), dict(num_blocks=0)])
def test_expand_rejects_bad_dims(lib, kw):
    d, i, b = _dims(**kw), _fake_in(), _fake_batch()
    assert lib.pd_expand_batch(ctypes.byref(d), ctypes.byref(i), ctypes.byref(b), None) == pdx.PD_EINVAL


def test_expand_rejects_null_and_misaligned(lib):
    d, i, b = _dims(), _fake_in(), _fake_batch()
    assert lib.pd_expand_batch(None, ctypes.byref(i), ctypes.byref(b), None) == pdx.PD_EINVAL
    assert lib.pd_expand_batch(ctypes.byref(d), None, ctypes.byref(b), None) == pdx.PD_EINVAL
    for f in [n for n, _ in pdx.ExpandIn._fields_ if n != "live_counts"]:   # live counts are optional
        i2 = _fake_in()
        setattr(i2, f, None)
        assert lib.pd_expand_batch(ctypes.byref(d), ctypes.byref(i2), ctypes.byref(b), None) == pdx.PD_EINVAL, f
    for f in [n for n, _ in pdx.Batch._fields_ if n != "status"]:
        b2 = _fake_batch()
        setattr(b2, f, None)
        assert lib.pd_expand_batch(ctypes.byref(d), ctypes.byref(i), ctypes.byref(b2), None) == pdx.PD_EINVAL, f
    i3 = _fake_in()
    i3.target_hidden = FAKE + 8
    assert lib.pd_expand_batch(ctypes.byref(d), ctypes.byref(i3), ctypes.byref(b), None) == pdx.PD_EINVAL


def test_expand_C0_is_noop(lib):
    d = _dims(C=0, T_in=0)
    assert lib.pd_expand_batch(ctypes.byref(d), ctypes.byref(_fake_in()), ctypes.byref(_fake_batch()), None) == 0


def _model(**kw):
    m = pdx.Model()
    vals = dict(d=256, Hq=4, Hkv=4, dh=64, F=688, N=4, V=4096, hidden3=768)
    vals.update(kw)
    for k, v in vals.items():
        setattr(m, k, v)
    m.rms_eps, m.rope_theta = 1e-5, 1e4
    for f in ("embed", "fc", "norm_emb", "norm_hid", "norm_final", "lm_head"):
        setattr(m, f, FAKE)
    for l in range(16):
        for f in ("norm_in", "w_qkv", "w_o", "norm_post", "w_gate", "w_up", "w_down"):
            getattr(m, f)[l] = FAKE
    return m


@pytest.mark.parametrize("kw", [dict(dh=96), dict(Hq=6, Hkv=4), dict(d=250, hidden3=750), dict(hidden3=700),
                                dict(N=0), dict(N=17), dict(V=4095), dict(F=690),
                                dict(d=4112, hidden3=12336)])
def test_forward_rejects_bad_model(lib, kw):
    h = ctypes.c_void_p(None)
    m, d, b = _model(**kw), _dims(hidden3=kw.get("hidden3", 768)), _fake_batch()
    rc = lib.pd_draft_forward(ctypes.byref(h), ctypes.byref(m), ctypes.byref(d), ctypes.byref(b),
                              FAKE, FAKE, FAKE, None, None)
    assert rc == pdx.PD_EINVAL and h.value is None


def test_forward_rejects_bad_call(lib):
    h = ctypes.c_void_p(None)
    m, b = _model(), _fake_batch()
    args = lambda d, bt=FAKE, kv=FAKE, di=FAKE: (ctypes.byref(h), ctypes.byref(m), ctypes.byref(d),
                                                 ctypes.byref(b), bt, kv, di, None, None)
    assert lib.pd_draft_forward(None, ctypes.byref(m), ctypes.byref(_dims(hidden3=768)), ctypes.byref(b),
                                FAKE, FAKE, FAKE, None, None) == pdx.PD_EINVAL
    assert lib.pd_draft_forward(*args(_dims(hidden3=768, block_size=8))) == pdx.PD_EINVAL
    assert lib.pd_draft_forward(*args(_dims(hidden3=24))) == pdx.PD_EINVAL  # hidden3 != 3d
    assert lib.pd_draft_forward(*args(_dims(hidden3=768), bt=None)) == pdx.PD_EINVAL
    assert lib.pd_draft_forward(*args(_dims(hidden3=768), kv=None)) == pdx.PD_EINVAL
    assert lib.pd_draft_forward(*args(_dims(hidden3=768), di=None)) == pdx.PD_EINVAL
    m.w_up[2] = None
    assert lib.pd_draft_forward(*args(_dims(hidden3=768))) == pdx.PD_EINVAL
    assert h.value is None
    m.w_up[2] = FAKE
    assert lib.pd_draft_forward(*args(_dims(C=0, T_in=0, hidden3=768))) == 0 and h.value is None


def test_handle_calls_reject_null(lib):
    lib.pd_free(None)
    out = ctypes.c_int32(0)
    assert lib.pd_status(None, ctypes.byref(out), None) == pdx.PD_EINVAL
    assert lib.pd_profile(None, 1) == pdx.PD_EINVAL
    ms, n = ctypes.c_double(0), ctypes.c_int64(0)
    assert lib.pd_profile_read(None, 0, ctypes.byref(ms), ctypes.byref(n)) == pdx.PD_EINVAL
    assert lib.pd_set_debug_resid(None, None) == pdx.PD_EINVAL


def test_binding_rejects_host_tensors(lib):
    dims = pdx.batch_dims(1, 2, 3, 9, 16, 2, 4)
    t = torch.zeros(4, dtype=torch.int32)
    inp = {k: t for k in ("num_tokens", "num_rejected", "target_ids", "target_pos", "next_token_ids",
                          "block_table")}
    inp["target_hidden"] = torch.zeros(64, dtype=torch.bfloat16)
    inp["h_shared"] = torch.zeros(16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pdx.pd_expand_batch(dims, inp, {})


def test_forward_ex_and_ar_advance_reject_bad_calls(lib):
    h = ctypes.c_void_p(None)
    m, b = _model(), _fake_batch()
    d = _dims(hidden3=768)
    opts = pdx.ForwardOpts(FAKE + 8, None)   # misaligned hidden_d
    assert lib.pd_draft_forward_ex(ctypes.byref(h), ctypes.byref(m), ctypes.byref(d), ctypes.byref(b),
                                   FAKE, FAKE, FAKE, None, ctypes.byref(opts), None) == pdx.PD_EINVAL
    b2 = _fake_batch()
    b2.hidden = None                          # no 3d rows: only allowed with hidden_d
    assert lib.pd_draft_forward_ex(ctypes.byref(h), ctypes.byref(m), ctypes.byref(d), ctypes.byref(b2),
                                   FAKE, FAKE, FAKE, None, None, None) == pdx.PD_EINVAL
    assert h.value is None
    assert lib.pd_ar_advance(ctypes.byref(d), ctypes.byref(b), None, FAKE, ctypes.byref(b), None) == pdx.PD_EINVAL
    assert lib.pd_ar_advance(ctypes.byref(d), None, FAKE, FAKE, ctypes.byref(b), None) == pdx.PD_EINVAL
    b3 = _fake_batch()
    b3.seq_lens = None
    assert lib.pd_ar_advance(ctypes.byref(d), ctypes.byref(b), FAKE, FAKE, ctypes.byref(b3), None) == pdx.PD_EINVAL
    assert lib.pd_ar_advance(ctypes.byref(_dims(C=0, T_in=0)), ctypes.byref(b), FAKE, FAKE,
                             ctypes.byref(b), None) == 0


def test_seq_partition_rejects_bad_calls(lib):
    P = pdx.PartitionDims

    def call(d, keep=FAKE, bnd=FAKE, seg=FAKE, off=FAKE, rows=FAKE, st=None):
        return lib.pd_seq_partition(ctypes.byref(d) if d is not None else None, keep, bnd, seg, off, rows, st, None)

    assert call(None) == pdx.PD_EINVAL
    for bad in (P(1, 0, 64, 2), P(1, 17, 64, 2), P(1, 4, 60, 2), P(1, 4, 0, 2), P(1, 4, 64, 0),
                P(1, 4, 64, 257), P(1, 16, 1 << 16, 2), P(-1, 4, 64, 2)):
        assert call(bad) == pdx.PD_EINVAL, (bad.B, bad.K, bad.n, bad.S)
    ok = P(1, 4, 64, 2)
    assert call(ok, keep=None) == pdx.PD_EINVAL
    assert call(ok, rows=None) == pdx.PD_EINVAL
    assert call(ok, keep=FAKE + 4) == pdx.PD_EINVAL     # keep must be 8-byte aligned
    assert call(ok, seg=FAKE + 8) == pdx.PD_EINVAL      # seg must be 16-byte aligned
    assert call(P(0, 4, 64, 2), keep=None, bnd=None, seg=None, off=None, rows=None) == pdx.PD_OK


def test_verify_stub_rejects_bad_calls(lib):
    d = _dims()
    b = pdx.Batch(*([FAKE] * len(pdx.Batch._fields_)))
    args = [FAKE] * 9
    assert lib.pd_verify_stub(None, ctypes.byref(b), *args, None) == pdx.PD_EINVAL
    assert lib.pd_verify_stub(ctypes.byref(d), None, *args, None) == pdx.PD_EINVAL
    for i in range(7):       # every pointer but status (the 8th) is required
        a = list(args)
        a[i] = None
        assert lib.pd_verify_stub(ctypes.byref(d), ctypes.byref(b), *a, None) == pdx.PD_EINVAL, i
    assert lib.pd_verify_stub(ctypes.byref(_dims(K=0)), ctypes.byref(b), *args, None) == pdx.PD_EINVAL
    assert lib.pd_verify_stub(ctypes.byref(_dims(C=0)), ctypes.byref(b), *args, None) == pdx.PD_OK


def test_forward_noalloc_rejects_bad_calls_and_oversize(lib):
    """The allocation-free forward checks its host arguments like
    pd_draft_forward_ex and refuses, before touching a device, a batch whose
    workspace exceeds the static scratch (PD_ESCRATCH)."""
    m, b = _model(), _fake_batch()
    d = _dims(hidden3=768)
    f = lib.pd_draft_forward_noalloc
    assert f(None, ctypes.byref(d), ctypes.byref(b), FAKE, FAKE, FAKE, None, None, None) == pdx.PD_EINVAL
    assert f(ctypes.byref(m), ctypes.byref(_dims(hidden3=768, K=0)), ctypes.byref(b), FAKE, FAKE, FAKE,
             None, None, None) == pdx.PD_EINVAL
    assert f(ctypes.byref(m), ctypes.byref(d), ctypes.byref(b), None, FAKE, FAKE, None, None, None) == pdx.PD_EINVAL
    assert f(ctypes.byref(m), ctypes.byref(_dims(C=0, T_in=0, hidden3=768)), ctypes.byref(b), FAKE, FAKE, FAKE,
             None, None, None) == pdx.PD_OK
    # the GPT-OSS-20B-scale drafter at 64 requests x K = 7 (896 expanded rows):
    # its split-K planes alone need more than the static array
    big = _model(d=2880, hidden3=8640, Hq=64, Hkv=8, dh=64, F=7680, N=4, V=201088)
    dbig = _dims(C=64, K=7, T_in=512, hidden3=8640, max_blocks=1280, num_blocks=90000)
    assert f(ctypes.byref(big), ctypes.byref(dbig), ctypes.byref(b), FAKE, FAKE, FAKE, None, None,
             None) == pdx.PD_ESCRATCH
    assert lib.pd_strerror(pdx.PD_ESCRATCH).startswith(b"workspace exceeds")
