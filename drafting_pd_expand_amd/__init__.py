"""Python binding of libpdexpand.so -- the P-EAGLE parallel-drafting step on MI355X.

Argument marshalling only: every step of the drafting path runs in the HIP
library (include/pd.h). The binding checks dtypes, devices, contiguity and
sizes on the host, turns torch tensors into device pointers and calls the
C ABI with the same names: pd_expand_batch, pd_draft_forward, pd_free.
There is no CPU fallback: without the built library every call raises.

Also here: helpers that allocate the expanded-batch buffers, move a model's
bf16 weights to the device, and convert a slot-addressed KV cache to and from
the library's paged layout (setup plumbing, outside the drafting step).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_int32, c_int64, c_void_p

import numpy as np
import torch

__all__ = [
    "PD_OK", "PD_EINVAL", "PD_ENOMEM", "PD_EHIP", "PD_ESCRATCH", "PD_PAGE", "PD_MAX_LAYERS",
    "NOALLOC_SCRATCH_BYTES", "pd_draft_forward_noalloc",
    "KERNEL_LMHEAD", "KERNEL_GEMM", "KERNEL_ATTN", "KERNEL_OTHER", "KERNEL_DECODE",
    "PdError", "library_path", "load", "pd_expand_batch", "pd_draft_forward", "pd_ar_advance", "pd_free",
    "Handle", "batch_dims", "alloc_batch", "device_model", "pack_kv_cache",
    "unpack_kv_cache", "kv_cache_elems",
]

PD_OK, PD_EINVAL, PD_ENOMEM, PD_EHIP, PD_ESCRATCH = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 64 << 20
PD_PAGE = 16
PD_MAX_LAYERS = 16
KERNEL_LMHEAD, KERNEL_GEMM, KERNEL_ATTN, KERNEL_OTHER, KERNEL_DECODE = 0, 1, 2, 3, 4
STATUS_BAD_CHAIN, STATUS_BAD_BOUNDS = 32, 64
PART_MAX_K, PART_MAX_S, PART_MAX_POS = 16, 256, 1 << 19

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.path.join(_HERE, "libpdexpand.so")


class PdError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_strerror(code)} ({code})")
        self.code = code


class BatchDims(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in
                ("C", "K", "T_in", "mask_token_id", "hidden3", "block_size", "max_blocks", "num_blocks")]


class ExpandIn(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in
                ("num_tokens", "num_rejected", "target_ids", "target_pos", "target_hidden",
                 "next_token_ids", "block_table", "h_shared", "live_counts")]


_BATCH_FIELDS = ("input_ids", "positions", "slot_mapping", "is_rejected", "is_masked",
                 "hidden_state_mapping", "new_token_indices", "cu_out", "seq_lens", "hidden", "status")


class Batch(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in _BATCH_FIELDS]


_L = c_void_p * PD_MAX_LAYERS


class ForwardOpts(ctypes.Structure):
    _fields_ = [("hidden_d", c_void_p), ("hidden_out", c_void_p), ("kv_fp8", c_int32),
                ("kv_scales", POINTER(ctypes.c_float))]


class PartitionDims(ctypes.Structure):
    _fields_ = [("B", c_int32), ("K", c_int32), ("n", c_int32), ("S", c_int32)]


class Model(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("d", "Hq", "Hkv", "dh", "F", "N", "V", "hidden3")] + [
        ("rms_eps", c_float), ("rope_theta", c_float),
        ("embed", c_void_p), ("fc", c_void_p), ("norm_emb", c_void_p), ("norm_hid", c_void_p),
        ("norm_in", _L), ("w_qkv", _L), ("w_o", _L), ("norm_post", _L),
        ("w_gate", _L), ("w_up", _L), ("w_down", _L),
        ("norm_final", c_void_p), ("lm_head", c_void_p),
    ]


def load():
    """Load the built library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run `python -m drafting_pd_expand_amd.build`)")
    lib = ctypes.CDLL(path)
    lib.pd_expand_batch.argtypes = [POINTER(BatchDims), POINTER(ExpandIn), POINTER(Batch), c_void_p]
    lib.pd_expand_batch.restype = c_int
    lib.pd_draft_forward.argtypes = [POINTER(c_void_p), POINTER(Model), POINTER(BatchDims),
                                     POINTER(Batch), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.pd_draft_forward.restype = c_int
    lib.pd_draft_forward_ex.argtypes = [POINTER(c_void_p), POINTER(Model), POINTER(BatchDims),
                                        POINTER(Batch), c_void_p, c_void_p, c_void_p, c_void_p,
                                        POINTER(ForwardOpts), c_void_p]
    lib.pd_draft_forward_ex.restype = c_int
    lib.pd_draft_forward_noalloc.argtypes = [POINTER(Model), POINTER(BatchDims), POINTER(Batch), c_void_p,
                                             c_void_p, c_void_p, c_void_p, POINTER(ForwardOpts), c_void_p]
    lib.pd_draft_forward_noalloc.restype = c_int
    lib.pd_ar_advance.argtypes = [POINTER(BatchDims), POINTER(Batch), c_void_p, c_void_p, POINTER(Batch),
                                  c_void_p]
    lib.pd_ar_advance.restype = c_int
    lib.pd_verify_stub.argtypes = [POINTER(BatchDims), POINTER(Batch)] + [c_void_p] * 9
    lib.pd_verify_stub.restype = c_int
    lib.pd_seq_partition.argtypes = [POINTER(PartitionDims), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p]
    lib.pd_seq_partition.restype = c_int
    lib.pd_free.argtypes = [c_void_p]
    lib.pd_free.restype = None
    lib.pd_strerror.argtypes = [c_int]
    lib.pd_strerror.restype = ctypes.c_char_p
    lib.pd_status.argtypes = [c_void_p, POINTER(c_int32), c_void_p]
    lib.pd_status.restype = c_int
    lib.pd_set_debug_resid.argtypes = [c_void_p, c_void_p]
    lib.pd_set_debug_resid.restype = c_int
    lib.pd_set_decode_timeline.argtypes = [c_void_p, c_void_p]
    lib.pd_set_decode_timeline.restype = c_int
    lib.pd_profile.argtypes = [c_void_p, c_int]
    lib.pd_profile.restype = c_int
    lib.pd_profile_read.argtypes = [c_void_p, c_int, POINTER(c_double), POINTER(c_int64)]
    lib.pd_profile_read.restype = c_int
    _LIB = lib
    return lib


def _strerror(code: int) -> str:
    try:
        return load().pd_strerror(code).decode()
    except Exception:  # pragma: no cover
        return "error"


def _check(code: int, what: str):
    if code != PD_OK:
        raise PdError(code, what)


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _dev(t, name, dtypes, numel=None, device=None, align=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device (cuda) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: has {t.numel()} elements, needs {numel}")
    if align is None:
        align = 16 if t.dtype in _BF16 or t.dtype == torch.float32 else 4
    if t.data_ptr() % align:
        raise ValueError(f"{name}: must be {align}-byte aligned")
    return t.data_ptr()


def batch_dims(C, K, T_in, mask_token_id, hidden3, max_blocks, num_blocks, block_size=PD_PAGE) -> dict:
    return dict(C=int(C), K=int(K), T_in=int(T_in), mask_token_id=int(mask_token_id),
                hidden3=int(hidden3), block_size=int(block_size), max_blocks=int(max_blocks),
                num_blocks=int(num_blocks))


def _dims_struct(d: dict) -> BatchDims:
    return BatchDims(*[int(d[n]) for n, _ in BatchDims._fields_])


def alloc_batch(dims: dict, device) -> dict:
    """Allocate the expanded-batch buffers for `dims` (contents undefined)."""
    C, K, T_in = dims["C"], dims["K"], dims["T_in"]
    T_out = T_in + C * (K - 1)
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=device)
    u8 = lambda n: torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    return {
        "input_ids": i32(T_out), "positions": i32(T_out), "slot_mapping": i32(T_out),
        "is_rejected": u8(T_out), "is_masked": u8(T_out), "hidden_state_mapping": i32(T_in),
        "new_token_indices": i32(C * K), "cu_out": i32(C + 1), "seq_lens": i32(C),
        "hidden": torch.empty((max(T_out, 1), dims["hidden3"]), dtype=torch.bfloat16, device=device),
        "status": torch.zeros(1, dtype=torch.int32, device=device),
    }


def _batch_struct(b: dict, dims: dict, device=None, hidden_optional: bool = False) -> Batch:
    C, K, T_in = dims["C"], dims["K"], dims["T_in"]
    T_out = T_in + C * (K - 1)
    sizes = {"input_ids": T_out, "positions": T_out, "slot_mapping": T_out, "is_rejected": T_out,
             "is_masked": T_out, "hidden_state_mapping": T_in, "new_token_indices": C * K,
             "cu_out": C + 1, "seq_lens": C, "hidden": T_out * dims["hidden3"], "status": 1}
    types = {"is_rejected": (torch.uint8,), "is_masked": (torch.uint8,), "hidden": _BF16}
    aligns = {"is_rejected": 1, "is_masked": 1}
    vals = []
    for n in _BATCH_FIELDS:
        if (n == "status" or (n == "hidden" and hidden_optional)) and b.get(n) is None:
            vals.append(None)
            continue
        vals.append(_dev(b[n], n, types.get(n, (torch.int32,)), sizes[n], device, aligns.get(n)))
    return Batch(*vals)


def pd_expand_batch(dims: dict, inp: dict, out: dict, stream=None) -> None:
    """Enqueue the batch expansion (include/pd.h: pd_expand_batch). inp may
    hold "live_counts" (int32 [2] device: live C and T_in of a bucketed
    batch whose capacity dims gives)."""
    lib = load()
    C, T_in = dims["C"], dims["T_in"]
    dev = inp["num_tokens"].device if C else None
    ein = ExpandIn(
        _dev(inp["num_tokens"], "num_tokens", (torch.int32,), C, dev),
        _dev(inp["num_rejected"], "num_rejected", (torch.int32,), C, dev),
        _dev(inp["target_ids"], "target_ids", (torch.int32,), T_in, dev),
        _dev(inp["target_pos"], "target_pos", (torch.int32,), T_in, dev),
        _dev(inp["target_hidden"], "target_hidden", _BF16, T_in * dims["hidden3"], dev),
        _dev(inp["next_token_ids"], "next_token_ids", (torch.int32,), C, dev),
        _dev(inp["block_table"], "block_table", (torch.int32,), C * dims["max_blocks"], dev),
        _dev(inp["h_shared"], "h_shared", _BF16, dims["hidden3"], dev),
        _dev(inp["live_counts"], "live_counts", (torch.int32,), 2, dev) if inp.get("live_counts") is not None
        else None,
    ) if C else ExpandIn()
    bs = _batch_struct(out, dims, dev) if C else Batch()
    d = _dims_struct(dims)
    _check(lib.pd_expand_batch(ctypes.byref(d), ctypes.byref(ein), ctypes.byref(bs),
                               c_void_p(_stream_ptr(stream))), "pd_expand_batch")


class Handle:
    """Owner of a pd_handle (library scratch for pd_draft_forward)."""

    def __init__(self):
        self.ptr = c_void_p(None)

    def free(self):
        if self.ptr.value:
            load().pd_free(self.ptr)
            self.ptr = c_void_p(None)

    def __del__(self):  # pragma: no cover
        try:
            self.free()
        except Exception:
            pass

    def status(self, stream=None) -> int:
        if not self.ptr.value:
            return 0
        out = c_int32(0)
        _check(load().pd_status(self.ptr, ctypes.byref(out), c_void_p(_stream_ptr(stream))), "pd_status")
        return int(out.value)

    def set_debug_resid(self, t):
        _check(load().pd_set_debug_resid(self.ptr, c_void_p(t.data_ptr() if t is not None else None)),
               "pd_set_debug_resid")

    def set_decode_timeline(self, t):
        """Phase timestamps of the persistent decode kernel into t (int64
        [(4 + 9 N) * CUs], device) on later calls; None stops."""
        _check(load().pd_set_decode_timeline(self.ptr, c_void_p(t.data_ptr() if t is not None else None)),
               "pd_set_decode_timeline")

    def profile(self, class_mask: int):
        """Record events around launches of the kernel classes in class_mask
        (bit 1 << KERNEL_*); 0 stops. Drops earlier records."""
        _check(load().pd_profile(self.ptr, int(class_mask)), "pd_profile")

    def profile_read(self, kernel_class: int):
        ms, n = c_double(0), c_int64(0)
        _check(load().pd_profile_read(self.ptr, int(kernel_class), ctypes.byref(ms), ctypes.byref(n)),
               "pd_profile_read")
        return float(ms.value), int(n.value)


def _model_struct(m: dict) -> Model:
    dm = m["dims"]
    st = Model()
    for n in ("d", "Hq", "Hkv", "dh", "F", "N", "V"):
        setattr(st, n, int(getattr(dm, n)))
    st.hidden3 = int(dm.hidden3)
    st.rms_eps = float(dm.rms_eps)
    st.rope_theta = float(dm.rope_theta)
    P = lambda t, n: _dev(t, n, _BF16)
    st.embed = P(m["embed"], "embed")
    st.fc = P(m["fc"], "fc")
    st.norm_emb = P(m["norm_emb"], "norm_emb")
    st.norm_hid = P(m["norm_hid"], "norm_hid")
    st.norm_final = P(m["norm_final"], "norm_final")
    st.lm_head = P(m["lm_head"], "lm_head")
    for l, L in enumerate(m["layers"]):
        st.norm_in[l] = P(L["norm_in"], "norm_in")
        st.w_qkv[l] = P(L["w_qkv"], "w_qkv")
        st.w_o[l] = P(L["w_o"], "w_o")
        st.norm_post[l] = P(L["norm_post"], "norm_post")
        st.w_gate[l] = P(L["w_gate"], "w_gate")
        st.w_up[l] = P(L["w_up"], "w_up")
        st.w_down[l] = P(L["w_down"], "w_down")
    return st


def _forward_args(model: dict, dims: dict, batch: dict, block_table, kv_cache, draft_ids, logits,
                  hidden_d, hidden_out, kv_scales):
    """Checked C arguments shared by the forward entry points: (model, dims,
    batch, block table, cache, draft ids, logits) structs / pointers and the
    options struct (None when no option is set)."""
    dm = model["dims"]
    C, K = dims["C"], dims["K"]
    dev = batch["input_ids"].device
    ms = model.get("_struct")
    if ms is None:
        ms = model["_struct"] = _model_struct(model)
    T_out = dims["T_in"] + C * (K - 1)
    if hidden_d is not None:
        batch = dict(batch)
        batch.setdefault("hidden", None)
    bs = _batch_struct(batch, dims, dev, hidden_optional=hidden_d is not None)
    d = _dims_struct(dims)
    bt = _dev(block_table, "block_table", (torch.int32,), C * dims["max_blocks"], dev)
    fp8 = kv_cache.dtype == torch.uint8
    kv = _dev(kv_cache, "kv_cache", (torch.uint8,) if fp8 else _BF16, kv_cache_elems(dm, dims["num_blocks"]), dev)
    di = _dev(draft_ids, "draft_ids", (torch.int32,), C * K, dev)
    lg = _dev(logits, "logits", (torch.float32,), C * K * dm.V, dev) if logits is not None else None
    refs = (ms, d, bs)
    args = [bt, kv, di, lg]
    if hidden_d is None and hidden_out is None and not fp8:
        return refs, args, None
    scales = None
    if fp8 and kv_scales is not None:
        sc = np.ascontiguousarray(np.asarray(kv_scales, dtype=np.float32).reshape(dm.N, 2))
        scales = (ctypes.c_float * (2 * dm.N))(*sc.reshape(-1).tolist())
    opts = ForwardOpts(
        _dev(hidden_d, "hidden_d", _BF16, T_out * dm.d, dev) if hidden_d is not None else None,
        _dev(hidden_out, "hidden_out", _BF16, C * K * dm.d, dev) if hidden_out is not None else None,
        1 if fp8 else 0, scales)
    opts._scales = scales   # keep the array alive with the struct
    return refs, args, opts


def pd_draft_forward_noalloc(model: dict, dims: dict, batch: dict, block_table, kv_cache, draft_ids,
                             logits=None, stream=None, hidden_d=None, hidden_out=None, kv_scales=None) -> None:
    """Enqueue the drafter pass without a handle and without any device
    allocation (include/pd.h: pd_draft_forward_noalloc): scratch is the
    library's static per-GPU array. Same arguments and results as
    pd_draft_forward; bad device data is reported in batch["status"].
    Raises PdError(PD_ESCRATCH) when the batch needs more scratch than the
    array holds."""
    lib = load()
    if dims["C"] == 0:
        return
    (ms, d, bs), args, opts = _forward_args(model, dims, batch, block_table, kv_cache, draft_ids, logits,
                                            hidden_d, hidden_out, kv_scales)
    _check(lib.pd_draft_forward_noalloc(ctypes.byref(ms), ctypes.byref(d), ctypes.byref(bs),
                                        *[c_void_p(a) for a in args],
                                        ctypes.byref(opts) if opts is not None else None,
                                        c_void_p(_stream_ptr(stream))), "pd_draft_forward_noalloc")


def pd_draft_forward(handle: Handle, model: dict, dims: dict, batch: dict, block_table, kv_cache,
                     draft_ids, logits=None, stream=None, hidden_d=None, hidden_out=None,
                     kv_scales=None) -> None:
    """Enqueue the drafter pass (include/pd.h: pd_draft_forward, or
    pd_draft_forward_ex when hidden_d / hidden_out are given or the cache is
    fp8). `model` is a dict made by device_model(); `batch` holds the
    expanded-batch tensors. kv_cache: bf16 (see pack_kv_cache) or uint8 E4M3
    codes (an fp8 cache; kv_scales then gives the [N][2] per-layer K and V
    scales, default 1.0).
    hidden_d: bf16 [T_out][d] projected hidden rows (fc skipped);
    hidden_out: bf16 [C*K][d] receives the sampled rows' final residual."""
    lib = load()
    if dims["C"] == 0:
        return
    (ms, d, bs), args, opts = _forward_args(model, dims, batch, block_table, kv_cache, draft_ids, logits,
                                            hidden_d, hidden_out, kv_scales)
    head = (ctypes.byref(handle.ptr), ctypes.byref(ms), ctypes.byref(d), ctypes.byref(bs),
            *[c_void_p(a) for a in args])
    if opts is None:
        _check(lib.pd_draft_forward(*head, c_void_p(_stream_ptr(stream))), "pd_draft_forward")
        return
    _check(lib.pd_draft_forward_ex(*head, ctypes.byref(opts), c_void_p(_stream_ptr(stream))),
           "pd_draft_forward_ex")


def pd_ar_advance(dims_prev: dict, prev: dict, draft_ids, block_table, nxt: dict, stream=None) -> None:
    """Enqueue the next autoregressive pass's batch (include/pd.h: pd_ar_advance).
    `nxt` is a batch allocated for {C, K = 1, T_in = C}; its hidden rows are
    not written."""
    lib = load()
    C, K = dims_prev["C"], dims_prev["K"]
    if C == 0:
        return
    dev = prev["input_ids"].device
    pb = _batch_struct(prev, dims_prev, dev, hidden_optional=True)
    nd = dict(dims_prev, K=1, T_in=C)
    nb = _batch_struct(dict(nxt, hidden=None), nd, dev, hidden_optional=True)
    d = _dims_struct(dims_prev)
    di = _dev(draft_ids, "draft_ids", (torch.int32,), C * K, dev)
    bt = _dev(block_table, "block_table", (torch.int32,), C * dims_prev["max_blocks"], dev)
    _check(lib.pd_ar_advance(ctypes.byref(d), ctypes.byref(pb), c_void_p(di), c_void_p(bt), ctypes.byref(nb),
                             c_void_p(_stream_ptr(stream))), "pd_ar_advance")


def pd_verify_stub(dims_prev: dict, prev: dict, prev_draft_ids, prev_next_token_ids, accepted, nxt: dict,
                   status=None, stream=None) -> None:
    """Enqueue the stand-in verifier (include/pd.h: pd_verify_stub). `nxt`
    holds the next round's num_tokens, num_rejected [C] and target_ids,
    target_pos [C*(K+1)] (int32, written)."""
    lib = load()
    C, K = dims_prev["C"], dims_prev["K"]
    if C == 0:
        return
    dev = prev["positions"].device
    pb = _batch_struct(prev, dims_prev, dev, hidden_optional=True)
    d = _dims_struct(dims_prev)
    I = (torch.int32,)
    args = (_dev(prev_draft_ids, "prev_draft_ids", I, C * K, dev),
            _dev(prev_next_token_ids, "prev_next_token_ids", I, C, dev),
            _dev(accepted, "accepted", I, C, dev),
            _dev(nxt["num_tokens"], "num_tokens", I, C, dev),
            _dev(nxt["num_rejected"], "num_rejected", I, C, dev),
            _dev(nxt["target_ids"], "target_ids", I, C * (K + 1), dev),
            _dev(nxt["target_pos"], "target_pos", I, C * (K + 1), dev),
            _dev(status, "status", I, 1, dev) if status is not None else None)
    _check(lib.pd_verify_stub(ctypes.byref(d), ctypes.byref(pb), *[c_void_p(x) for x in args],
                              c_void_p(_stream_ptr(stream))), "pd_verify_stub")


def pd_seq_partition(keep, boundaries, seg, seg_offsets, rows, status=None, stream=None) -> None:
    """Enqueue the sequence partitioning (include/pd.h: pd_seq_partition).
    keep: uint8 [B][K][n]; boundaries: int32 [B][S+1]; seg: int32 [B][K][n] out;
    seg_offsets: int32 [B][S+1] out; rows: int32 [B][K*n] out; status: int32 [1] or None."""
    lib = load()
    if keep.dim() != 3 or boundaries.dim() != 2:
        raise ValueError("keep must be [B][K][n] and boundaries [B][S+1]")
    B, K, n = (int(x) for x in keep.shape)
    S = int(boundaries.shape[1]) - 1
    if boundaries.shape[0] != B:
        raise ValueError("boundaries must have one row per sequence")
    dims = PartitionDims(B, K, n, S)
    if B == 0:
        _check(lib.pd_seq_partition(ctypes.byref(dims), None, None, None, None, None, None,
                                    c_void_p(_stream_ptr(stream))), "pd_seq_partition")
        return
    dev = keep.device
    args = (_dev(keep, "keep", (torch.uint8,), B * K * n, dev, 8),
            _dev(boundaries, "boundaries", (torch.int32,), B * (S + 1), dev),
            _dev(seg, "seg", (torch.int32,), B * K * n, dev, 16),
            _dev(seg_offsets, "seg_offsets", (torch.int32,), B * (S + 1), dev),
            _dev(rows, "rows", (torch.int32,), B * K * n, dev),
            _dev(status, "status", (torch.int32,), 1, dev) if status is not None else None)
    _check(lib.pd_seq_partition(ctypes.byref(dims), *[c_void_p(a) for a in args],
                                c_void_p(_stream_ptr(stream))), "pd_seq_partition")


def pd_free(handle: Handle) -> None:
    handle.free()


# ----------------------------------------------------------------------------- setup plumbing

def _to_dev_bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(device).view(
        torch.bfloat16)


def device_model(model_np: dict, device) -> dict:
    """Upload bf16-bit numpy weights (synth.make_model layout) to the device."""
    up = lambda a: _to_dev_bf16(a, device)
    out = {"dims": model_np["dims"], "layers": []}
    for k in ("embed", "fc", "norm_emb", "norm_hid", "norm_final", "lm_head", "h_shared"):
        out[k] = up(model_np[k])
    for L in model_np["layers"]:
        out["layers"].append({k: up(v) for k, v in L.items()})
    return out


def kv_cache_elems(dm, num_blocks: int) -> int:
    return dm.N * 2 * num_blocks * dm.Hkv * PD_PAGE * dm.dh


def pack_kv_cache(k_slots: torch.Tensor, v_slots: torch.Tensor) -> torch.Tensor:
    """Slot-addressed K/V [N][num_blocks*16][Hkv][dh] -> the library's paged
    cache [N][2][num_blocks][Hkv][16*dh] (K pages token-major, V pages
    dim-major)."""
    N, S, Hkv, dh = k_slots.shape
    nb = S // PD_PAGE
    kp = k_slots.reshape(N, nb, PD_PAGE, Hkv, dh).permute(0, 1, 3, 2, 4).reshape(N, nb, Hkv, PD_PAGE * dh)
    vp = v_slots.reshape(N, nb, PD_PAGE, Hkv, dh).permute(0, 1, 3, 4, 2).reshape(N, nb, Hkv, PD_PAGE * dh)
    return torch.stack([kp, vp], dim=1).contiguous()


def pack_kv_cache_fp8(k_codes: torch.Tensor, v_codes: torch.Tensor) -> torch.Tensor:
    """Like pack_kv_cache for uint8 E4M3 codes (an fp8 cache)."""
    return pack_kv_cache(k_codes, v_codes)


def unpack_kv_cache(cache: torch.Tensor, Hkv: int, dh: int):
    """Inverse of pack_kv_cache: returns (k_slots, v_slots)."""
    N, _, nb = cache.shape[:3]
    kp = cache[:, 0].reshape(N, nb, Hkv, PD_PAGE, dh).permute(0, 1, 3, 2, 4).reshape(N, nb * PD_PAGE, Hkv, dh)
    vp = cache[:, 1].reshape(N, nb, Hkv, dh, PD_PAGE).permute(0, 1, 4, 2, 3).reshape(N, nb * PD_PAGE, Hkv, dh)
    return kp, vp
