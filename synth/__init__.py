"""Seeded synthetic inputs for the P-EAGLE parallel drafting step.

This module is shared by the oracle-side tests and the GPU-side callers. It
holds only workload shapes and random draws: no step of the drafting method is
computed here. Every floating-point tensor is drawn in fp32 and rounded once,
to nearest-even, to bf16 (returned as uint16 bit patterns), so both sides read
the very same bf16 values.

Pages cited:
  [Paper]  "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training" (summary page)
  [Blog]   "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding in
           vLLM" (summary page of the vLLM blog post)
  [arXiv]  ScienceStack page for arXiv 2602.01469 (same paper as [Paper])

Recipe (stand-ins for the pages' datasets, which are not available here):
  * matrices and embedding rows ~ N(0, 0.02); RMSNorm gains 1 + N(0, 0.1);
    h_shared and target hidden rows ~ N(0, 1); prior-context K/V ~ N(0, 1).
  * token ids and sampled tokens uniform in [0, V-1); the MASK id is V-1.
  * context lengths either fixed or lognormal with the median (3,891) and P90
    (10,800) of the length distribution in [arXiv] Figure 1 / [Blog] "training
    on long sequences", clipped to [128, 20000] (20,000 is that figure's P99).
  * decode steps carry n_r = K+1 verify tokens with an accepted-draft count
    a_r ~ U{0..K}, so n_r - (a_r + 1) of them are rejected.
  * KV pages (16 tokens) are handed out as a random permutation of the pool,
    so one request's pages are scattered; a few spare pages are never used.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "ModelDims", "Workload", "WORKLOADS", "MODELS", "get_workload",
    "make_model", "make_batch", "make_kv_pool", "kv_fp8_scales", "make_cod_keep", "make_rounds",
    "f32_to_bf16_bits",
]

_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


@dataclass(frozen=True)
class ModelDims:
    """Drafter shape: d model width, hidden3 = 3d target-feature width."""
    name: str
    d: int
    Hq: int
    Hkv: int
    dh: int
    F: int
    N: int
    V: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def hidden3(self) -> int:
        return 3 * self.d

    @property
    def qkv_out(self) -> int:
        return (self.Hq + 2 * self.Hkv) * self.dh

    def qkv_in(self, layer: int) -> int:
        return 2 * self.d if layer == 0 else self.d


@dataclass(frozen=True)
class Workload:
    """One draft step's batch: C requests, depth K, context recipe."""
    name: str
    model: ModelDims
    C: int
    K: int
    context: str          # "fixed" or "lognormal"
    L: int = 0            # fixed context length (tokens already cached)
    n_verify: int = 0     # verify tokens per request; 0 means K+1
    accept: str = "uniform"  # "uniform" (a_r ~ U{0..K}) or "all" (no rejection)
    seed: int = 0
    spare_pages: int = 8

    @property
    def n(self) -> int:
        return self.n_verify if self.n_verify else self.K + 1


MODELS = {
    "tiny": ModelDims("tiny", d=256, Hq=4, Hkv=4, dh=64, F=688, N=4, V=4096),
    "gptoss20b": ModelDims("gptoss20b", d=2880, Hq=64, Hkv=8, dh=64, F=7680, N=4, V=201088),
    "qwen3coder30b": ModelDims("qwen3coder30b", d=2048, Hq=32, Hkv=4, dh=128, F=6144, N=4, V=151936),
}

WORKLOADS = {
    # prefill of a 128-token prompt (nothing cached yet), K=4
    "tiny": Workload("tiny", MODELS["tiny"], C=1, K=4, context="fixed", L=0,
                     n_verify=128, accept="all", seed=0),
    "g_c1": Workload("g_c1", MODELS["gptoss20b"], C=1, K=7, context="fixed", L=4096, seed=1),
    "g_c4": Workload("g_c4", MODELS["gptoss20b"], C=4, K=7, context="lognormal", seed=2),
    "g_c64_k3": Workload("g_c64_k3", MODELS["gptoss20b"], C=64, K=3, context="lognormal", seed=3),
    "g_c64_k5": Workload("g_c64_k5", MODELS["gptoss20b"], C=64, K=5, context="lognormal", seed=3),
    "g_c64": Workload("g_c64", MODELS["gptoss20b"], C=64, K=7, context="lognormal", seed=3),
    "q_c16": Workload("q_c16", MODELS["qwen3coder30b"], C=16, K=7, context="fixed", L=20000, seed=4),
}


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


# ----------------------------------------------------------------------------
# parallel, thread-count-independent draws

def _fill(shape, seed: int, tag: int, kind: str, scale: float = 1.0, shift: float = 0.0) -> np.ndarray:
    """bf16 bits of `shift + scale * N(0,1)` (kind='normal'), chunked so that
    the values depend only on (seed, tag, chunk) and not on the thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nch = max(1, (n + _CHUNK - 1) // _CHUNK)

    def work(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tag, c)))
        if kind != "normal":
            raise ValueError(kind)
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        if shift != 0.0:
            v += np.float32(shift)
        out[lo:hi] = f32_to_bf16_bits(v)

    if nch == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nch)))
    return out.reshape(shape)


def make_model(m: ModelDims, seed: int = 1234) -> dict:
    """Random-init drafter weights, all bf16 bits, row-major [out][in].

    h_shared (the learned MTP hidden state, [Paper] sec. 2 architecture,
    [Blog] "hidden state management") is 3d wide and part of the model.
    """
    tag = iter(range(1000))
    W = lambda shape: _fill(shape, seed, next(tag), "normal", 0.02)
    G = lambda n: _fill((n,), seed, next(tag), "normal", 0.1, 1.0)
    model = {
        "dims": m,
        "embed": W((m.V, m.d)),
        "fc": W((m.d, m.hidden3)),
        "norm_emb": G(m.d),
        "norm_hid": G(m.d),
        "layers": [],
    }
    for l in range(m.N):
        model["layers"].append({
            "norm_in": G(m.d),      # unused at layer 0 (the two input norms replace it)
            "w_qkv": W((m.qkv_out, m.qkv_in(l))),
            "w_o": W((m.d, m.Hq * m.dh)),
            "norm_post": G(m.d),
            "w_gate": W((m.F, m.d)),
            "w_up": W((m.F, m.d)),
            "w_down": W((m.d, m.F)),
        })
    model["norm_final"] = G(m.d)
    model["lm_head"] = W((m.V, m.d))
    model["h_shared"] = _fill((m.hidden3,), seed, next(tag), "normal", 1.0)
    return model


def _context_lengths(w: Workload, rng) -> np.ndarray:
    if w.context == "fixed":
        return np.full(w.C, w.L, dtype=np.int64)
    if w.context == "lognormal":
        sigma = math.log(10800.0 / 3891.0) / 1.2815515655446004
        L = np.exp(rng.normal(math.log(3891.0), sigma, size=w.C))
        return np.clip(np.rint(L), 128, 20000).astype(np.int64)
    raise ValueError(w.context)


def make_batch(w: Workload, seed: int | None = None, block_size: int = 16, extra_positions: int = 0) -> dict:
    """The verify-batch side of one draft step (all integer data + target rows).

    Returns int32 numpy arrays in the layout the expansion consumes, the
    target hidden rows as bf16 bits, and the page pool description.
    extra_positions: block-table room for that many more positions per
    request (later rounds of a multi-round run).
    """
    seed = w.seed if seed is None else seed
    m = w.model
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(7,)))
    L = _context_lengths(w, rng)
    n = np.full(w.C, w.n, dtype=np.int64)
    if w.accept == "uniform":
        a = rng.integers(0, w.K + 1, size=w.C)            # accepted drafts 0..K
        v = np.minimum(a + 1, n)
    elif w.accept == "all":
        v = n.copy()
    else:
        raise ValueError(w.accept)
    rho = n - v
    T_in = int(n.sum())
    target_ids = rng.integers(0, m.V - 1, size=T_in)
    next_ids = rng.integers(0, m.V - 1, size=w.C)
    target_pos = np.concatenate([np.arange(L[r], L[r] + n[r]) for r in range(w.C)]) if w.C else np.zeros(0, np.int64)
    # pages: enough for every position this step can touch
    pages = [int(-(-(L[r] + n[r] + w.K + extra_positions) // block_size)) for r in range(w.C)]
    num_blocks = int(sum(pages)) + w.spare_pages
    max_blocks = max(pages) if pages else 1
    perm = rng.permutation(num_blocks)
    block_table = np.full((w.C, max_blocks), -1, dtype=np.int64)
    used = 0
    for r in range(w.C):
        block_table[r, : pages[r]] = perm[used: used + pages[r]]
        used += pages[r]
    hidden = _fill((T_in, m.hidden3), seed, 11, "normal", 1.0)
    i32 = lambda x: np.ascontiguousarray(x, dtype=np.int32)
    return {
        "C": w.C, "K": w.K, "T_in": T_in, "mask_id": m.V - 1,
        "block_size": block_size, "max_blocks": max_blocks, "num_blocks": num_blocks,
        "context_lens": i32(L),
        "num_tokens": i32(n), "num_rejected": i32(rho),
        "target_ids": i32(target_ids), "target_pos": i32(target_pos),
        "target_hidden": hidden, "next_token_ids": i32(next_ids),
        "block_table": i32(block_table.reshape(w.C, max_blocks)),
        "spare_pages": i32(perm[used:]),
    }


def make_kv_pool(m: ModelDims, num_blocks: int, seed: int, block_size: int = 16, fp8: bool = False) -> dict:
    """Prior KV-cache contents, slot-addressed: k, v bf16 bits of shape
    [N layers][num_blocks * block_size slots][Hkv][dh], all ~ N(0, 1).
    (Slots past a request's context hold stale values that the step must
    overwrite before it reads them.)
    fp8: the same draws stored as E4M3 codes (uint8), rounded to nearest by
    the library's float8_e4m3fn type; with the scales of kv_fp8_scales they
    read back as code value * scale."""
    shape = (m.N, num_blocks * block_size, m.Hkv, m.dh)
    if not fp8:
        return {"k": _fill(shape, seed, 21, "normal", 1.0),
                "v": _fill(shape, seed, 22, "normal", 1.0)}
    import torch
    out = {}
    for name, tag in (("k", 23), ("v", 24)):
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tag,)))
        x = np.clip(rng.standard_normal(shape, dtype=np.float32), -448.0, 448.0)
        out[name] = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out


def kv_fp8_scales(m: ModelDims, seed: int) -> dict:
    """Per-layer scales of an fp8 KV cache (stored code = value / scale):
    k_scale and v_scale uniform in [0.5, 2), float32."""
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(25,)))
    return {"k_scale": rng.uniform(0.5, 2.0, m.N).astype(np.float32),
            "v_scale": rng.uniform(0.5, 2.0, m.N).astype(np.float32)}


def make_cod_keep(B: int, n: int, K: int, r: float, seed: int, lengths=None) -> np.ndarray:
    """Kept-position masks of B training sequences, uint8 [B][K][n] (1 = kept).

    Stand-in for COD sampling's output ([Paper] sec. 3 challenge analysis:
    deeper depths keep positions with geometric decay r): depth 0 keeps every
    position below the sequence's length; position p is kept at depth d >= 1
    with probability r, and only if position p-1 is kept at depth d-1, so
    depth d keeps about r^d of the positions and every kept position's
    dependency is kept. At n = 8192, K = 8, r = 0.8 that is about
    8192 * (1 - 0.8^8) / 0.2 = 34,080 positions, the pages' ~34K.
    lengths: optional [B] sequence lengths <= n (positions past them are
    padding, never kept); default n.
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed, 31]))
    u = rng.random((B, K, n), dtype=np.float32)
    L = np.full(B, n) if lengths is None else np.asarray(lengths)
    keep = np.zeros((B, K, n), dtype=bool)
    keep[:, 0, :] = np.arange(n)[None, :] < L[:, None]
    for d in range(1, K):
        keep[:, d, 1:] = keep[:, d - 1, :-1] & (u[:, d, 1:] < r)
    return keep.astype(np.uint8)


def make_rounds(w: Workload, R: int, seed: int | None = None) -> list:
    """Inputs of rounds 2..R of a multi-round run (the verifier stand-in's
    draws): per round, accepted-draft counts a_r ~ U{0..K}, the token the
    target samples after verification (uniform in [0, V-1)) and the target
    hidden rows of the K+1-token verify windows (~ N(0, 1), bf16 bits)."""
    seed = w.seed if seed is None else seed
    m = w.model
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(41,)))
    out = []
    for t in range(R - 1):
        out.append({
            "accepted": np.ascontiguousarray(rng.integers(0, w.K + 1, size=w.C), dtype=np.int32),
            "next_token_ids": np.ascontiguousarray(rng.integers(0, m.V - 1, size=w.C), dtype=np.int32),
            "target_hidden": _fill((w.C * (w.K + 1), m.hidden3), seed * 1000 + t, 43, "normal", 1.0),
        })
    return out
