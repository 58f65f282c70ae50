"""CPU oracle for the P-EAGLE parallel drafting step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy definitions of what the drafting step computes:
  * ``expand``        -- the batch expansion (ids, positions, MASK slots, the
                         rejected / masked masks, new-token indices, the
                         hidden-state map, slot mapping with -1 for rejected
                         tokens, per-request starts) and the hidden-row fill.
  * ``draft_forward`` -- fc projection, the N decoder layers (RMSNorm, RoPE,
                         paged causal GQA attention, SwiGLU MLP), final norm,
                         LM head and greedy argmax.
  * ``ar_advance``    -- the next pass of autoregressive EAGLE-style drafting
                         (one row per request, fed back token and hidden), and
  * ``ar_draft``      -- K such serial passes: the baseline that parallel
                         drafting replaces.
  * ``verify_stub``, ``draft_rounds`` -- several draft/verify rounds in a
                         row with a stand-in verifier (accepted counts and
                         target outputs are inputs), KV carried over.
  * ``fp8``           -- the E4M3 codec of the fp8 KV cache (``draft_forward``
                         and the drivers take ``kv_fp8`` scales).
  * ``seq_partition`` -- the training-side sequence partitioning: every kept
                         (depth, position) of a long sequence assigned to a
                         segment with its dependencies, plus each segment's
                         causal-completion context.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports it, and this package imports nothing from
the product path: the two share only the seeded input generator ``synth``.

Pages cited (by title; section names are those printed on the pages):
  [Paper]  "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training" (summary page)
  [Blog]   "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding in
           vLLM" (summary page of the vLLM blog post)
  [arXiv]  ScienceStack page for arXiv 2602.01469

Parity pins (tests/test_oracle_*.py) tie each function to something other than
itself: a hand-derived expansion example (tests/golden), the pages' own
hidden-state fill code run in torch, RoPE's closed form and its
relative-position identity ([Paper] appendix B / [arXiv] Theorem 2.3), a dense
library causal-attention forward on prefill, brute-force softmax, invariants
(a)-(e) and request independence. Full-forward logits at random init have no
printed values on the pages: beyond those pins they are "parity unpinned".
"""
from .expand import expand, ar_advance
from .forward import draft_forward, ar_draft, rope_rotate, rms_norm, silu
from .bf16 import bf16_to_f64
from . import fp8
from .partition import seq_partition, equal_boundaries
from .rounds import verify_stub, draft_rounds

__all__ = ["expand", "ar_advance", "draft_forward", "ar_draft", "rope_rotate", "rms_norm", "silu", "bf16_to_f64",
           "seq_partition", "equal_boundaries", "verify_stub", "draft_rounds"]
