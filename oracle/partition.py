"""Oracle: sequence partitioning for within-sequence gradient accumulation
-- TEST INFRASTRUCTURE ONLY (plain Python loops, small inputs).

[Paper] sec. 3.2 "Sequence Partitioning"; [Blog] "training on long sequences"
(the sequence partition algorithm paragraph); [arXiv] Figure 4 caption.

Training P-EAGLE on a sequence of n tokens with K prediction depths lays out
up to n x K positions: depth 0 holds every position, deeper depths only the
positions COD sampling kept. Position p at depth d (d >= 1) depends on
position p-1 at depth d-1 (it must attend to it). A long sequence is cut into
S segments, each processed on its own, so every dependency has to stay inside
one segment. The steps, in the pages' order:

  1. the S segments and their boundaries 0 = b_0 <= b_1 <= ... <= b_S = n are
     given (the pages set them from the memory limit); segment s covers the
     depth-0 indices [b_s, b_{s+1});
  2. positions at depths 0 and 1 go to the segment their index falls in;
  3. for d = 2, 3, ... in turn, position p at depth d goes to the segment its
     dependency (p-1, d-1) was given;
  4. causal completion: each segment also carries every depth-0 position up
     to its boundary -- the ones before b_s, which the segment does not own --
     as attention context.

Readings (the pages leave these open):
  * a kept position whose dependency is not kept cannot be placed; COD never
    produces one. Such a position (and everything that depends on it) gets no
    segment and the input is reported bad. Depth-0 positions have no
    dependency; a depth-1 position p needs (p-1, 0).
  * a segment's own rows are listed depth by depth, positions ascending.
"""
from __future__ import annotations

import numpy as np


def _segment_of_index(boundaries, i: int) -> int:
    """The segment whose depth-0 index range [b_s, b_{s+1}) holds i."""
    for s in range(len(boundaries) - 1):
        if boundaries[s] <= i < boundaries[s + 1]:
            return s
    return -1


def seq_partition(keep, boundaries) -> dict:
    """Assign every kept position (depth d, index p) of one sequence to a
    segment ([Paper] sec. 3.2 steps 1-4).

    keep: [K][n] booleans, position p kept at depth d.
    boundaries: S+1 ints, 0 = b_0 <= ... <= b_S = n.
    Returns {"seg": [K][n] int (-1: not kept or not placeable), "owned": S
    lists of (d, p), "context": S lists of depth-0 indices (causal
    completion), "offsets": S+1 prefix counts of the owned lists, "bad":
    True if the boundaries are invalid or a kept position lacks its
    dependency}.
    """
    keep = np.asarray(keep, dtype=bool)
    K, n = keep.shape
    b = [int(x) for x in boundaries]
    S = len(b) - 1
    seg = np.full((K, n), -1, dtype=np.int64)
    ok_bounds = S >= 1 and b[0] == 0 and b[-1] == n and all(b[s] <= b[s + 1] for s in range(S))
    if not ok_bounds:
        return {"seg": seg, "owned": [[] for _ in range(max(S, 0))], "context": [[] for _ in range(max(S, 0))],
                "offsets": [0] * (max(S, 0) + 1), "bad": True}
    bad = False
    # step 2: depths 0 and 1 by index (a depth-1 position needs (p-1, 0) kept)
    for p in range(n):
        if keep[0][p]:
            seg[0][p] = _segment_of_index(b, p)
    if K > 1:
        for p in range(n):
            if not keep[1][p]:
                continue
            if p >= 1 and keep[0][p - 1]:
                seg[1][p] = _segment_of_index(b, p)
            else:
                bad = True
    # step 3: deeper positions follow their dependency, depth after depth
    for d in range(2, K):
        for p in range(n):
            if not keep[d][p]:
                continue
            dep = seg[d - 1][p - 1] if p >= 1 else -1
            if dep >= 0:
                seg[d][p] = dep
            else:
                bad = True
    owned = [[] for _ in range(S)]
    for d in range(K):
        for p in range(n):
            if seg[d][p] >= 0:
                owned[seg[d][p]].append((d, p))
    # step 4: causal completion -- the depth-0 positions before the segment
    context = [[p for p in range(b[s]) if keep[0][p]] for s in range(S)]
    offsets = [0]
    for s in range(S):
        offsets.append(offsets[-1] + len(owned[s]))
    return {"seg": seg, "owned": owned, "context": context, "offsets": offsets, "bad": bad}


def equal_boundaries(n: int, S: int) -> list:
    """S segments of (nearly) equal depth-0 length: b_s = floor(s * n / S).
    The pages set the boundaries from the memory limit; equal lengths are the
    plainest such choice."""
    return [(s * n) // S for s in range(S + 1)]
