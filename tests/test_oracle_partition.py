"""Pins for the oracle's sequence partitioning (CPU only).

[Paper] sec. 3.2 "Sequence Partitioning"; [arXiv] Figure 4 caption. Pins,
each against something other than the assignment loop itself:
  * the Figure 4 setting worked by hand (tests/golden): position 8 at depth 2
    stays with position 7 at depth 1, where a split by index would separate
    them; a kept position without its dependency is reported;
  * closure: from the attention pattern alone (a depth-d position attends to
    the depth-0 positions up to its anchor p-d and to its chain (p-j, d-j)),
    every position a segment owns finds everything it attends to among the
    segment's own rows and its context -- the property the partition exists
    for -- while no segment is given more context than the depth-0 positions
    before it;
  * every placeable kept position is owned exactly once; depths 0 and 1 sit
    by index; following the chain d-1 steps down lands on depth-1 index
    p-d+1 (closed form);
  * one segment owns everything; bad boundaries are reported;
  * the COD stand-in reproduces the pages' position count (~34K at 8192,
    K = 8, r = 0.8).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "partition_fig4_example.json")


def _keep_from(spec, K, n):
    keep = np.zeros((K, n), bool)
    for d, ps in spec.items():
        keep[int(d), ps] = True
    return keep


def _attends_to(d, p, keep):
    """Everything position (d, p) attends to under the parallel-prediction
    mask: the real context (depth-0 positions 0..p-d) and its own chain of
    earlier-depth rows (p-j, d-j), j = 1..d-1, plus itself."""
    a = p - d
    need = {(0, q) for q in range(a + 1) if keep[0][q]}
    need |= {(d - j, p - j) for j in range(1, d)}
    need.add((d, p))
    return need


def check_closure(res, keep, boundaries):
    S = len(boundaries) - 1
    for s in range(S):
        have = set(map(tuple, res["owned"][s])) | {(0, q) for q in res["context"][s]}
        for (d, p) in res["owned"][s]:
            missing = _attends_to(d, p, keep) - have
            assert not missing, f"segment {s}: ({d}, {p}) attends to {sorted(missing)[:4]} outside the segment"
        # causal completion adds the depth-0 positions before b_s and nothing else
        assert res["context"][s] == [q for q in range(boundaries[s]) if keep[0][q]]


def check_assignment(res, keep, boundaries):
    K, n = keep.shape
    S = len(boundaries) - 1
    seen = {}
    for s in range(S):
        for dp in res["owned"][s]:
            assert tuple(dp) not in seen, f"{dp} owned twice"
            seen[tuple(dp)] = s
    # placeable = kept with an unbroken chain down to depth 0
    for d in range(K):
        for p in range(n):
            ok = all(p - j >= 0 and keep[d - j][p - j] for j in range(d + 1))
            assert ((d, p) in seen) == ok, (d, p)
            if not ok:
                assert res["seg"][d][p] == -1
                continue
            s = seen[(d, p)]
            assert res["seg"][d][p] == s
            q = p if d == 0 else p - d + 1      # depth-1 index at the chain's start
            assert boundaries[s] <= q < boundaries[s + 1], (d, p, s)
    assert res["offsets"] == list(np.cumsum([0] + [len(o) for o in res["owned"]]))
    # each segment's rows are listed depth by depth, positions ascending
    for s in range(S):
        assert res["owned"][s] == sorted(res["owned"][s])


def test_figure4_example_by_hand():
    g = json.load(open(GOLD))
    K, n, b = g["K"], g["n"], g["boundaries"]
    keep = _keep_from(g["keep"], K, n)
    res = oracle.seq_partition(keep, b)
    assert not res["bad"]
    assert list(res["seg"][0]) == g["expected_seg"]["0"]
    for d in ("1", "2", "3"):
        for p, s in g["expected_seg"][d].items():
            assert res["seg"][int(d)][int(p)] == s, (d, p)
    assert [[list(x) for x in o] for o in res["owned"]] == g["expected_owned"]
    assert res["context"] == g["expected_context"]
    check_closure(res, keep, b)
    # the by-index split separates the caption's pair, and breaks closure
    for key, s_naive in g["naive_by_index_seg_of"].items():
        d, p = json.loads(key)
        assert res["seg"][d][p] != s_naive
    naive = {"owned": [[], []], "context": res["context"]}
    for d in range(K):
        for p in range(n):
            if keep[d][p]:
                naive["owned"][0 if p < b[1] else 1].append((d, p))
    with pytest.raises(AssertionError):
        check_closure(naive, keep, b)


def test_figure4_broken_chain_reported():
    g = json.load(open(GOLD))
    keep = _keep_from(g["broken"]["keep"], g["K"], g["n"])
    res = oracle.seq_partition(keep, g["boundaries"])
    assert res["bad"]
    for d, p in g["broken"]["unplaced"]:
        assert res["seg"][d][p] == -1
    placed = sum(len(o) for o in res["owned"])
    assert placed == int(keep.sum()) - len(g["broken"]["unplaced"])
    check_closure(res, keep, g["boundaries"])


@pytest.mark.parametrize("n,K,S,r,seed", [
    (40, 4, 3, 0.8, 1), (64, 6, 5, 0.9, 2), (33, 3, 1, 0.7, 3), (50, 5, 50, 0.8, 4), (24, 8, 4, 1.0, 5),
])
def test_random_cod_closure_and_assignment(n, K, S, r, seed):
    rng = np.random.default_rng(seed)
    keep = synth.make_cod_keep(1, n, K, r, seed, lengths=[n - int(rng.integers(0, 5))])[0].astype(bool)
    for b in (oracle.equal_boundaries(n, S),
              sorted([0, n] + list(rng.integers(0, n + 1, size=S - 1)))):   # uneven, possibly empty segments
        res = oracle.seq_partition(keep, b)
        assert not res["bad"]
        check_closure(res, keep, b)
        check_assignment(res, keep, b)


def test_one_segment_owns_everything():
    keep = synth.make_cod_keep(1, 30, 5, 0.8, 9)[0].astype(bool)
    res = oracle.seq_partition(keep, [0, 30])
    assert res["owned"][0] == sorted((d, p) for d in range(5) for p in range(30) if keep[d][p])
    assert res["context"] == [[]]


def test_random_broken_chains_reported():
    rng = np.random.default_rng(11)
    keep = synth.make_cod_keep(1, 48, 5, 0.8, 12)[0].astype(bool)
    holes = keep.copy()
    for _ in range(6):
        d, p = int(rng.integers(1, 4)), int(rng.integers(0, 48))
        holes[d][p] = False
    extra = holes.copy()
    extra[3][1] = True           # no depth-2 position 0 can exist: never placeable
    for k in (holes, extra):
        res = oracle.seq_partition(k, [0, 16, 30, 48])
        broken = any(k[d][p] and not all(p - j >= 0 and k[d - j][p - j] for j in range(d + 1))
                     for d in range(5) for p in range(48))
        assert res["bad"] == broken
        check_closure(res, k, [0, 16, 30, 48])
        check_assignment(res, k, [0, 16, 30, 48])


@pytest.mark.parametrize("b", [[1, 5, 10], [0, 5, 9], [0, 6, 5, 10], [0]])
def test_bad_boundaries_reported(b):
    keep = np.ones((2, 10), bool)
    keep[1][0] = False
    res = oracle.seq_partition(keep, b)
    assert res["bad"]
    assert (res["seg"] == -1).all()


def test_cod_standin_matches_pages_position_count():
    keep = synth.make_cod_keep(8, 8192, 8, 0.8, 3)
    per = keep.reshape(8, -1).sum(axis=1)
    # [Paper] sec. 3.2: 8192 tokens, K = 8, r = 0.8 give about 34K positions
    assert abs(per.mean() - 34000) < 400
    # every kept position's dependency is kept
    k = keep.astype(bool)
    assert not (k[:, 1:, 1:] & ~k[:, :-1, :-1]).any() and not k[:, 1:, 0].any()
