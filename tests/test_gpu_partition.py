"""GPU parity of the sequence partitioning (pd_seq_partition, through the C
ABI) against the oracle ([Paper] sec. 3.2 "Sequence Partitioning").

Integer work: every output is compared bit for bit -- the per-position
segment ids, the per-segment offsets and the row lists -- on small and
multi-tile sequences, uneven and empty segments, one to 256 segments, depths
1 to 16, broken chains and bad boundaries (reported, never read out of
bounds), the Figure 4 example, and at the benchmark's full size (256
sequences of 8192 tokens, K = 8, r = 0.8, 4 segments) on sampled sequences
against the oracle and on every sequence against the closed form (a
position's segment is the one holding depth-1 index p-d+1).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "partition_fig4_example.json")
SENT = -7


def _say(msg):
    print(msg, flush=True)


def run_gpu(keep: np.ndarray, bnd: np.ndarray):
    import drafting_pd_expand_amd as pdx
    dev = torch.device("cuda:0")
    B, K, n = keep.shape
    S = bnd.shape[1] - 1
    k = torch.from_numpy(np.ascontiguousarray(keep, dtype=np.uint8)).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(bnd, dtype=np.int32)).to(dev)
    seg = torch.full((B, K, n), SENT, dtype=torch.int32, device=dev)
    off = torch.full((B, S + 1), SENT, dtype=torch.int32, device=dev)
    rows = torch.full((B, K * n), SENT, dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    pdx.pd_seq_partition(k, b, seg, off, rows, st)
    torch.cuda.synchronize()
    return seg.cpu().numpy(), off.cpu().numpy(), rows.cpu().numpy(), int(st.item())


def check_against_oracle(keep, bnd, seg, off, rows, seqs=None):
    B, K, n = keep.shape
    bad = False
    for i in (range(B) if seqs is None else seqs):
        res = oracle.seq_partition(keep[i].astype(bool), bnd[i])
        bad |= res["bad"]
        assert np.array_equal(seg[i], res["seg"]), f"sequence {i}: segment ids differ"
        assert list(off[i]) == res["offsets"], f"sequence {i}: offsets {list(off[i])[:8]} vs {res['offsets'][:8]}"
        want = [d * n + p for o in res["owned"] for (d, p) in o]
        tot = res["offsets"][-1]
        assert np.array_equal(rows[i][:tot], np.asarray(want, dtype=np.int64)), f"sequence {i}: row lists differ"
        assert (rows[i][tot:] == SENT).all(), f"sequence {i}: rows written past the end"
    return bad


def closed_form(keep, bnd):
    """Vectorized closed form (any size): validity down the chains, segment of
    depth-1 index p-d+1, rows ordered by (segment, depth, p)."""
    B, K, n = keep.shape
    k = keep.astype(bool)
    valid = k.copy()
    for d in range(1, K):
        valid[:, d, 0] = False
        valid[:, d, 1:] = k[:, d, 1:] & valid[:, d - 1, :-1]
    seg = np.full((B, K, n), -1, np.int64)
    p = np.arange(n)
    for i in range(B):
        for d in range(K):
            q = p - max(d - 1, 0)
            s = np.searchsorted(bnd[i], q, side="right") - 1
            seg[i, d] = np.where(valid[i, d], s, -1)
    return seg


@pytest.mark.parametrize("B,n,K,S,r,seed", [
    (3, 16, 4, 2, 0.8, 1), (4, 40, 5, 3, 0.8, 2), (2, 64, 1, 4, 0.8, 3), (3, 96, 16, 7, 0.9, 4),
    (2, 8200, 8, 4, 0.8, 5), (2, 16384, 4, 256, 0.8, 6), (5, 256, 8, 1, 0.8, 7),
], ids=["n16", "n40", "k1", "k16", "two-tiles", "s256", "s1"])
def test_partition_matches_oracle(B, n, K, S, r, seed):
    rng = np.random.default_rng(seed)
    lengths = [n - int(rng.integers(0, min(n, 40))) for _ in range(B)]
    keep = synth.make_cod_keep(B, n, K, r, seed, lengths=lengths)
    bnd = np.zeros((B, S + 1), np.int32)
    for i in range(B):
        if i % 2 == 0:
            bnd[i] = oracle.equal_boundaries(n, S)
        else:   # uneven, possibly empty segments
            bnd[i] = sorted([0, n] + list(rng.integers(0, n + 1, size=S - 1)))
    _say(f"[partition] B={B} n={n} K={K} S={S}")
    seg, off, rows, st = run_gpu(keep, bnd)
    assert st == 0
    assert not check_against_oracle(keep, bnd, seg, off, rows)


def test_figure4_example_and_broken_chain():
    g = json.load(open(GOLD))
    K, n = g["K"], g["n"]
    keep = np.zeros((2, K, n), np.uint8)
    for j, spec in enumerate((g["keep"], g["broken"]["keep"])):
        for d, ps in spec.items():
            keep[j, int(d), ps] = 1
    bnd = np.array([g["boundaries"]] * 2, np.int32)
    _say("[partition] figure-4 example")
    seg, off, rows, st = run_gpu(keep, bnd)
    assert st == 32      # the second sequence has a broken chain
    assert check_against_oracle(keep, bnd, seg, off, rows)
    assert seg[0][2][8] == 0 and seg[0][3][9] == 0
    for d, p in g["broken"]["unplaced"]:
        assert seg[1][d][p] == -1


def test_random_broken_chains_and_bad_boundaries():
    rng = np.random.default_rng(21)
    B, n, K, S = 4, 48, 5, 3
    keep = synth.make_cod_keep(B, n, K, 0.8, 22)
    for _ in range(10):
        keep[int(rng.integers(0, B)), int(rng.integers(1, K)), int(rng.integers(0, n))] ^= 1
    keep[0, 3, 1] = 1                        # a depth-3 position with no possible chain
    bnd = np.array([[0, 16, 30, 48]] * B, np.int32)
    bnd[2] = [0, 30, 16, 48]                 # decreasing: reported, sequence left unassigned
    _say("[partition] broken chains + bad boundaries")
    seg, off, rows, st = run_gpu(keep, bnd)
    assert st & 32 and st & 64
    assert (seg[2] == -1).all() and (off[2] == 0).all() and (rows[2] == SENT).all()
    check_against_oracle(keep, bnd, seg, off, rows, seqs=[0, 1, 3])


def test_full_size_sampled_and_closed_form():
    B, n, K, S = 256, 8192, 8, 4
    keep = synth.make_cod_keep(B, n, K, 0.8, 99)
    bnd = np.array([oracle.equal_boundaries(n, S)] * B, np.int32)
    _say(f"[partition] full size B={B} n={n} K={K} S={S}")
    seg, off, rows, st = run_gpu(keep, bnd)
    assert st == 0
    check_against_oracle(keep, bnd, seg, off, rows, seqs=[0, 131, 255])
    want = closed_form(keep, bnd)
    assert np.array_equal(seg, want)
    for i in range(B):
        s = want[i].reshape(-1)
        idx = np.nonzero(s >= 0)[0]
        order = idx[np.lexsort((idx, s[idx]))]    # (segment, then d * n + p)
        assert np.array_equal(rows[i][:len(order)], order), f"sequence {i}"
        cnt = np.bincount(s[idx], minlength=S)
        assert np.array_equal(off[i], np.concatenate([[0], np.cumsum(cnt)])), f"sequence {i}"
    # deterministic: a second run is bit-identical
    seg2, off2, rows2, _ = run_gpu(keep, bnd)
    assert np.array_equal(seg, seg2) and np.array_equal(off, off2) and np.array_equal(rows, rows2)
