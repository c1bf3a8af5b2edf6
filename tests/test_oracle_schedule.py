"""Pins for the oracle's schedule: brute force, invariants, property tests."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import plan_dynamic, plan_static, tiles_per_sequence, default_static_splits


def brute_force_dynamic(seq_lens, P):
    """Enumerate tiles one by one: find each tile's worker by scanning the
    worker boundaries, then cut maximal runs of equal (worker, sequence)."""
    n = [-(-L // 64) for L in seq_lens]
    owner_seq, local = [], []
    for b, nb in enumerate(n):
        for t in range(nb):
            owner_seq.append(b)
            local.append(t)
    T = len(owner_seq)
    bounds = [w * T // P for w in range(P + 1)]
    owner_w = []
    for i in range(T):
        w = 0
        while not (bounds[w] <= i < bounds[w + 1]):
            w += 1
        owner_w.append(w)
    chunks = []
    i = 0
    while i < T:
        j = i
        while j + 1 < T and owner_w[j + 1] == owner_w[i] and owner_seq[j + 1] == owner_seq[i]:
            j += 1
        chunks.append((owner_seq[i], local[i], local[j] + 1, owner_w[i]))
        i = j + 1
    return chunks


def check_plan_invariants(plan, seq_lens):
    n = tiles_per_sequence(seq_lens)
    B = n.size
    cover = [np.zeros(nb, dtype=np.int64) for nb in n]
    ch = plan.chunks
    for c in range(ch.shape[0]):
        b, t0, t1, w = ch[c]
        assert 0 <= t0 < t1 <= n[b]
        cover[b][t0:t1] += 1
        assert plan.worker_chunk[w] <= c < plan.worker_chunk[w + 1]
    for b in range(B):
        assert np.all(cover[b] == 1), f"sequence {b} tiles not covered exactly once"
        lo, hi = plan.seq_chunk[b], plan.seq_chunk[b + 1]
        assert hi > lo and np.all(ch[lo:hi, 0] == b)
        assert ch[lo, 1] == 0 and ch[hi - 1, 2] == n[b]
        assert np.all(ch[lo + 1:hi, 1] == ch[lo:hi - 1, 2])
    assert np.all(np.diff(plan.worker_chunk) >= 0)
    assert plan.seq_chunk[B] == ch.shape[0] == plan.worker_chunk[-1]
    assert np.array_equal(plan.cu_tiles, np.concatenate([[0], np.cumsum(n)]))


def test_dynamic_matches_brute_force_small():
    rng = np.random.default_rng(0)
    for _ in range(300):
        B = int(rng.integers(1, 7))
        P = int(rng.integers(1, 9))
        lens = rng.integers(1, 700, B).tolist()
        plan = plan_dynamic(lens, P)
        assert [tuple(c) for c in plan.chunks.tolist()] == brute_force_dynamic(lens, P)
        check_plan_invariants(plan, lens)


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(1, 5000), min_size=1, max_size=40), st.integers(1, 600))
def test_dynamic_properties(lens, P):
    plan = plan_dynamic(lens, P)
    check_plan_invariants(plan, lens)
    T = int(tiles_per_sequence(lens).sum())
    loads = np.zeros(P, dtype=np.int64)
    for b, t0, t1, w in plan.chunks:
        loads[w] += t1 - t0
    assert loads.sum() == T
    assert set(np.unique(loads)) <= {T // P, -(-T // P)}       # balanced to one tile
    assert plan.num_chunks <= P + len(lens) - 1


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(1, 5000), min_size=1, max_size=40), st.integers(1, 16))
def test_static_properties(lens, S):
    plan = plan_static(lens, S)
    check_plan_invariants(plan, lens)
    n = tiles_per_sequence(lens)
    assert plan.num_workers == len(lens) * S
    for b, t0, t1, w in plan.chunks:
        assert w // S == b
        s = w % S
        assert t0 == s * n[b] // S and t1 == (s + 1) * n[b] // S
    # per sequence, split sizes differ by at most one tile
    for b in range(len(lens)):
        sizes = [t1 - t0 for bb, t0, t1, _ in plan.chunks if bb == b]
        assert max(sizes) - min(sizes) <= 1


def test_mixed_batch_figures():
    """1 x 131072 + 31 x 4096 tokens on 256 workers: 2048 + 31*64 tiles."""
    lens = [131072] + [4096] * 31
    plan = plan_dynamic(lens, 256)
    assert plan.cu_tiles[-1] == 2048 + 31 * 64
    loads = np.bincount(plan.chunks[:, 3], weights=plan.chunks[:, 2] - plan.chunks[:, 1], minlength=256)
    assert loads.max() == 16 and loads.min() == 15          # 4032 / 256 = 15.75
    # workers w with floor(w*4032/256) < 2048, i.e. w <= 130, touch the long sequence
    assert plan.seq_chunk[1] - plan.seq_chunk[0] == 131
    # 256 workers + 31 interior sequence starts, minus the one start that falls on a
    # worker boundary: floor(191*4032/256) = 3008 = 2048 + 15*64
    assert plan.num_chunks == 256 + 31 - 1
    static = plan_static(lens, default_static_splits(32, 256))
    # static: 8 splits each; the long sequence's splits hold 256 tiles
    assert default_static_splits(32, 256) == 8
    assert max(t1 - t0 for _, t0, t1, _ in static.chunks) == 256


def test_loguniform_batch_figures():
    """The log-uniform FP8 batch: 64 lengths rint(exp(U(ln 512, ln 262144))) from
    default_rng(5) hold 2,771,856 tokens in 43,341 tiles; on 256 workers each
    takes 169 or 170 tiles (43341 / 256 = 169.3), cut into 318 chunks, at most
    25 of them in one sequence."""
    from load_balanced_split_rope_amd import workloads as wl
    lens = wl.named("loguniform").seq_lens
    assert len(lens) == 64 and min(lens) >= 512 and max(lens) <= 262144
    assert sum(lens) == 2771856
    plan = plan_dynamic(lens, 256)
    assert plan.cu_tiles[-1] == 43341
    loads = np.bincount(plan.chunks[:, 3], weights=plan.chunks[:, 2] - plan.chunks[:, 1], minlength=256)
    assert loads.min() == 169 and loads.max() == 170
    assert plan.num_chunks == 318
    assert np.diff(plan.seq_chunk).max() == 25


def test_uniform_batch_dynamic_equals_static():
    """With equal lengths both schedules give the same chunks (the control case)."""
    lens = [4096] * 32
    d = plan_dynamic(lens, 256)
    s = plan_static(lens, 8)
    assert np.array_equal(d.chunks, s.chunks)


def test_rejects_empty_sequences():
    with pytest.raises(ValueError):
        plan_dynamic([5, 0], 4)


# ---- XCD-weighted dynamic schedule ----

def _golden_weighted():
    path = os.path.join(os.path.dirname(__file__), "golden", "weighted_schedule_examples.txt")
    cases = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, tail = line.split(":")
        nums = [int(x) for x in head.split()]
        cases.append((nums[0], nums[1], tuple(nums[2:]), [int(x) for x in tail.split()]))
    return cases


def _tiles_per_worker(plan):
    out = np.zeros(plan.num_workers, dtype=np.int64)
    for b, t0, t1, w in plan.chunks:
        out[w] += t1 - t0
    return out


@pytest.mark.parametrize("T,P,weights,expect", _golden_weighted())
def test_weighted_hand_examples(T, P, weights, expect):
    # T tiles as T one-tile sequences (any split of T gives the same counts)
    plan = plan_dynamic([64] * T, P, weights)
    assert _tiles_per_worker(plan).tolist() == expect
    check_plan_invariants(plan, [64] * T)


def _dispatch_sim(P):
    """Simulate the launch: workgroup i goes to XCD i % 8; XCDs take worker ids
    in turn, XCD 0's whole run first.  Returns the XCD of every worker."""
    per_xcd = [[i for i in range(P) if i % 8 == x] for x in range(8)]
    xcd_of = []
    for x in range(8):
        xcd_of += [x] * len(per_xcd[x])
    return xcd_of


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(1, 3000), min_size=1, max_size=40), st.integers(1, 300),
       st.lists(st.integers(1, 65536), min_size=8, max_size=8))
def test_weighted_shares_and_invariants(lens, P, weights):
    plan = plan_dynamic(lens, P, weights)
    check_plan_invariants(plan, lens)
    T = int(tiles_per_sequence(lens).sum())
    xcd_of = _dispatch_sim(P)
    wts = [weights[x] for x in xcd_of]
    total = sum(wts)
    got = _tiles_per_worker(plan)
    for w in range(P):
        # floor of a running share: within one tile of the exact share
        assert abs(Fraction(int(got[w])) - Fraction(T * wts[w], total)) < 1
    # exact bounds from fractions
    run = 0
    for w in range(P):
        lo = math.floor(Fraction(T * run, total))
        run += wts[w]
        hi = math.floor(Fraction(T * run, total))
        assert got[w] == hi - lo


@pytest.mark.parametrize("c", [1, 7, 65536])
def test_equal_weights_are_the_unweighted_plan(c):
    rng = np.random.default_rng(3)
    for _ in range(20):
        lens = rng.integers(1, 20000, size=int(rng.integers(1, 50))).tolist()
        P = int(rng.integers(1, 400))
        a, b = plan_dynamic(lens, P), plan_dynamic(lens, P, [c] * 8)
        assert np.array_equal(a.chunks, b.chunks) and np.array_equal(a.worker_chunk, b.worker_chunk)


def test_weighted_rejects_bad_weights():
    with pytest.raises(ValueError):
        plan_dynamic([100], 8, [1] * 7)
    with pytest.raises(ValueError):
        plan_dynamic([100], 8, [1] * 7 + [0])
