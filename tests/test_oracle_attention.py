"""Pins for the oracle's attention: brute force, a library routine, closed forms,
and the split-then-merge invariant."""

import math

import numpy as np
import pytest
import torch

from oracle import attend_full, combine_lse


def brute_force(q, k, v, scale):
    """Scalar loops straight from the definition of softmax attention."""
    G, D = len(q), len(q[0])
    L = len(k)
    out, lses = [], []
    for h in range(G):
        s = [scale * sum(q[h][d] * k[j][d] for d in range(D)) for j in range(L)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        out.append([sum(e[j] * v[j][d] for j in range(L)) / z for d in range(D)])
        lses.append(m + math.log(z))
    return np.array(out), np.array(lses)


def test_matches_brute_force_tiny():
    rng = np.random.default_rng(0)
    for G, L, D in [(1, 1, 4), (3, 7, 8), (8, 13, 16), (2, 64, 8)]:
        q, k, v = (rng.standard_normal(s) for s in ((G, D), (L, D), (L, D)))
        o, lse = attend_full(q, k, v, 0.37)
        bo, bl = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.37)
        assert np.allclose(o, bo, rtol=1e-13, atol=1e-14)
        assert np.allclose(lse, bl, rtol=1e-13, atol=1e-14)


def test_matches_torch_sdpa_float64():
    """Library routine: torch's scaled_dot_product_attention in float64 on CPU."""
    rng = np.random.default_rng(1)
    for G, L in [(8, 1), (8, 63), (8, 200), (16, 1000)]:
        q, k, v = (rng.standard_normal(s) for s in ((G, 128), (L, 128), (L, 128)))
        o, _ = attend_full(q, k, v, 1 / math.sqrt(128))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0]
        assert np.allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_single_key_returns_v():
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal((8, 128)), rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    o, lse = attend_full(q, k, v, 0.1)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))
    assert np.allclose(lse, 0.1 * q @ k[0], rtol=1e-15)


def test_zero_query_gives_mean_and_log_length():
    rng = np.random.default_rng(3)
    for L in (1, 2, 64, 4097):
        k, v = rng.standard_normal((L, 128)), rng.standard_normal((L, 128))
        o, lse = attend_full(np.zeros((8, 128)), k, v, 0.088)
        assert np.allclose(o, v.mean(axis=0), rtol=1e-12, atol=1e-15)
        assert np.allclose(lse, math.log(L), rtol=0, atol=1e-12)


def test_split_then_merge_equals_unsplit():
    rng = np.random.default_rng(4)
    for trial in range(30):
        L = int(rng.integers(2, 600))
        q, k, v = rng.standard_normal((8, 128)) * 2, rng.standard_normal((L, 128)), rng.standard_normal((L, 128))
        cuts = np.unique(np.concatenate([[0, L], rng.integers(1, L, int(rng.integers(1, 6)))]))
        parts = [attend_full(q, k[a:b], v[a:b], 0.088) for a, b in zip(cuts[:-1], cuts[1:])]
        o, lse = combine_lse(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        ro, rl = attend_full(q, k, v, 0.088)
        assert np.allclose(o, ro, rtol=1e-12, atol=1e-14)
        assert np.allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_merge_of_one_part_is_identity_and_key_order_is_irrelevant():
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((8, 128)), rng.standard_normal((50, 128)), rng.standard_normal((50, 128))
    o, lse = attend_full(q, k, v, 0.088)
    mo, ml = combine_lse(o[None], lse[None])
    assert np.allclose(mo, o, rtol=1e-15) and np.allclose(ml, lse, rtol=1e-15)
    p = rng.permutation(50)
    po, pl = attend_full(q, k[p], v[p], 0.088)
    assert np.allclose(po, o, rtol=1e-12, atol=1e-15) and np.allclose(pl, lse, rtol=1e-14)


def test_one_dropped_tile_moves_lse_measurably():
    """With q = 0, lse = ln L exactly; dropping one 64-token tile of a 131072-token
    sequence moves it by ln(131072/131008) = 4.9e-4, far above fp32 noise."""
    L = 131072
    assert abs(math.log(L) - math.log(L - 64)) > 4.8e-4
