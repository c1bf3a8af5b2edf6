"""The device schedule equals the oracle's, bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from gpu_util import device

pytestmark = pytest.mark.gpu


def device_plan(lens, sched, max_blocks=None):
    dev = device()
    lens = [int(x) for x in lens]
    mb = max_blocks or max(-(-L // 64) for L in lens)
    cfg = lb.DecodeConfig(64, 8, "bf16", max_blocks_per_seq=mb, num_pages=1)
    ws = lb.alloc_workspace(cfg, len(lens), sched, device=dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    lb.plan(cfg, sl, sched, ws)
    torch.cuda.synchronize()
    return lb.read_plan(cfg, len(lens), sched, ws)


def assert_same(got, ref):
    assert np.array_equal(got["cu_tiles"], ref.cu_tiles)
    assert np.array_equal(got["worker_chunk"], ref.worker_chunk)
    assert np.array_equal(got["chunks"], ref.chunks)
    assert np.array_equal(got["seq_chunk"], ref.seq_chunk)


@pytest.mark.parametrize("name", wl.NAMES)
@pytest.mark.parametrize("P", [1, 7, 256, 512, 1024])
def test_named_workloads_dynamic(name, P):
    lens = wl.named(name).seq_lens
    got = device_plan(lens, lb.Schedule("dynamic", num_workers=P))
    assert got["error_word"] == 0
    assert_same(got, oracle.plan_dynamic(lens, P))


@pytest.mark.parametrize("name", wl.NAMES)
@pytest.mark.parametrize("S", [0, 1, 3, 8, 64])
def test_named_workloads_static(name, S):
    lens = wl.named(name).seq_lens
    got = device_plan(lens, lb.Schedule("static", num_workers=256, static_splits=S))
    assert_same(got, oracle.plan_static(lens, S or max(1, 256 // len(lens))))


def test_random_batches():
    rng = np.random.default_rng(123)
    for i in range(300):
        B = int(rng.integers(1, 200)) if i % 3 else int(rng.integers(1, 3000))
        lens = rng.integers(1, int(rng.choice([100, 5000, 300_000])), B)
        P = int(rng.integers(1, 1025))
        assert_same(device_plan(lens, lb.Schedule("dynamic", num_workers=P)),
                    oracle.plan_dynamic(lens, P))
        S = int(rng.integers(1, 20))
        assert_same(device_plan(lens, lb.Schedule("static", num_workers=P, static_splits=S)),
                    oracle.plan_static(lens, S))


def test_largest_batch():
    lens = np.random.default_rng(5).integers(1, 70_000, 16384)
    assert_same(device_plan(lens, lb.Schedule("dynamic", num_workers=1024)),
                oracle.plan_dynamic(lens, 1024))


def test_out_of_range_lengths_are_clamped_and_flagged():
    got = device_plan([0, 5, 700], lb.Schedule("dynamic", num_workers=4), max_blocks=4)
    assert got["error_word"] & lb._binding.DEV_ERR_SEQ_LEN
    assert got["seq_len_eff"].tolist() == [1, 5, 256]
    assert_same(got, oracle.plan_dynamic([1, 5, 256], 4))


WEIGHT_SETS = [(1,) * 8, (9, 10, 9, 10, 9, 10, 9, 10), (1, 65536, 3, 700, 2, 1, 65536, 5),
               (65536,) * 8, (10, 9, 10, 9, 10, 9, 10, 9)]


@pytest.mark.parametrize("name", wl.NAMES)
@pytest.mark.parametrize("P", [1, 7, 256, 1000])
@pytest.mark.parametrize("wi", range(len(WEIGHT_SETS)))
def test_named_workloads_weighted(name, P, wi):
    lens = wl.named(name).seq_lens
    wts = WEIGHT_SETS[wi]
    got = device_plan(lens, lb.Schedule("dynamic", num_workers=P, xcd_weights=wts))
    assert got["error_word"] == 0
    assert_same(got, oracle.plan_dynamic(lens, P, wts))


def test_random_weighted_batches():
    rng = np.random.default_rng(321)
    for i in range(150):
        B = int(rng.integers(1, 300)) if i % 3 else int(rng.integers(1, 3000))
        lens = rng.integers(1, int(rng.choice([100, 5000, 300_000])), B)
        P = int(rng.integers(1, 1025))
        wts = tuple(int(x) for x in rng.integers(1, int(rng.choice([3, 1000, 65537])), 8))
        assert_same(device_plan(lens, lb.Schedule("dynamic", num_workers=P, xcd_weights=wts)),
                    oracle.plan_dynamic(lens, P, wts))


def test_largest_weighted():
    """Largest sizes: 16384 sequences of up to 262144 tokens, 1024 workers,
    maximal weights (T * C(P) near 2^53)."""
    lens = np.random.default_rng(6).integers(1, 262_145, 16384)
    wts = (65536, 65535, 65536, 65535, 65534, 65536, 65533, 65536)
    assert_same(device_plan(lens, lb.Schedule("dynamic", num_workers=1024, xcd_weights=wts)),
                oracle.plan_dynamic(lens, 1024, wts))
