"""Host logic of the XCD weight calibration (no GPU): rates from synthetic traces."""

import numpy as np
import pytest

import load_balanced_split_rope_amd as lb


def _trace(durs_us, xcds):
    n = len(durs_us)
    tr = np.zeros((n, 4), dtype=np.int64)
    tr[:, 0] = 1000
    tr[:, 1] = 1000 + np.rint(np.asarray(durs_us) * 100).astype(np.int64)
    tr[:, 3] = xcds
    return tr


def test_rates_and_weights_from_synthetic_trace():
    # 16 workers, 2 per XCD, 10 tiles each; odd XCDs take 10% longer
    xcds = np.repeat(np.arange(8), 2)
    durs = np.where(xcds % 2 == 1, 110.0, 100.0)
    plan = {"chunks": np.array([(0, 10 * w, 10 * w + 10, w) for w in range(16)])}
    rates = lb.xcd_rates([_trace(durs, xcds)], plan)
    assert np.allclose(rates, np.where(np.arange(8) % 2, 20 / 220, 20 / 200))
    wts = lb.xcd_weights_from_rates(rates, scale=1000)
    assert wts == (1000, 909, 1000, 909, 1000, 909, 1000, 909)


def test_worker_with_several_chunks_counts_all_tiles():
    xcds = np.arange(8)
    plan = {"chunks": np.array([(0, 0, 3, 0), (1, 0, 5, 0)] +
                               [(1, 5 + w, 6 + w, w) for w in range(1, 8)])}
    rates = lb.xcd_rates([_trace(np.full(8, 10.0), xcds)], plan)
    assert rates[0] == pytest.approx(0.8) and np.allclose(rates[1:], 0.1)


def test_rejects_idle_xcd_and_bad_rates():
    plan = {"chunks": np.array([(0, 0, 1, 0)])}
    with pytest.raises(ValueError):
        lb.xcd_rates([_trace([5.0], [0])], plan)
    with pytest.raises(ValueError):
        lb.xcd_weights_from_rates([1.0] * 7)
    with pytest.raises(ValueError):
        lb.xcd_weights_from_rates([1.0] * 7 + [0.0])
