"""Pins for the ragged-batch oracle (R22): each sequence has its own number
of new tokens, packed along one token axis.

* packed starts, positions and cache slots by hand;
* every token's output against torch's fp64 scaled-dot-product attention with
  an explicit boolean mask (a library routine), on batches with empty,
  one-token and many-token sequences;
* equal counts reduce to the uniform multi-token oracle;
* a planted mistake (two sequences' counts swapped) is caught.
"""

import numpy as np
import pytest

from oracle import multitoken as mt
from load_balanced_split_rope_amd import workloads as wl
from checks import poison_cache, host_pools, host_step_inputs, oracle_cfg
from test_oracle_multitoken import _masked_sdpa
import oracle


def test_starts_and_positions_by_hand():
    assert mt.query_starts([3, 0, 2, 1]).tolist() == [0, 3, 3, 5, 6]
    assert mt.query_starts([]).tolist() == [0]
    # sequence lengths 10, 4, 5 with 3, 0, 2 new tokens
    assert mt.varlen_positions([10, 4, 5], [3, 0, 2]).tolist() == [7, 8, 9, 3, 4]
    assert mt.varlen_positions([1], [1]).tolist() == [0]
    with pytest.raises(ValueError):
        mt.query_starts([1, -1])
    with pytest.raises(ValueError):
        mt.varlen_positions([2, 5], [3, 1])


def _setup(lens, counts, Hq=16, Hkv=2, dtype="bf16", seed=21):
    w = wl.custom(lens, num_q_heads=Hq, num_kv_heads=Hkv, kv_dtype=dtype, seed=seed,
                  new_tokens=counts)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    h = host_step_inputs(inp)
    assert np.array_equal(inp["q_start"].numpy(), mt.query_starts(counts))
    assert np.array_equal(h["positions"], mt.varlen_positions(lens, counts))
    pro = mt.prologue_varlen(h["q"], h["k"], h["v"], h["positions"], counts, h["wq"], h["wk"],
                             h["block_table"], theta=w.rope_theta, eps=w.rms_eps,
                             kv_dtype=w.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    return w, inp, h, host_pools(inp, w), pro, oracle_cfg(inp, w)


def test_slots_by_hand():
    lens, counts = [70, 5, 130], [3, 0, 66]
    w, inp, h, pools, pro, cfg = _setup(lens, counts)
    bt = h["block_table"]
    want = []
    for b, (L, n) in enumerate(zip(lens, counts)):
        for j in range(n):
            p = L - n + j
            want.append((bt[b][p // 64], p % 64))
    assert [tuple(map(int, s)) for s in pro["slots"]] == want


CASES = [([70, 5, 130, 1], [3, 0, 66, 1], "bf16"),
         ([64, 200, 33], [64, 1, 7], "fp8"),
         ([9, 129], [9, 128], "bf16")]


@pytest.mark.parametrize("lens,counts,dtype", CASES)
def test_varlen_against_masked_sdpa(lens, counts, dtype):
    w, inp, h, pools, pro, cfg = _setup(lens, counts, dtype=dtype)
    got = mt.attention_varlen(pro["q_out"], pools, pro, h["seq_lens"], counts, h["block_table"],
                              cfg)
    assert len(got) == sum(counts) * w.num_q_heads
    G = w.num_q_heads // w.num_kv_heads
    starts = mt.query_starts(counts)
    for b, (L, n) in enumerate(zip(lens, counts)):
        if n == 0:
            continue
        rows = slice(int(starts[b]), int(starts[b + 1]))
        for g in range(w.num_kv_heads):
            K, V = oracle.step._sequence_kv(pools, pro, b, g, h["seq_lens"], h["block_table"], cfg)
            assert np.all(np.isfinite(K)) and np.all(np.isfinite(V))
            o_ref, l_ref = _masked_sdpa(pro["q_out"][rows, g * G:(g + 1) * G], K, V, L, n,
                                        cfg["sm_scale"])
            for j in range(n):
                for i in range(G):
                    o, l = got[(b, j, g * G + i)]
                    np.testing.assert_allclose(o, o_ref[j, i], rtol=1e-12, atol=1e-12)
                    assert abs(l - l_ref[j, i]) <= 1e-12 * max(1.0, abs(l_ref[j, i]))


def test_equal_counts_reduce_to_uniform():
    lens, Tq = [40, 3, 100], 3
    w, inp, h, pools, pro, cfg = _setup(lens, [Tq] * 3)
    got = mt.attention_varlen(pro["q_out"], pools, pro, h["seq_lens"], [Tq] * 3,
                              h["block_table"], cfg)
    q_out = pro["q_out"].reshape(3, Tq, w.num_q_heads, 128)
    ref = mt.decode_attention_tokens(q_out, pools, pro, h["seq_lens"], h["block_table"], cfg)
    assert got.keys() == ref.keys()
    for key in ref:
        assert np.array_equal(got[key][0], ref[key][0]) and got[key][1] == ref[key][1]


def test_swapped_counts_are_caught():
    lens, counts = [80, 90], [5, 2]
    w, inp, h, pools, pro, cfg = _setup(lens, counts)
    wrong = mt.attention_varlen(pro["q_out"], pools, pro, h["seq_lens"], [2, 5],
                                h["block_table"], cfg)
    right = mt.attention_varlen(pro["q_out"], pools, pro, h["seq_lens"], counts,
                                h["block_table"], cfg)
    # sequence 1 token 0 reads packed row 5 (right) vs row 2 (wrong): different queries
    assert not np.allclose(wrong[(1, 0, 0)][0], right[(1, 0, 0)][0])
