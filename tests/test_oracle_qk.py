"""Pins for the FP8 Q.K^T reading (R23): q codes RNE(clamp(fl32(q * fl32(1/q_scale)),
+-448)), scores of the decoded codes times q_scale.

* codes worked by hand (a rounding, a tie to even, saturation, the scale);
* the quantiser against an exhaustive nearest-code search over all 256 E4M3
  codes (ties to the even mantissa), on random BF16 queries and scales;
* queries that E4M3 represents exactly give the BF16 path's attention bit
  for bit (the reduction to the pinned path), and a planted wrong scale fails.
"""

import numpy as np
import pytest

import oracle
from oracle import qk
from oracle.formats import e4m3_to_f64, f64_to_bf16_bits


def bits(x):
    return f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def test_codes_by_hand():
    # 1.0 at scale 1 -> 0x38; 0.30078125 (BF16 of 0.3) * 8 = 2.40625 -> 2.5 = 0x42
    assert qk.quantize_query(bits([1.0]), 1.0).tolist() == [0x38]
    assert qk.quantize_query(bits([0.3]), 0.125).tolist() == [0x42]
    # 2.375 lies halfway between 2.25 (mantissa 001) and 2.5 (010): ties to even -> 2.5
    assert qk.quantize_query(bits([2.375]), 1.0).tolist() == [0x42]
    # -2.125 halfway between -2 (000) and -2.25 (001) -> -2 = 0xC0
    assert qk.quantize_query(bits([-2.125]), 1.0).tolist() == [0xC0]
    # beyond 448 saturates to the largest finite code, either sign
    assert qk.quantize_query(bits([1000.0, -600.0]), 1.0).tolist() == [0x7E, 0xFE]
    # the scale divides: 3 at scale 0.5 -> 6 = 0x4C; values decode to code * q_scale
    assert qk.quantize_query(bits([3.0]), 0.5).tolist() == [0x4C]
    v = qk.query_values(bits([3.0]), {"qk_dtype": "fp8", "q_scale": 0.5})
    assert v.tolist() == [3.0]


def _nearest_code(x):
    """Exhaustive: the finite E4M3 code nearest to x, ties to the even code
    (even mantissa LSB), after clamping to +-448."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_to_f64(codes)
    x = min(max(float(x), -448.0), 448.0)
    d = np.abs(vals - x)
    best = np.flatnonzero(d == d.min())
    if len(best) > 1:                     # a tie: +0/-0 or two neighbours
        even = [i for i in best if (codes[i] & 1) == 0]
        best = even if even else best
    c = int(codes[best[0]])
    return 0 if vals[best[0]] == 0 and x >= 0 else c


@pytest.mark.parametrize("seed", range(4))
def test_quantiser_against_exhaustive_search(seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(400) * rng.choice([0.01, 1, 30, 300], 400)
    qb = bits(q)
    for q_scale in (1.0, 0.037, 2.0 ** -4, 3.0):
        got = qk.quantize_query(qb, q_scale)
        inv = np.float32(1.0) / np.float32(q_scale)
        x = oracle.bf16_bits_to_f64(qb).astype(np.float32) * inv
        want = [_nearest_code(v) for v in x.astype(np.float64)]
        vals_got, vals_want = e4m3_to_f64(got), e4m3_to_f64(np.array(want, dtype=np.uint8))
        assert np.array_equal(vals_got, vals_want), q_scale      # +0 / -0 compare equal


def test_representable_queries_reduce_to_the_bf16_path():
    """q = code * 2^-3 for random E4M3 codes: quantisation at q_scale 2^-3 is
    exact, so the FP8 scores equal the BF16 ones and attention is identical."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (3, 8, 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30                       # no NaN codes
    qv = e4m3_to_f64(codes) * 2.0 ** -3
    qb = bits(qv)
    assert np.array_equal(oracle.bf16_bits_to_f64(qb), qv)      # BF16 holds them exactly
    K = rng.standard_normal((3, 200, 128))
    V = rng.standard_normal((3, 200, 128))
    base = {"qk_dtype": "bf16"}
    fp8 = {"qk_dtype": "fp8", "q_scale": 2.0 ** -3}
    wrong = {"qk_dtype": "fp8", "q_scale": 3 * 2.0 ** -3}       # a planted wrong scale
    for b in range(3):
        o0, l0 = oracle.attend_full(qk.query_values(qb[b], base), K[b], V[b], 128 ** -0.5)
        o1, l1 = oracle.attend_full(qk.query_values(qb[b], fp8), K[b], V[b], 128 ** -0.5)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
        q2 = qk.query_values(qb[b], wrong)
        assert not np.array_equal(q2, qv[b])                     # re-rounded: values move
        o2, _ = oracle.attend_full(q2, K[b], V[b], 128 ** -0.5)
        assert np.abs(o2 - o0).max() > 1e-3


def test_fp8_lse_slack_is_the_measured_bound_times_the_largest_product_sum():
    """The FP8-score lse slack (R23's tolerance term for the FP8 matrix cores'
    accumulation) equals 2^-15 * sm * max over the keys of sum_d |q_d k_d|:
    brute force over a two-sequence step, both sequences, every head."""
    import oracle
    from load_balanced_split_rope_amd import workloads as wl
    from checks import fp8_lse_slack_for, host_step_inputs, host_pools, FP8_SCORE_REL
    from oracle.step import apply_prologue_writes, gather_kv
    w = wl.custom([1, 70], num_q_heads=16, num_kv_heads=2, kv_dtype="fp8", seed=5)
    inp = wl.make_inputs(w)
    h = host_step_inputs(inp)
    pro = oracle.prologue(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                          h["block_table"], theta=w.rope_theta, eps=w.rms_eps, kv_dtype="fp8",
                          k_scale=w.k_scale, v_scale=w.v_scale)
    got = fp8_lse_slack_for(inp, w, pro, 0.3, np.arange(2))
    kp, vp = (np.array(p, copy=True) for p in host_pools(inp, w))
    apply_prologue_writes(kp, vp, pro, kv_dtype="fp8", page_stride=inp["page_stride"],
                          head_stride=inp["head_stride"])
    qv = qk.query_values(pro["q_out"], {"qk_dtype": "fp8", "q_scale": 0.3})
    for b in range(2):
        L = int(h["seq_lens"][b])
        for hh in range(16):
            K = gather_kv(kp, "k", "fp8", h["block_table"][b], L, hh // 8,
                          page_stride=inp["page_stride"], head_stride=inp["head_stride"],
                          scale=float(np.float32(w.k_scale)))
            want = max(np.sum(np.abs(qv[b, hh] * K[i])) for i in range(L))
            assert np.isclose(got[b, hh], FP8_SCORE_REL / np.sqrt(128.0) * want, rtol=1e-12)
