"""FP8 Q.K^T (R23) against the fp64 oracle: with an FP8 cache and qk_dtype
FP8, q is quantised with a per-tensor q_scale and the scores run on FP8
matrix cores.  Decode (both schedules, several new tokens, groups 8 and 16),
prefill and ragged prefill; outputs and lse to the R14 FP8 tolerance.  Each
case also checks that the GPU result is closer to the quantised-q oracle than
to the BF16-q one (so the FP8 path is the one that ran)."""

import numpy as np
import pytest
import torch

import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import check_output, poison_cache, to_f64, fp8_lse_slack, fp8_lse_slack_for
from gpu_util import device, to_device, run_step, config_for
from test_gpu_step import oracle_step
from test_gpu_prefill import run_prefill, oracle_prefill
from test_gpu_varlen import run_varlen, oracle_varlen, check_against

pytestmark = pytest.mark.gpu

COARSE = 0.3          # q codes about 0.3 apart near |q| = 4: the quantisation shows
FINE = 2.0 ** -6


def qk_cfg(w, g, q_scale):
    cfg = config_for(w, g)
    cfg.qk_dtype, cfg.q_scale = "fp8", q_scale
    return cfg


def closer_to_quantised(got, ref_q8, ref_bf16):
    e8 = np.abs(got - ref_q8).max()
    e16 = np.abs(got - ref_bf16).max()
    assert e8 < 0.5 * e16, (e8, e16)


DECODE = [
    dict(seq_lens=[65, 1000, 4097, 3], num_q_heads=64, num_kv_heads=8),
    dict(seq_lens=[2000, 70, 129], num_q_heads=32, num_kv_heads=2),
    dict(seq_lens=[130, 1500], num_q_heads=64, num_kv_heads=8, tokens=2),
    dict(seq_lens=[130, 1500, 67], num_q_heads=64, num_kv_heads=8, tokens=4),   # two blocks per wave
]


@pytest.mark.parametrize("case", range(len(DECODE)))
@pytest.mark.parametrize("sched", ["dynamic5", "dynamic256", "static"])
def test_decode_fp8_scores(case, sched):
    dev = device()
    w = wl.custom(seed=740 + case, kv_dtype="fp8", **DECODE[case])
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    g = to_device(inp, dev)
    s = {"dynamic5": lb.Schedule("dynamic", num_workers=5),
         "dynamic256": lb.Schedule("dynamic", num_workers=256),
         "static": lb.Schedule("static", num_workers=256)}[sched]
    print(f"fp8 scores decode case {case} {sched}", flush=True)
    res = run_step(w, g, s, cfg=qk_cfg(w, g, COARSE))
    assert res["error"] == 0
    pro, ro, rl = oracle_step(w, inp, {"qk_dtype": "fp8", "q_scale": COARSE})
    got = to_f64(res["out"]).reshape(ro.shape)
    check_output(got, ro, "fp8", "fp8-score output")
    lse = to_f64(res["lse"]).reshape(rl.shape)
    slack = fp8_lse_slack_for(inp, w, pro, COARSE, np.repeat(np.arange(w.batch), w.tokens))
    assert np.all(np.abs(lse - rl) <= 1e-4 + 1e-5 * np.abs(rl) + slack.reshape(rl.shape)), \
        float(np.abs(lse - rl).max())
    _, rb, _ = oracle_step(w, inp)
    closer_to_quantised(got, ro, rb)


def test_decode_fine_scale():
    """A fine q_scale: codes track q closely and the result stays in tolerance."""
    dev = device()
    w = wl.custom([300, 4100, 64], kv_dtype="fp8", seed=750)
    inp = wl.make_inputs(w)
    g = to_device(inp, dev)
    res = run_step(w, g, lb.Schedule("dynamic", num_workers=64), cfg=qk_cfg(w, g, FINE))
    pro, ro, rl = oracle_step(w, inp, {"qk_dtype": "fp8", "q_scale": FINE})
    check_output(to_f64(res["out"]), ro, "fp8", "fine-scale output")
    slack = fp8_lse_slack_for(inp, w, pro, FINE, np.arange(w.batch))
    assert np.all(np.abs(to_f64(res["lse"]) - rl) <= 1e-4 + 1e-5 * np.abs(rl) + slack)


@pytest.mark.parametrize("case", [
    dict(seq_lens=[100, 300], tokens=100),
    dict(seq_lens=[65, 129, 4096], num_q_heads=16, num_kv_heads=4, tokens=65),
])
def test_prefill_fp8_scores(case):
    dev = device()
    c = dict(case)
    c.setdefault("num_q_heads", 64)
    c.setdefault("num_kv_heads", 8)
    w = wl.custom(seed=760, kv_dtype="fp8", **c)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    g = to_device(inp, dev)
    res = run_prefill(w, g, qk_cfg(w, g, COARSE))
    assert res["error"] == 0
    pro, ro, rl = oracle_prefill(w, inp, {"qk_dtype": "fp8", "q_scale": COARSE})
    got = to_f64(res["out"]).reshape(ro.shape)
    check_output(got, ro, "fp8", "fp8-score prefill output")
    lse = to_f64(res["lse"]).reshape(rl.shape)
    slack = fp8_lse_slack_for(inp, w, pro, COARSE, np.repeat(np.arange(w.batch), w.tokens))
    assert np.all(np.abs(lse - rl) <= 1e-4 + 1e-5 * np.abs(rl) + slack.reshape(rl.shape))
    _, rb, _ = oracle_prefill(w, inp)
    closer_to_quantised(got, ro, rb)


def test_ragged_prefill_fp8_scores():
    dev = device()
    w = wl.custom([300, 5, 700, 64], kv_dtype="fp8", seed=770, new_tokens=[300, 0, 33, 1])
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    g = to_device(inp, dev)
    res = run_varlen(w, g, cfg=qk_cfg(w, g, COARSE))
    assert res["error"] == 0
    pro, ref = oracle_varlen(w, inp, extra={"qk_dtype": "fp8", "q_scale": COARSE})
    seq_of_row = np.repeat(np.arange(w.batch), w.new_tokens)
    check_against(w, res, ref, fp8_lse_slack_for(inp, w, pro, COARSE, seq_of_row))


@pytest.mark.slow
def test_full_mix_fp8_scores_sampled():
    """mix_fp8 in the benchmark's launch configuration with FP8 scores."""
    import oracle
    from checks import host_step_inputs, oracle_cfg
    from gpu_util import compact_pools, remap_slots
    dev = device()
    w = wl.named("mix_fp8")
    g = wl.make_inputs(w, device=dev)
    q_scale = 2.0 ** -5
    res = run_step(w, g, lb.Schedule("dynamic"), cfg=qk_cfg(w, g, q_scale))
    assert res["error"] == 0
    h = host_step_inputs(g)
    pro = oracle.prologue(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                          h["block_table"], theta=w.rope_theta, eps=w.rms_eps,
                          kv_dtype=w.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    seqs = [0, 7, 31]
    kp, vp, bt, pmap = compact_pools(g, w, seqs)
    cfg = dict(oracle_cfg(g, w), qk_dtype="fp8", q_scale=q_scale)
    ref = oracle.decode_attention(pro["q_out"], (kp, vp), remap_slots(pro, pmap), h["seq_lens"],
                                  bt, cfg, seqs=seqs, heads=list(range(64)))
    out, lse = to_f64(res["out"]), to_f64(res["lse"])
    # the cache as read back holds the step's new keys (bit-exact to the oracle's)
    slack = fp8_lse_slack(w, kp, bt, h["seq_lens"], g["page_stride"], g["head_stride"],
                          pro["q_out"], q_scale, np.arange(w.batch), seqs=seqs)
    for (b, hh), (o, l) in ref.items():
        check_output(out[b, hh], o, "fp8", f"seq {b} head {hh}")
        assert abs(lse[b, hh] - l) <= 1e-4 + 1e-5 * abs(l) + slack[b, hh]


@pytest.mark.parametrize("q_scale", [2.0 ** -6, 2.0 ** -5, 2.0 ** -3, COARSE])
def test_fp8_score_error_within_the_accumulation_bound(q_scale):
    """One-row sequences, so each lse is a single score: its error against the
    oracle's exact dot product of the same codes stays within FP8_SCORE_REL
    times sm * sum_d |q_d k_d| with no absolute floor (the bound the FP8-score
    lse checks add), and the BF16-score step on the same inputs is exact to
    fp32 rounding."""
    dev = device()
    w = wl.custom([1] * 64, num_q_heads=64, num_kv_heads=8, kv_dtype="fp8", seed=4242)
    inp = wl.make_inputs(w)
    g = to_device(inp, dev)
    res = run_step(w, g, lb.Schedule("dynamic", num_workers=256), cfg=qk_cfg(w, g, q_scale))
    assert res["error"] == 0
    pro, _, rl = oracle_step(w, inp, {"qk_dtype": "fp8", "q_scale": q_scale})
    slack = fp8_lse_slack_for(inp, w, pro, q_scale, np.arange(w.batch))
    err = np.abs(to_f64(res["lse"]) - rl)
    assert np.all(err <= slack), float(np.max(err / slack))
    rb = run_step(w, to_device(inp, dev), lb.Schedule("dynamic", num_workers=256))
    _, _, lb16 = oracle_step(w, inp)
    assert np.max(np.abs(to_f64(rb["lse"]) - lb16)) < 2e-6
