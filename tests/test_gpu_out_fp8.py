"""FP8 attention output (R21): out holds E4M3 codes of o / out_scale.

* One-row sequences: the output is V exactly, so with power-of-two scales the
  codes must equal the oracle's encoding bit for bit -- this pins the
  kernel's rounding (BF16 values include exact E4M3 ties) and saturation.
* Steps with split sequences, both caches, several new tokens: codes within
  the R14 tolerance plus half an E4M3 step; lse unchanged from the BF16 run.
* The full mix in the benchmark's launch configuration, sampled heads.
"""

import numpy as np
import pytest
import torch

import oracle
import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import check_output_fp8, to_f64, bits_u16, poison_cache, host_step_inputs, oracle_cfg
from gpu_util import device, to_device, run_step, config_for, compact_pools, remap_slots
from test_gpu_step import oracle_step

pytestmark = pytest.mark.gpu


def fp8_cfg(w, g, out_scale):
    cfg = config_for(w, g)
    cfg.out_dtype, cfg.out_scale = "fp8", out_scale
    return cfg


@pytest.mark.parametrize("kv_dtype,out_scale", [("bf16", 2.0 ** -3), ("bf16", 2.0 ** -8),
                                                ("fp8", 2.0 ** -2), ("fp8", 2.0 ** -9)])
def test_single_row_codes_are_exact(kv_dtype, out_scale):
    """L = 1: out = v (the new token's value), so the codes are E4M3(v / out_scale)."""
    dev = device()
    w = wl.custom([1, 1, 1, 1, 1], num_q_heads=64, num_kv_heads=8, kv_dtype=kv_dtype, seed=710)
    inp = wl.make_inputs(w)
    g = to_device(inp, dev)
    res = run_step(w, g, lb.Schedule("dynamic", num_workers=3), cfg=fp8_cfg(w, g, out_scale))
    assert res["error"] == 0
    h = host_step_inputs(inp)
    pro = oracle.prologue(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                          h["block_table"], theta=w.rope_theta, eps=w.rms_eps,
                          kv_dtype=kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    # the value attention reads back for the one row: the stored v, decoded
    v = oracle.step.decode_values(pro["v_store"], kv_dtype, w.v_scale)       # [B, Hkv, D]
    want = oracle.encode_output(np.repeat(v, 8, axis=1), "fp8", out_scale)   # [B, Hq, D]
    got = res["out"].cpu().numpy()
    assert np.array_equal(got, want), int((got != want).sum())
    if out_scale <= 2.0 ** -8:                        # |v| > 1.75 (BF16) or > 0.875 (FP8)
        assert np.any((want & 0x7F) == 0x7E)          # saturated codes were exercised


CASES = [
    dict(seq_lens=[65, 1000, 4097, 3], num_q_heads=64, num_kv_heads=8),
    dict(seq_lens=[2000, 70, 129], num_q_heads=16, num_kv_heads=2, kv_dtype="fp8"),
    dict(seq_lens=[130, 1500], num_q_heads=64, num_kv_heads=8, tokens=2),
    dict(seq_lens=[130, 1500, 66], num_q_heads=64, num_kv_heads=8, tokens=4,
         kv_dtype="fp8"),                                    # two blocks per wave
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("workers", [1, 5, 256])
def test_fp8_output_steps(case, workers):
    dev = device()
    w = wl.custom(seed=720 + case, **CASES[case])
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    out_scale = 2.0 ** -6 * 1.37          # not a power of two: the general path
    g = to_device(inp, dev)
    sched = lb.Schedule("dynamic", num_workers=workers)
    res = run_step(w, g, sched, cfg=fp8_cfg(w, g, out_scale))
    assert res["error"] == 0
    _, ro, rl = oracle_step(w, inp)
    err = check_output_fp8(res["out"].cpu().numpy(), ro, w.kv_dtype, out_scale)
    lse = to_f64(res["lse"])
    assert np.all(np.abs(lse - rl) <= 1e-4 + 1e-5 * np.abs(rl))
    # the same step with a BF16 output gives the same lse, bit for bit
    g2 = to_device(inp, dev)
    res2 = run_step(w, g2, sched)
    assert torch.equal(res["lse"], res2["lse"])
    print(f"fp8 out case {case}, {workers} workers: max err {err:.3e}", flush=True)


@pytest.mark.slow
def test_full_mix_fp8_output():
    dev = device()
    w = wl.named("mix")
    g = wl.make_inputs(w, device=dev)
    out_scale = 2.0 ** -7
    res = run_step(w, g, lb.Schedule("dynamic"), cfg=fp8_cfg(w, g, out_scale))
    assert res["error"] == 0
    h = host_step_inputs(g)
    pro = oracle.prologue(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                          h["block_table"], theta=w.rope_theta, eps=w.rms_eps,
                          kv_dtype=w.kv_dtype)
    seqs = [0, 7, 31]
    kp, vp, bt, pmap = compact_pools(g, w, seqs)
    ref = oracle.decode_attention(pro["q_out"], (kp, vp), remap_slots(pro, pmap), h["seq_lens"],
                                  bt, oracle_cfg(g, w), seqs=seqs, heads=list(range(64)))
    out = res["out"].cpu().numpy()
    for (b, hh), (o, l) in ref.items():
        check_output_fp8(out[b, hh], o, "bf16", out_scale, f"seq {b} head {hh}")
