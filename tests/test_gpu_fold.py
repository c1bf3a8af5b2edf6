"""The merge folded into the split-attention launch (LBSR_SCHED_FOLD_MERGE):
the same steps as the two-launch form against the fp64 oracle, at small
sizes under every schedule shape and at full size (sampled), plus error
reporting, determinism and the standalone lbsr_attention call."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import poison_cache, host_step_inputs, check_output, to_f64, bits_u16
from gpu_util import device, to_device, run_step, config_for
from test_gpu_step import SMALL, SCHEDS, check_step
from test_gpu_full import sampled_checks

pytestmark = pytest.mark.gpu


def folded(sched):
    return dataclasses.replace(sched, fold_merge=True)


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("si", range(len(SCHEDS)))
def test_small_steps_folded(case, si):
    w = wl.custom(seed=200 + case, **SMALL[case])
    check_step(w, folded(SCHEDS[si]), "folded merge")


@pytest.mark.parametrize("P", [3, 40, 256])
def test_more_kv_heads_than_waves_folded(P):
    """16 KV heads on 8 waves: two lockstep passes over each chunk, each with
    its own arrival counter."""
    w = wl.custom([3000, 70, 900, 129], num_q_heads=32, num_kv_heads=16, seed=25)
    check_step(w, lb.Schedule("dynamic", num_workers=P, fold_merge=True), "16 KV heads folded")
    w8 = wl.custom([2000, 65], num_q_heads=32, num_kv_heads=16, kv_dtype="fp8", seed=26)
    check_step(w8, lb.Schedule("static", num_workers=P, fold_merge=True), "16 KV heads static")


def test_random_small_batches_folded():
    rng = np.random.default_rng(77)
    for i in range(12):
        B = int(rng.integers(1, 9))
        lens = [int(x) for x in rng.integers(1, 3000, B)]
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2, 8]))
        w = wl.custom(lens, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                      kv_dtype=str(rng.choice(["bf16", "fp8"])), seed=300 + i)
        P = int(rng.integers(1, 300))
        check_step(w, lb.Schedule("dynamic", num_workers=P, fold_merge=True), f"P={P} folded")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mix", "mix_fp8", "uniform", "loguniform"])
def test_full_workload_folded(name):
    dev = device()
    w = wl.named(name)
    print(f"full workload {name} folded: B={w.batch} {w.kv_dtype}", flush=True)
    g = wl.make_inputs(w, device=dev)
    poison_cache(g, w, spare_pages=False)
    h = host_step_inputs(g)
    pro = oracle.prologue(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                          h["block_table"], theta=w.rope_theta, eps=w.rms_eps,
                          kv_dtype=w.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    res = run_step(w, g, lb.Schedule("dynamic", fold_merge=True))
    assert res["error"] == 0
    got_q = bits_u16(res["q_out"]).reshape(pro["q_out"].shape)
    assert np.array_equal(got_q, pro["q_out"]) or np.mean(got_q != pro["q_out"]) < 1e-6
    n = sampled_checks(w, g, res, h, pro)
    print(f"  {n} sampled heads match", flush=True)


def test_folded_matches_two_launches():
    """Both forms merge the same partials with the same weights; only the
    order of the additions differs."""
    dev = device()
    w = wl.custom([5000, 77, 129, 64, 3000], num_q_heads=64, num_kv_heads=8, seed=21)
    inp = wl.make_inputs(w)
    r2 = run_step(w, to_device(inp, dev), lb.Schedule("dynamic", num_workers=64))
    r1 = run_step(w, to_device(inp, dev), lb.Schedule("dynamic", num_workers=64, fold_merge=True))
    assert torch.equal(r1["q_out"], r2["q_out"])
    a, b = to_f64(r1["out"]), to_f64(r2["out"])
    assert np.max(np.abs(a - b)) <= 2 ** -7 * max(1.0, float(np.max(np.abs(b))))
    assert np.max(np.abs(to_f64(r1["lse"]) - to_f64(r2["lse"]))) <= 1e-5


def test_folded_repeat_runs_are_bit_identical():
    """Which wave merges a sequence varies from run to run; the result does not."""
    dev = device()
    w = wl.custom([9000, 77, 129, 4000], num_q_heads=64, num_kv_heads=8, kv_dtype="fp8", seed=22)
    g = to_device(wl.make_inputs(w), dev)
    sched = lb.Schedule("dynamic", num_workers=256, fold_merge=True)
    r1 = run_step(w, g, sched)
    outs = [run_step(w, g, sched) for _ in range(3)]   # idempotent re-runs
    for r in outs:
        assert torch.equal(r1["out"], r["out"]) and torch.equal(r1["lse"], r["lse"])


def test_folded_errors_are_reported():
    """Bad pages (split kernel) and bad positions (the prologue's per-token
    status, folded by the split launch) reach the error word."""
    dev = device()
    w = wl.custom([100, 70, 1000], num_q_heads=8, num_kv_heads=1, seed=23)
    sched = lb.Schedule("dynamic", num_workers=9, fold_merge=True)
    inp = wl.make_inputs(w)
    inp["block_table"][0, 0] = -5
    assert run_step(w, to_device(inp, dev), sched)["error"] == lb._binding.DEV_ERR_PAGE
    inp = wl.make_inputs(w)
    inp["positions"][2] = 10_000                      # a split sequence's token
    assert run_step(w, to_device(inp, dev), sched)["error"] == lb._binding.DEV_ERR_POSITION
    inp = wl.make_inputs(w)
    inp["positions"][1] = 10_000                      # a one-chunk sequence's token
    assert run_step(w, to_device(inp, dev), sched)["error"] == lb._binding.DEV_ERR_POSITION
    assert run_step(w, to_device(wl.make_inputs(w), dev), sched)["error"] == 0


def test_standalone_attention_folded():
    """lbsr_plan then lbsr_attention with the flag: one launch after the plan,
    the same outputs as the step's attention."""
    dev = device()
    w = wl.custom([3000, 1, 640, 65], num_q_heads=32, num_kv_heads=4, seed=24)
    inp = wl.make_inputs(w)
    g = to_device(inp, dev)
    cfg = config_for(w, g)
    sched = lb.Schedule("dynamic", num_workers=40, fold_merge=True)
    res = run_step(w, g, sched)            # writes the new tokens; q_out for the call below
    ws = lb.alloc_workspace(cfg, w.batch, sched, device=dev)
    out = torch.empty_like(res["out"])
    lse = torch.empty_like(res["lse"])
    lb.plan(cfg, g["seq_lens"], sched, ws)
    lb.attention(cfg, res["q_out"], g["k_cache"], g["v_cache"], g["block_table"], sched, ws, out,
                 lse)
    torch.cuda.synchronize()
    assert torch.equal(out, res["out"]) and torch.equal(lse, res["lse"])
    assert lb.read_error(cfg, w.batch, sched, ws) == 0


@pytest.mark.parametrize("lens,Hq,Hkv,kv_dtype", [
    ([65, 1000, 4097, 3], 64, 8, "bf16"),
    ([2000, 70, 129], 16, 2, "fp8"),
])
@pytest.mark.parametrize("workers", [5, 256])
def test_folded_fp8_output(lens, Hq, Hkv, kv_dtype, workers):
    """The folded merge writes E4M3 codes of o / out_scale like the merge kernel:
    within the tolerance plus half an E4M3 step of the oracle."""
    from checks import check_output_fp8
    from test_gpu_out_fp8 import fp8_cfg
    from test_gpu_step import oracle_step
    dev = device()
    w = wl.custom(lens, num_q_heads=Hq, num_kv_heads=Hkv, kv_dtype=kv_dtype, seed=27)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    out_scale = 2.0 ** -6 * 1.37
    g = to_device(inp, dev)
    res = run_step(w, g, lb.Schedule("dynamic", num_workers=workers, fold_merge=True),
                   cfg=fp8_cfg(w, g, out_scale))
    assert res["error"] == 0
    _, ro, rl = oracle_step(w, inp)
    check_output_fp8(res["out"].cpu().numpy(), ro, w.kv_dtype, out_scale)
    assert np.all(np.abs(to_f64(res["lse"]) - rl) <= 1e-4 + 1e-5 * np.abs(rl))


@pytest.mark.parametrize("Hq,Hkv", [(32, 4), (32, 16), (48, 12)])
def test_folded_plan_reused_by_two_attention_calls(Hq, Hkv):
    """One lbsr_plan, then lbsr_attention twice with the flag (as every layer
    of a step would reuse one plan): the arrival counters must start from zero
    again, so the second call merges its split sequences too.  Covers the
    lockstep kernels (4 and 16 KV heads, one counter per pass) and the
    per-wave form (12 KV heads on 8 waves)."""
    from test_gpu_step import oracle_step
    dev = device()
    w = wl.custom([3000, 1, 640, 65, 2500], num_q_heads=Hq, num_kv_heads=Hkv, seed=28)
    inp = wl.make_inputs(w)
    _, ro, rl = oracle_step(w, inp)
    g = to_device(inp, dev)
    cfg = config_for(w, g)
    sched = lb.Schedule("dynamic", num_workers=40, fold_merge=True)
    res = run_step(w, g, sched)            # writes the new tokens; q_out for the calls below
    check_output(to_f64(res["out"]), ro, w.kv_dtype, "step output")
    ws = lb.alloc_workspace(cfg, w.batch, sched, device=dev)
    lb.plan(cfg, g["seq_lens"], sched, ws)
    for call in range(2):
        out = torch.full_like(res["out"], float("nan"))
        lse = torch.full_like(res["lse"], float("nan"))
        lb.attention(cfg, res["q_out"], g["k_cache"], g["v_cache"], g["block_table"], sched, ws,
                     out, lse)
        torch.cuda.synchronize()
        check_output(to_f64(out), ro, w.kv_dtype, f"attention call {call}")
        assert np.all(np.abs(to_f64(lse) - rl) <= 1e-4 + 1e-5 * np.abs(rl)), call
        assert torch.equal(out, res["out"]) and torch.equal(lse, res["lse"]), call
    assert lb.read_error(cfg, w.batch, sched, ws) == 0
