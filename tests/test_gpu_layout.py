"""A cache in another layout against the fp64 oracle: each (page, KV head)'s V
tile right after its K tile in one device allocation (head stride two tiles,
page stride 2 Hkv tiles; k_cache and v_cache are views one tile apart, so the
prologue's K and V writes land in the same buffer).  Decode (one and several
new tokens, both caches, both schedules), prefill through each way the
prefill kernel stages its tiles (BF16 by global-to-LDS loads, FP8 converted
in registers, FP8 codes for FP8 scores) and a ragged prefill.  Every element
the step must not read (unowned tiles, rows past each length, the new
tokens' own slots) holds NaN beforehand; the oracle reads a host copy taken
before the step."""

import numpy as np
import pytest
import torch

import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import check_output, poison_cache, to_f64, bits_u16, fp8_lse_slack_for
from gpu_util import device, run_step, config_for
from test_gpu_step import oracle_step
from test_gpu_prefill import run_prefill, oracle_prefill
from test_gpu_varlen import run_varlen, oracle_varlen, check_against

pytestmark = pytest.mark.gpu


def interleaved_inputs(w, dev):
    """Inputs on the device in the interleaved layout (NaN where nothing may be
    read), and a host copy of them for the oracle."""
    g = wl.make_inputs(w, device=dev, kv_interleave=True)
    assert g["k_cache"].untyped_storage().data_ptr() == g["v_cache"].untyped_storage().data_ptr()
    poison_cache(g, w)
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in g.items()}
    return g, host


def check_lse(got, ref, slack=0.0):
    got = to_f64(got).reshape(ref.shape)
    assert np.all(np.abs(got - ref) <= 1e-4 + 1e-5 * np.abs(ref) + slack), \
        float(np.max(np.abs(got - ref)))


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tokens", [1, 4])
@pytest.mark.parametrize("kind", ["dynamic", "static"])
def test_decode_interleaved(kv_dtype, tokens, kind):
    dev = device()
    w = wl.custom([3000, 130, 64, 4, 700], num_q_heads=64, num_kv_heads=8, kv_dtype=kv_dtype,
                  seed=1200 + tokens, tokens=tokens)
    g, host = interleaved_inputs(w, dev)
    print(f"interleaved decode: {kv_dtype}, {tokens} new tokens, {kind}", flush=True)
    res = run_step(w, g, lb.Schedule(kind, num_workers=256))
    assert res["error"] == 0
    pro, ro, rl = oracle_step(w, host)
    assert np.array_equal(bits_u16(res["q_out"]).reshape(-1), pro["q_out"].reshape(-1))
    check_output(to_f64(res["out"]).reshape(ro.shape), ro, kv_dtype, "interleaved decode output")
    check_lse(res["lse"], rl)


@pytest.mark.parametrize("kv_dtype,qk", [("bf16", "bf16"), ("fp8", "bf16"), ("fp8", "fp8")])
def test_prefill_interleaved(kv_dtype, qk):
    dev = device()
    w = wl.custom([200, 333, 65], num_q_heads=64, num_kv_heads=8, kv_dtype=kv_dtype,
                  seed=1210, tokens=65)
    g, host = interleaved_inputs(w, dev)
    cfg = config_for(w, g)
    extra = None
    if qk == "fp8":
        cfg.qk_dtype, cfg.q_scale = "fp8", 2.0 ** -5
        extra = {"qk_dtype": "fp8", "q_scale": 2.0 ** -5}
    print(f"interleaved prefill: {kv_dtype} cache, {qk} scores", flush=True)
    res = run_prefill(w, g, cfg)
    assert res["error"] == 0
    pro, ro, rl = oracle_prefill(w, host, extra)
    assert np.array_equal(bits_u16(res["q_out"]).reshape(-1), pro["q_out"].reshape(-1))
    check_output(to_f64(res["out"]).reshape(ro.shape), ro, kv_dtype, "interleaved prefill output")
    slack = 0.0
    if qk == "fp8":
        slack = fp8_lse_slack_for(host, w, pro, 2.0 ** -5,
                                  np.repeat(np.arange(w.batch), w.tokens)).reshape(rl.shape)
    check_lse(res["lse"], rl, slack)


def test_ragged_prefill_interleaved():
    dev = device()
    w = wl.custom([300, 5, 1200, 64], num_q_heads=64, num_kv_heads=8, seed=1220,
                  new_tokens=[300, 0, 33, 1])
    g, host = interleaved_inputs(w, dev)
    print("interleaved ragged prefill", flush=True)
    res = run_varlen(w, g)
    assert res["error"] == 0
    pro, ref = oracle_varlen(w, host)
    assert np.array_equal(bits_u16(res["q_out"]), pro["q_out"])
    check_against(w, res, ref)
