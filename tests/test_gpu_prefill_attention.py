"""The attention-only prefill entry points (lbsr_prefill_attention and
lbsr_prefill_attention_varlen) on their own, against the fp64 oracle: q_out
and the caches holding the new tokens' k and v come from the oracle's
prologue (written into a host copy of the pools and uploaded), so these
calls are checked apart from the GPU prologue that the fused step runs
before them.  Each staging path of the prefill kernel (BF16 tiles, an FP8
cache with BF16 scores, FP8 scores), with the workspace's work list and
without it (the uniform call's grid)."""

import numpy as np
import pytest
import torch

import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from oracle.step import apply_prologue_writes
from checks import check_output, poison_cache, host_pools, to_f64, fp8_lse_slack_for
from gpu_util import device, config_for
from test_gpu_prefill import oracle_prefill
from test_gpu_varlen import oracle_varlen, check_against

pytestmark = pytest.mark.gpu

Q_SCALE = 2.0 ** -5


def device_inputs(w, inp, pro, dev):
    """q_out from the oracle's prologue bits; pools with its k/v writes applied."""
    kp, vp = (p.copy() for p in host_pools(inp, w))
    apply_prologue_writes(kp, vp, pro, kv_dtype=w.kv_dtype, page_stride=inp["page_stride"],
                          head_stride=inp["head_stride"])

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a.copy()).to(dev)

    q_out = up(np.ascontiguousarray(pro["q_out"], dtype=np.uint16))
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    g["k_cache"], g["v_cache"] = up(kp), up(vp)
    return q_out, g


def scores_cfg(w, g, qk):
    cfg = config_for(w, g)
    if qk == "fp8":
        cfg.qk_dtype, cfg.q_scale = "fp8", Q_SCALE
    return cfg, ({"qk_dtype": "fp8", "q_scale": Q_SCALE} if qk == "fp8" else None)


@pytest.mark.parametrize("kv_dtype,qk", [("bf16", "bf16"), ("fp8", "bf16"), ("fp8", "fp8")])
@pytest.mark.parametrize("listed", [True, False])
def test_prefill_attention_alone(kv_dtype, qk, listed):
    dev = device()
    w = wl.custom([300, 1000, 129], num_q_heads=64, num_kv_heads=8, kv_dtype=kv_dtype,
                  seed=1300, tokens=129)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    extra = {"qk_dtype": "fp8", "q_scale": Q_SCALE} if qk == "fp8" else None
    pro, ro, rl = oracle_prefill(w, inp, extra)
    q_out, g = device_inputs(w, inp, pro, dev)
    cfg, _ = scores_cfg(w, g, qk)
    q_out = q_out.reshape(cfg.tokens_shape(w.batch, w.num_q_heads, 128))
    out = torch.empty(q_out.shape, dtype=cfg.out_torch_dtype, device=dev)
    lse = torch.empty(cfg.tokens_shape(w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = lb.alloc_prefill_workspace(cfg, w.batch, w.batch * w.tokens, device=dev) if listed else None
    print(f"prefill attention alone: {kv_dtype} cache, {qk} scores, work list {listed}", flush=True)
    lb.prefill_attention(cfg, q_out, g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"],
                         out, lse, err, workspace=ws)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    check_output(to_f64(out).reshape(ro.shape), ro, kv_dtype, "prefill attention output")
    slack = 0.0
    if qk == "fp8":
        slack = fp8_lse_slack_for(inp, w, pro, Q_SCALE,
                                  np.repeat(np.arange(w.batch), w.tokens)).reshape(rl.shape)
    got = to_f64(lse).reshape(rl.shape)
    assert np.all(np.abs(got - rl) <= 1e-4 + 1e-5 * np.abs(rl) + slack), \
        float(np.max(np.abs(got - rl)))


@pytest.mark.parametrize("kv_dtype,qk", [("bf16", "bf16"), ("fp8", "bf16"), ("fp8", "fp8")])
def test_prefill_attention_varlen_alone(kv_dtype, qk):
    dev = device()
    w = wl.custom([300, 5, 1200, 64, 1], num_q_heads=64, num_kv_heads=8, kv_dtype=kv_dtype,
                  seed=1310, new_tokens=[300, 0, 33, 64, 1])
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    extra = {"qk_dtype": "fp8", "q_scale": Q_SCALE} if qk == "fp8" else None
    pro, ref = oracle_varlen(w, inp, extra=extra)
    q_out, g = device_inputs(w, inp, pro, dev)
    cfg, _ = scores_cfg(w, g, qk)
    total = q_out.shape[0]
    out = torch.empty(q_out.shape, dtype=cfg.out_torch_dtype, device=dev)
    lse = torch.empty(q_out.shape[:2], dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = lb.alloc_prefill_workspace(cfg, w.batch, total, device=dev)
    print(f"ragged prefill attention alone: {kv_dtype} cache, {qk} scores", flush=True)
    lb.prefill_attention_varlen(cfg, g["q_start"], q_out, g["k_cache"], g["v_cache"],
                                g["block_table"], g["seq_lens"], ws, out, lse, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    slack = None
    if qk == "fp8":
        slack = fp8_lse_slack_for(inp, w, pro, Q_SCALE, np.repeat(np.arange(w.batch), w.new_tokens))
    check_against(w, {"out": out, "lse": lse}, ref, slack)
