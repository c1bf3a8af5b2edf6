"""The decode step that allocates nothing (lbsr_decode_step_noalloc), through
the C ABI: on three calls in a row -- the second with a smaller input, the
third larger again with the merge folded into the split launch -- its q_out,
cache writes, output and lse equal lbsr_decode_step's with a caller
workspace bit for bit, and meet the oracle's tolerance rule."""

import numpy as np
import pytest
import torch

import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import check_output, to_f64
from gpu_util import device, to_device, run_step, config_for
from test_gpu_step import oracle_step

pytestmark = pytest.mark.gpu

CALLS = [
    (dict(seq_lens=[5000, 77, 129, 64, 3000, 1], num_q_heads=64, num_kv_heads=8),
     lb.Schedule("dynamic", num_workers=256)),
    (dict(seq_lens=[200, 63, 1, 64], num_q_heads=8, num_kv_heads=1, kv_dtype="fp8"),
     lb.Schedule("static", num_workers=8)),
    (dict(seq_lens=[9000, 640, 65, 3], num_q_heads=32, num_kv_heads=4),
     lb.Schedule("dynamic", num_workers=100, fold_merge=True)),
]


def noalloc_step(w, g, sched):
    cfg = config_for(w, g)
    dev = g["q"].device
    q_out = torch.empty_like(g["q"])
    out = torch.empty(g["q"].shape, dtype=cfg.out_torch_dtype, device=dev)
    lse = torch.empty(cfg.tokens_shape(w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    lb.decode_step_noalloc(cfg, g["q"], g["k"], g["v"], g["positions"], g["seq_lens"],
                           g["q_norm_w"], g["k_norm_w"], g["block_table"], g["k_cache"],
                           g["v_cache"], q_out, sched, out, lse)
    torch.cuda.synchronize()
    return q_out, out, lse


def test_noalloc_step_matches_the_workspace_step():
    dev = device()
    for i, (kw, sched) in enumerate(CALLS):
        w = wl.custom(seed=400 + i, **kw)
        print(f"no-alloc call {i}: lengths {w.seq_lens}, {w.num_q_heads}q/{w.num_kv_heads}kv "
              f"{w.kv_dtype}, {sched}", flush=True)
        inp = wl.make_inputs(w)
        g_ref = to_device(inp, dev)
        ref = run_step(w, g_ref, sched)
        assert ref["error"] == 0
        g = to_device(inp, dev)
        q_out, out, lse = noalloc_step(w, g, sched)
        assert torch.equal(q_out, ref["q_out"])
        assert torch.equal(g["k_cache"], g_ref["k_cache"]) and torch.equal(g["v_cache"], g_ref["v_cache"])
        assert torch.equal(out, ref["out"]) and torch.equal(lse, ref["lse"])
        _, ro, rl = oracle_step(w, inp)
        check_output(to_f64(out), ro, w.kv_dtype, f"no-alloc call {i}")
        assert np.all(np.abs(to_f64(lse) - rl) <= 1e-4 + 1e-5 * np.abs(rl))
