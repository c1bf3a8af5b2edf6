"""Full-size workloads, in the launch configuration the benchmark times
(dynamic over every CU, and the static baseline): the schedule bit-exact,
every new token's q_out, every head of sampled sequences (the longest,
shortest and median) against the fp64 oracle, and a zero-query run whose
lse must be ln L for every sequence."""

import numpy as np
import pytest
import torch

import oracle
from oracle import multitoken as mt
import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import (poison_cache, host_step_inputs, oracle_cfg, check_output, to_f64, bits_u16)
from gpu_util import device, run_step, compact_pools, remap_slots

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

FULL = ["uniform", "mix", "mix_fp8", "loguniform", "mix_mtp2", "mix_mtp4"]


def sampled_checks(w, g, res, h, pro):
    lens = np.asarray(w.seq_lens)
    order = np.argsort(lens)
    seqs = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2])})
    heads = list(range(w.num_q_heads))     # every q head, so every KV head is compared
    kp, vp, bt, pmap = compact_pools(g, w, seqs)
    cfg = oracle_cfg(g, w)
    pro_c = remap_slots(pro, pmap)
    out = to_f64(res["out"])
    lse = to_f64(res["lse"])
    if w.tokens == 1:
        ref = oracle.decode_attention(pro["q_out"], (kp, vp), pro_c, h["seq_lens"], bt, cfg,
                                      seqs=seqs, heads=heads)
        ref = {(b, 0, hh): v for (b, hh), v in ref.items()}
        out, lse = out[:, None], lse[:, None]
    else:
        q_out = pro["q_out"].reshape(w.batch, w.tokens, w.num_q_heads, 128)
        ref = mt.decode_attention_tokens(q_out, (kp, vp), pro_c, h["seq_lens"], bt, cfg,
                                         seqs=seqs, heads=heads)
    worst = 0.0
    for (b, j, hh), (o, l) in ref.items():
        _, rl2 = check_output(out[b, j, hh], o, w.kv_dtype, f"output seq {b} token {j} head {hh}")
        worst = max(worst, rl2)
        assert abs(lse[b, j, hh] - l) <= 1e-4 + 1e-5 * abs(l), (b, j, hh, lse[b, j, hh], l)
    print(f"    worst relative L2 over {len(ref)} heads: {worst:.2e}", flush=True)
    return len(ref)


@pytest.mark.parametrize("name", FULL)
def test_full_workload(name):
    dev = device()
    w = wl.named(name)
    print(f"full workload {name}: B={w.batch} {w.kv_dtype}, generating on device", flush=True)
    g = wl.make_inputs(w, device=dev)
    poison_cache(g, w, spare_pages=False)
    h = host_step_inputs(g)
    kw = dict(theta=w.rope_theta, eps=w.rms_eps, kv_dtype=w.kv_dtype, k_scale=w.k_scale,
              v_scale=w.v_scale)
    if w.tokens == 1:
        pro = oracle.prologue(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                              h["block_table"], **kw)
    else:
        pro = mt.prologue_tokens(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                                 h["block_table"], **kw)
    P = lb.device_workers(0)
    for sched in (lb.Schedule("dynamic"), lb.Schedule("static"),
                  lb.Schedule("dynamic", xcd_weights=(9, 10, 9, 10, 9, 10, 9, 10))):
        # the pools keep the pre-step contents the oracle reads: run on a copy
        gg = dict(g)
        gg["k_cache"], gg["v_cache"] = g["k_cache"].clone(), g["v_cache"].clone()
        res = run_step(w, gg, sched)
        assert res["error"] == 0
        ref_plan = (oracle.plan_dynamic(w.seq_lens, P, sched.xcd_weights)
                    if sched.kind == "dynamic"
                    else oracle.plan_static(w.seq_lens, max(1, P // w.batch)))
        got = res["plan"]
        for key in ("cu_tiles", "worker_chunk", "chunks", "seq_chunk"):
            assert np.array_equal(got[key], getattr(ref_plan, key)), key
        got_q = bits_u16(res["q_out"]).reshape(pro["q_out"].shape)
        assert np.array_equal(got_q, pro["q_out"]) or np.mean(got_q != pro["q_out"]) < 1e-6
        n = sampled_checks(w, gg, res, h, pro)
        print(f"  {sched}: plan exact, {n} sampled heads match", flush=True)
        del gg, res
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["mix", "mix_fp8", "loguniform", "mix_mtp2", "mix_mtp4"])
def test_full_zero_query_lse(name):
    """Every (sequence, head) at full size: with q = 0 the lse is ln of the
    number of rows attended (L, or L - Tq + j + 1 for new token j)."""
    dev = device()
    w = wl.named(name)
    g = wl.make_inputs(w, device=dev)
    g["q_norm_w"].zero_()
    res = run_step(w, g, lb.Schedule("dynamic"))
    lse = to_f64(res["lse"])
    lens = np.asarray(w.seq_lens, dtype=np.float64)
    if w.tokens == 1:
        want = np.log(lens)[:, None]
    else:
        want = np.log(lens[:, None] - w.tokens + np.arange(w.tokens)[None, :] + 1)[:, :, None]
    err = np.abs(lse - want)
    print(f"{name}: max |lse - ln L| = {err.max():.2e}", flush=True)
    assert np.all(err <= 16 * np.finfo(np.float32).eps * np.maximum(want, 1))
