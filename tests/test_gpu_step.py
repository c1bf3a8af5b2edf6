"""Whole decode steps through lbsr_decode_step vs the fp64 oracle, at sizes
the oracle finishes in seconds, plus the invariants the method has."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import multitoken as mt
import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import (poison_cache, host_pools, host_step_inputs, oracle_cfg, check_output,
                    to_f64, bits_u16)
from gpu_util import device, to_device, run_step

pytestmark = pytest.mark.gpu


def oracle_step(w, inp, extra=None):
    """The oracle's step; outputs [B, Hq, D] / [B, Hq], or [B, Tq, Hq, D] /
    [B, Tq, Hq] with several new tokens per sequence.  extra: more oracle cfg
    entries (e.g. the FP8 Q.K^T reading's qk_dtype and q_scale)."""
    h = host_step_inputs(inp)
    pools = host_pools(inp, w)
    kw = dict(theta=w.rope_theta, eps=w.rms_eps, kv_dtype=w.kv_dtype,
              k_scale=np.float32(w.k_scale).item(), v_scale=np.float32(w.v_scale).item(),
              norm_before_rope=w.norm_before_rope)
    cfg = oracle_cfg(inp, w)
    cfg["k_scale"] = np.float32(w.k_scale).item()
    cfg["v_scale"] = np.float32(w.v_scale).item()
    cfg.update(extra or {})
    B, Hq, Tq = w.batch, w.num_q_heads, w.tokens
    if Tq == 1:
        pro = oracle.prologue(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                              h["block_table"], **kw)
        ref = oracle.decode_attention(pro["q_out"], pools, pro, h["seq_lens"], h["block_table"],
                                      cfg)
        o = np.stack([np.stack([ref[(b, hh)][0] for hh in range(Hq)]) for b in range(B)])
        lse = np.array([[ref[(b, hh)][1] for hh in range(Hq)] for b in range(B)])
        return pro, o, lse
    pro = mt.prologue_tokens(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                             h["block_table"], **kw)
    q_out = pro["q_out"].reshape(B, Tq, Hq, 128)
    ref = mt.decode_attention_tokens(q_out, pools, pro, h["seq_lens"], h["block_table"], cfg)
    o = np.array([[[ref[(b, j, hh)][0] for hh in range(Hq)] for j in range(Tq)] for b in range(B)])
    lse = np.array([[[ref[(b, j, hh)][1] for hh in range(Hq)] for j in range(Tq)]
                    for b in range(B)])
    return pro, o, lse


def check_step(w, sched, seed_note=""):
    dev = device()
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    print(f"step: lens {w.seq_lens[:8]}{'...' if w.batch > 8 else ''} B={w.batch} "
          f"{w.num_q_heads}q/{w.num_kv_heads}kv {w.kv_dtype} tokens {w.tokens} {sched} "
          f"{seed_note}", flush=True)
    g = to_device(inp, dev)
    res = run_step(w, g, sched)
    pro, ro, rl = oracle_step(w, inp)
    assert res["error"] == 0
    max_abs, rel = check_output(to_f64(res["out"]), ro, w.kv_dtype, "attention output")
    lse = to_f64(res["lse"])
    assert np.all(np.abs(lse - rl) <= 1e-4 + 1e-5 * np.abs(rl)), float(np.max(np.abs(lse - rl)))
    return res, ro, rl


SMALL = [
    dict(seq_lens=[1, 63, 64, 200], num_q_heads=8, num_kv_heads=1),           # the tiny shape
    dict(seq_lens=[65, 128, 129, 1000, 1, 4097], num_q_heads=64, num_kv_heads=8),
    dict(seq_lens=[2000, 3, 700], num_q_heads=16, num_kv_heads=2, kv_dtype="fp8"),
    dict(seq_lens=[1, 1, 1, 64, 64], num_q_heads=8, num_kv_heads=2, kv_dtype="fp8"),
    dict(seq_lens=[513, 31, 8191], num_q_heads=32, num_kv_heads=4, norm_before_rope=True),
    dict(seq_lens=[300, 5], num_q_heads=12, num_kv_heads=3),                   # group 4
    dict(seq_lens=[900, 70], num_q_heads=32, num_kv_heads=2),                  # group 16
    dict(seq_lens=[1500, 2], num_q_heads=80, num_kv_heads=10, kv_dtype="fp8"), # > 8 KV heads
]
SCHEDS = [lb.Schedule("dynamic", num_workers=1), lb.Schedule("dynamic", num_workers=5),
          lb.Schedule("dynamic", num_workers=256), lb.Schedule("static", num_workers=256),
          lb.Schedule("static", num_workers=8, static_splits=3),
          lb.Schedule("dynamic", num_workers=256, xcd_weights=(9, 10, 9, 10, 9, 10, 9, 10)),
          lb.Schedule("dynamic", num_workers=13, xcd_weights=(1, 5, 2, 9, 1, 1, 7, 3))]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("si", range(len(SCHEDS)))
def test_small_steps(case, si):
    w = wl.custom(seed=200 + case, **SMALL[case])
    check_step(w, SCHEDS[si])


# Several new tokens per sequence (multi-token decode).  Lengths 64k + 1 and
# 64k + 2 leave the last tile with fewer rows than new tokens, so with many
# workers the last chunk holds no row of the early tokens (empty partials).
MULTI = [
    dict(seq_lens=[2, 65, 129, 1000, 4097], num_q_heads=64, num_kv_heads=8, tokens=2),
    dict(seq_lens=[4, 66, 700, 130], num_q_heads=16, num_kv_heads=4, tokens=4, kv_dtype="fp8"),
    dict(seq_lens=[3, 2000, 193], num_q_heads=8, num_kv_heads=2, tokens=3),
    dict(seq_lens=[16, 64 * 9 + 1], num_q_heads=8, num_kv_heads=8, tokens=16),   # group 1
    dict(seq_lens=[300, 65], num_q_heads=32, num_kv_heads=4, tokens=2, norm_before_rope=True,
         kv_dtype="fp8"),
    # 17 to 32 columns per KV head: both blocks of 16 on the head's wave, one
    # accumulator parked in LDS; lockstep with 8 and 16 KV heads, not with 12
    dict(seq_lens=[5, 66, 1000, 131], num_q_heads=64, num_kv_heads=8, tokens=4),        # 32
    dict(seq_lens=[3, 700, 64 * 3 + 2], num_q_heads=8, num_kv_heads=1, tokens=3),       # 24
    dict(seq_lens=[5, 66, 1000, 64 * 20 + 1], num_q_heads=64, num_kv_heads=8, tokens=4,
         kv_dtype="fp8"),                                                                # 32
    dict(seq_lens=[17, 64 * 7 + 2, 2500], num_q_heads=32, num_kv_heads=16, tokens=16),  # 32
    dict(seq_lens=[9, 800, 64 * 4 + 1], num_q_heads=36, num_kv_heads=12, tokens=8),     # 24
    # more: blocks of 16 on neighbouring waves
    dict(seq_lens=[8, 520, 2000], num_q_heads=16, num_kv_heads=2, tokens=8, kv_dtype="fp8"),  # 64
    dict(seq_lens=[40, 300], num_q_heads=12, num_kv_heads=4, tokens=11),               # 33
]
MULTI_SCHEDS = [lb.Schedule("dynamic", num_workers=1), lb.Schedule("dynamic", num_workers=7),
                lb.Schedule("dynamic", num_workers=256), lb.Schedule("static", num_workers=256),
                lb.Schedule("dynamic", num_workers=256, xcd_weights=(9, 10, 9, 10, 9, 10, 9, 10))]


@pytest.mark.parametrize("case", range(len(MULTI)))
@pytest.mark.parametrize("si", range(len(MULTI_SCHEDS)))
def test_multi_token_steps(case, si):
    w = wl.custom(seed=600 + case, **MULTI[case])
    res, ro, rl = check_step(w, MULTI_SCHEDS[si])
    assert res["out"].shape == (w.batch, w.tokens, w.num_q_heads, 128)


def test_multi_token_last_token_matches_one_token_step():
    """The last new token attends the whole sequence: its output equals a
    one-token step's on the same cache contents and query."""
    dev = device()
    w = wl.custom([1000, 65, 4100], num_q_heads=64, num_kv_heads=8, tokens=2, seed=650)
    inp = wl.make_inputs(w)
    g = to_device(inp, dev)
    r2 = run_step(w, g, lb.Schedule("dynamic", num_workers=256))
    # the one-token step over the caches the first step wrote, with the last
    # token's inputs: its prologue rewrites that token's slot with the same bits
    w1 = wl.custom([1000, 65, 4100], num_q_heads=64, num_kv_heads=8, seed=650)
    g1 = dict(g)
    for key in ("q", "k", "v"):
        g1[key] = g[key][:, 1].contiguous()
    g1["positions"] = g["positions"][:, 1].contiguous()
    r1 = run_step(w1, g1, lb.Schedule("dynamic", num_workers=256))
    assert torch.equal(r1["q_out"], r2["q_out"][:, 1])
    d = (r1["out"].float() - r2["out"][:, 1].float()).abs().max().item()
    assert d <= 2 ** -7, d                  # same math, other chunk boundaries in P.V rounding
    assert (r1["lse"] - r2["lse"][:, 1]).abs().max().item() < 1e-5


def test_tiny_named_workload():
    check_step(wl.named("tiny"), lb.Schedule("dynamic", num_workers=3))


def test_random_small_batches():
    rng = np.random.default_rng(7)
    for i in range(12):
        B = int(rng.integers(1, 9))
        lens = rng.integers(1, 3000, B).tolist()
        hkv = int(rng.choice([1, 2, 8]))
        w = wl.custom(lens, num_q_heads=8 * hkv, num_kv_heads=hkv,
                      kv_dtype=str(rng.choice(["bf16", "fp8"])), seed=300 + i)
        check_step(w, lb.Schedule("dynamic", num_workers=int(rng.integers(1, 40))), f"iter {i}")


def test_single_token_returns_v_exactly():
    dev = device()
    w = wl.custom([1, 1, 1], num_q_heads=64, num_kv_heads=8, seed=11)
    inp = wl.make_inputs(w)
    g = to_device(inp, dev)
    res = run_step(w, g, lb.Schedule("dynamic", num_workers=4))
    v = bits_u16(inp["v"])                                      # [B, Hkv, D]
    got = bits_u16(res["out"]).reshape(3, 8, 8, 128)            # [B, Hkv, G, D]
    assert np.array_equal(got, np.broadcast_to(v[:, :, None, :], got.shape))


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_zero_query_gives_log_length(kv_dtype):
    """q-norm weight 0 makes every score 0: lse = ln L exactly in exact arithmetic;
    a dropped or repeated 64-token tile would move it by >= ln(1 + 64/L)."""
    dev = device()
    lens = [1, 64, 65, 4096, 40000]
    w = wl.custom(lens, num_q_heads=16, num_kv_heads=2, kv_dtype=kv_dtype, seed=12)
    inp = wl.make_inputs(w)
    inp["q_norm_w"].zero_()
    g = to_device(inp, dev)
    for sched in (lb.Schedule("dynamic", num_workers=7), lb.Schedule("static", num_workers=64)):
        res = run_step(w, g, sched)
        lse = to_f64(res["lse"])
        want = np.log(np.asarray(lens, dtype=np.float64))[:, None]
        assert np.all(np.abs(lse - want) <= 16 * np.finfo(np.float32).eps * np.maximum(want, 1))


def test_page_relabelling_is_bit_identical():
    dev = device()
    w = wl.custom([3000, 130, 64], num_q_heads=16, num_kv_heads=2, seed=13)
    inp = wl.make_inputs(w)
    g1 = to_device(inp, dev)
    r1 = run_step(w, g1, lb.Schedule("dynamic", num_workers=6))
    n, ps = inp["num_pages"], inp["page_stride"]
    perm = torch.from_numpy(np.random.default_rng(1).permutation(n)).to(dev)
    g2 = to_device(inp, dev)
    for key in ("k_cache", "v_cache"):
        moved = torch.empty_like(g2[key]).view(n, ps)
        moved[perm] = g2[key].view(n, ps)
        g2[key] = moved.view(-1)
    bt = g2["block_table"].clone()
    mask = bt >= 0
    bt[mask] = perm[bt[mask].long()].to(torch.int32)
    g2["block_table"] = bt
    r2 = run_step(w, g2, lb.Schedule("dynamic", num_workers=6))
    assert torch.equal(r1["out"], r2["out"]) and torch.equal(r1["lse"], r2["lse"])


def test_dynamic_and_static_agree():
    dev = device()
    w = wl.custom([20000, 300, 4096, 1], num_q_heads=64, num_kv_heads=8, seed=14)
    inp = wl.make_inputs(w)
    rd = run_step(w, to_device(inp, dev), lb.Schedule("dynamic", num_workers=256))
    rs = run_step(w, to_device(inp, dev), lb.Schedule("static", num_workers=256))
    ld, ls = to_f64(rd["lse"]), to_f64(rs["lse"])
    assert np.max(np.abs(ld - ls)) <= 1e-5 * max(1.0, np.max(np.abs(ld)))
    od, os_ = to_f64(rd["out"]), to_f64(rs["out"])
    # The probabilities enter P.V as BF16, rounded after subtracting each chunk's
    # own running max, so the two schedules differ by that rounding (2^-9 relative
    # per term, averaging out over a row), plus the final BF16 rounding.
    assert np.all(np.abs(od - os_) <= 2.0 ** -7 * np.abs(od) + 5e-4)
    assert np.linalg.norm(od - os_) <= 2e-3 * np.linalg.norm(od)


def test_repeat_runs_are_bit_identical():
    dev = device()
    w = wl.custom([5000, 77, 129], num_q_heads=64, num_kv_heads=8, kv_dtype="fp8", seed=15)
    inp = wl.make_inputs(w)
    g = to_device(inp, dev)
    r1 = run_step(w, g, lb.Schedule("dynamic", num_workers=256))
    r2 = run_step(w, g, lb.Schedule("dynamic", num_workers=256))   # idempotent re-run
    assert torch.equal(r1["out"], r2["out"]) and torch.equal(r1["lse"], r2["lse"])


def test_bad_inputs_are_flagged_not_faulted():
    dev = device()
    w = wl.custom([100, 70], num_q_heads=8, num_kv_heads=1, seed=16)
    inp = wl.make_inputs(w)
    inp["block_table"][0, 0] = -5
    g = to_device(inp, dev)
    res = run_step(w, g, lb.Schedule("dynamic", num_workers=2))
    assert res["error"] == lb._binding.DEV_ERR_PAGE
    # a position past the block table: the fused prologue reports it through the step
    inp = wl.make_inputs(w)
    inp["positions"][1] = 10_000
    res = run_step(w, to_device(inp, dev), lb.Schedule("dynamic", num_workers=2))
    assert res["error"] == lb._binding.DEV_ERR_POSITION
    # and a clean step afterwards on the same inputs reports nothing
    res = run_step(w, to_device(wl.make_inputs(w), dev), lb.Schedule("dynamic", num_workers=2))
    assert res["error"] == 0


def test_worker_trace_records_every_worker():
    dev = device()
    w = wl.custom([3000, 130, 64, 9000], num_q_heads=64, num_kv_heads=8, seed=17)
    g = to_device(wl.make_inputs(w), dev)
    from gpu_util import config_for
    cfg = config_for(w, g)
    sched = lb.Schedule("dynamic", num_workers=37)
    ws = lb.alloc_workspace(cfg, w.batch, sched, device=dev)
    q_out, out = torch.empty_like(g["q"]), torch.empty_like(g["q"])
    tr = torch.zeros(37, 4, dtype=torch.int64, device=dev)
    ms = lb.decode_step_timed(cfg, g["q"], g["k"], g["v"], g["positions"], g["seq_lens"],
                              g["q_norm_w"], g["k_norm_w"], g["block_table"], g["k_cache"],
                              g["v_cache"], q_out, sched, ws, out, None, trace=tr)
    t = tr.cpu().numpy()
    assert len(ms) == 3 and all(x > 0 for x in ms)
    assert np.all(t[:, 0] > 0) and np.all(t[:, 1] >= t[:, 0])
    # the split kernel's span, in the 100 MHz clock, fits inside its event time
    span_us = (t[:, 1].max() - t[:, 0].min()) / 100.0
    assert span_us <= ms[1] * 1e3 * 1.5 + 5
