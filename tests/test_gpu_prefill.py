"""Prefill and chunked prefill (lbsr_prefill_step) against the fp64 oracle:
every new token attends its causal prefix (R20's reading, with any number of
new tokens).  q_out is bit-exact; outputs and lse to the R14 tolerance."""

import numpy as np
import pytest
import torch

from oracle import multitoken as mt, attend_full, bf16_bits_to_f64
from oracle.step import _sequence_kv
import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import (check_output, check_output_fp8, poison_cache, host_pools, host_step_inputs,
                    oracle_cfg, to_f64, bits_u16)
from gpu_util import device, to_device, config_for, run_step

pytestmark = pytest.mark.gpu


def run_prefill(w, g, cfg=None, sorted_list=True):
    """lbsr_prefill_step; sorted_list: with a workspace (the longest-first work
    list), else the workspace-free grid."""
    dev = g["q"].device
    cfg = cfg or config_for(w, g)
    q_out = torch.empty_like(g["q"])
    out = torch.empty(g["q"].shape, dtype=cfg.out_torch_dtype, device=dev)
    lse = torch.empty(cfg.tokens_shape(w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = (lb.alloc_prefill_workspace(cfg, w.batch, w.batch * w.tokens, device=dev)
          if sorted_list else None)
    lb.prefill_step(cfg, g["q"], g["k"], g["v"], g["positions"], g["seq_lens"], g["q_norm_w"],
                    g["k_norm_w"], g["block_table"], g["k_cache"], g["v_cache"], q_out, out,
                    lse, err, workspace=ws)
    torch.cuda.synchronize()
    return {"q_out": q_out, "out": out, "lse": lse, "error": int(err.item()), "cfg": cfg}


def oracle_prefill(w, inp, extra=None):
    h = host_step_inputs(inp)
    B, Tq, Hq = w.batch, w.tokens, w.num_q_heads
    q = h["q"].reshape(B, Tq, Hq, 128)
    k = h["k"].reshape(B, Tq, w.num_kv_heads, 128)
    v = h["v"].reshape(B, Tq, w.num_kv_heads, 128)
    pos = h["positions"].reshape(B, Tq)
    pro = mt.prologue_tokens(q, k, v, pos, h["wq"], h["wk"], h["block_table"],
                             theta=w.rope_theta, eps=w.rms_eps, kv_dtype=w.kv_dtype,
                             k_scale=np.float32(w.k_scale).item(),
                             v_scale=np.float32(w.v_scale).item(),
                             norm_before_rope=w.norm_before_rope)
    cfg = oracle_cfg(inp, w)
    cfg["k_scale"], cfg["v_scale"] = np.float32(w.k_scale).item(), np.float32(w.v_scale).item()
    cfg.update(extra or {})
    q_out = pro["q_out"].reshape(B, Tq, Hq, 128)
    ref = mt.decode_attention_tokens(q_out, host_pools(inp, w), pro, h["seq_lens"],
                                     h["block_table"], cfg)
    o = np.array([[[ref[(b, j, hh)][0] for hh in range(Hq)] for j in range(Tq)] for b in range(B)])
    lse = np.array([[[ref[(b, j, hh)][1] for hh in range(Hq)] for j in range(Tq)]
                    for b in range(B)])
    return pro, o, lse


CASES = [
    dict(seq_lens=[100, 300], num_q_heads=64, num_kv_heads=8, tokens=100),        # prefill + chunk
    dict(seq_lens=[37, 500, 1000], num_q_heads=64, num_kv_heads=8, tokens=37),    # partial block
    dict(seq_lens=[300, 2000], num_q_heads=8, num_kv_heads=8, tokens=300),         # group 1
    dict(seq_lens=[65, 129, 4096], num_q_heads=16, num_kv_heads=4, tokens=65, kv_dtype="fp8"),
    dict(seq_lens=[50, 700], num_q_heads=32, num_kv_heads=2, tokens=50),           # group 16
    dict(seq_lens=[90, 91], num_q_heads=12, num_kv_heads=4, tokens=90, norm_before_rope=True),
    dict(seq_lens=[1, 64, 65], num_q_heads=8, num_kv_heads=1, tokens=1),           # one token
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_matches_oracle(case):
    dev = device()
    w = wl.custom(seed=800 + case, **CASES[case])
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    print(f"prefill case {case}: lens {w.seq_lens} tokens {w.tokens} "
          f"{w.num_q_heads}q/{w.num_kv_heads}kv {w.kv_dtype}", flush=True)
    res = run_prefill(w, to_device(inp, dev))
    assert res["error"] == 0
    pro, ro, rl = oracle_prefill(w, inp)
    assert np.array_equal(bits_u16(res["q_out"]).reshape(pro["q_out"].shape), pro["q_out"])
    check_output(to_f64(res["out"]).reshape(ro.shape), ro, w.kv_dtype, "prefill output")
    lse = to_f64(res["lse"]).reshape(rl.shape)
    assert np.all(np.abs(lse - rl) <= 1e-4 + 1e-5 * np.abs(rl)), float(np.max(np.abs(lse - rl)))


@pytest.mark.parametrize("case", [0, 1, 3])
def test_workspace_free_grid_is_bit_identical(case):
    """Without a workspace the blocks run in another order, on the same
    arithmetic: outputs, lse and q_out are identical bit for bit."""
    dev = device()
    w = wl.custom(seed=800 + case, **CASES[case])
    inp = wl.make_inputs(w)
    a = run_prefill(w, to_device(inp, dev), sorted_list=True)
    b = run_prefill(w, to_device(inp, dev), sorted_list=False)
    for key in ("q_out", "out", "lse"):
        assert torch.equal(a[key], b[key]), key


def test_prefill_agrees_with_decode_path():
    """With few new tokens both paths apply; they agree to fp32 reassociation
    (the decode path splits the KV range into chunks and merges them)."""
    dev = device()
    w = wl.custom([70, 4100, 700], num_q_heads=64, num_kv_heads=8, tokens=8, seed=820)
    inp = wl.make_inputs(w)
    rp = run_prefill(w, to_device(inp, dev))
    rd = run_step(w, to_device(inp, dev), lb.Schedule("dynamic", num_workers=256))
    assert torch.equal(rp["q_out"], rd["q_out"])
    d = (rp["out"].float() - rd["out"].float()).abs().max().item()
    assert d <= 2 ** -6, d
    assert (rp["lse"] - rd["lse"]).abs().max().item() < 1e-4


def test_prefill_fp8_output():
    dev = device()
    w = wl.custom([200, 333], num_q_heads=64, num_kv_heads=8, tokens=200, seed=830)
    inp = wl.make_inputs(w)
    g = to_device(inp, dev)
    cfg = config_for(w, g)
    cfg.out_dtype, cfg.out_scale = "fp8", 2.0 ** -6 * 1.21
    res = run_prefill(w, g, cfg)
    _, ro, _ = oracle_prefill(w, inp)
    check_output_fp8(res["out"].cpu().numpy(), ro, "bf16", cfg.out_scale)


def test_prefill_flags_short_length():
    """A length below the new-token count is clamped up and flagged, not faulted."""
    dev = device()
    w = wl.custom([40, 90], num_q_heads=8, num_kv_heads=1, tokens=40, seed=840)
    g = to_device(wl.make_inputs(w), dev)
    g["seq_lens"][0] = 3
    res = run_prefill(w, g)
    assert res["error"] & lb._binding.DEV_ERR_SEQ_LEN


@pytest.mark.slow
@pytest.mark.parametrize("name", [n for n in wl.PREFILL_NAMES if not wl.named(n).varlen])
def test_prefill_full_size_sampled(name):
    """The benchmark's prefill workloads at full size: q_out of every token
    bit-exact on sampled sequences, outputs and lse of sampled (token, head)
    pairs against the oracle."""
    dev = device()
    w = wl.named(name)
    g = wl.make_inputs(w, device=dev)
    pools = host_pools(g, w)              # the caches before the step writes them
    print(f"prefill full size {name}", flush=True)
    res = run_prefill(w, g)
    assert res["error"] == 0
    h = host_step_inputs(g)
    B, Tq, Hq, Hkv = w.batch, w.tokens, w.num_q_heads, w.num_kv_heads
    seqs = [0, B - 1]
    pick = [0, 1, Tq // 2 - 1, Tq - 1]
    pos = h["positions"].reshape(B, Tq)[seqs]
    # prologue on every token of the sampled sequences (all their k/v rows are read)
    pro = mt.prologue_tokens(h["q"].reshape(B, Tq, Hq, 128)[seqs],
                             h["k"].reshape(B, Tq, Hkv, 128)[seqs],
                             h["v"].reshape(B, Tq, Hkv, 128)[seqs], pos, h["wq"], h["wk"],
                             h["block_table"][seqs], theta=w.rope_theta, eps=w.rms_eps,
                             kv_dtype=w.kv_dtype, k_scale=np.float32(w.k_scale).item(),
                             v_scale=np.float32(w.v_scale).item())
    q_out = pro["q_out"].reshape(len(seqs), Tq, Hq, 128)
    got_q = bits_u16(res["q_out"]).reshape(B, Tq, Hq, 128)
    assert np.array_equal(got_q[seqs], q_out)
    cfg = oracle_cfg(g, w)
    cfg["k_scale"], cfg["v_scale"] = np.float32(w.k_scale).item(), np.float32(w.v_scale).item()
    out, lse = to_f64(res["out"]), to_f64(res["lse"])
    lens = h["seq_lens"][seqs]
    for i, b in enumerate(seqs):
        for hh in (0, 9, 63):
            K, V = _sequence_kv(pools, pro, i, hh // (Hq // Hkv), lens, h["block_table"][seqs],
                                cfg)
            for j in pick:
                lim = mt.causal_limit(w.seq_lens[b], Tq, j)
                o_ref, l_ref = attend_full(bf16_bits_to_f64(q_out[i, j, [hh]]), K[:lim], V[:lim],
                                           cfg["sm_scale"])
                check_output(out[b, j, hh], o_ref[0], w.kv_dtype, f"seq {b} token {j} head {hh}")
                assert abs(lse[b, j, hh] - l_ref[0]) <= 1e-4 + 1e-5 * abs(l_ref[0])


@pytest.mark.slow
def test_prefill_longest_prompt():
    """One prompt at the 2^18-token maximum (4096 pages, 8 q / 1 KV head) beside a
    short one: q_out of sampled tokens bit-exact, sampled outputs and lse
    against the oracle (its prologue runs on every token: all k/v rows are read)."""
    dev = device()
    T = 1 << 18
    w = wl.custom([T, T], num_q_heads=8, num_kv_heads=1, tokens=T, seed=855)
    g = wl.make_inputs(w, device=dev)
    pools = host_pools(g, w)
    print("prefill 2 x 262144 tokens, 8q/1kv", flush=True)
    res = run_prefill(w, g)
    assert res["error"] == 0
    h = host_step_inputs(g)
    b = 0
    pro = mt.prologue_tokens(h["q"].reshape(2, T, 8, 128)[[b]], h["k"].reshape(2, T, 1, 128)[[b]],
                             h["v"].reshape(2, T, 1, 128)[[b]],
                             h["positions"].reshape(2, T)[[b]], h["wq"], h["wk"],
                             h["block_table"][[b]], theta=w.rope_theta, eps=w.rms_eps,
                             kv_dtype="bf16")
    q_out = pro["q_out"].reshape(1, T, 8, 128)
    got_q = bits_u16(res["q_out"]).reshape(2, T, 8, 128)
    pick = [0, 1, 4095, 65536, T // 2 + 7, T - 2, T - 1]
    assert np.array_equal(got_q[b, pick], q_out[0, pick])
    cfg = oracle_cfg(g, w)
    K, V = _sequence_kv(pools, pro, 0, 0, h["seq_lens"][[b]], h["block_table"][[b]], cfg)
    out, lse = to_f64(res["out"]), to_f64(res["lse"])
    for j in pick:
        lim = mt.causal_limit(T, T, j)
        o_ref, l_ref = attend_full(bf16_bits_to_f64(q_out[0, j]), K[:lim], V[:lim], cfg["sm_scale"])
        for hh in (0, 5, 7):
            check_output(out[b, j, hh], o_ref[hh], "bf16", f"token {j} head {hh}")
            assert abs(lse[b, j, hh] - l_ref[hh]) <= 1e-4 + 1e-5 * abs(l_ref[hh])
