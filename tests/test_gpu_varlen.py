"""Ragged (varlen) prefill against the fp64 oracle (R22): every sequence has
its own number of new tokens, packed along one token axis.

* prologue + attention of ragged batches (empty, one-token and long
  sequences; both caches; several head groups): q_out and cache bits exact,
  outputs and lse to the R14 tolerance;
* equal counts give bit-identical results to the uniform prefill call;
* a mixed batch: decoding sequences through the decode step, prompts through
  the ragged prefill, on one stream and one cache;
* malformed q_start ranges are flagged and skipped, not faulted.
"""

import numpy as np
import pytest
import torch

from oracle import multitoken as mt
import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import (check_output, poison_cache, host_pools, host_step_inputs, oracle_cfg, to_f64,
                    bits_u16)
from gpu_util import device, to_device, config_for, run_step

pytestmark = pytest.mark.gpu


def run_varlen(w, g, cfg=None, q_start=None, total=None):
    dev = g["q"].device
    cfg = cfg or config_for(w, g)
    q_out = torch.empty_like(g["q"])
    out = torch.zeros(g["q"].shape, dtype=cfg.out_torch_dtype, device=dev)
    lse = torch.zeros(g["q"].shape[:2], dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = lb.alloc_prefill_workspace(cfg, g["seq_lens"].shape[0], g["q"].shape[0], device=dev)
    lb.prefill_step_varlen(cfg, g["q_start"] if q_start is None else q_start, g["q"], g["k"],
                           g["v"], g["positions"], g["seq_lens"], g["q_norm_w"], g["k_norm_w"],
                           g["block_table"], g["k_cache"], g["v_cache"], q_out, ws, out, lse, err)
    torch.cuda.synchronize()
    return {"q_out": q_out, "out": out, "lse": lse, "error": int(err.item()), "cfg": cfg}


def oracle_varlen(w, inp, seqs=None, extra=None):
    h = host_step_inputs(inp)
    kw = dict(theta=w.rope_theta, eps=w.rms_eps, kv_dtype=w.kv_dtype,
              k_scale=np.float32(w.k_scale).item(), v_scale=np.float32(w.v_scale).item(),
              norm_before_rope=w.norm_before_rope)
    pro = mt.prologue_varlen(h["q"], h["k"], h["v"], h["positions"], w.new_tokens, h["wq"],
                             h["wk"], h["block_table"], **kw)
    cfg = oracle_cfg(inp, w)
    cfg["k_scale"], cfg["v_scale"] = kw["k_scale"], kw["v_scale"]
    cfg.update(extra or {})
    ref = mt.attention_varlen(pro["q_out"], host_pools(inp, w), pro, h["seq_lens"], w.new_tokens,
                              h["block_table"], cfg, seqs=seqs)
    return pro, ref


def check_against(w, res, ref, lse_slack=None):
    """res's output and lse rows against the oracle's; lse_slack [rows, Hq]: the
    FP8-score term added to lse's bound (R23), per packed row."""
    starts = mt.query_starts(w.new_tokens)
    out, lse = to_f64(res["out"]), to_f64(res["lse"])
    rows = sorted({(b, j) for (b, j, _) in ref})
    for b, j in rows:
        r = int(starts[b]) + j
        o_ref = np.stack([ref[(b, j, hh)][0] for hh in range(w.num_q_heads)])
        l_ref = np.array([ref[(b, j, hh)][1] for hh in range(w.num_q_heads)])
        check_output(out[r], o_ref, w.kv_dtype, f"seq {b} token {j}")
        slack = 0.0 if lse_slack is None else lse_slack[r]
        assert np.all(np.abs(lse[r] - l_ref) <= 1e-4 + 1e-5 * np.abs(l_ref) + slack), (b, j)


CASES = [
    dict(seq_lens=[300, 5, 700, 64, 1], new_tokens=[300, 0, 33, 1, 1]),         # G = 8
    dict(seq_lens=[65, 129, 4096, 20], new_tokens=[65, 100, 7, 20], kv_dtype="fp8"),
    dict(seq_lens=[50, 700, 640], num_q_heads=32, num_kv_heads=2, new_tokens=[50, 257, 640]),
    dict(seq_lens=[90, 91, 2], num_q_heads=12, num_kv_heads=4, new_tokens=[90, 3, 2],
         norm_before_rope=True),
    dict(seq_lens=[1, 64, 65, 500], num_q_heads=8, num_kv_heads=8, new_tokens=[1, 64, 0, 500]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_varlen_matches_oracle(case):
    dev = device()
    c = dict(CASES[case])
    c.setdefault("num_q_heads", 64)
    c.setdefault("num_kv_heads", 8)
    w = wl.custom(seed=860 + case, **c)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    print(f"varlen case {case}: lens {w.seq_lens} new {w.new_tokens} "
          f"{w.num_q_heads}q/{w.num_kv_heads}kv {w.kv_dtype}", flush=True)
    res = run_varlen(w, to_device(inp, dev))
    assert res["error"] == 0
    pro, ref = oracle_varlen(w, inp)
    assert np.array_equal(bits_u16(res["q_out"]), pro["q_out"])
    check_against(w, res, ref)


def test_equal_counts_match_uniform_call():
    """A ragged batch with every count = Tq runs the same kernels as the
    uniform call, on the same packed rows: results are bit-identical."""
    dev = device()
    lens, Tq = [300, 1000, 77], 77
    wv = wl.custom(lens, seed=870, new_tokens=[Tq] * 3)
    wu = wl.custom(lens, seed=870, tokens=Tq)
    gv, gu = to_device(wl.make_inputs(wv), dev), to_device(wl.make_inputs(wu), dev)
    assert torch.equal(gv["q"].view(3, Tq, 64, 128), gu["q"])
    rv = run_varlen(wv, gv)
    cfg = config_for(wu, gu)
    q_out, out = torch.empty_like(gu["q"]), torch.empty_like(gu["q"])
    lse = torch.empty(cfg.tokens_shape(3, 64), dtype=torch.float32, device=dev)
    lb.prefill_step(cfg, gu["q"], gu["k"], gu["v"], gu["positions"], gu["seq_lens"],
                    gu["q_norm_w"], gu["k_norm_w"], gu["block_table"], gu["k_cache"],
                    gu["v_cache"], q_out, out, lse)                   # the workspace-free grid
    torch.cuda.synchronize()
    assert torch.equal(rv["q_out"].view(q_out.shape), q_out)
    assert torch.equal(rv["out"].view(out.shape), out)
    assert torch.equal(rv["lse"].view(lse.shape), lse)


def test_work_list_is_grouped_by_sequence_longest_first():
    """The plan's work list, read from the workspace (white box: the item
    count in its first word, (sequence, block) int32 pairs from byte 256):
    every item once; each sequence's items contiguous, from its last block
    (the longest) down; sequences ordered by their longest item's tile count,
    longest first.  The order decides only which workgroup runs an item, not
    any result; this pins the grouping that lets the blocks of one sequence
    share its prefix tiles in L2."""
    dev = device()
    lens = [300, 5, 700, 64, 1, 4096, 2000, 129, 4160, 33]
    counts = [300, 0, 33, 1, 1, 1000, 64, 129, 65, 33]
    w = wl.custom(lens, seed=890, new_tokens=counts)
    g = to_device(wl.make_inputs(w), dev)
    cfg = config_for(w, g)
    ws = lb.alloc_prefill_workspace(cfg, len(lens), g["q"].shape[0], device=dev)
    q_out = torch.empty_like(g["q"])
    out = torch.zeros(g["q"].shape, dtype=cfg.out_torch_dtype, device=dev)
    lb.prefill_step_varlen(cfg, g["q_start"], g["q"], g["k"], g["v"], g["positions"],
                           g["seq_lens"], g["q_norm_w"], g["k_norm_w"], g["block_table"],
                           g["k_cache"], g["v_cache"], q_out, ws, out)
    torch.cuda.synchronize()
    words = ws.cpu().numpy().view(np.int32)
    tpb = 256 // (w.num_q_heads // w.num_kv_heads)
    items = [-(-n // tpb) for n in counts]
    n = int(words[0])
    assert n == sum(items)
    lst = words[64:64 + 2 * n].reshape(n, 2)
    assert sorted(map(tuple, lst.tolist())) == sorted((b, q) for b in range(len(lens))
                                                     for q in range(items[b]))
    first = {}
    for pos, (b, q) in enumerate(lst.tolist()):
        first.setdefault(b, pos)
        assert pos == first[b] + (items[b] - 1 - q), (pos, b, q)   # contiguous, last block first
    order = sorted(first, key=first.get)
    keys = [-(-lens[b] // 64) for b in order]
    assert keys == sorted(keys, reverse=True), (order, keys)


def test_mixed_batch_decode_and_prefill():
    """Sequences 0-2 decode one token (split-KV decode step, dynamic schedule);
    sequences 3-4 prefill a chunk (ragged prefill); one cache, one stream."""
    dev = device()
    lens, counts = [3000, 70, 5000, 600, 1000], [1, 1, 1, 600, 200]
    w = wl.custom(lens, seed=880, new_tokens=counts)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    g = to_device(inp, dev)
    cfg = config_for(w, g)
    dec = [0, 1, 2]
    wd = wl.custom([lens[b] for b in dec], seed=880)
    gd = dict(g, q=g["q"][:3].contiguous(), k=g["k"][:3].contiguous(), v=g["v"][:3].contiguous(),
              positions=g["positions"][:3].contiguous(), seq_lens=g["seq_lens"][:3].contiguous(),
              block_table=g["block_table"][:3].contiguous())
    rd = run_step(wd, gd, lb.Schedule("dynamic", num_workers=64), cfg=lb.DecodeConfig(
        64, 8, "bf16", g["max_blocks"], g["num_pages"]))
    assert rd["error"] == 0
    pre = slice(3, 5)
    qs = g["q_start"][3:] - g["q_start"][3]
    gp = dict(g, q=g["q"][3:].contiguous(), k=g["k"][3:].contiguous(), v=g["v"][3:].contiguous(),
              positions=g["positions"][3:].contiguous(), seq_lens=g["seq_lens"][pre].contiguous(),
              block_table=g["block_table"][pre].contiguous())
    cfg_p = lb.DecodeConfig(64, 8, "bf16", g["max_blocks"], g["num_pages"], tokens_per_seq=600)
    rp = run_varlen(w, gp, cfg=cfg_p, q_start=qs.contiguous())
    assert rp["error"] == 0
    pro, ref = oracle_varlen(w, inp)
    got_q = torch.cat([rd["q_out"], rp["q_out"]])
    assert np.array_equal(bits_u16(got_q), pro["q_out"])
    res = {"out": torch.cat([rd["out"], rp["out"]]), "lse": torch.cat([rd["lse"], rp["lse"]])}
    check_against(w, res, ref)


def test_malformed_q_start_is_flagged():
    """A range past total_tokens or above the bound skips that sequence and sets
    LBSR_DEV_ERR_QUERY_START; the well-formed sequences are still right."""
    dev = device()
    lens, counts = [40, 90, 30], [4, 6, 2]
    w = wl.custom(lens, seed=890, new_tokens=counts, num_q_heads=8, num_kv_heads=1)
    inp = wl.make_inputs(w)
    pro, ref = oracle_varlen(w, inp, seqs=[0])
    for bad, bound in (([0, 4, 13, 12], 6),     # sequence 1 ends past total_tokens = 12
                       ([0, 4, 10, 12], 5)):    # sequence 1 has 6 > 5 new tokens
        g = to_device(inp, dev)
        cfg = config_for(w, g)
        cfg.tokens_per_seq = bound
        qs = torch.tensor(bad, dtype=torch.int32, device=dev)
        res = run_varlen(w, g, cfg=cfg, q_start=qs)
        assert res["error"] & lb._binding.DEV_ERR_QUERY_START
        check_against(w, res, ref)                 # sequence 0 unaffected


@pytest.mark.slow
@pytest.mark.parametrize("name,seqs", [("ragged_prefill", [0, 3, 7]),   # no prefix; 8192; 20000
                                       ("mixed_prefill", [0, 3])])      # 8192-token prefixes
def test_ragged_prefill_full_size_sampled(name, seqs):
    """The benchmark's ragged prefills (8 prompts and 25,788 packed new tokens;
    the mixed batch's 4 x 1024 after 8192 cached) in their launch
    configuration: q_out of sampled sequences bit-exact, sampled (token, head)
    outputs and lse against the oracle."""
    dev = device()
    w = wl.named(name)
    g = wl.make_inputs(w, device=dev)
    pools = host_pools(g, w)              # the caches before the step writes them
    print(f"{name} full size", flush=True)
    res = run_varlen(w, g)
    assert res["error"] == 0
    h = host_step_inputs(g)
    starts = mt.query_starts(w.new_tokens)
    rows = np.concatenate([np.arange(starts[b], starts[b + 1]) for b in seqs])
    sub_counts = [w.new_tokens[b] for b in seqs]
    kw = dict(theta=w.rope_theta, eps=w.rms_eps, kv_dtype=w.kv_dtype)
    pro = mt.prologue_varlen(h["q"][rows], h["k"][rows], h["v"][rows], h["positions"][rows],
                             sub_counts, h["wq"], h["wk"], h["block_table"][seqs], **kw)
    assert np.array_equal(bits_u16(res["q_out"])[rows], pro["q_out"])
    cfg = oracle_cfg(g, w)
    picks = [[0, n // 2, n - 1] for n in sub_counts]
    ref = mt.attention_varlen(pro["q_out"], pools, pro, h["seq_lens"][seqs], sub_counts,
                              h["block_table"][seqs], cfg, heads=[0, 9, 63], tokens=picks)
    out, lse = to_f64(res["out"]), to_f64(res["lse"])
    for (i, j, hh), (o, l) in ref.items():
        r = int(starts[seqs[i]]) + j
        check_output(out[r, hh], o, "bf16", f"seq {seqs[i]} token {j} head {hh}")
        assert abs(lse[r, hh] - l) <= 1e-4 + 1e-5 * abs(l)


@pytest.mark.slow
def test_ragged_largest_batch():
    """16384 sequences (the batch limit) with 0 to 3 new tokens each: the plan's
    per-sequence prefix sums fill its LDS; sampled sequences against the oracle."""
    dev = device()
    rng = np.random.default_rng(905)
    B = 16384
    counts = rng.integers(0, 4, B).tolist()
    lens = (np.array(counts) + rng.integers(1, 200, B)).tolist()
    w = wl.custom(lens, num_q_heads=8, num_kv_heads=1, seed=905, new_tokens=counts)
    inp = wl.make_inputs(w)
    print(f"ragged batch of {B}, {sum(counts)} new tokens", flush=True)
    res = run_varlen(w, to_device(inp, dev))
    assert res["error"] == 0
    seqs = sorted({0, B - 1} | {int(b) for b in rng.choice(np.nonzero(np.array(counts))[0], 40)})
    pro, ref = oracle_varlen(w, inp, seqs=seqs)
    assert np.array_equal(bits_u16(res["q_out"]), pro["q_out"])
    check_against(w, res, ref)
