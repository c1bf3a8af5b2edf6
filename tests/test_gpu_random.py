"""Decode steps on seeded random configurations vs the fp64 oracle: batch
size, lengths (with the page-boundary values 1, 63, 64, 65 and multiples of
64 mixed in), head shapes within the API's limits (G <= 16, G * Tq <= 64),
cache dtype, new tokens per sequence, RoPE/RMSNorm order and the schedule
(dynamic with any worker count and optional XCD weights, static with any
split count, the folded merge where it applies).  The configurations are
drawn once from fixed seeds, so a failure names a reproducible case."""

import numpy as np
import pytest

import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from test_gpu_step import check_step
from test_gpu_varlen import run_varlen, oracle_varlen, check_against
from checks import poison_cache, bits_u16
from gpu_util import device, to_device

pytestmark = pytest.mark.gpu

HEADS = [(8, 1), (8, 2), (8, 8), (16, 2), (12, 3), (24, 8), (32, 2), (32, 4), (64, 8), (48, 12),
         (16, 16), (40, 10)]


def draw(i):
    rng = np.random.default_rng(7000 + i)
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    g = hq // hkv
    tokens = int(rng.choice([t for t in (1, 1, 1, 2, 3, 4) if g * t <= 64]))
    batch = int(rng.integers(1, 17))
    special = [1, 63, 64, 65, 128, 129, 640, 4096]
    lens = []
    for _ in range(batch):
        L = int(special[rng.integers(len(special))]) if rng.random() < 0.35 else \
            int(np.exp(rng.uniform(0, np.log(6000))))
        lens.append(max(L, tokens))
    kv = "fp8" if rng.random() < 0.35 else "bf16"
    norm_first = bool(rng.random() < 0.25)
    r = rng.random()
    if r < 0.55:
        P = int(rng.choice([1, 2, 3, 7, 37, 100, 256, 513, 1024]))
        wts = tuple(int(x) for x in rng.integers(1, 20, 8)) if rng.random() < 0.3 else None
        fold = tokens == 1 and (g & (g - 1)) == 0 and rng.random() < 0.3
        sched = lb.Schedule("dynamic", num_workers=P, xcd_weights=wts, fold_merge=fold)
    else:
        S = int(rng.choice([1, 2, 3, 7, 16, 64]))
        sched = lb.Schedule("static", static_splits=S)
    w = wl.custom(lens, num_q_heads=hq, num_kv_heads=hkv, kv_dtype=kv, seed=7000 + i,
                  tokens=tokens, norm_before_rope=norm_first)
    return w, sched


@pytest.mark.parametrize("i", range(60))
def test_random_configuration(i):
    w, sched = draw(i)
    check_step(w, sched, seed_note=f"(random case {i})")


def draw_ragged(i):
    rng = np.random.default_rng(9000 + i)
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    batch = int(rng.integers(1, 7))
    counts = [int(rng.choice([0, 1, 2, 31, 32, 33, 100, 257])) for _ in range(batch)]
    if sum(counts) == 0:
        counts[0] = 5
    lens = [n + int(rng.choice([0, 0, 1, 63, 64, 500, 2000])) for n in counts]
    lens = [max(L, 1) for L in lens]
    kv = "fp8" if rng.random() < 0.35 else "bf16"
    return wl.custom(lens, num_q_heads=hq, num_kv_heads=hkv, kv_dtype=kv, seed=9000 + i,
                     new_tokens=counts, norm_before_rope=bool(rng.random() < 0.25))


@pytest.mark.parametrize("i", range(16))
def test_random_ragged_prefill(i):
    """Ragged prefill (random per-sequence counts, zero included, after random
    prefixes) vs the oracle: q_out bits, outputs and lse."""
    dev = device()
    w = draw_ragged(i)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    print(f"random ragged case {i}: lens {w.seq_lens} new {w.new_tokens} "
          f"{w.num_q_heads}q/{w.num_kv_heads}kv {w.kv_dtype}", flush=True)
    res = run_varlen(w, to_device(inp, dev))
    assert res["error"] == 0
    pro, ref = oracle_varlen(w, inp)
    assert np.array_equal(bits_u16(res["q_out"]), pro["q_out"])
    check_against(w, res, ref)


def draw_prefill(i):
    rng = np.random.default_rng(11000 + i)
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    batch = int(rng.integers(1, 5))
    tokens = int(rng.choice([1, 2, 17, 31, 32, 33, 47, 48, 49, 64, 65, 130, 300]))
    lens = [tokens + int(rng.choice([0, 0, 1, 63, 64, 65, 700, 3000])) for _ in range(batch)]
    kv = "fp8" if rng.random() < 0.5 else "bf16"
    qk = "fp8" if kv == "fp8" and rng.random() < 0.5 else "bf16"
    w = wl.custom(lens, num_q_heads=hq, num_kv_heads=hkv, kv_dtype=kv, seed=11000 + i,
                  tokens=tokens, norm_before_rope=bool(rng.random() < 0.25))
    return w, qk, bool(rng.random() < 0.5)


@pytest.mark.parametrize("i", range(20))
def test_random_uniform_prefill(i):
    """Uniform prefill (every sequence the same count of new tokens, block
    widths of 256/G and, with FP8 scores, 384/G columns crossed at random) vs
    the oracle: q_out bits, outputs and lse (FP8 scores: with the matrix
    cores' accumulation term), with and without the work list."""
    from test_gpu_prefill import run_prefill, oracle_prefill
    from checks import check_output, to_f64, fp8_lse_slack_for
    from gpu_util import config_for
    dev = device()
    w, qk, listed = draw_prefill(i)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    g = to_device(inp, dev)
    cfg = config_for(w, g)
    extra = None
    if qk == "fp8":
        cfg.qk_dtype, cfg.q_scale = "fp8", 2.0 ** -5
        extra = {"qk_dtype": "fp8", "q_scale": 2.0 ** -5}
    print(f"random prefill case {i}: lens {w.seq_lens} tokens {w.tokens} "
          f"{w.num_q_heads}q/{w.num_kv_heads}kv {w.kv_dtype} scores {qk} list {listed}", flush=True)
    res = run_prefill(w, g, cfg, sorted_list=listed)
    assert res["error"] == 0
    pro, ro, rl = oracle_prefill(w, inp, extra)
    assert np.array_equal(bits_u16(res["q_out"]).reshape(-1), pro["q_out"].reshape(-1))
    check_output(to_f64(res["out"]).reshape(ro.shape), ro, w.kv_dtype, "random prefill output")
    slack = 0.0
    if qk == "fp8":
        slack = fp8_lse_slack_for(inp, w, pro, 2.0 ** -5,
                                  np.repeat(np.arange(w.batch), w.tokens)).reshape(rl.shape)
    lse = to_f64(res["lse"]).reshape(rl.shape)
    assert np.all(np.abs(lse - rl) <= 1e-4 + 1e-5 * np.abs(rl) + slack), \
        float(np.max(np.abs(lse - rl)))
