"""The fused prologue against the oracle: q_out bits, the cache slot each new
token lands in (bit-exact indexing), the stored values, and that nothing else
in the cache changes."""

import numpy as np
import pytest
import torch

import oracle
from oracle import multitoken as mt
import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import host_pools, host_step_inputs, bits_u16, poison_cache
from gpu_util import device, to_device, config_for

pytestmark = pytest.mark.gpu


def near_tie(pre, kind):
    """True where an fp64 value lies within 2^-40 (relative) of a rounding
    midpoint of the stored format: there the GPU's fp64 (different sum order,
    pow/sin implementations) may round the other way."""
    pre = np.asarray(pre, dtype=np.float64)
    a = np.abs(pre)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    bits = 7 if kind == "bf16" else 3
    lo_e = -126 if kind == "bf16" else -6
    q = np.ldexp(1.0, (np.maximum(e, lo_e) - bits).astype(np.int64))
    frac = a / q - np.floor(a / q)
    return np.abs(frac - 0.5) < 2.0 ** -40 * np.maximum(a / q, 1.0)


def run_prologue(w, inp_cpu, dev, error_word=None):
    g = to_device(inp_cpu, dev)
    cfg = config_for(w, g)
    q_out = torch.empty_like(g["q"])
    lb.rope_norm_kv_write(cfg, g["q"], g["k"], g["v"], g["positions"], g["q_norm_w"],
                          g["k_norm_w"], g["block_table"], g["k_cache"], g["v_cache"], q_out,
                          error_word=error_word)
    torch.cuda.synchronize()
    return g, q_out


CASES = [
    ("tiny", None),
    ("custom", dict(seq_lens=[1, 64, 65, 4096, 20000, 200], num_q_heads=64, num_kv_heads=8)),
    ("custom", dict(seq_lens=[3, 129, 262144], num_q_heads=16, num_kv_heads=2, kv_dtype="fp8")),
    ("custom", dict(seq_lens=[77, 5000], num_q_heads=32, num_kv_heads=4, norm_before_rope=True)),
    ("custom", dict(seq_lens=[300, 1, 64], num_q_heads=8, num_kv_heads=2, kv_dtype="fp8",
                    k_scale=0.0371, v_scale=0.0113)),
    # several new tokens per sequence, some pairs straddling a page boundary
    ("custom", dict(seq_lens=[2, 64, 65, 130, 4096], num_q_heads=64, num_kv_heads=8, tokens=2)),
    ("custom", dict(seq_lens=[4, 66, 1000, 129], num_q_heads=16, num_kv_heads=4, kv_dtype="fp8",
                    tokens=4)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prologue_matches_oracle(case):
    dev = device()
    name, kw = CASES[case]
    w = wl.named("tiny") if name == "tiny" else wl.custom(seed=100 + case, **kw)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    before_k, before_v = host_pools(inp, w)
    h = host_step_inputs(inp)
    print(f"prologue case {case}: lens {w.seq_lens} {w.num_q_heads}q/{w.num_kv_heads}kv "
          f"{w.kv_dtype} tokens {w.tokens}", flush=True)
    g, q_out = run_prologue(w, inp, dev)

    kw = dict(theta=w.rope_theta, eps=w.rms_eps, kv_dtype=w.kv_dtype,
              k_scale=np.float32(w.k_scale).item(), v_scale=np.float32(w.v_scale).item(),
              norm_before_rope=w.norm_before_rope)
    if w.tokens == 1:
        pro = oracle.prologue(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                              h["block_table"], **kw)
    else:
        pro = mt.prologue_tokens(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                                 h["block_table"], **kw)
    # q_out: the fp64 result's BF16 rounding, except at near-ties (token-major flat)
    got_q = bits_u16(q_out).reshape(pro["q_out"].shape)
    diff = got_q != pro["q_out"]
    assert not np.any(diff & ~near_tie(pro["q_f64"], "bf16")), int(diff.sum())

    # the cache: expected = before + the oracle's writes at the oracle's slots
    after_k, after_v = host_pools(g, w)
    exp_k, exp_v = before_k.copy(), before_v.copy()
    oracle.step.apply_prologue_writes(exp_k, exp_v, pro, kv_dtype=w.kv_dtype,
                                      page_stride=g["page_stride"], head_stride=g["head_stride"])
    B, Hkv, D = pro["k_store"].shape
    for got, exp, pre, kind in ((after_k, exp_k, pro["k_pre"], "k"),
                                (after_v, exp_v, pro["v_pre"], "v")):
        # fp64 value that was rounded into each written element (NaN elsewhere)
        pre_flat = np.full(exp.size, np.nan)
        for b in range(B):
            page, row = pro["slots"][b]
            for gg in range(Hkv):
                off = page * g["page_stride"] + gg * g["head_stride"] + \
                    oracle.tile_offset(kind, w.kv_dtype, row, np.arange(D))
                pre_flat[off] = pre[b, gg]
        mism = np.nonzero(got != exp)[0]
        assert not np.isnan(pre_flat[mism]).any(), f"{kind} cache changed outside the new slots"
        assert near_tie(pre_flat[mism], w.kv_dtype).all(), \
            f"{kind} cache: {mism.size} stored values differ away from rounding ties"


def test_prologue_flags_bad_position_and_page():
    dev = device()
    w = wl.custom([10, 70], num_q_heads=8, num_kv_heads=1, seed=9)
    inp = wl.make_inputs(w)
    inp["positions"][0] = 10_000               # past max_blocks * 64
    inp["block_table"][1, 1] = 99_999          # not a page of the pool
    before_k, before_v = host_pools(inp, w)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    g, _ = run_prologue(w, inp, dev, error_word=err)
    e = int(err.item())
    assert e & lb._binding.DEV_ERR_POSITION and e & lb._binding.DEV_ERR_PAGE
    after_k, after_v = host_pools(g, w)
    assert np.array_equal(after_k, before_k) and np.array_equal(after_v, before_v)
