"""Decode steps at the limits the library accepts, against the fp64 oracle:
the largest batch (16384 sequences), the most workers (1024), a static split
into 1024 parts (a merge over 1024 rows), the longest sequence (262144
tokens), and 16 KV heads (two per wave, in lockstep)."""

import numpy as np
import pytest
import torch

import oracle
import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from checks import check_output, to_f64, host_step_inputs, oracle_cfg, poison_cache, bits_u16
from gpu_util import device, run_step, compact_pools, remap_slots, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def sampled(w, g, res, seqs, heads):
    """Oracle outputs of (seqs x heads) on compacted host copies of their pages."""
    h = host_step_inputs(g)
    pro = oracle.prologue(h["q"], h["k"], h["v"], h["positions"], h["wq"], h["wk"],
                          h["block_table"], theta=w.rope_theta, eps=w.rms_eps,
                          kv_dtype=w.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    kp, vp, bt, pmap = compact_pools(g, w, seqs)
    ref = oracle.decode_attention(pro["q_out"], (kp, vp), remap_slots(pro, pmap), h["seq_lens"],
                                  bt, oracle_cfg(g, w), seqs=seqs, heads=heads)
    out, lse = to_f64(res["out"]), to_f64(res["lse"])
    for (b, hh), (o, l) in ref.items():
        check_output(out[b, hh], o, w.kv_dtype, f"seq {b} head {hh}")
        assert abs(lse[b, hh] - l) <= 1e-4 + 1e-5 * abs(l), (b, hh)
    return pro


def test_largest_batch():
    dev = device()
    lens = np.random.default_rng(900).integers(1, 131, 16384).tolist()
    w = wl.custom(lens, num_q_heads=8, num_kv_heads=1, seed=900)
    g = wl.make_inputs(w, device=dev)
    print("16384 sequences, 8q/1kv", flush=True)
    res = run_step(w, g, lb.Schedule("dynamic", num_workers=256))
    assert res["error"] == 0
    assert np.array_equal(res["plan"]["chunks"], oracle.plan_dynamic(lens, 256).chunks)
    seqs = sorted(set(np.random.default_rng(1).integers(0, 16384, 200).tolist()) | {0, 16383})
    sampled(w, g, res, seqs, list(range(8)))


def test_most_workers():
    dev = device()
    w = wl.named("mix")
    g = wl.make_inputs(w, device=dev)
    res = run_step(w, g, lb.Schedule("dynamic", num_workers=1024))
    assert res["error"] == 0
    assert np.array_equal(res["plan"]["chunks"], oracle.plan_dynamic(w.seq_lens, 1024).chunks)
    sampled(w, g, res, [0, 5, 31], [0, 33, 63])


def test_static_split_into_1024_parts():
    """Sequence 0 (1094 tiles) is cut into 1024 parts, so the merge combines 1024
    rows; sequence 1 has one tile and one non-empty part."""
    dev = device()
    w = wl.custom([70000, 5], num_q_heads=64, num_kv_heads=8, seed=901)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    g = to_device(inp, dev)
    sched = lb.Schedule("static", num_workers=8, static_splits=1024)
    res = run_step(w, g, sched)
    assert res["error"] == 0
    plan = oracle.plan_static(w.seq_lens, 1024)
    assert np.array_equal(res["plan"]["chunks"], plan.chunks)
    assert plan.seq_chunk[1] - plan.seq_chunk[0] == 1024
    sampled(w, g, res, [0, 1], list(range(64)))


def test_longest_sequence():
    """One sequence at the 262144-token maximum (4096 pages) beside a short one."""
    dev = device()
    w = wl.custom([262144, 77], num_q_heads=64, num_kv_heads=8, seed=902)
    g = wl.make_inputs(w, device=dev)
    poison_cache(g, w, spare_pages=False)
    res = run_step(w, g, lb.Schedule("dynamic", num_workers=256))
    assert res["error"] == 0
    sampled(w, g, res, [0, 1], [0, 7, 8, 40, 63])


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sixteen_kv_heads(kv_dtype):
    """Hkv = 16 with 8 waves per workgroup: each wave runs two KV heads, in lockstep."""
    dev = device()
    w = wl.custom([4100, 65, 1, 700], num_q_heads=64, num_kv_heads=16, kv_dtype=kv_dtype, seed=903)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    g = to_device(inp, dev)
    for P in (1, 37, 256):
        res = run_step(w, dict(g, k_cache=g["k_cache"].clone(), v_cache=g["v_cache"].clone()),
                       lb.Schedule("dynamic", num_workers=P))
        assert res["error"] == 0
        sampled(w, dict(g, k_cache=g["k_cache"], v_cache=g["v_cache"]), res, [0, 1, 2, 3],
                list(range(64)))
