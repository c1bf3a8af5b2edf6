"""Pins for the multi-token decode oracle (R20): several new tokens per
sequence, each attending its causal prefix.

* positions and limits by hand;
* each token's output against torch's fp64 scaled-dot-product attention with
  an explicit boolean mask built from the positions (a library routine);
* the prefix property: token j equals the single-token step on the first
  L - Tq + j + 1 rows;
* split-then-merge equals unsplit, on plans where some chunks hold no row of
  an early token (empty partials);
* a planted off-by-one in the causal limit is caught.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import multitoken as mt
from load_balanced_split_rope_amd import workloads as wl
from checks import poison_cache, host_pools, host_step_inputs, oracle_cfg


def test_positions_and_limits_by_hand():
    assert mt.token_positions([10, 3], 3).tolist() == [[7, 8, 9], [0, 1, 2]]
    assert mt.token_positions([5], 1).tolist() == [[4]]
    # token j of a length-L sequence attends rows [0, L - Tq + j + 1)
    assert [mt.causal_limit(10, 3, j) for j in range(3)] == [8, 9, 10]
    with pytest.raises(ValueError):
        mt.token_positions([2, 5], 3)


def _setup(lens, tokens, Hq=16, Hkv=2, dtype="bf16", seed=11):
    w = wl.custom(lens, num_q_heads=Hq, num_kv_heads=Hkv, kv_dtype=dtype, seed=seed,
                  tokens=tokens)
    inp = wl.make_inputs(w)
    poison_cache(inp, w)
    h = host_step_inputs(inp)
    q = h["q"].reshape(w.batch, tokens, Hq, 128)
    k = h["k"].reshape(w.batch, tokens, Hkv, 128)
    v = h["v"].reshape(w.batch, tokens, Hkv, 128)
    pos = h["positions"].reshape(w.batch, tokens)
    assert np.array_equal(pos, mt.token_positions(h["seq_lens"], tokens))
    pro = mt.prologue_tokens(q, k, v, pos, h["wq"], h["wk"], h["block_table"],
                             theta=w.rope_theta, eps=w.rms_eps, kv_dtype=w.kv_dtype,
                             k_scale=w.k_scale, v_scale=w.v_scale)
    q_out = pro["q_out"].reshape(w.batch, tokens, Hq, 128)
    return w, inp, h, host_pools(inp, w), pro, q_out, oracle_cfg(inp, w)


def _masked_sdpa(q_bits, K, V, L, Tq, sm_scale):
    """torch fp64 SDPA of the Tq x G queries of one KV group over K, V [L, D]
    with mask[j, r] = r <= L - Tq + j, and the log-sum-exp of the masked scores."""
    Tq_, G, D = q_bits.shape
    q = torch.from_numpy(oracle.bf16_bits_to_f64(q_bits).reshape(Tq * G, D))
    k = torch.from_numpy(np.ascontiguousarray(K))
    v = torch.from_numpy(np.ascontiguousarray(V))
    pos = torch.arange(L)
    limit = (L - Tq + torch.arange(Tq)).repeat_interleave(G)        # last attended row
    mask = pos[None, :] <= limit[:, None]                            # [Tq*G, L]
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None],
                                                         attn_mask=mask[None], scale=sm_scale)[0]
    s = (q @ k.T) * sm_scale
    lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=1)
    return o.numpy().reshape(Tq, G, D), lse.numpy().reshape(Tq, G)


@pytest.mark.parametrize("lens,tokens,dtype", [([5, 64, 65, 130], 2, "bf16"),
                                               ([4, 66, 200], 4, "fp8"),
                                               ([3, 129], 3, "bf16")])
def test_tokens_against_masked_sdpa(lens, tokens, dtype):
    w, inp, h, pools, pro, q_out, cfg = _setup(lens, tokens, dtype=dtype)
    got = mt.decode_attention_tokens(q_out, pools, pro, h["seq_lens"], h["block_table"], cfg)
    G = w.num_q_heads // w.num_kv_heads
    for b, L in enumerate(lens):
        for g in range(w.num_kv_heads):
            K, V = oracle.step._sequence_kv(pools, pro, b, g, h["seq_lens"], h["block_table"], cfg)
            assert np.all(np.isfinite(K)) and np.all(np.isfinite(V))
            o_ref, l_ref = _masked_sdpa(q_out[b, :, g * G:(g + 1) * G], K, V, L, tokens,
                                        cfg["sm_scale"])
            for j in range(tokens):
                for i in range(G):
                    o, l = got[(b, j, g * G + i)]
                    assert np.allclose(o, o_ref[j, i], rtol=1e-12, atol=1e-13)
                    assert abs(l - l_ref[j, i]) <= 1e-12 * max(1.0, abs(l_ref[j, i]))


def test_prefix_property():
    """Token j of a step equals the one-token step over the first L - Tq + j + 1 rows."""
    lens, Tq = [70, 9, 128], 3
    w, inp, h, pools, pro, q_out, cfg = _setup(lens, Tq, Hq=8, Hkv=1)
    got = mt.decode_attention_tokens(q_out, pools, pro, h["seq_lens"], h["block_table"], cfg)
    for j in range(Tq):
        trunc = np.asarray(lens) - Tq + j + 1
        one = oracle.decode_attention(q_out[:, j], pools, pro, trunc, h["block_table"], cfg)
        for (b, hh), (o, l) in one.items():
            assert np.array_equal(o, got[(b, j, hh)][0]) and l == got[(b, j, hh)][1]


@pytest.mark.parametrize("tokens", [2, 4])
def test_split_equals_full_with_empty_partials(tokens):
    # L = 64k + 1: the last tile holds one row, so with a worker per tile the
    # last chunk holds no row of the early tokens
    lens = [129, 65, 64 * 5 + 2]
    w, inp, h, pools, pro, q_out, cfg = _setup(lens, tokens, Hq=8, Hkv=2)
    full = mt.decode_attention_tokens(q_out, pools, pro, h["seq_lens"], h["block_table"], cfg)
    B, Hq = len(lens), w.num_q_heads
    ref_o = np.array([[[full[(b, j, hh)][0] for hh in range(Hq)] for j in range(tokens)]
                      for b in range(B)])
    ref_l = np.array([[[full[(b, j, hh)][1] for hh in range(Hq)] for j in range(tokens)]
                      for b in range(B)])
    saw_empty = False
    for plan in (oracle.plan_dynamic(lens, 1), oracle.plan_dynamic(lens, 11),
                 oracle.plan_dynamic(lens, 256), oracle.plan_static(lens, 3)):
        o, lse, parts = mt.split_attention_tokens(q_out, pools, pro, h["seq_lens"],
                                                  h["block_table"], cfg, plan)
        assert np.allclose(o, ref_o, rtol=1e-12, atol=1e-14)
        assert np.allclose(lse, ref_l, rtol=1e-13, atol=1e-13)
        for oc, lc in parts.values():
            empty = np.isneginf(lc)
            saw_empty |= bool(empty.any())
            assert np.all(oc[empty] == 0)
    assert saw_empty


def test_prologue_tokens_slots_and_queries():
    lens, Tq = [63, 64, 200], 2
    w, inp, h, pools, pro, q_out, cfg = _setup(lens, Tq, Hq=8, Hkv=1)
    qf = oracle.bf16_bits_to_f64(h["q"]).reshape(len(lens), Tq, 8, 128)
    wq = oracle.bf16_bits_to_f64(h["wq"])
    for b, L in enumerate(lens):
        for j in range(Tq):
            pos = L - Tq + j
            t = b * Tq + j
            assert tuple(pro["slots"][t]) == (h["block_table"][b][pos // 64], pos % 64)
            ref = oracle.qk_transform(qf[b, j], wq, pos, w.rope_theta, w.rms_eps, False)
            assert np.array_equal(pro["q_f64"][t], ref)


def test_planted_off_by_one_is_caught(monkeypatch):
    """A causal limit one row too far must fail the masked-SDPA comparison."""
    lens, Tq = [70, 130], 2
    w, inp, h, pools, pro, q_out, cfg = _setup(lens, Tq, Hq=8, Hkv=1)
    monkeypatch.setattr(mt, "causal_limit", lambda L, T, j: int(L) - int(T) + int(j) + 2
                        if j < T - 1 else int(L))
    bad = mt.decode_attention_tokens(q_out, pools, pro, h["seq_lens"], h["block_table"], cfg)
    K, V = oracle.step._sequence_kv(pools, pro, 0, 0, h["seq_lens"], h["block_table"], cfg)
    o_ref, _ = _masked_sdpa(q_out[0, :, 0:8], K, V, lens[0], Tq, cfg["sm_scale"])
    assert not np.allclose(bad[(0, 0, 0)][0], o_ref[0, 0], rtol=1e-6, atol=1e-8)
