"""Shared test helpers: input poisoning, tolerance rule, exact comparisons.

Tolerance (reading R14 of the values the step must match):
* BF16 cache: every element |got - ref| <= 2e-2 + 1e-2 |ref|, and for the
  attention output also ||got - ref||_2 / ||ref||_2 <= 1e-2 (the elementwise
  bound alone is looser than the signal at long lengths).
* FP8 cache: every element |got - ref| <= 6e-2 on the attention output, and
  ||got - ref||_2 / ||ref||_2 <= 2e-2.  The same codes are decoded exactly on
  both sides, so the relative error is of the size the BF16 path shows; the
  elementwise bound alone passes an all-zero output once |o| < 6e-2, which
  N(0,1) values reach at a few thousand rows.
* FP8 output: the codes within the bound above plus half an E4M3 step of the
  value, and in L2 within the half-step norm plus the cache's relative bound.
* The schedule and every cache index: bit-exact.
"""

import numpy as np
import torch

from oracle import tile_offset, PAGE_SIZE, BF16_NAN_BITS, E4M3_NAN_CODE
from oracle.qk import query_values
from oracle.step import apply_prologue_writes, gather_kv

# R23 with FP8 scores: the FP8 matrix cores accumulate a score's 128 products
# with less than fp32 precision.  Measured on the device over 16,384 one-row
# scores (four q scales; with one row, lse is the score itself), the error was
# at most 2^-16.05 of M = sm * sum_d |q_d k_d|.  An lse is a softmax-weighted
# mean of its row's scores, so its error is at most the largest score error;
# FP8-score lse checks add twice the measured bound times the row's largest M.
FP8_SCORE_REL = 2.0 ** -15

BF16_ATOL, BF16_RTOL, BF16_REL_L2 = 2e-2, 1e-2, 1e-2
FP8_ATOL, FP8_REL_L2 = 6e-2, 2e-2


def to_f64(t):
    """A torch tensor (bf16/fp32) -> fp64 numpy on the host."""
    return t.detach().to("cpu", torch.float64).numpy()


def bits_u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def check_output(got, ref, kv_dtype, what="output", rel_l2=True):
    """Apply the tolerance rule; return (max_abs, rel_l2) or raise AssertionError."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    rl2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    if kv_dtype == "bf16":
        bad = err > BF16_ATOL + BF16_RTOL * np.abs(ref)
        assert not bad.any(), f"{what}: {int(bad.sum())} elements out of tolerance, max abs {max_abs:.3e}"
        if rel_l2:
            assert rl2 <= BF16_REL_L2, f"{what}: relative L2 {rl2:.3e} > {BF16_REL_L2}"
    else:
        assert max_abs <= FP8_ATOL, f"{what}: max abs {max_abs:.3e} > {FP8_ATOL}"
        if rel_l2:
            assert rl2 <= FP8_REL_L2, f"{what}: relative L2 {rl2:.3e} > {FP8_REL_L2}"
    return max_abs, rl2


def e4m3_step(x):
    """Spacing of OCP E4M3 values around |x| (2^-9 in the subnormal range)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.ldexp(1.0, (np.maximum(e, -6) - 3).astype(np.int64))


def check_output_fp8(codes, ref, kv_dtype, out_scale, what="output", rel_l2=True):
    """FP8 output (R21): the decoded codes times out_scale must lie within the
    R14 tolerance of the fp64 result plus half an E4M3 step of the output;
    where |ref| / out_scale exceeds 448 the code must be the saturated one.
    In L2 (unsaturated elements): ||got - ref|| <= ||half steps|| + r ||ref||,
    r the cache's relative L2 bound -- rounding moves each element by at most
    half a step, so the triangle inequality gives this bound."""
    from oracle import e4m3_to_f64
    got = e4m3_to_f64(np.asarray(codes, dtype=np.uint8)) * out_scale
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: NaN codes"
    x = ref / out_scale
    sat = np.abs(x) > 448
    assert np.all(np.abs(got[sat]) == 448 * out_scale), f"{what}: saturation"
    base = BF16_ATOL + BF16_RTOL * np.abs(ref) if kv_dtype == "bf16" else np.full(ref.shape, FP8_ATOL)
    tol = base + 0.5 * e4m3_step(np.minimum(np.abs(x), 448)) * out_scale
    err = np.abs(got - ref)
    bad = (err > tol) & ~sat
    assert not bad.any(), f"{what}: {int(bad.sum())} codes out of tolerance, max err {err.max():.3e}"
    if rel_l2 and (~sat).any():
        r = BF16_REL_L2 if kv_dtype == "bf16" else FP8_REL_L2
        half = 0.5 * e4m3_step(np.minimum(np.abs(x[~sat]), 448)) * out_scale
        lim = np.linalg.norm(half) + r * np.linalg.norm(ref[~sat])
        dist = np.linalg.norm(got[~sat] - ref[~sat])
        assert dist <= lim, f"{what}: L2 distance {dist:.3e} > {lim:.3e}"
    return float(err[~sat].max()) if (~sat).any() else 0.0


def poison_indices(inp, w, kind, spare_pages=True):
    """Pool indices (one pool) of every element the step must not read.

    Pages no sequence owns, the rows at or past L_b of each sequence's last
    page, and the new tokens' own slots (the prologue must overwrite them
    before attention reads them).
    """
    counts = w.new_tokens if w.varlen else [int(w.tokens)] * w.batch
    bt = inp["block_table"].cpu().numpy()
    lens = [int(L) for L in w.seq_lens]
    Hkv, ps, hs = w.num_kv_heads, inp["page_stride"], inp["head_stride"]
    owned = set()
    for b, L in enumerate(lens):
        owned.update(bt[b, :-(-L // PAGE_SIZE)].tolist())
    idx = [np.zeros(0, dtype=np.int64)]
    if spare_pages:
        # the tile of this kind for every (unowned page, KV head): with K and V
        # interleaved in one allocation the page's other tiles belong to the
        # other kind (and one view's range past them to the next page)
        tile = PAGE_SIZE * 128
        idx += [np.arange(p * ps + g * hs, p * ps + g * hs + tile)
                for p in range(inp["num_pages"]) if p not in owned for g in range(Hkv)]
    d = np.arange(128)
    for b, L in enumerate(lens):
        t = (L - 1) // PAGE_SIZE
        slots = [(t, r) for r in range(L - t * PAGE_SIZE, PAGE_SIZE)]
        slots += [(pos // PAGE_SIZE, pos % PAGE_SIZE) for pos in range(L - int(counts[b]), L)]
        for tile, r in slots:
            page = int(bt[b, tile])
            for g in range(Hkv):
                off = tile_offset(kind, w.kv_dtype, np.array([[r]]), d[None, :]).reshape(-1)
                idx.append(page * ps + g * hs + off)
    return np.concatenate(idx)


def poison_cache(inp, w, spare_pages=True):
    """Fill every cache element the step must not read with NaN, in place
    (spare_pages=False leaves unowned pages alone, for very large pools)."""
    nan = BF16_NAN_BITS if w.kv_dtype == "bf16" else E4M3_NAN_CODE
    for key, kind in (("k_cache", "k"), ("v_cache", "v")):
        pool = inp[key]
        ti = torch.from_numpy(poison_indices(inp, w, kind, spare_pages).astype(np.int64)).to(pool.device)
        if pool.dtype == torch.bfloat16:
            pool.view(torch.int16).index_fill_(0, ti, int(np.int16(np.uint16(nan).view(np.int16))))
        else:
            pool.index_fill_(0, ti, nan)


def oracle_cfg(inp, w):
    return {"kv_dtype": w.kv_dtype, "k_scale": w.k_scale, "v_scale": w.v_scale,
            "sm_scale": 1.0 / np.sqrt(128.0), "page_stride": inp["page_stride"],
            "head_stride": inp["head_stride"], "num_kv_heads": w.num_kv_heads}


def host_pools(inp, w):
    """Host numpy views of the pools: uint16 BF16 bits or uint8 codes."""
    if w.kv_dtype == "bf16":
        return bits_u16(inp["k_cache"]), bits_u16(inp["v_cache"])
    return inp["k_cache"].cpu().numpy(), inp["v_cache"].cpu().numpy()


def host_step_inputs(inp):
    """The small per-step arrays as host numpy (BF16 as uint16 bits)."""
    return {
        "q": bits_u16(inp["q"]), "k": bits_u16(inp["k"]), "v": bits_u16(inp["v"]),
        "wq": bits_u16(inp["q_norm_w"]), "wk": bits_u16(inp["k_norm_w"]),
        "positions": inp["positions"].cpu().numpy().astype(np.int64),
        "seq_lens": inp["seq_lens"].cpu().numpy().astype(np.int64),
        "block_table": inp["block_table"].cpu().numpy().astype(np.int64),
    }


def fp8_lse_slack(w, k_pool, block_table, seq_lens, page_stride, head_stride, q_out_bits,
                  q_scale, seq_of_row, seqs=None):
    """FP8-score lse slack, [rows, Hq]: FP8_SCORE_REL * sm * max over the L_b keys of
    sum_d |q_d k_d|, for query row r of sequence b = seq_of_row[r] (q_out_bits
    [rows, Hq, D] BF16 bits, quantised under R23 as the scores use them).
    k_pool holds the new tokens' keys; seqs: only these sequences (0 elsewhere)."""
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, 128
    G = Hq // Hkv
    seq_of_row = np.asarray(seq_of_row)
    qv = np.abs(query_values(q_out_bits, {"qk_dtype": "fp8", "q_scale": q_scale}))
    qv = qv.reshape(len(seq_of_row), Hq, D)
    k_scale = float(np.float32(w.k_scale))
    out = np.zeros((len(seq_of_row), Hq))
    for b in (np.unique(seq_of_row) if seqs is None else seqs):
        rs = np.nonzero(seq_of_row == b)[0]
        if rs.size == 0:
            continue
        for g in range(Hkv):
            K = np.abs(gather_kv(k_pool, "k", w.kv_dtype, block_table[b], int(seq_lens[b]), g,
                                 page_stride=page_stride, head_stride=head_stride, scale=k_scale))
            M = qv[rs, g * G:(g + 1) * G].reshape(-1, D) @ K.T          # [rows * G, L]
            out[rs, g * G:(g + 1) * G] = M.max(axis=1).reshape(rs.size, G)
    return FP8_SCORE_REL / np.sqrt(128.0) * out


def fp8_lse_slack_for(inp, w, pro, q_scale, seq_of_row):
    """fp8_lse_slack for host inputs ``inp`` and the oracle's prologue ``pro``
    (its k and v written into copies of the pools)."""
    kp, vp = (np.array(p, copy=True) for p in host_pools(inp, w))
    apply_prologue_writes(kp, vp, pro, kv_dtype=w.kv_dtype, page_stride=inp["page_stride"],
                          head_stride=inp["head_stride"])
    h = host_step_inputs(inp)
    return fp8_lse_slack(w, kp, h["block_table"], h["seq_lens"], inp["page_stride"],
                         inp["head_stride"], pro["q_out"], q_scale, seq_of_row)
