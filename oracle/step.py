"""One whole decode step in fp64: prologue, cache write, attention, split+merge.

Page A, "Why does dynamic scheduling matter in attention?", and page B,
"Code analysis 2": the new token's q and k are rotated (RoPE) and normalised
(QK-Norm), and the new k and v are written into the KV cache, as one fused
pass; page B adds that the op writes a caller-provided output (here q_out).
The attention then reads the cache through the block table.

Readings used here:

* R5 -- sequence b's new token sits at position positions[b] = L_b - 1 and is
  attended to (attention covers rows [0, L_b)).
* R6 -- tile t of sequence b is page block_table[b][t]; the new token goes to
  page block_table[b][pos // 64], row pos % 64 (layout in ``layout.py``).
* R9 -- FP8 cache: code = E4M3(x / scale) with clamping; value = code * scale;
  separate per-tensor scales for k and v.
* R10 -- values are rounded only where the data path stores a narrow type:
  q_out (BF16), the cache slot (BF16 or E4M3) and the final output (BF16).
  Everything else is fp64.  Tests compare GPU results with these fp64 values.
* R17 -- rows at or past L_b inside the last page are never used.
* R21 -- with an FP8 output the attention output is stored as E4M3 codes of
  o / out_scale (clamp to +-448, then round to nearest even); lse stays fp32.
"""

import numpy as np

from .qk import query_values
from .formats import bf16_bits_to_f64, f64_to_bf16_bits, e4m3_to_f64, f64_to_e4m3
from .rope_norm import qk_transform
from .layout import tile_offset, PAGE_SIZE, HEAD_DIM
from .schedule import plan_dynamic, plan_static
from .attention import attend_full, attend_chunk, combine_lse


def cache_slot(block_table, pos):
    """(page, row) of the cache slot that holds position ``pos`` (R6)."""
    return int(block_table[pos // PAGE_SIZE]), int(pos % PAGE_SIZE)


def prologue(q, k, v, positions, wq, wk, block_table, *, theta, eps, kv_dtype,
             k_scale=1.0, v_scale=1.0, norm_before_rope=False):
    """RoPE + QK-Norm on q and k, and the values the cache write stores.

    q: [B, Hq, D] BF16 bits; k, v: [B, Hkv, D] BF16 bits; positions: [B];
    wq, wk: [D] BF16 bits; block_table: [B, max_blocks].

    Returns a dict with
      q_f64   [B, Hq, D]  RoPE+norm of q before rounding
      q_out   [B, Hq, D]  its BF16 bits (the caller-visible output)
      k_f64   [B, Hkv, D] RoPE+norm of k before rounding
      k_store, v_store    what the cache slot holds: BF16 bits or E4M3 codes
      k_pre, v_pre        the value that was rounded into k_store/v_store
                          (k_f64 or k_f64/k_scale; v or v/v_scale)
      slots   [B, 2]      (page, row) of each new token
    """
    qf = bf16_bits_to_f64(q)
    kf = bf16_bits_to_f64(k)
    vf = bf16_bits_to_f64(v)
    wqf = bf16_bits_to_f64(wq)
    wkf = bf16_bits_to_f64(wk)
    B = qf.shape[0]
    q_f64 = np.empty_like(qf)
    k_f64 = np.empty_like(kf)
    slots = np.zeros((B, 2), dtype=np.int64)
    for b in range(B):
        pos = int(positions[b])
        q_f64[b] = qk_transform(qf[b], wqf, pos, theta, eps, norm_before_rope)
        k_f64[b] = qk_transform(kf[b], wkf, pos, theta, eps, norm_before_rope)
        slots[b] = cache_slot(block_table[b], pos)
    out = {"q_f64": q_f64, "q_out": f64_to_bf16_bits(q_f64), "k_f64": k_f64,
           "slots": slots}
    if kv_dtype == "bf16":
        out["k_pre"], out["v_pre"] = k_f64, vf
        out["k_store"] = f64_to_bf16_bits(k_f64)
        out["v_store"] = np.asarray(v, dtype=np.uint16).copy()   # exact: v is already BF16
    elif kv_dtype == "fp8":
        out["k_pre"], out["v_pre"] = k_f64 / k_scale, vf / v_scale
        out["k_store"] = f64_to_e4m3(out["k_pre"])
        out["v_store"] = f64_to_e4m3(out["v_pre"])
    else:
        raise ValueError(kv_dtype)
    return out


def encode_output(o, out_dtype="bf16", out_scale=1.0):
    """The stored attention output (R10, R21): BF16 bits of o, or -- FP8 output,
    page B "Code analysis 1" (the output dtype is passed explicitly) -- the E4M3
    codes of o / out_scale, clamped to +-448 and rounded to nearest even."""
    o = np.asarray(o, dtype=np.float64)
    if out_dtype == "bf16":
        return f64_to_bf16_bits(o)
    if out_dtype == "fp8":
        return f64_to_e4m3(o / out_scale)
    raise ValueError(out_dtype)


def decode_values(stored, kv_dtype, scale):
    """Cache contents -> fp64 values (BF16 exact; E4M3 times its scale)."""
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(stored)
    return e4m3_to_f64(stored) * scale


def apply_prologue_writes(k_pool, v_pool, pro, *, kv_dtype, page_stride, head_stride):
    """Write each new token's k and v into (copies of) the pools, in place."""
    B, Hkv, D = pro["k_store"].shape
    r_idx = np.arange(D)
    for b in range(B):
        page, row = pro["slots"][b]
        for g in range(Hkv):
            base = page * page_stride + g * head_stride
            k_pool[base + tile_offset("k", kv_dtype, row, r_idx)] = pro["k_store"][b, g]
            v_pool[base + tile_offset("v", kv_dtype, row, r_idx)] = pro["v_store"][b, g]


def gather_kv(pool, kind, kv_dtype, block_row, length, g, *, page_stride,
              head_stride, scale=1.0):
    """Rows [0, length) of KV head g of one sequence, decoded to fp64 [length, D]."""
    rows = np.arange(length)
    pages = np.asarray(block_row, dtype=np.int64)[rows // PAGE_SIZE]
    base = pages * page_stride + g * head_stride               # [length]
    off = tile_offset(kind, kv_dtype, (rows % PAGE_SIZE)[:, None],
                      np.arange(HEAD_DIM)[None, :])           # [length, D]
    stored = np.asarray(pool)[base[:, None] + off]
    return decode_values(stored, kv_dtype, scale)


def _sequence_kv(pools, pro, b, g, seq_lens, block_table, cfg):
    """K and V rows of sequence b, head g, after the prologue's writes.

    The pools are the caches *before* the step; every slot the prologue wrote
    that falls inside this sequence's pages is replaced by the stored value.
    """
    k_pool, v_pool = pools
    L = int(seq_lens[b])
    kd = dict(page_stride=cfg["page_stride"], head_stride=cfg["head_stride"])
    K = gather_kv(k_pool, "k", cfg["kv_dtype"], block_table[b], L, g, scale=cfg["k_scale"], **kd)
    V = gather_kv(v_pool, "v", cfg["kv_dtype"], block_table[b], L, g, scale=cfg["v_scale"], **kd)
    if pro is not None:
        n_b = (L + PAGE_SIZE - 1) // PAGE_SIZE
        row_pages = np.asarray(block_table[b][:n_b], dtype=np.int64)
        for bb in range(pro["slots"].shape[0]):
            page, row = pro["slots"][bb]
            for t in np.nonzero(row_pages == page)[0]:
                j = int(t) * PAGE_SIZE + int(row)
                if j < L:
                    K[j] = decode_values(pro["k_store"][bb, g], cfg["kv_dtype"], cfg["k_scale"])
                    V[j] = decode_values(pro["v_store"][bb, g], cfg["kv_dtype"], cfg["v_scale"])
    return K, V


def decode_attention(q_out_bits, pools, pro, seq_lens, block_table, cfg,
                     seqs=None, heads=None):
    """Full-softmax decode attention for the requested (sequence, q head) pairs.

    q_out_bits: [B, Hq, D] BF16 bits of the rotated, normalised queries.
    cfg: dict with kv_dtype, k_scale, v_scale, sm_scale, page_stride,
    head_stride, num_kv_heads.  Returns {(b, h): (o [D], lse)} in fp64.
    """
    B, Hq, D = q_out_bits.shape
    G = Hq // cfg["num_kv_heads"]
    seqs = range(B) if seqs is None else seqs
    result = {}
    for b in seqs:
        hs = range(Hq) if heads is None else heads
        by_group = {}
        for h in hs:
            by_group.setdefault(h // G, []).append(h)
        for g, hlist in by_group.items():
            K, V = _sequence_kv(pools, pro, b, g, seq_lens, block_table, cfg)
            qg = query_values(q_out_bits[b, hlist], cfg)
            o, lse = attend_full(qg, K, V, cfg["sm_scale"])
            for i, h in enumerate(hlist):
                result[(b, h)] = (o[i], lse[i])
    return result


def split_attention(q_out_bits, pools, pro, seq_lens, block_table, cfg, plan):
    """Attention computed per chunk of ``plan`` and merged (R13).

    Returns (o [B, Hq, D], lse [B, Hq], partials) where partials[c] is
    (o_c [Hq, D], lse_c [Hq]) for chunk c.  Must equal ``decode_attention``.
    """
    B, Hq, D = q_out_bits.shape
    Hkv = cfg["num_kv_heads"]
    G = Hq // Hkv
    o = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    partials = {}
    for b in range(B):
        kv = [_sequence_kv(pools, pro, b, g, seq_lens, block_table, cfg) for g in range(Hkv)]
        c_lo, c_hi = int(plan.seq_chunk[b]), int(plan.seq_chunk[b + 1])
        L = int(seq_lens[b])
        for c in range(c_lo, c_hi):
            _, t0, t1, _ = plan.chunks[c]
            j0, j1 = int(t0) * PAGE_SIZE, min(int(t1) * PAGE_SIZE, L)
            oc = np.zeros((Hq, D))
            lc = np.zeros(Hq)
            for g in range(Hkv):
                K, V = kv[g]
                qg = query_values(q_out_bits[b, g * G:(g + 1) * G], cfg)
                og, lg = attend_chunk(qg, K[j0:j1], V[j0:j1], cfg["sm_scale"])
                oc[g * G:(g + 1) * G] = og
                lc[g * G:(g + 1) * G] = lg
            partials[c] = (oc, lc)
        po = np.stack([partials[c][0] for c in range(c_lo, c_hi)])
        pl = np.stack([partials[c][1] for c in range(c_lo, c_hi)])
        o[b], lse[b] = combine_lse(po, pl)
    return o, lse, partials


def make_plan(seq_lens, sched, num_workers, static_splits=0, xcd_weights=None):
    """Dynamic (optionally XCD-weighted) or static plan (static_splits 0 -> the default S)."""
    if sched == "dynamic":
        return plan_dynamic(seq_lens, num_workers, xcd_weights)
    S = static_splits or max(1, int(num_workers) // len(seq_lens))
    return plan_static(seq_lens, S)
