"""Multi-token decode steps (several new tokens per sequence), in fp64.

Page A, "Two new HPC backends in the vLLM ecosystem": the model carries a
speculative-decoding (MTP) layer.  Verifying drafted tokens means that one
decode step brings several new tokens per sequence, which attend to the cache
and, causally, to each other.

Reading R20: every sequence of the step has the same number Tq of new tokens
(Tq = 1 is the ordinary step).  L_b counts all of them; new token j (0-based)
of sequence b sits at position L_b - Tq + j, is rotated with that position,
has its k and v written to that slot, and attends rows [0, L_b - Tq + j]:
the prefix and new tokens 0..j.  Arrays of new tokens are token-major:
q [B, Tq, Hq, D], k and v [B, Tq, Hkv, D], positions [B, Tq]; outputs are
[B, Tq, Hq, D] and lse [B, Tq, Hq].

Ragged batches (R22, at the end of this module) give every sequence its own
number of new tokens, packed along one token axis.

The prologue and the per-sequence KV gather are the single-token ones applied
to the flattened token list (``step.prologue`` / ``step._sequence_kv``); what
is new here is the causal limit per token and the chunk partial of a token
that has no rows in a chunk: it is empty, with o = 0 and lse = -inf, and the
log-sum-exp merge gives it weight 0.
"""

import numpy as np

from .qk import query_values
from .layout import PAGE_SIZE
from .attention import attend_full, combine_lse
from .step import prologue, _sequence_kv


def token_positions(seq_lens, tokens):
    """positions[b, j] = L_b - Tq + j (R20)."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    Tq = int(tokens)
    if Tq < 1 or np.any(lens < Tq):
        raise ValueError("every sequence must hold its Tq new tokens")
    return lens[:, None] - Tq + np.arange(Tq)[None, :]


def causal_limit(L, tokens, j):
    """Rows [0, limit) that new token j of a length-L sequence attends (R20)."""
    return int(L) - int(tokens) + int(j) + 1


def prologue_tokens(q, k, v, positions, wq, wk, block_table, **kw):
    """The fused prologue on every new token: the single-token prologue over the
    token-major flattened list, each token using its own sequence's table row.

    Returns the prologue dict with arrays over B * Tq tokens (token b*Tq + j).
    """
    q = np.asarray(q)
    B, Tq = q.shape[0], q.shape[1]
    flat = lambda a: np.asarray(a).reshape((B * Tq,) + np.asarray(a).shape[2:])
    bt = np.repeat(np.asarray(block_table), Tq, axis=0)
    return prologue(flat(q), flat(k), flat(v), np.asarray(positions).reshape(-1), wq, wk, bt,
                    **kw)


def decode_attention_tokens(q_out_bits, pools, pro, seq_lens, block_table, cfg,
                            seqs=None, heads=None):
    """Full-softmax attention of every new token over its causal prefix (R20).

    q_out_bits: [B, Tq, Hq, D] BF16 bits.  Returns {(b, j, h): (o [D], lse)}.
    """
    B, Tq, Hq, D = q_out_bits.shape
    G = Hq // cfg["num_kv_heads"]
    result = {}
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        hs = range(Hq) if heads is None else heads
        by_group = {}
        for h in hs:
            by_group.setdefault(h // G, []).append(h)
        for g, hlist in by_group.items():
            K, V = _sequence_kv(pools, pro, b, g, seq_lens, block_table, cfg)
            for j in range(Tq):
                lim = causal_limit(L, Tq, j)
                o, lse = attend_full(query_values(q_out_bits[b, j, hlist], cfg), K[:lim],
                                     V[:lim], cfg["sm_scale"])
                for i, h in enumerate(hlist):
                    result[(b, j, h)] = (o[i], lse[i])
    return result


def chunk_partial(q, K, V, row0, row1, limit, sm_scale):
    """Partial result of one chunk (rows [row0, row1)) for one token whose
    causal limit is `limit`: attention over rows [row0, min(row1, limit)), or
    the empty partial (o = 0, lse = -inf) when that range is empty."""
    r1 = min(row1, limit)
    if r1 <= row0:
        q = np.asarray(q)
        return np.zeros(q.shape), np.full(q.shape[0], -np.inf)
    return attend_full(q, K[row0:r1], V[row0:r1], sm_scale)


def split_attention_tokens(q_out_bits, pools, pro, seq_lens, block_table, cfg, plan):
    """Per-chunk partials of every new token, merged (R13, R20).

    Returns (o [B, Tq, Hq, D], lse [B, Tq, Hq], partials) with partials[c] =
    (o_c [Tq, Hq, D], lse_c [Tq, Hq]).  Must equal ``decode_attention_tokens``.
    """
    B, Tq, Hq, D = q_out_bits.shape
    Hkv = cfg["num_kv_heads"]
    G = Hq // Hkv
    o = np.zeros((B, Tq, Hq, D))
    lse = np.zeros((B, Tq, Hq))
    partials = {}
    for b in range(B):
        kv = [_sequence_kv(pools, pro, b, g, seq_lens, block_table, cfg) for g in range(Hkv)]
        c_lo, c_hi = int(plan.seq_chunk[b]), int(plan.seq_chunk[b + 1])
        L = int(seq_lens[b])
        for c in range(c_lo, c_hi):
            _, t0, t1, _ = plan.chunks[c]
            row0, row1 = int(t0) * PAGE_SIZE, min(int(t1) * PAGE_SIZE, L)
            oc = np.zeros((Tq, Hq, D))
            lc = np.zeros((Tq, Hq))
            for g in range(Hkv):
                K, V = kv[g]
                for j in range(Tq):
                    qg = query_values(q_out_bits[b, j, g * G:(g + 1) * G], cfg)
                    og, lg = chunk_partial(qg, K, V, row0, row1, causal_limit(L, Tq, j),
                                           cfg["sm_scale"])
                    oc[j, g * G:(g + 1) * G] = og
                    lc[j, g * G:(g + 1) * G] = lg
            partials[c] = (oc, lc)
        po = np.stack([partials[c][0] for c in range(c_lo, c_hi)])   # [C, Tq, Hq, D]
        pl = np.stack([partials[c][1] for c in range(c_lo, c_hi)])   # [C, Tq, Hq]
        for j in range(Tq):
            o[b, j], lse[b, j] = combine_lse(po[:, j], pl[:, j])
    return o, lse, partials


# ---------------------------------------------------------------------------
# Ragged batches (reading R22): sequence b has its own count n_b >= 0 of new
# tokens.  The new tokens of all sequences are packed along one axis: those of
# sequence b are rows q_start[b] .. q_start[b+1]-1, q_start being the running
# sum of the counts.  New token j of sequence b sits at position L_b - n_b + j
# and attends rows [0, L_b - n_b + j], exactly as R20 with Tq = n_b.

def query_starts(new_tokens):
    """q_start[b] = n_0 + ... + n_{b-1}, b = 0..B (so q_start[B] = N)."""
    counts = np.asarray(new_tokens, dtype=np.int64)
    if np.any(counts < 0):
        raise ValueError("negative new-token count")
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def varlen_positions(seq_lens, new_tokens):
    """Packed positions: the new tokens of sequence b are L_b - n_b, ..., L_b - 1."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    counts = np.asarray(new_tokens, dtype=np.int64)
    if np.any(lens < counts):
        raise ValueError("every sequence must hold its new tokens")
    out = [np.arange(L - n, L) for L, n in zip(lens, counts)]
    return np.concatenate(out + [np.zeros(0, dtype=np.int64)])


def prologue_varlen(q, k, v, positions, new_tokens, wq, wk, block_table, **kw):
    """The fused prologue on the packed tokens [N, H, D]: the single-token
    prologue, each token with its own sequence's block-table row."""
    seq = np.repeat(np.arange(len(new_tokens)), np.asarray(new_tokens, dtype=np.int64))
    bt = np.asarray(block_table)[seq]
    return prologue(np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(positions), wq, wk,
                    bt, **kw)


def attention_varlen(q_out_bits, pools, pro, seq_lens, new_tokens, block_table, cfg,
                     seqs=None, heads=None, tokens=None):
    """Full-softmax attention of every packed new token over its causal prefix.

    q_out_bits: [N, Hq, D] BF16 bits.  tokens: optional per-sequence lists of
    token indices j to compute (all by default).  Returns {(b, j, h): (o, lse)}.
    """
    Hq = q_out_bits.shape[1]
    G = Hq // cfg["num_kv_heads"]
    starts = query_starts(new_tokens)
    result = {}
    for b in (range(len(new_tokens)) if seqs is None else seqs):
        L, n = int(seq_lens[b]), int(new_tokens[b])
        js = range(n) if tokens is None else tokens[b]
        by_group = {}
        for h in (range(Hq) if heads is None else heads):
            by_group.setdefault(h // G, []).append(h)
        for g, hlist in by_group.items():
            K, V = _sequence_kv(pools, pro, b, g, seq_lens, block_table, cfg)
            for j in js:
                lim = causal_limit(L, n, j)
                row = int(starts[b]) + j
                o, lse = attend_full(query_values(q_out_bits[row, hlist], cfg), K[:lim],
                                     V[:lim], cfg["sm_scale"])
                for i, h in enumerate(hlist):
                    result[(b, j, h)] = (o[i], lse[i])
    return result
