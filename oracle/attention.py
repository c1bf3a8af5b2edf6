"""Decode attention for one sequence and one KV head, in fp64.

Page A, "Two new HPC backends in the vLLM ecosystem": 64 query heads share 8
KV heads (head dim 128), i.e. groups of 8 query heads read one KV head (R7:
query head h uses KV head floor(h / G), G = Hq / Hkv).  Page A, "Why does
dynamic scheduling matter in attention?": the KV range of a sequence may be
split across compute units (split-KV), which implies the partial results are
merged afterwards; the merge is the usual log-sum-exp one (R13).

Reading R8: scores are sigma * <q, k> with sigma = 1/sqrt(D); no soft-cap,
window, ALiBi or sink terms.  The oracle computes the *full* softmax; the
split form below is the definition of a partial result plus its merge, used
to check that splitting changes nothing.
"""

import numpy as np


def attend_full(q, k, v, sm_scale):
    """Full-softmax attention of G query rows over L keys.

    q: [G, D]; k, v: [L, D] (already decoded and scaled).  Returns
    (o [G, D], lse [G]) with o = softmax(sm_scale * q k^T) v and
    lse = ln sum_j exp(sm_scale * <q, k_j>), both in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] < 1:
        raise ValueError("attention needs at least one key")
    s = sm_scale * (q @ k.T)                     # [G, L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    denom = p.sum(axis=1, keepdims=True)
    o = (p @ v) / denom
    lse = m[:, 0] + np.log(denom[:, 0])
    return o, lse


def attend_chunk(q, k, v, sm_scale):
    """A split's partial result: attention restricted to the split's keys."""
    return attend_full(q, k, v, sm_scale)


def combine_lse(partial_o, partial_lse):
    """Merge partial results (R13), in ascending split order.

    partial_o: [C, G, D]; partial_lse: [C, G].  With M = max_c lse_c:
    lse = M + ln sum_c exp(lse_c - M) and o = sum_c exp(lse_c - lse) o_c.
    """
    po = np.asarray(partial_o, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    m = pl.max(axis=0)
    w = np.exp(pl - m)                           # [C, G]
    lse = m + np.log(w.sum(axis=0))
    o = np.zeros(po.shape[1:], dtype=np.float64)
    for c in range(po.shape[0]):                 # ascending order, as stated
        o += np.exp(pl[c] - lse)[:, None] * po[c]
    return o, lse
