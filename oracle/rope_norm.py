"""RoPE and QK-Norm (RMSNorm) in fp64.

Page A, "Why does dynamic scheduling matter in attention?", and page B,
"Code analysis 2": the prologue applies a RoPE rotation and QK-Norm to the new
token and writes the KV cache, in that order, as one fused pass.  The pages
name neither the RoPE variant nor the norm's formula; the readings are:

* R1 -- rotate-half ("NeoX") RoPE over the whole head dimension D: channel i
  pairs with channel i + D/2, frequency w_i = theta**(-2i/D), angle pos*w_i.
* R2 -- RoPE first, then the norm (the order the pages list the operations
  in).  ``norm_before_rope`` selects the other order.  RoPE is an isometry and
  the RMS is rotation invariant, so the two orders differ only through the
  per-channel weight; with weight 1 they agree exactly.  Which order the
  pages mean is parity unpinned (they do not say); the composition of each
  order is pinned by an invariant it alone satisfies for any weights (norm
  last: y / w has the RMS of a normalised vector; RoPE last: so does y
  rotated back, divided by w).
* R3 -- RMSNorm y = x / sqrt(mean(x**2) + eps) * w, eps inside the root, one
  weight vector of length D for all q heads and one for all k heads.
* R4 -- v is neither rotated nor normalised.
"""

import numpy as np


def rope_neox(x, pos, theta):
    """Rotate-half RoPE of ``x[..., D]`` at integer position ``pos`` (R1).

    out[i]       = x[i] cos(a_i) - x[i + D/2] sin(a_i)
    out[i + D/2] = x[i + D/2] cos(a_i) + x[i] sin(a_i),   a_i = pos * theta**(-2i/D)
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    omega = np.power(float(theta), -2.0 * i / d)
    a = float(pos) * omega
    c, s = np.cos(a), np.sin(a)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rms_norm(x, w, eps):
    """RMSNorm over the last axis (R3): x / sqrt(mean(x**2) + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(w, dtype=np.float64)


def qk_transform(x, w, pos, theta, eps, norm_before_rope=False):
    """The q/k part of the prologue for one token: RoPE then RMSNorm (R2)."""
    if norm_before_rope:
        return rope_neox(rms_norm(x, w, eps), pos, theta)
    return rms_norm(rope_neox(x, pos, theta), w, eps)
