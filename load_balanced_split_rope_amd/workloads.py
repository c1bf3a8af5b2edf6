"""Seeded synthetic decode-step inputs.

This module only draws random inputs of the right shapes; it holds none of
the step's arithmetic (no RoPE, norm, quantiser, layout or schedule), so both
the HIP library's tests and the fp64 oracle can use it.  Conversions of the
random draws to BF16 and FP8 E4M3 use torch's own dtype casts.

Workloads (shapes of the model the pages name: 64 query heads, 8 KV heads,
head dim 128; 64-token pages):

* ``tiny``        batch 4, lengths {1, 63, 64, 200}, 8 q heads / 1 KV head, BF16
* ``uniform``     batch 32, every length 4096, 64/8 heads, BF16
* ``mix``         1 x 131072 + 31 x 4096, 64/8 heads, BF16
* ``mix_fp8``     the same mix with an FP8 E4M3 cache (k scale 2**-5, v scale 2**-4)
* ``loguniform``  batch 64, lengths log-uniform in [512, 262144], FP8 E4M3
* ``mix_mtp2``    the BF16 mix with 2 new tokens per sequence (multi-token
                  decode, as when one drafted token is verified)
* ``mix_mtp4``    the same with 4 new tokens per sequence (three drafted)
* ``prefill``     prefill of 4 prompts of 8192 tokens (every token is new), BF16
* ``prefill_fp8`` the same with an FP8 E4M3 cache
* ``chunked_prefill``  32 sequences of 4608 tokens whose last 512 are new
                  (a 512-token prefill chunk after a 4096-token prefix)
* ``ragged_prefill``  8 prompts with their own chunk lengths (8192, 4096,
                  2048, 1024, 512, 3072, 6144, 700 new tokens) after prefixes
                  of 0, 4096, 0, 8192, 0, 1024, 0, 20000 tokens (packed)
* ``mixed_prefill``  the prefill half of a mixed batch: 4 sequences each
                  prefilling 1024 new tokens after 8192 cached (packed)

Recipe (per workload, seed s): ``numpy.random.SeedSequence(s)`` spawns child
streams, in order: 0 lengths (unused: fixed lists, or for ``loguniform``
``default_rng(5)`` itself), 1 q, 2 k, 3 v, 4 q-norm weight, 5 k-norm weight,
6 page permutation, 7 K-cache contents, 8 V-cache contents.  q, k, v and the
cache values are N(0, 1); norm weights are 1 + 0.1 N(0, 1); all rounded to
BF16 (the cache to E4M3 after dividing by its scale).  The pool has
T + max(16, ceil(T/16)) pages; sequence b gets pages perm[cu[b]:cu[b+1]] of a
random permutation; unused block-table entries are -1; positions[b] = L_b - 1.
With Tq > 1 new tokens per sequence, q, k and v gain a token axis after the
batch axis (drawn as [B, Tq, H, D], so Tq = 1 draws the same values) and
positions[b, j] = L_b - Tq + j.  A ragged batch (new_tokens = [n_b]) packs
its N = sum n_b new tokens along one axis: q, k, v drawn as [N, H, D],
positions[q_start[b] + j] = L_b - n_b + j, q_start the prefix sums of n_b.
On a GPU the cache contents (up to 5.7 GB) are drawn on the device with a
torch generator seeded from children 7 and 8, in fixed 2**26-element blocks.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

PAGE = 64
HEAD_DIM = 128
TILE = PAGE * HEAD_DIM


@dataclass
class Workload:
    name: str
    seq_lens: list
    num_q_heads: int = 64
    num_kv_heads: int = 8
    kv_dtype: str = "bf16"
    k_scale: float = 1.0
    v_scale: float = 1.0
    rope_theta: float = 1e4
    rms_eps: float = 1e-6
    norm_before_rope: bool = False
    seed: int = 0
    tokens: int = 1            # new tokens per sequence (multi-token decode)
    new_tokens: list = None    # per-sequence new-token counts of a ragged (varlen) batch
    extra: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.seq_lens)

    @property
    def tiles(self):
        return [-(-int(L) // PAGE) for L in self.seq_lens]

    @property
    def varlen(self):
        return self.new_tokens is not None

    @property
    def max_new_tokens(self):
        """The bound on any sequence's new tokens (a ragged batch's tokens_per_seq)."""
        return max(1, max(self.new_tokens)) if self.varlen else self.tokens


def loguniform_lengths(seed, batch=64, lo=512, hi=262144):
    """Lengths rint(exp(U(ln lo, ln hi))), clipped, drawn by default_rng(seed)
    itself rather than a spawned child: with seed 5 this is the batch of
    2,771,856 tokens in 43,341 pages the log-uniform workload is quoted on."""
    u = np.random.default_rng(seed).uniform(np.log(lo), np.log(hi), batch)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64).tolist()


def named(name):
    """The named workloads listed above."""
    if name == "tiny":
        return Workload("tiny", [1, 63, 64, 200], num_q_heads=8, num_kv_heads=1, seed=1)
    if name == "uniform":
        return Workload("uniform", [4096] * 32, seed=2)
    if name == "mix":
        return Workload("mix", [131072] + [4096] * 31, seed=3)
    if name == "mix_fp8":
        return Workload("mix_fp8", [131072] + [4096] * 31, kv_dtype="fp8",
                        k_scale=2.0 ** -5, v_scale=2.0 ** -4, seed=4)
    if name == "loguniform":
        return Workload("loguniform", loguniform_lengths(5), kv_dtype="fp8",
                        k_scale=2.0 ** -5, v_scale=2.0 ** -4, seed=5)
    if name == "mix_mtp2":
        return Workload("mix_mtp2", [131072] + [4096] * 31, seed=6, tokens=2)
    if name == "mix_mtp4":
        return Workload("mix_mtp4", [131072] + [4096] * 31, seed=7, tokens=4)
    if name == "prefill":
        return Workload("prefill", [8192] * 4, seed=8, tokens=8192)
    if name == "prefill_fp8":
        return Workload("prefill_fp8", [8192] * 4, kv_dtype="fp8", k_scale=2.0 ** -5,
                        v_scale=2.0 ** -4, seed=9, tokens=8192)
    if name == "chunked_prefill":
        return Workload("chunked_prefill", [4608] * 32, seed=10, tokens=512)
    if name == "ragged_prefill":
        new = [8192, 4096, 2048, 1024, 512, 3072, 6144, 700]
        prefix = [0, 4096, 0, 8192, 0, 1024, 0, 20000]
        return Workload("ragged_prefill", [p + n for p, n in zip(prefix, new)], seed=11,
                        new_tokens=new)
    if name == "mixed_prefill":
        # the prefill half of a mixed batch: 4 sequences each prefilling a
        # 1024-token chunk after 8192 cached tokens (ragged call)
        return Workload("mixed_prefill", [9216] * 4, seed=12, new_tokens=[1024] * 4)
    raise KeyError(name)


NAMES = ("tiny", "uniform", "mix", "mix_fp8", "loguniform")
MULTI_TOKEN_NAMES = ("mix_mtp2", "mix_mtp4")
PREFILL_NAMES = ("prefill", "prefill_fp8", "chunked_prefill", "ragged_prefill")


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _fill_pool(out, children, scale, kv_dtype, device):
    """Fill a flat pool tensor (bf16 or uint8 codes) with N(0,1) draws."""
    n = out.numel()
    seed = int(children.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)
    if device.type == "cpu":
        vals = np.random.default_rng(children).standard_normal(n, dtype=np.float32)
        t = torch.from_numpy(vals)
        if kv_dtype == "bf16":
            out.copy_(t.to(torch.bfloat16))
        else:
            out.copy_((t / scale).clamp_(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8))
        return
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    block = 1 << 26
    for s in range(0, n, block):
        m = min(block, n - s)
        v = torch.randn(m, generator=gen, device=device, dtype=torch.float32)
        if kv_dtype == "bf16":
            out[s:s + m].copy_(v.to(torch.bfloat16))
        else:
            out[s:s + m].copy_((v / scale).clamp_(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8))


def make_inputs(w: Workload, device="cpu", spare_pages=None, kv_interleave=False):
    """Draw one step's inputs for workload ``w`` on ``device``.

    Returns a dict of tensors: q [B,Hq,D] bf16, k/v [B,Hkv,D] bf16 (with a
    token axis, [B,Tq,H,D], when w.tokens > 1), q_norm_w/k_norm_w [D] bf16,
    positions [B] int32 ([B,Tq] when w.tokens > 1), seq_lens [B] int32,
    block_table [B, max_blocks] int32, k_cache/v_cache flat pools (bf16 or
    uint8 E4M3 codes) of num_pages * Hkv * 8192 elements, and metadata.

    kv_interleave: K and V share one allocation, the V tile of every (page,
    KV head) right after its K tile (head stride 16384, page stride
    Hkv * 16384 elements); k_cache and v_cache are views 8192 elements apart.
    """
    device = torch.device(device)
    ss = np.random.SeedSequence(w.seed).spawn(9)
    B, Hq, Hkv, D = w.batch, w.num_q_heads, w.num_kv_heads, HEAD_DIM
    lens = np.asarray(w.seq_lens, dtype=np.int64)
    n = np.asarray(w.tiles, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(n)])
    T = int(cu[-1])
    spare = max(16, -(-T // 16)) if spare_pages is None else int(spare_pages)
    num_pages = T + spare
    perm = np.random.default_rng(ss[6]).permutation(num_pages)
    max_blocks = int(n.max())
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    for b in range(B):
        bt[b, :n[b]] = perm[cu[b]:cu[b + 1]]
    if w.varlen:
        counts = np.asarray(w.new_tokens, dtype=np.int64)
        if counts.shape != (B,) or np.any(counts < 0) or np.any(lens < counts):
            raise ValueError("every sequence must hold its new tokens")
        q_start = np.concatenate([[0], np.cumsum(counts)])
        N = int(q_start[-1])
        q = np.random.default_rng(ss[1]).standard_normal((N, Hq, D), dtype=np.float32)
        k = np.random.default_rng(ss[2]).standard_normal((N, Hkv, D), dtype=np.float32)
        v = np.random.default_rng(ss[3]).standard_normal((N, Hkv, D), dtype=np.float32)
        positions = np.concatenate([np.arange(L - n, L) for L, n in zip(lens, counts)]
                                   + [np.zeros(0, dtype=np.int64)])
    else:
        Tq = int(w.tokens)
        if Tq < 1 or np.any(lens < Tq):
            raise ValueError("every sequence must hold its new tokens")
        shape = (lambda H: (B, H, D)) if Tq == 1 else (lambda H: (B, Tq, H, D))
        q = np.random.default_rng(ss[1]).standard_normal((B, Tq, Hq, D), dtype=np.float32).reshape(shape(Hq))
        k = np.random.default_rng(ss[2]).standard_normal((B, Tq, Hkv, D), dtype=np.float32).reshape(shape(Hkv))
        v = np.random.default_rng(ss[3]).standard_normal((B, Tq, Hkv, D), dtype=np.float32).reshape(shape(Hkv))
        positions = (lens - 1) if Tq == 1 else lens[:, None] - Tq + np.arange(Tq)[None, :]
    wq = 1 + 0.1 * np.random.default_rng(ss[4]).standard_normal(D, dtype=np.float32)
    wk = 1 + 0.1 * np.random.default_rng(ss[5]).standard_normal(D, dtype=np.float32)
    pool_elems = num_pages * Hkv * TILE
    cache_dtype = torch.bfloat16 if w.kv_dtype == "bf16" else torch.uint8
    if kv_interleave:
        both = torch.empty(2 * pool_elems, dtype=cache_dtype, device=device)
        tiles = both.view(num_pages * Hkv, 2, TILE)
        k_tmp = torch.empty(pool_elems, dtype=cache_dtype, device=device)
        _fill_pool(k_tmp, ss[7], w.k_scale, w.kv_dtype, device)
        tiles[:, 0].copy_(k_tmp.view(-1, TILE))
        _fill_pool(k_tmp, ss[8], w.v_scale, w.kv_dtype, device)
        tiles[:, 1].copy_(k_tmp.view(-1, TILE))
        del k_tmp
        k_cache = both[:2 * pool_elems - TILE]
        v_cache = both[TILE:]
        page_stride, head_stride = 2 * Hkv * TILE, 2 * TILE
    else:
        k_cache = torch.empty(pool_elems, dtype=cache_dtype, device=device)
        v_cache = torch.empty(pool_elems, dtype=cache_dtype, device=device)
        _fill_pool(k_cache, ss[7], w.k_scale, w.kv_dtype, device)
        _fill_pool(v_cache, ss[8], w.v_scale, w.kv_dtype, device)
        page_stride, head_stride = Hkv * TILE, TILE
    return {
        "q": _bf16(q).to(device), "k": _bf16(k).to(device), "v": _bf16(v).to(device),
        "q_norm_w": _bf16(wq).to(device), "k_norm_w": _bf16(wk).to(device),
        "positions": torch.from_numpy(np.ascontiguousarray(positions, dtype=np.int32)).to(device),
        "seq_lens": torch.from_numpy(lens.astype(np.int32)).to(device),
        "block_table": torch.from_numpy(bt).to(device),
        "k_cache": k_cache, "v_cache": v_cache,
        "num_pages": num_pages, "page_stride": page_stride, "head_stride": head_stride,
        "max_blocks": max_blocks, "total_tiles": T, "tokens": w.max_new_tokens,
        **({"q_start": torch.from_numpy(q_start.astype(np.int32)).to(device),
            "total_tokens": N} if w.varlen else {}),
    }


def custom(seq_lens, num_q_heads=64, num_kv_heads=8, kv_dtype="bf16", seed=0, **kw):
    """A workload with explicit lengths (for tests); FP8 defaults to scales 2**-5 / 2**-4."""
    if kv_dtype == "fp8":
        kw.setdefault("k_scale", 2.0 ** -5)
        kw.setdefault("v_scale", 2.0 ** -4)
    return Workload(f"custom{seed}", list(map(int, seq_lens)), num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, kv_dtype=kv_dtype, seed=seed, **kw)
