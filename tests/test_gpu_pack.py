"""lbsr_pack_cache / lbsr_unpack_cache against the oracle's restatement of the
tile layout: a row-major cache (token-major or head-major, contiguous or with
padded strides) packed on the GPU must equal, bit for bit, the pool that
oracle.layout.tile_offset places each element in, for K and V, BF16 and FP8,
into the default pool layout and into one with K and V interleaved; and
unpacking must give the rows back bit for bit.  Byte movement only, so the
bar is exact; the data are random bit patterns (NaN codes included)."""

import numpy as np
import pytest
import torch

import load_balanced_split_rope_amd as lb
from oracle.layout import tile_offset, PAGE_SIZE, HEAD_DIM
from gpu_util import device

pytestmark = pytest.mark.gpu

TILE = PAGE_SIZE * HEAD_DIM


def cfg_for(dtype, pages, heads, page_stride=None, head_stride=None):
    return lb.DecodeConfig(heads * 8, heads, dtype, 4, pages,
                           page_stride=page_stride or heads * TILE, head_stride=head_stride or TILE)


def random_rows(dtype, pages, heads, layout, pad, seed):
    """Row-major cache [pages, 64, H, 128] (NHD) or [pages, H, 64, 128] (HND) of
    random bit patterns; pad > 0 makes it a view with padded rows."""
    rng = np.random.default_rng(seed)
    shape = [pages, PAGE_SIZE, heads, HEAD_DIM] if layout == "NHD" else \
        [pages, heads, PAGE_SIZE, HEAD_DIM]
    full = list(shape)
    full[3] += pad
    if dtype == "bf16":
        bits = rng.integers(0, 1 << 16, size=full, dtype=np.uint16).view(np.int16)
        t = torch.from_numpy(bits).view(torch.bfloat16)
    else:
        t = torch.from_numpy(rng.integers(0, 256, size=full, dtype=np.uint8))
    return t[..., :HEAD_DIM]


def as_bits(t):
    t = t.cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


def expected_pool(rows_nhd, kind, dtype, cfg):
    """The pool the oracle's layout puts rows_nhd [pages, 64, H, 128] in."""
    pages, _, heads, _ = rows_nhd.shape
    pool = np.zeros(cfg.pool_elems(), dtype=rows_nhd.dtype)
    r = np.arange(PAGE_SIZE)[:, None]
    d = np.arange(HEAD_DIM)[None, :]
    off = tile_offset(kind, dtype, r, d)                          # [64, 128]
    for p in range(pages):
        for g in range(heads):
            pool[p * cfg.page_stride + g * cfg.head_stride + off] = rows_nhd[p, :, g, :]
    return pool


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("layout,pad", [("NHD", 0), ("HND", 0), ("NHD", 32), ("HND", 64)])
def test_pack_matches_layout_and_unpack_restores(dtype, kind, layout, pad):
    dev = device()
    pages, heads = 37, 8
    cfg = cfg_for(dtype, pages, heads)
    seed = 100 * ["bf16", "fp8"].index(dtype) + 10 * ["k", "v"].index(kind) + pad
    rows = random_rows(dtype, pages, heads, layout, pad, seed=seed + (layout == "HND"))
    # on the device with the same (possibly padded) strides
    full = torch.empty(rows.shape[:3] + (HEAD_DIM + pad,), dtype=rows.dtype, device=dev)
    rows_d = full[..., :HEAD_DIM]
    rows_d.copy_(rows.to(dev))
    cache = torch.empty(cfg.pool_elems(), dtype=cfg.cache_dtype, device=dev)
    print(f"pack {dtype} {kind} {layout} pad {pad}: strides {rows_d.stride()}", flush=True)
    lb.pack_cache(cfg, kind, rows_d, cache, layout=layout)
    torch.cuda.synchronize()
    nhd = as_bits(rows) if layout == "NHD" else as_bits(rows).transpose(0, 2, 1, 3)
    assert np.array_equal(as_bits(cache), expected_pool(nhd, kind, dtype, cfg))
    back = torch.empty_like(rows_d)
    if dtype == "bf16":
        back.view(torch.int16).fill_(0x7FC1)
    else:
        back.fill_(0x7F)
    lb.unpack_cache(cfg, kind, cache, back, layout=layout)
    torch.cuda.synchronize()
    assert np.array_equal(as_bits(back), as_bits(rows))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_pack_into_interleaved_pools(dtype):
    """K and V packed into one allocation with each (page, head)'s V tile right
    after its K tile: each call writes only its own kind's tiles."""
    dev = device()
    pages, heads = 19, 4
    cfg = cfg_for(dtype, pages, heads, page_stride=2 * heads * TILE, head_stride=2 * TILE)
    rk = random_rows(dtype, pages, heads, "NHD", 0, seed=11)
    rv = random_rows(dtype, pages, heads, "NHD", 0, seed=12)
    n = cfg.pool_elems()
    both = torch.empty(n + TILE, dtype=cfg.cache_dtype, device=dev)
    lb.pack_cache(cfg, "k", rk.to(dev), both[:n], layout="NHD")
    lb.pack_cache(cfg, "v", rv.to(dev), both[TILE:], layout="NHD")
    torch.cuda.synchronize()
    tiles = as_bits(both).reshape(pages * heads, 2, TILE)
    # expected pools in each view's coordinates, padded to whole (K, V) pairs:
    # a view's tiles are its even ones
    pair = lambda e: np.concatenate([e, np.zeros(TILE, e.dtype)]).reshape(-1, 2, TILE)[:, 0]
    assert np.array_equal(tiles[:, 0], pair(expected_pool(as_bits(rk), "k", dtype, cfg)))
    assert np.array_equal(tiles[:, 1], pair(expected_pool(as_bits(rv), "v", dtype, cfg)))


def test_packed_cache_feeds_the_step():
    """A cache packed from rows on the GPU and the one the step tests build in
    the tile layout directly give the same step, bit for bit."""
    from load_balanced_split_rope_amd import workloads as wl
    from gpu_util import to_device, run_step
    dev = device()
    w = wl.custom([700, 64, 1, 130], num_q_heads=64, num_kv_heads=8, seed=1400)
    inp = wl.make_inputs(w)
    g = to_device(inp, dev)
    cfg = cfg_for("bf16", inp["num_pages"], 8)
    # the rows of the existing pools, by the oracle's layout (inverse of expected_pool)
    r = np.arange(PAGE_SIZE)[:, None]
    d = np.arange(HEAD_DIM)[None, :]
    g2 = to_device(inp, dev)
    for key, kind in (("k_cache", "k"), ("v_cache", "v")):
        pool = as_bits(inp[key])
        off = tile_offset(kind, "bf16", r, d)
        rows = np.stack([np.stack([pool[p * cfg.page_stride + h * TILE + off] for h in range(8)], 1)
                         for p in range(inp["num_pages"])])
        rows_t = torch.from_numpy(np.ascontiguousarray(rows)).view(torch.bfloat16).to(dev)
        g2[key] = torch.empty_like(g[key])
        lb.pack_cache(cfg, kind, rows_t, g2[key], layout="NHD")
    torch.cuda.synchronize()
    assert torch.equal(g2["k_cache"].view(torch.int16), g["k_cache"].view(torch.int16))
    a = run_step(w, g, lb.Schedule("dynamic", num_workers=256))
    b = run_step(w, g2, lb.Schedule("dynamic", num_workers=256))
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["lse"], b["lse"])
