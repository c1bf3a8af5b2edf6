"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-only parts (layout, validation) behave as documented.  Nothing here
launches a kernel."""

import ctypes
import os
import re

import pytest

from load_balanced_split_rope_amd import _binding as B
from load_balanced_split_rope_amd import DecodeConfig, Schedule, workspace_layout, LbsrError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "lbsr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lbsr_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("liblbsr.so is not built (run __graft_entry__.build())")
    return B.lib()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 11
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_strings(lib):
    assert lib.lbsr_abi_version() == 7
    for st in range(5):
        assert lib.lbsr_status_string(st).startswith(b"LBSR_")
    assert lib.lbsr_status_string(99) == b"unknown lbsr_status"


def cfg_mix():
    return DecodeConfig(64, 8, "bf16", max_blocks_per_seq=2048, num_pages=4300)


def test_workspace_layout_dynamic_and_static():
    lay = workspace_layout(cfg_mix(), 32, Schedule("dynamic", num_workers=256))
    assert lay.num_workers == 256 and lay.max_chunks == 256 + 31
    offs = [lay.error_word, lay.cu_tiles, lay.worker_chunk, lay.chunks, lay.seq_chunk,
            lay.seq_len_eff, lay.token_status, lay.partial_o, lay.partial_lse, lay.arrivals,
            lay.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.total - lay.arrivals >= 4 * 32 * 8
    assert lay.partial_lse - lay.partial_o >= 4 * 287 * 64 * 128
    st = workspace_layout(cfg_mix(), 32, Schedule("static", num_workers=256))
    assert st.static_splits == 8 and st.num_workers == 256 and st.max_chunks == 256
    st = workspace_layout(cfg_mix(), 32, Schedule("static", num_workers=256, static_splits=3))
    assert st.static_splits == 3 and st.num_workers == 96


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, B.E_UNSUPPORTED), ("page_size", 16, B.E_UNSUPPORTED),
    ("num_kv_heads", 3, B.E_INVALID), ("num_q_heads", 8 * 17, B.E_UNSUPPORTED),
    ("kv_dtype", 7, B.E_INVALID), ("max_blocks_per_seq", 0, B.E_INVALID),
    ("num_pages", 0, B.E_INVALID), ("page_stride", 100, B.E_INVALID),
    ("head_stride", 8192 * 1000, B.E_INVALID),
])
def test_shape_validation(lib, field, value, status):
    s = cfg_mix().shape()
    setattr(s, field, value)
    c = Schedule("dynamic", num_workers=256).cfg()
    out = B.WsLayout()
    got = lib.lbsr_workspace_layout(ctypes.byref(s), 32, ctypes.byref(c), ctypes.byref(out))
    assert got == status, lib.lbsr_last_error()
    assert lib.lbsr_last_error() != b""


def test_batch_and_schedule_validation(lib):
    s = cfg_mix().shape()
    out = B.WsLayout()
    for batch, cfg, status in [
        (0, B.SchedCfg(0, 256, 0, 0), B.E_INVALID),
        (20000, B.SchedCfg(0, 256, 0, 0), B.E_UNSUPPORTED),
        (32, B.SchedCfg(5, 256, 0, 0), B.E_INVALID),
        (32, B.SchedCfg(0, -1, 0, 0), B.E_INVALID),
        (32, B.SchedCfg(0, 256, 0, 2), B.E_INVALID),          # unknown flag bit
    ]:
        assert lib.lbsr_workspace_layout(ctypes.byref(s), batch, ctypes.byref(cfg),
                                         ctypes.byref(out)) == status


@pytest.mark.parametrize("kind,weights,status", [
    ("dynamic", None, B.OK),
    ("dynamic", (1,) * 8, B.OK),
    ("dynamic", (B.MAX_XCD_WEIGHT,) * 8, B.OK),
    ("dynamic", (9, 10, 9, 10, 9, 10, 9, 10), B.OK),
    ("dynamic", (1, 1, 1, 1, 1, 1, 1, 0), B.E_INVALID),        # some zero, some not
    ("dynamic", (1, 1, 1, 1, 1, 1, 1, -3), B.E_INVALID),
    ("dynamic", (1, 1, 1, 1, 1, 1, 1, B.MAX_XCD_WEIGHT + 1), B.E_INVALID),
    ("static", (1,) * 8, B.E_INVALID),                         # weights are dynamic-only
    ("static", None, B.OK),
])
def test_xcd_weight_validation(lib, kind, weights, status):
    s = cfg_mix().shape()
    c = Schedule(kind, num_workers=256, xcd_weights=weights).cfg()
    out = B.WsLayout()
    got = lib.lbsr_workspace_layout(ctypes.byref(s), 32, ctypes.byref(c), ctypes.byref(out))
    assert got == status, lib.lbsr_last_error()


def test_sched_cfg_struct_matches_header():
    """lbsr_sched_cfg is 4 int32 fields and the 8 XCD weights: 48 bytes."""
    assert ctypes.sizeof(B.SchedCfg) == 48
    assert B.SchedCfg.xcd_weight.offset == 16


def test_entry_points_reject_bad_pointers_before_any_launch(lib):
    """Null or misaligned pointers return LBSR_E_INVALID without touching a device."""
    s = cfg_mix().shape()
    p = cfg_mix().params()
    c = Schedule("dynamic", num_workers=256).cfg()
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x10002)
    assert lib.lbsr_plan(ctypes.byref(s), 32, nul, ctypes.byref(c), fake, 1 << 30, nul) == B.E_INVALID
    assert lib.lbsr_plan(ctypes.byref(s), 32, fake, ctypes.byref(c), odd, 1 << 30, nul) == B.E_INVALID
    assert lib.lbsr_plan(ctypes.byref(s), 32, fake, ctypes.byref(c), fake, 16, nul) == B.E_WORKSPACE
    # q, k, v, positions, q_norm_w, k_norm_w, block_table, k_cache, v_cache, q_out, error_word
    args = [fake] * 11
    args[9] = odd                          # q_out misaligned
    assert lib.lbsr_rope_norm_kv_write(ctypes.byref(s), ctypes.byref(p), 32, *args, nul) == B.E_INVALID
    args = [fake] * 11
    args[9] = args[0]                      # q_out aliases q
    assert lib.lbsr_rope_norm_kv_write(ctypes.byref(s), ctypes.byref(p), 32, *args, nul) == B.E_INVALID
    args = [fake] * 11
    args[3] = nul                          # positions missing
    assert lib.lbsr_rope_norm_kv_write(ctypes.byref(s), ctypes.byref(p), 32, *args, nul) == B.E_INVALID
    assert lib.lbsr_attention(ctypes.byref(s), ctypes.byref(p), 32, fake, fake, fake, fake,
                              ctypes.byref(c), fake, 1 << 30, nul, nul, nul) == B.E_INVALID


def test_params_validation(lib):
    s = cfg_mix().shape()
    s.kv_dtype = B.KV_FP8_E4M3
    c = Schedule("dynamic", num_workers=256).cfg()
    fake = ctypes.c_void_p(0x10000)
    for field, value in [("rope_theta", 0.0), ("rms_eps", -1.0), ("k_scale", 0.0),
                         ("v_scale", float("inf")), ("sm_scale", float("nan")),
                         ("norm_before_rope", 2)]:
        p = DecodeConfig(64, 8, "fp8", 2048, 4300).params()
        setattr(p, field, value)
        got = lib.lbsr_attention(ctypes.byref(s), ctypes.byref(p), 32, fake, fake, fake, fake,
                                 ctypes.byref(c), fake, 1 << 30, fake, fake, ctypes.c_void_p(0))
        assert got == B.E_INVALID, field


def test_python_layer_raises_on_status():
    bad = DecodeConfig(64, 8, "bf16", max_blocks_per_seq=0, num_pages=10)
    with pytest.raises(LbsrError, match="LBSR_E_INVALID"):
        workspace_layout(bad, 4, Schedule("dynamic", num_workers=8))


def test_binding_signatures_match_header(lib):
    """Each ctypes prototype has as many parameters as the header declares."""
    text = open(os.path.join(ROOT, "include", "lbsr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    seen = 0
    for m in re.finditer(r"\b(lbsr_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        name, params = m.group(1), m.group(2).strip()
        n = 0 if params in ("void", "") else len(params.split(","))
        assert len(getattr(lib, name).argtypes) == n, name
        seen += 1
    assert seen == len(B.EXPORTS)


def test_shape_struct_matches_header():
    """lbsr_shape: 8 int32 fields (tokens_per_seq and reserved after
    max_blocks_per_seq), then the three int64: 56 bytes."""
    assert ctypes.sizeof(B.Shape) == 56
    assert B.Shape.tokens_per_seq.offset == 24 and B.Shape.num_pages.offset == 32


@pytest.mark.parametrize("Hq,Hkv,tokens,reserved,workers,status", [
    (64, 8, 1, 0, 256, B.OK), (64, 8, 2, 0, 256, B.OK), (16, 4, 4, 0, 256, B.OK),
    (8, 8, 16, 0, 256, B.OK), (64, 8, 3, 0, 256, B.OK), (64, 8, 8, 0, 256, B.OK),
    (8, 8, 64, 0, 256, B.OK),
    (64, 8, 0, 0, 256, B.E_INVALID), (64, 8, -1, 0, 256, B.E_INVALID),
    (64, 8, 9, 0, 256, B.E_UNSUPPORTED),          # 8 heads x 9 tokens > 64 columns
    (8, 8, 65, 0, 256, B.E_UNSUPPORTED),
    (64, 8, 4, 0, 1024, B.E_UNSUPPORTED),         # 1024 chunks x 32 columns > the merge's LDS
    (64, 8, 2, 0, 1024, B.OK),                    # 1024 x 16 x 4 B = 64 KiB: fits
    (64, 8, 1, 5, 256, B.E_INVALID),
])
def test_tokens_per_seq_validation(lib, Hq, Hkv, tokens, reserved, workers, status):
    s = DecodeConfig(Hq, Hkv, "bf16", 2048, 4300, tokens_per_seq=tokens).shape()
    s.reserved = reserved
    c = Schedule("dynamic", num_workers=workers).cfg()
    out = B.WsLayout()
    got = lib.lbsr_workspace_layout(ctypes.byref(s), 32, ctypes.byref(c), ctypes.byref(out))
    assert got == status, lib.lbsr_last_error()


def test_workspace_grows_with_tokens(lib):
    """Partials, their lse and the per-token status scale with the new tokens."""
    c = Schedule("dynamic", num_workers=256).cfg()
    lays = []
    for tokens in (1, 2):
        s = DecodeConfig(64, 8, "bf16", 2048, 4300, tokens_per_seq=tokens).shape()
        out = B.WsLayout()
        assert lib.lbsr_workspace_layout(ctypes.byref(s), 32, ctypes.byref(c),
                                         ctypes.byref(out)) == B.OK
        lays.append(out)
    one, two = lays
    cmax = one.max_chunks
    assert two.partial_lse - two.partial_o >= 2 * cmax * 64 * 128 * 4
    assert two.total - two.partial_lse >= 2 * cmax * 64 * 4
    assert two.total > one.total


def test_params_struct_matches_header():
    """lbsr_params: double, float, int32, 3 floats, int32 out_dtype, float out_scale,
    int32 qk_dtype, float q_scale: 48 bytes."""
    assert ctypes.sizeof(B.Params) == 48
    assert B.Params.out_dtype.offset == 28 and B.Params.out_scale.offset == 32
    assert B.Params.qk_dtype.offset == 36 and B.Params.q_scale.offset == 40


@pytest.mark.parametrize("out_dtype,out_scale,status", [
    (B.OUT_BF16, 0.0, B.OK), (B.OUT_FP8_E4M3, 0.5, B.OK), (B.OUT_FP8_E4M3, 0.0, B.E_INVALID),
    (B.OUT_FP8_E4M3, float("inf"), B.E_INVALID), (B.OUT_FP8_E4M3, -1.0, B.E_INVALID),
    (7, 1.0, B.E_INVALID),
])
def test_out_dtype_validation(lib, out_dtype, out_scale, status):
    s = cfg_mix().shape()
    c = Schedule("dynamic", num_workers=256).cfg()
    p = cfg_mix().params()
    p.out_dtype, p.out_scale = out_dtype, out_scale
    fake = ctypes.c_void_p(0x10000)
    got = lib.lbsr_attention(ctypes.byref(s), ctypes.byref(p), 32, fake, fake, fake, fake,
                             ctypes.byref(c), fake, 16, fake, fake, ctypes.c_void_p(0))
    # a valid configuration fails only at the (too small) workspace, before any launch
    assert got == (B.E_WORKSPACE if status == B.OK else status), lib.lbsr_last_error()


def test_tokens_beyond_block_table_reach_rejected(lib):
    """New tokens must fit the block table: tokens_per_seq > max_blocks * 64 is
    refused before any launch (a kernel would otherwise walk past the row)."""
    s = DecodeConfig(8, 8, "bf16", 2, 100, tokens_per_seq=129).shape()
    p = DecodeConfig(8, 8, "bf16", 2, 100).params()
    fake = ctypes.c_void_p(0x10000)
    nul = ctypes.c_void_p(0)
    # q_out, k_cache, v_cache, block_table, seq_lens, workspace, ws_bytes, out, lse, err, stream
    got = lib.lbsr_prefill_attention(ctypes.byref(s), ctypes.byref(p), 4, *([fake] * 5), nul, 0,
                                     fake, nul, nul, nul)
    assert got == B.E_INVALID and b"max_blocks_per_seq" in lib.lbsr_last_error()
    s = DecodeConfig(8, 8, "bf16", 2, 100, tokens_per_seq=128).shape()
    got = lib.lbsr_prefill_attention(ctypes.byref(s), ctypes.byref(p), 4, ctypes.c_void_p(0x10002),
                                     *([fake] * 4), nul, 0, fake, nul, nul, nul)
    assert got == B.E_INVALID and b"q_out" in lib.lbsr_last_error()   # shape accepted


def test_varlen_entry_points_validate_before_any_launch(lib):
    """Negative token counts, a missing or misaligned q_start or workspace, a
    short workspace and too many packed rows return errors without touching a
    device; the workspace size follows its formula."""
    cfg = DecodeConfig(64, 8, "bf16", 200, 4000, tokens_per_seq=512)
    s, p = cfg.shape(), cfg.params()
    fake, odd, nul = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10002), ctypes.c_void_p(0)
    n = ctypes.c_size_t()
    assert lib.lbsr_prefill_workspace_size(ctypes.byref(s), 8, 100, ctypes.byref(n)) == B.OK
    assert n.value == 256 + 8 * (-(-100 // 32) + 8)          # 32 tokens per block at G = 8
    big = 1 << 20
    attn = lambda total, qs, ws, nb: lib.lbsr_prefill_attention_varlen(
        ctypes.byref(s), ctypes.byref(p), 8, total, qs, *([fake] * 5), ws, nb, fake, nul, nul, nul)
    assert attn(-1, fake, fake, big) == B.E_INVALID
    assert attn(100, nul, fake, big) == B.E_INVALID and b"q_start" in lib.lbsr_last_error()
    assert attn(100, odd, fake, big) == B.E_INVALID
    assert attn(100, fake, nul, big) == B.E_INVALID and b"workspace" in lib.lbsr_last_error()
    assert attn(100, fake, ctypes.c_void_p(0x10040), big) == B.E_INVALID     # not 256-aligned
    assert attn(100, fake, fake, n.value - 1) == B.E_WORKSPACE
    assert attn(1 << 26, fake, fake, big) == B.E_UNSUPPORTED      # 2^26 tokens x 80 rows
    # q, k, v, positions, seq_lens, q_norm_w, k_norm_w, block_table, k_cache, v_cache, q_out
    args = [fake] * 11
    step = lambda qs, a: lib.lbsr_prefill_step_varlen(
        ctypes.byref(s), ctypes.byref(p), 8, 100, qs, *a, fake, big, fake, nul, nul, nul)
    assert step(nul, args) == B.E_INVALID
    a2 = list(args)
    a2[10] = a2[0]                                         # q_out aliases q
    assert step(fake, a2) == B.E_INVALID and b"alias" in lib.lbsr_last_error()


@pytest.mark.parametrize("kv_dtype,qk_dtype,q_scale,status", [
    ("fp8", B.QK_BF16, 0.0, B.OK), ("fp8", B.QK_FP8_E4M3, 0.25, B.OK),
    ("bf16", B.QK_FP8_E4M3, 0.25, B.E_UNSUPPORTED),      # FP8 scores need an FP8 cache
    ("fp8", B.QK_FP8_E4M3, 0.0, B.E_INVALID), ("fp8", B.QK_FP8_E4M3, float("nan"), B.E_INVALID),
    ("fp8", B.QK_FP8_E4M3, 1e-45, B.E_INVALID),         # 1/q_scale overflows fp32
    ("fp8", 5, 1.0, B.E_INVALID),
])
def test_qk_dtype_validation(lib, kv_dtype, qk_dtype, q_scale, status):
    """Checked before any launch: fake pointers are never dereferenced."""
    cfg = DecodeConfig(64, 8, kv_dtype, 2048, 4300, k_scale=0.5, v_scale=0.5)
    s, p = cfg.shape(), cfg.params()
    p.qk_dtype, p.q_scale = qk_dtype, q_scale
    c = Schedule("dynamic", num_workers=256).cfg()
    fake = ctypes.c_void_p(0x10000)
    got = lib.lbsr_attention(ctypes.byref(s), ctypes.byref(p), 32, fake, fake, fake, fake,
                             ctypes.byref(c), fake, 1 << 30, fake, fake, ctypes.c_void_p(0))
    if status == B.OK:
        # valid params: validation proceeds past them (and then needs a device)
        assert b"qk_dtype" not in lib.lbsr_last_error() and b"q_scale" not in lib.lbsr_last_error()
    else:
        assert got == status, lib.lbsr_last_error()


def test_uniform_prefill_workspace_validation(lib):
    """The uniform calls' workspace is optional; given, it must be 256-byte
    aligned and hold the work list of batch * tokens_per_seq tokens."""
    cfg = DecodeConfig(64, 8, "bf16", 200, 4000, tokens_per_seq=512)
    s, p = cfg.shape(), cfg.params()
    fake, nul = ctypes.c_void_p(0x10000), ctypes.c_void_p(0)
    n = ctypes.c_size_t()
    assert lib.lbsr_prefill_workspace_size(ctypes.byref(s), 8, 8 * 512, ctypes.byref(n)) == B.OK
    assert n.value == 256 + 8 * (8 * 512 // 32 + 8)
    call = lambda ws, nb: lib.lbsr_prefill_attention(ctypes.byref(s), ctypes.byref(p), 8,
                                                     *([fake] * 5), ws, nb, fake, nul, nul, nul)
    assert call(ctypes.c_void_p(0x10040), n.value) == B.E_INVALID     # not 256-byte aligned
    assert call(fake, n.value - 1) == B.E_WORKSPACE
    for ws, nb in ((fake, n.value), (nul, 0)):                        # valid: fails later (no GPU)
        call(ws, nb)
        assert b"workspace" not in lib.lbsr_last_error()


@pytest.mark.parametrize("Hq,Hkv,tokens,status", [
    (64, 8, 1, B.OK),                 # the pages' shape, one new token
    (8, 1, 1, B.OK),
    (64, 4, 1, B.OK),                 # group 16
    (64, 8, 2, B.E_UNSUPPORTED),      # multi-token steps keep the merge launch
    (48, 8, 1, B.E_UNSUPPORTED),      # group 6: not a power of two
])
def test_fold_merge_validation(lib, Hq, Hkv, tokens, status):
    """LBSR_SCHED_FOLD_MERGE: one new token per sequence and a power-of-two group."""
    cfg = DecodeConfig(Hq, Hkv, "bf16", max_blocks_per_seq=64, num_pages=100, tokens_per_seq=tokens)
    s = cfg.shape()
    c = Schedule("dynamic", num_workers=256, fold_merge=True).cfg()
    assert c.flags == B.SCHED_FOLD_MERGE
    out = B.WsLayout()
    got = lib.lbsr_workspace_layout(ctypes.byref(s), 16, ctypes.byref(c), ctypes.byref(out))
    assert got == status, lib.lbsr_last_error()


def test_readers_validate_before_touching_the_device(lib):
    """lbsr_read_plan / lbsr_read_device_error check their arguments on the
    host before any synchronisation or copy."""
    cfg = cfg_mix()
    s = cfg.shape()
    sched = Schedule("dynamic", num_workers=256)
    c = sched.cfg()
    lay = workspace_layout(cfg, 32, sched)
    host = B.PlanHost()
    n = ctypes.c_int32()
    fake = ctypes.c_void_p(1 << 20)        # never dereferenced: validation fails first
    cases = [
        (lambda: lib.lbsr_read_plan(ctypes.byref(s), 32, ctypes.byref(c), fake, lay.total, None,
                                    ctypes.byref(n), None), B.E_INVALID),       # out NULL
        (lambda: lib.lbsr_read_plan(ctypes.byref(s), 32, ctypes.byref(c), None, lay.total,
                                    ctypes.byref(host), ctypes.byref(n), None), B.E_INVALID),
        (lambda: lib.lbsr_read_plan(ctypes.byref(s), 32, ctypes.byref(c), ctypes.c_void_p((1 << 20) + 4),
                                    lay.total, ctypes.byref(host), ctypes.byref(n), None),
         B.E_INVALID),                                                           # misaligned
        (lambda: lib.lbsr_read_plan(ctypes.byref(s), 32, ctypes.byref(c), fake, lay.total - 1,
                                    ctypes.byref(host), ctypes.byref(n), None), B.E_WORKSPACE),
        (lambda: lib.lbsr_read_plan(ctypes.byref(s), 0, ctypes.byref(c), fake, lay.total,
                                    ctypes.byref(host), ctypes.byref(n), None), B.E_INVALID),
        (lambda: lib.lbsr_read_device_error(fake, None, None), B.E_INVALID),    # code NULL
        (lambda: lib.lbsr_read_device_error(None, ctypes.byref(n), None), B.E_INVALID),
        (lambda: lib.lbsr_read_device_error(ctypes.c_void_p((1 << 20) + 8), ctypes.byref(n), None),
         B.E_INVALID),
    ]
    for i, (call, want) in enumerate(cases):
        assert call() == want, (i, lib.lbsr_last_error())
        assert lib.lbsr_last_error() != b""


def test_plan_host_struct_matches_header():
    """lbsr_plan_host: five host pointers in the header's order."""
    assert [f for f, _ in B.PlanHost._fields_] == ["cu_tiles", "worker_chunk", "chunks",
                                                   "seq_chunk", "seq_len_eff"]
    assert ctypes.sizeof(B.PlanHost) == 5 * ctypes.sizeof(ctypes.c_void_p)


def test_stream_read_validates_before_any_launch(lib):
    fake = ctypes.c_void_p(1 << 20)
    sink = ctypes.c_void_p(1 << 21)
    for args, want in [((None, 1 << 15, 0, 0, sink, None), B.E_INVALID),
                       ((fake, 1 << 15, 0, 0, None, None), B.E_INVALID),
                       ((ctypes.c_void_p((1 << 20) + 8), 1 << 15, 0, 0, sink, None), B.E_INVALID),
                       ((fake, 0, 0, 0, sink, None), B.E_INVALID),
                       ((fake, (1 << 15) + 16, 0, 0, sink, None), B.E_INVALID),
                       ((fake, 1 << 15, -1, 0, sink, None), B.E_INVALID),
                       ((fake, 1 << 15, 0, 3, sink, None), B.E_INVALID)]:
        assert lib.lbsr_stream_read(*args) == want, lib.lbsr_last_error()


def test_noalloc_step_refuses_beyond_its_scratch_before_any_launch(lib):
    """lbsr_decode_step_noalloc: a step whose workspace exceeds the library's
    scratch (4096 sequences: about 142 MB) is refused with LBSR_E_WORKSPACE
    on the host, before any pointer is touched or kernel launched."""
    s = cfg_mix().shape()
    p = cfg_mix().params()
    c = Schedule("dynamic", num_workers=256).cfg()
    lay = workspace_layout(cfg_mix(), 4096, Schedule("dynamic", num_workers=256))
    assert lay.total > B.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000)
    got = lib.lbsr_decode_step_noalloc(ctypes.byref(s), ctypes.byref(p), 4096, *([fake] * 11),
                                       ctypes.byref(c), fake, fake, None)
    assert got == B.E_WORKSPACE and b"scratch" in lib.lbsr_last_error()
    # the mix itself fits
    assert workspace_layout(cfg_mix(), 32, Schedule("dynamic", num_workers=256)).total \
        <= B.NOALLOC_SCRATCH_BYTES


C_CALLER = r"""
#include <stdio.h>
#include <string.h>
#include "lbsr.h"

int main(void) {
  lbsr_shape s;
  lbsr_sched_cfg c;
  lbsr_ws_layout l;
  size_t bytes = 0;
  lbsr_status st;
  memset(&s, 0, sizeof s);
  memset(&c, 0, sizeof c);
  s.num_q_heads = 64; s.num_kv_heads = 8; s.head_dim = 128; s.page_size = 64;
  s.kv_dtype = LBSR_KV_BF16; s.max_blocks_per_seq = 2048; s.tokens_per_seq = 1;
  s.num_pages = 4096; s.page_stride = 8 * 8192; s.head_stride = 8192;
  c.sched = LBSR_SCHED_DYNAMIC; c.num_workers = 256;
  st = lbsr_workspace_layout(&s, 32, &c, &l);
  printf("%d %d %zu %d %d\n", lbsr_abi_version(), (int)st, l.total, l.num_workers, l.max_chunks);
  s.head_dim = 64;
  st = lbsr_workspace_size(&s, 32, &c, &bytes);
  printf("%s|%s\n", lbsr_status_string(st), lbsr_last_error());
  return 0;
}
"""


def test_header_is_c_and_the_library_links_from_c(lib, tmp_path):
    """include/lbsr.h is a C header (pedantic C99, warnings as errors), and a C
    program linked against liblbsr.so gets the same host-side answers as the
    binding: the workspace layout of a decode step, and a refused shape."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(B.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", libdir, "-l:" + os.path.basename(B.LIB_PATH),
                    "-Wl,-rpath," + libdir], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    abi, st, total, workers, max_chunks = out[0].split()
    cfg = DecodeConfig(64, 8, "bf16", 2048, 4096)
    ref = workspace_layout(cfg, 32, Schedule("dynamic", num_workers=256))
    assert (int(abi), int(st)) == (lib.lbsr_abi_version(), 0)
    assert (int(total), int(workers), int(max_chunks)) == (ref.total, ref.num_workers, ref.max_chunks)
    assert out[1].startswith("LBSR_E_UNSUPPORTED") and "head_dim 64" in out[1], out[1]


def test_config_structs_follow_field_changes():
    """The binding builds each config's ctypes structs once; assigning a field
    rebuilds them, and a struct handed to a caller is the caller's copy."""
    c = DecodeConfig(64, 8, "bf16", 2048, 4300)
    s = c.shape()
    s.head_dim = 64
    assert c.shape().head_dim == 128
    c.num_pages = 10
    assert c.shape().num_pages == 10
    assert c.pool_elems() == 9 * 8 * 8192 + 7 * 8192 + 8192
    c.out_dtype = "fp8"
    assert c.params().out_dtype == B.OUT_FP8_E4M3
    sched = Schedule("dynamic", num_workers=5)
    before = sched.cfg()
    sched.num_workers = 7
    assert sched.cfg().num_workers == 7 and before.num_workers == 5


def test_pack_cache_validates_before_any_launch(lib):
    """lbsr_pack_cache / lbsr_unpack_cache check the kind, the pointers and the
    row-major strides (positive, 16-byte multiples, rows not overlapping) on
    the host: each refusal comes back without touching a device, and a valid
    call gets past validation (it fails only where a device is needed)."""
    cfg = DecodeConfig(64, 8, "bf16", 4, 100)
    s = cfg.shape()
    fake, odd, nul = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10008), ctypes.c_void_p(0)
    H = 8
    nhd = (64 * H * 128, H * 128, 128)        # token-major rows
    hnd = (H * 64 * 128, 128, 64 * 128)       # head-major rows
    for fn in (lib.lbsr_pack_cache, lib.lbsr_unpack_cache):
        def call(kind=0, a=fake, b=fake, st=nhd, shape=s):
            return fn(ctypes.byref(shape), kind, a, *st, b, nul) if fn is lib.lbsr_pack_cache \
                else fn(ctypes.byref(shape), kind, a, b, *st, nul)
        assert call(kind=2) == B.E_INVALID and b"kind" in lib.lbsr_last_error()
        assert call(a=nul) == B.E_INVALID
        assert call(b=odd) == B.E_INVALID and b"aligned" in lib.lbsr_last_error()
        assert call(st=(nhd[0], nhd[1], 4)) == B.E_INVALID          # 8-byte head stride
        assert call(st=(nhd[0], 0, 128)) == B.E_INVALID             # zero token stride
        assert call(st=(1 << 40, nhd[1], 128)) == B.E_INVALID       # pages would span > 2^46
        assert call(st=(nhd[0], 128, 128)) == B.E_INVALID           # token and head rows collide
        assert b"overlaps" in lib.lbsr_last_error()
        assert call(st=(64 * 128, H * 128, 128)) == B.E_INVALID     # pages overlap
        bad = DecodeConfig(64, 8, "bf16", 4, 100).shape()
        bad.head_dim = 64
        assert call(shape=bad) == B.E_UNSUPPORTED
        for st in (nhd, hnd, (2 * nhd[0], 2 * nhd[1], 2 * 128)):    # padded rows are fine
            got = call(st=st)
            assert got not in (B.E_INVALID, B.E_UNSUPPORTED), lib.lbsr_last_error()
    # FP8 rows: one-byte elements, 16-element alignment
    s8 = DecodeConfig(64, 8, "fp8", 4, 100).shape()
    assert lib.lbsr_pack_cache(ctypes.byref(s8), 1, fake, 64 * H * 128, H * 128, 120, fake,
                               nul) == B.E_INVALID


@pytest.mark.parametrize("field,value", [("kv_dtype", "bf8"), ("kv_dtype", "BF16"),
                                         ("out_dtype", "fp16"), ("qk_dtype", "e4m3")])
def test_binding_refuses_unknown_dtype_names(field, value):
    """The binding names dtypes by string; an unknown name is refused rather than
    read as the other type."""
    cfg = cfg_mix()
    setattr(cfg, field, value)
    with pytest.raises(ValueError, match=field):
        cfg.shape() if field == "kv_dtype" else cfg.params()


@pytest.mark.parametrize("page_stride,head_stride", [
    (1 << 62, 8192),                      # would overflow int64 in num_pages * page_stride
    (8192 * 8, (1 << 46) // 4),           # 8 KV heads x head_stride > 2^46
    ((1 << 46) // 4000 // 8192 * 8192 + 8192 * 8, 8192)])   # just above the bound at 4000 pages
def test_huge_strides_are_refused(lib, page_stride, head_stride):
    """Strides whose pool would pass 2^46 elements are refused on the host,
    before any product of them could overflow."""
    cfg = DecodeConfig(64, 8, "bf16", max_blocks_per_seq=64, num_pages=4000,
                       page_stride=page_stride, head_stride=head_stride)
    s = cfg.shape()
    out = B.WsLayout()
    c = Schedule("dynamic", num_workers=256).cfg()
    got = lib.lbsr_workspace_layout(ctypes.byref(s), 16, ctypes.byref(c), ctypes.byref(out))
    assert got == B.E_INVALID and b"2^46" in lib.lbsr_last_error()


def test_large_strides_within_the_bound_are_accepted(lib):
    cfg = DecodeConfig(64, 8, "bf16", max_blocks_per_seq=64, num_pages=4000,
                       page_stride=(1 << 46) // 4000 // 8192 * 8192, head_stride=8192)
    s = cfg.shape()
    out = B.WsLayout()
    c = Schedule("dynamic", num_workers=256).cfg()
    assert lib.lbsr_workspace_layout(ctypes.byref(s), 16, ctypes.byref(c),
                                     ctypes.byref(out)) == B.OK, lib.lbsr_last_error()
