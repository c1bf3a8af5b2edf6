"""Python face of the decode step: the same calls as include/lbsr.h, on torch tensors.

Nothing here computes: it validates tensors, marshals pointers and the current
torch stream, and calls liblbsr.  Device memory comes from torch.
"""

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _binding as B


class _Memo:
    """The ctypes structs a config marshals to, built once and rebuilt after any
    field is assigned (the dataclasses below stay mutable)."""

    def __setattr__(self, name, value):
        object.__setattr__(self, name, value)
        object.__setattr__(self, "_memo", {})

    def _memoised(self, key, build):
        memo = self.__dict__.get("_memo")
        if memo is None:
            memo = {}
            object.__setattr__(self, "_memo", memo)
        if key not in memo:
            memo[key] = build()
        return memo[key]


@dataclass
class DecodeConfig(_Memo):
    """Geometry of the KV pools and the per-step constants (lbsr_shape + lbsr_params)."""
    num_q_heads: int
    num_kv_heads: int
    kv_dtype: str                 # "bf16" or "fp8"
    max_blocks_per_seq: int
    num_pages: int
    page_stride: int = 0          # elements; 0 -> num_kv_heads * 8192 (page-major pools)
    head_stride: int = 0          # elements; 0 -> 8192
    rope_theta: float = 1e4
    rms_eps: float = 1e-6
    norm_before_rope: bool = False
    k_scale: float = 1.0
    v_scale: float = 1.0
    sm_scale: float = 0.0         # 0 -> 1/sqrt(128)
    tokens_per_seq: int = 1       # new tokens per sequence (multi-token decode)
    out_dtype: str = "bf16"       # "bf16", or "fp8": E4M3 codes of out / out_scale
    out_scale: float = 1.0
    qk_dtype: str = "bf16"        # "bf16", or "fp8" (FP8 cache): q quantised with q_scale and
    q_scale: float = 1.0          # Q.K^T on FP8 matrix cores

    def shape(self):
        """lbsr_shape of this config (a fresh struct the caller may modify)."""
        return B.Shape.from_buffer_copy(self._shape())

    def _shape(self):
        # shared by the binding's calls; never modified
        if self.kv_dtype not in ("bf16", "fp8"):
            raise ValueError(f"kv_dtype {self.kv_dtype!r}: 'bf16' or 'fp8'")
        return self._memoised("shape", lambda: B.Shape(
            self.num_q_heads, self.num_kv_heads, B.HEAD_DIM, B.PAGE_SIZE,
            B.KV_BF16 if self.kv_dtype == "bf16" else B.KV_FP8_E4M3,
            self.max_blocks_per_seq, self.tokens_per_seq, 0, self.num_pages,
            self.page_stride or self.num_kv_heads * B.TILE_ELEMS,
            self.head_stride or B.TILE_ELEMS))

    def tokens_shape(self, batch, *rest):
        """Shape of a per-new-token array: (batch, *rest), or (batch, Tq, *rest) when Tq > 1."""
        Tq = self.tokens_per_seq
        return (batch,) + rest if Tq == 1 else (batch, Tq) + rest

    def params(self):
        """lbsr_params of this config (a fresh struct the caller may modify)."""
        return B.Params.from_buffer_copy(self._params())

    def _params(self):
        for name in ("out_dtype", "qk_dtype"):
            if getattr(self, name) not in ("bf16", "fp8"):
                raise ValueError(f"{name} {getattr(self, name)!r}: 'bf16' or 'fp8'")
        return self._memoised("params", lambda: B.Params(
            self.rope_theta, self.rms_eps, int(self.norm_before_rope), self.k_scale,
            self.v_scale, self.sm_scale,
            B.OUT_BF16 if self.out_dtype == "bf16" else B.OUT_FP8_E4M3, self.out_scale,
            B.QK_BF16 if self.qk_dtype == "bf16" else B.QK_FP8_E4M3, self.q_scale))

    @property
    def out_torch_dtype(self):
        """dtype of `out`: bfloat16, or uint8 E4M3 codes."""
        return torch.bfloat16 if self.out_dtype == "bf16" else torch.uint8

    @property
    def cache_dtype(self):
        return torch.bfloat16 if self.kv_dtype == "bf16" else torch.uint8

    def pool_elems(self):
        """Elements a pool must hold: one past the last element of the last tile."""
        def count():
            s = self._shape()
            return ((s.num_pages - 1) * s.page_stride + (s.num_kv_heads - 1) * s.head_stride
                    + B.TILE_ELEMS)
        return self._memoised("pool_elems", count)


@dataclass
class Schedule(_Memo):
    """lbsr_sched_cfg: "dynamic" (P workers, 0 = CU count) or "static" (S splits, 0 = P/B).

    xcd_weights: None (equal shares) or 8 integer weights in [1, 65536], the
    relative streaming rate of each XCD's compute units (dynamic only).
    fold_merge: merge split sequences inside the split-attention launch
    (LBSR_SCHED_FOLD_MERGE; one new token per sequence) instead of a second launch.
    """
    kind: str = "dynamic"
    num_workers: int = 0
    static_splits: int = 0
    xcd_weights: tuple = None
    fold_merge: bool = False

    def cfg(self):
        """lbsr_sched_cfg of this schedule (a fresh struct the caller may modify)."""
        return B.SchedCfg.from_buffer_copy(self._cfg())

    def _cfg(self):
        if self.kind not in ("dynamic", "static"):
            raise ValueError(f"unknown schedule {self.kind!r}")
        wts = [0] * B.NUM_XCDS if self.xcd_weights is None else [int(x) for x in self.xcd_weights]
        if len(wts) != B.NUM_XCDS:
            raise ValueError(f"xcd_weights needs {B.NUM_XCDS} entries, got {len(wts)}")
        return self._memoised("cfg", lambda: B.SchedCfg(
            B.SCHED_DYNAMIC if self.kind == "dynamic" else B.SCHED_STATIC, self.num_workers,
            self.static_splits, B.SCHED_FOLD_MERGE if self.fold_merge else 0,
            (ctypes.c_int32 * B.NUM_XCDS)(*wts)))


def device_workers(device=0):
    out = ctypes.c_int32()
    B._check(B.lib().lbsr_device_workers(int(device), ctypes.byref(out)))
    return out.value


def workspace_layout(cfg: DecodeConfig, batch: int, sched: Schedule):
    out = B.WsLayout()
    s, c = cfg._shape(), sched._cfg()
    B._check(B.lib().lbsr_workspace_layout(ctypes.byref(s), int(batch), ctypes.byref(c),
                                           ctypes.byref(out)))
    return out


def alloc_workspace(cfg: DecodeConfig, batch: int, sched: Schedule, device="cuda"):
    lay = workspace_layout(cfg, batch, sched)
    return torch.empty(lay.total, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- checks

def _need(t, name, dtype, shape=None, numel=None):
    # the common case in one comparison chain; the diagnosis below only on failure
    if (type(t) is torch.Tensor and t.dtype is dtype and t.is_cuda and t.is_contiguous()
            and (shape is None or t.shape == shape) and (numel is None or t.numel() >= numel)):
        return
    _diagnose(t, name, dtype, shape, numel)


def _diagnose(t, name, dtype, shape=None, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} must hold at least {numel} elements, has {t.numel()}")


def _check_pools(cfg, k_cache, v_cache):
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, cfg.cache_dtype, numel=cfg.pool_elems())


def _check_table(cfg, block_table, batch):
    _need(block_table, "block_table", torch.int32, shape=(batch, cfg.max_blocks_per_seq))


# ---------------------------------------------------------------- entry points

def rope_norm_kv_write(cfg: DecodeConfig, q, k, v, positions, q_norm_w, k_norm_w, block_table,
                       k_cache, v_cache, q_out, error_word=None, stream=None):
    """lbsr_rope_norm_kv_write: RoPE + QK-Norm + cache write of the new tokens."""
    batch = q.shape[0]
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, B.HEAD_DIM
    _need(q, "q", torch.bfloat16, shape=cfg.tokens_shape(batch, Hq, D))
    _need(k, "k", torch.bfloat16, shape=cfg.tokens_shape(batch, Hkv, D))
    _need(v, "v", torch.bfloat16, shape=cfg.tokens_shape(batch, Hkv, D))
    _need(q_out, "q_out", torch.bfloat16, shape=cfg.tokens_shape(batch, Hq, D))
    _need(positions, "positions", torch.int32, shape=cfg.tokens_shape(batch))
    _need(q_norm_w, "q_norm_w", torch.bfloat16, shape=(D,))
    _need(k_norm_w, "k_norm_w", torch.bfloat16, shape=(D,))
    _check_table(cfg, block_table, batch)
    _check_pools(cfg, k_cache, v_cache)
    if error_word is not None:
        _need(error_word, "error_word", torch.int32, numel=1)
    s, p = cfg._shape(), cfg._params()
    B._check(B.lib().lbsr_rope_norm_kv_write(
        ctypes.byref(s), ctypes.byref(p), batch, B._ptr(q), B._ptr(k), B._ptr(v),
        B._ptr(positions), B._ptr(q_norm_w), B._ptr(k_norm_w), B._ptr(block_table),
        B._ptr(k_cache), B._ptr(v_cache), B._ptr(q_out), B._ptr(error_word), B._stream(stream)))


def plan(cfg: DecodeConfig, seq_lens, sched: Schedule, workspace, stream=None):
    """lbsr_plan: the step's tile schedule, written into ``workspace``."""
    batch = seq_lens.shape[0]
    _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
    _need(workspace, "workspace", torch.uint8)
    s, c = cfg._shape(), sched._cfg()
    B._check(B.lib().lbsr_plan(ctypes.byref(s), batch, B._ptr(seq_lens), ctypes.byref(c),
                               B._ptr(workspace), workspace.numel(), B._stream(stream)))


def attention(cfg: DecodeConfig, q_out, k_cache, v_cache, block_table, sched: Schedule,
              workspace, out, lse_out=None, stream=None):
    """lbsr_attention: split attention + merge over the planned schedule."""
    batch = q_out.shape[0]
    Hq, D = cfg.num_q_heads, B.HEAD_DIM
    _need(q_out, "q_out", torch.bfloat16, shape=cfg.tokens_shape(batch, Hq, D))
    _need(out, "out", cfg.out_torch_dtype, shape=cfg.tokens_shape(batch, Hq, D))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, shape=cfg.tokens_shape(batch, Hq))
    _check_table(cfg, block_table, batch)
    _check_pools(cfg, k_cache, v_cache)
    _need(workspace, "workspace", torch.uint8)
    s, p, c = cfg._shape(), cfg._params(), sched._cfg()
    B._check(B.lib().lbsr_attention(
        ctypes.byref(s), ctypes.byref(p), batch, B._ptr(q_out), B._ptr(k_cache),
        B._ptr(v_cache), B._ptr(block_table), ctypes.byref(c), B._ptr(workspace),
        workspace.numel(), B._ptr(out), B._ptr(lse_out), B._stream(stream)))


def _step_args(cfg, q, k, v, positions, seq_lens, q_norm_w, k_norm_w, block_table, k_cache,
               v_cache, q_out, sched, workspace, out, lse_out):
    batch = q.shape[0]
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, B.HEAD_DIM
    _need(q, "q", torch.bfloat16, shape=cfg.tokens_shape(batch, Hq, D))
    _need(k, "k", torch.bfloat16, shape=cfg.tokens_shape(batch, Hkv, D))
    _need(v, "v", torch.bfloat16, shape=cfg.tokens_shape(batch, Hkv, D))
    _need(q_out, "q_out", torch.bfloat16, shape=cfg.tokens_shape(batch, Hq, D))
    _need(out, "out", cfg.out_torch_dtype, shape=cfg.tokens_shape(batch, Hq, D))
    _need(positions, "positions", torch.int32, shape=cfg.tokens_shape(batch))
    _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
    _need(q_norm_w, "q_norm_w", torch.bfloat16, shape=(D,))
    _need(k_norm_w, "k_norm_w", torch.bfloat16, shape=(D,))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, shape=cfg.tokens_shape(batch, Hq))
    _check_table(cfg, block_table, batch)
    _check_pools(cfg, k_cache, v_cache)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    s, p, c = cfg._shape(), cfg._params(), sched._cfg()
    head = (ctypes.byref(s), ctypes.byref(p), batch, B._ptr(q), B._ptr(k), B._ptr(v),
            B._ptr(positions), B._ptr(seq_lens), B._ptr(q_norm_w), B._ptr(k_norm_w),
            B._ptr(block_table), B._ptr(k_cache), B._ptr(v_cache), B._ptr(q_out),
            ctypes.byref(c))
    ws = () if workspace is None else (B._ptr(workspace), workspace.numel())
    return head + ws + (B._ptr(out), B._ptr(lse_out)), (s, p, c)


def decode_step(cfg: DecodeConfig, q, k, v, positions, seq_lens, q_norm_w, k_norm_w, block_table,
                k_cache, v_cache, q_out, sched: Schedule, workspace, out, lse_out=None,
                stream=None):
    """lbsr_decode_step: plan, prologue, split attention and merge on one stream."""
    args, keep = _step_args(cfg, q, k, v, positions, seq_lens, q_norm_w, k_norm_w, block_table,
                            k_cache, v_cache, q_out, sched, workspace, out, lse_out)
    B._check(B.lib().lbsr_decode_step(*args, B._stream(stream)))
    del keep


def decode_step_noalloc(cfg: DecodeConfig, q, k, v, positions, seq_lens, q_norm_w, k_norm_w,
                        block_table, k_cache, v_cache, q_out, sched: Schedule, out, lse_out=None,
                        stream=None):
    """lbsr_decode_step_noalloc: the decode step with the library's own per-GPU
    scratch as its workspace (for callers that cannot allocate).  Raises
    LbsrError (LBSR_E_WORKSPACE) when the step needs more than the scratch."""
    args, keep = _step_args(cfg, q, k, v, positions, seq_lens, q_norm_w, k_norm_w, block_table,
                            k_cache, v_cache, q_out, sched, None, out, lse_out)
    B._check(B.lib().lbsr_decode_step_noalloc(*args, B._stream(stream)))
    del keep


def decode_step_timed(cfg: DecodeConfig, q, k, v, positions, seq_lens, q_norm_w, k_norm_w,
                      block_table, k_cache, v_cache, q_out, sched: Schedule, workspace, out,
                      lse_out=None, stream=None, trace=None):
    """lbsr_decode_step_timed: the step with HIP events around each kernel (synchronises).

    Returns milliseconds of (schedule + prologue, split attention, merge).  ``trace``
    (int64 [W, 4] on the GPU) receives per-worker {start, end, HW_ID, XCC_ID}."""
    args, keep = _step_args(cfg, q, k, v, positions, seq_lens, q_norm_w, k_norm_w, block_table,
                            k_cache, v_cache, q_out, sched, workspace, out, lse_out)
    if trace is not None:
        W = workspace_layout(cfg, q.shape[0], sched).num_workers
        _need(trace, "trace", torch.int64, shape=(W, 4))
    ms = (ctypes.c_float * 3)()
    B._check(B.lib().lbsr_decode_step_timed(*args, B._stream(stream), ms, B._ptr(trace)))
    del keep
    return list(ms)


def prefill_attention(cfg: DecodeConfig, q_out, k_cache, v_cache, block_table, seq_lens, out,
                      lse_out=None, error_word=None, stream=None, workspace=None):
    """lbsr_prefill_attention: every new token (cfg.tokens_per_seq per sequence)
    attends its causal prefix.  workspace (from alloc_prefill_workspace with
    batch * tokens_per_seq tokens) runs the blocks longest first, which pays
    when the sequences' lengths differ; None keeps the workspace-free grid."""
    batch = q_out.shape[0]
    Hq, D = cfg.num_q_heads, B.HEAD_DIM
    _need(q_out, "q_out", torch.bfloat16, shape=cfg.tokens_shape(batch, Hq, D))
    _need(out, "out", cfg.out_torch_dtype, shape=cfg.tokens_shape(batch, Hq, D))
    _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, shape=cfg.tokens_shape(batch, Hq))
    if error_word is not None:
        _need(error_word, "error_word", torch.int32, numel=1)
    _check_table(cfg, block_table, batch)
    _check_pools(cfg, k_cache, v_cache)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    s, p = cfg._shape(), cfg._params()
    B._check(B.lib().lbsr_prefill_attention(
        ctypes.byref(s), ctypes.byref(p), batch, B._ptr(q_out), B._ptr(k_cache), B._ptr(v_cache),
        B._ptr(block_table), B._ptr(seq_lens), B._ptr(workspace), _nbytes(workspace),
        B._ptr(out), B._ptr(lse_out), B._ptr(error_word), B._stream(stream)))


def prefill_step(cfg: DecodeConfig, q, k, v, positions, seq_lens, q_norm_w, k_norm_w,
                 block_table, k_cache, v_cache, q_out, out, lse_out=None, error_word=None,
                 stream=None, workspace=None):
    """lbsr_prefill_step: the prologue on every new token, then prefill
    attention (workspace as for prefill_attention)."""
    batch = q.shape[0]
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, B.HEAD_DIM
    _need(q, "q", torch.bfloat16, shape=cfg.tokens_shape(batch, Hq, D))
    _need(k, "k", torch.bfloat16, shape=cfg.tokens_shape(batch, Hkv, D))
    _need(v, "v", torch.bfloat16, shape=cfg.tokens_shape(batch, Hkv, D))
    _need(q_out, "q_out", torch.bfloat16, shape=cfg.tokens_shape(batch, Hq, D))
    _need(out, "out", cfg.out_torch_dtype, shape=cfg.tokens_shape(batch, Hq, D))
    _need(positions, "positions", torch.int32, shape=cfg.tokens_shape(batch))
    _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
    _need(q_norm_w, "q_norm_w", torch.bfloat16, shape=(D,))
    _need(k_norm_w, "k_norm_w", torch.bfloat16, shape=(D,))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, shape=cfg.tokens_shape(batch, Hq))
    if error_word is not None:
        _need(error_word, "error_word", torch.int32, numel=1)
    _check_table(cfg, block_table, batch)
    _check_pools(cfg, k_cache, v_cache)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    s, p = cfg._shape(), cfg._params()
    B._check(B.lib().lbsr_prefill_step(
        ctypes.byref(s), ctypes.byref(p), batch, B._ptr(q), B._ptr(k), B._ptr(v),
        B._ptr(positions), B._ptr(seq_lens), B._ptr(q_norm_w), B._ptr(k_norm_w),
        B._ptr(block_table), B._ptr(k_cache), B._ptr(v_cache), B._ptr(q_out),
        B._ptr(workspace), _nbytes(workspace), B._ptr(out), B._ptr(lse_out),
        B._ptr(error_word), B._stream(stream)))


def prefill_workspace_size(cfg: DecodeConfig, batch: int, total_tokens: int) -> int:
    """Bytes of a prefill's workspace (its longest-first work list): total_tokens
    is the packed count of a ragged batch, or batch * tokens_per_seq."""
    n = ctypes.c_size_t()
    s = cfg._shape()
    B._check(B.lib().lbsr_prefill_workspace_size(ctypes.byref(s), batch, total_tokens,
                                                 ctypes.byref(n)))
    return n.value


def alloc_prefill_workspace(cfg: DecodeConfig, batch: int, total_tokens: int, device="cuda"):
    n = prefill_workspace_size(cfg, batch, total_tokens)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _check_varlen(cfg, q_start, batch, total, workspace):
    _need(q_start, "q_start", torch.int32, shape=(batch + 1,))
    if total < 0:
        raise ValueError(f"total_tokens {total} < 0")
    _need(workspace, "workspace", torch.uint8)


def prefill_attention_varlen(cfg: DecodeConfig, q_start, q_out, k_cache, v_cache, block_table,
                             seq_lens, workspace, out, lse_out=None, error_word=None,
                             stream=None):
    """lbsr_prefill_attention_varlen: a ragged batch.  Sequence b's new tokens
    are packed rows [q_start[b], q_start[b+1]) of q_out/out [N, Hq, D];
    cfg.tokens_per_seq bounds every sequence's count; workspace from
    alloc_prefill_workspace."""
    batch, total = seq_lens.shape[0], q_out.shape[0]
    Hq, D = cfg.num_q_heads, B.HEAD_DIM
    _check_varlen(cfg, q_start, batch, total, workspace)
    _need(q_out, "q_out", torch.bfloat16, shape=(total, Hq, D))
    _need(out, "out", cfg.out_torch_dtype, shape=(total, Hq, D))
    _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, shape=(total, Hq))
    if error_word is not None:
        _need(error_word, "error_word", torch.int32, numel=1)
    _check_table(cfg, block_table, batch)
    _check_pools(cfg, k_cache, v_cache)
    s, p = cfg._shape(), cfg._params()
    B._check(B.lib().lbsr_prefill_attention_varlen(
        ctypes.byref(s), ctypes.byref(p), batch, total, B._ptr(q_start), B._ptr(q_out),
        B._ptr(k_cache), B._ptr(v_cache), B._ptr(block_table), B._ptr(seq_lens),
        B._ptr(workspace), workspace.numel(), B._ptr(out), B._ptr(lse_out), B._ptr(error_word),
        B._stream(stream)))


def prefill_step_varlen(cfg: DecodeConfig, q_start, q, k, v, positions, seq_lens, q_norm_w,
                        k_norm_w, block_table, k_cache, v_cache, q_out, workspace, out,
                        lse_out=None, error_word=None, stream=None):
    """lbsr_prefill_step_varlen: the prologue on every packed new token, then
    ragged prefill attention."""
    batch, total = seq_lens.shape[0], q.shape[0]
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, B.HEAD_DIM
    _check_varlen(cfg, q_start, batch, total, workspace)
    _need(q, "q", torch.bfloat16, shape=(total, Hq, D))
    _need(k, "k", torch.bfloat16, shape=(total, Hkv, D))
    _need(v, "v", torch.bfloat16, shape=(total, Hkv, D))
    _need(q_out, "q_out", torch.bfloat16, shape=(total, Hq, D))
    _need(out, "out", cfg.out_torch_dtype, shape=(total, Hq, D))
    _need(positions, "positions", torch.int32, shape=(total,))
    _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
    _need(q_norm_w, "q_norm_w", torch.bfloat16, shape=(D,))
    _need(k_norm_w, "k_norm_w", torch.bfloat16, shape=(D,))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, shape=(total, Hq))
    if error_word is not None:
        _need(error_word, "error_word", torch.int32, numel=1)
    _check_table(cfg, block_table, batch)
    _check_pools(cfg, k_cache, v_cache)
    s, p = cfg._shape(), cfg._params()
    B._check(B.lib().lbsr_prefill_step_varlen(
        ctypes.byref(s), ctypes.byref(p), batch, total, B._ptr(q_start), B._ptr(q), B._ptr(k),
        B._ptr(v), B._ptr(positions), B._ptr(seq_lens), B._ptr(q_norm_w), B._ptr(k_norm_w),
        B._ptr(block_table), B._ptr(k_cache), B._ptr(v_cache), B._ptr(q_out),
        B._ptr(workspace), workspace.numel(), B._ptr(out), B._ptr(lse_out), B._ptr(error_word),
        B._stream(stream)))


def read_plan(cfg: DecodeConfig, batch: int, sched: Schedule, workspace, stream=None):
    """The plan arrays of a workspace, through lbsr_read_plan (synchronises the
    stream; for tests and tools)."""
    lay = workspace_layout(cfg, batch, sched)
    W = lay.num_workers
    arrs = {"cu_tiles": np.zeros(batch + 1, np.int32),
            "worker_chunk": np.zeros(W + 1, np.int32),
            "chunks": np.zeros((lay.max_chunks, 4), np.int32),
            "seq_chunk": np.zeros(batch + 1, np.int32),
            "seq_len_eff": np.zeros(batch, np.int32)}
    host = B.PlanHost(*(a.ctypes.data for a in arrs.values()))
    n = ctypes.c_int32(0)
    s = cfg._shape()
    B._check(B.lib().lbsr_read_plan(ctypes.byref(s), batch, ctypes.byref(sched._cfg()),
                                    B._ptr(workspace), workspace.numel(), ctypes.byref(host),
                                    ctypes.byref(n), B._stream(stream)))
    arrs["chunks"] = arrs["chunks"][:n.value].copy()
    return {"error_word": read_error(cfg, batch, sched, workspace, stream), **arrs,
            "num_workers": W, "max_chunks": lay.max_chunks}


def read_error(cfg: DecodeConfig, batch: int, sched: Schedule, workspace, stream=None):
    """The workspace's sticky device error bits, through lbsr_read_device_error
    (synchronises the stream)."""
    code = ctypes.c_int32(0)
    B._check(B.lib().lbsr_read_device_error(B._ptr(workspace), ctypes.byref(code),
                                            B._stream(stream)))
    return int(code.value)


def stream_read(buf, sink, workgroups=0, mode=0, stream=None):
    """The streaming-read probe (lbsr_stream_read): reads all of ``buf`` (a
    device tensor whose size is a multiple of 32 KiB); ``sink`` is a device
    buffer of at least ``workgroups`` (or CU count) 32-bit words.  mode 0: the
    split kernel's load pattern; 1: a plain grid-wide sweep; 2: mode 0's
    bursts loaded straight into LDS.  Asynchronous."""
    if buf.device.type != "cuda" or sink.device.type != "cuda":
        raise ValueError("stream_read needs device tensors")
    if sink.dtype not in (torch.int32, torch.uint32) or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous int32 or uint32 tensor")
    n = int(workgroups) or device_workers(buf.device.index or 0)
    if sink.numel() < n:
        raise ValueError(f"sink holds {sink.numel()} words; the probe writes one per workgroup ({n})")
    B._check(B.lib().lbsr_stream_read(B._ptr(buf), _nbytes(buf), int(workgroups), int(mode),
                                      B._ptr(sink), B._stream(stream)))


_ROW_AXES = {"NHD": (0, 1, 2), "HND": (0, 2, 1)}   # (page, token, head) axis of each form
_KINDS = {"k": 0, "v": 1}


def _row_strides(cfg, rows, layout):
    """Element strides (page, token, head) of a row-major cache view: a tensor
    [num_pages, 64, Hkv, 128] ("NHD") or [num_pages, Hkv, 64, 128] ("HND") of
    the cache dtype, with contiguous channels (other strides are free)."""
    if layout not in _ROW_AXES:
        raise ValueError(f"layout must be 'NHD' or 'HND', not {layout!r}")
    pa, ta, ha = _ROW_AXES[layout]
    want = [cfg.num_pages, 0, 0, B.HEAD_DIM]
    want[ta], want[ha] = B.PAGE_SIZE, cfg.num_kv_heads
    if not isinstance(rows, torch.Tensor) or not rows.is_cuda or rows.dtype != cfg.cache_dtype:
        raise ValueError(f"rows must be a device tensor of {cfg.cache_dtype}")
    if tuple(rows.shape) != tuple(want) or rows.stride(3) != 1:
        raise ValueError(f"rows must be {layout} {tuple(want)} with contiguous channels, "
                         f"got {tuple(rows.shape)} strides {rows.stride()}")
    st = rows.stride()
    return st[pa], st[ta], st[ha]


def pack_cache(cfg: DecodeConfig, kind, rows, cache, layout="NHD", stream=None):
    """lbsr_pack_cache: a row-major paged K or V cache (``kind`` "k" or "v";
    ``rows`` a [num_pages, 64, Hkv, 128] "NHD" or [num_pages, Hkv, 64, 128]
    "HND" view, any strides with contiguous channels) into ``cache``, a pool of
    the library's tile layout with cfg's geometry.  Asynchronous."""
    ps, ts, hs = _row_strides(cfg, rows, layout)
    _need(cache, "cache", cfg.cache_dtype, numel=cfg.pool_elems())
    B._check(B.lib().lbsr_pack_cache(ctypes.byref(cfg._shape()), _KINDS[kind], B._ptr(rows),
                                     ps, ts, hs, B._ptr(cache), B._stream(stream)))


def unpack_cache(cfg: DecodeConfig, kind, cache, rows, layout="NHD", stream=None):
    """lbsr_unpack_cache: the inverse of pack_cache (``rows`` receives the
    row-major form).  Asynchronous."""
    ps, ts, hs = _row_strides(cfg, rows, layout)
    _need(cache, "cache", cfg.cache_dtype, numel=cfg.pool_elems())
    B._check(B.lib().lbsr_unpack_cache(ctypes.byref(cfg._shape()), _KINDS[kind], B._ptr(cache),
                                       B._ptr(rows), ps, ts, hs, B._stream(stream)))


def xcd_rates(traces, plans):
    """Measured tile rate (tiles per microsecond of busy time) of each XCD.

    traces: per-worker records of split-attention launches, int64 [W, 4] =
    (start, end) of the 100 MHz constant clock, HW_ID, XCC_ID, as written by
    decode_step_timed(trace=...); plans: the matching read_plan() dicts (one
    per trace, or a single one for all).  XCD x's rate is the tiles its
    workers processed over the sum of their busy times.
    """
    if isinstance(plans, dict):
        plans = [plans] * len(traces)
    tiles = np.zeros(B.NUM_XCDS)
    busy = np.zeros(B.NUM_XCDS)
    for tr, pl in zip(traces, plans):
        tr = np.asarray(tr)
        per_worker = np.zeros(tr.shape[0])
        ch = np.asarray(pl["chunks"])
        np.add.at(per_worker, ch[:, 3], ch[:, 2] - ch[:, 1])
        x = tr[:, 3] & 0xF
        dur = (tr[:, 1] - tr[:, 0]) / 100.0
        for i in range(B.NUM_XCDS):
            m = x == i
            tiles[i] += per_worker[m].sum()
            busy[i] += dur[m].sum()
    if np.any(busy <= 0):
        raise ValueError("every XCD must have run a worker with work")
    return tiles / busy


def xcd_weights_from_rates(rates, scale=4096):
    """Integer weights for Schedule.xcd_weights: scale * rate / max(rate), at least 1."""
    r = np.asarray(rates, dtype=np.float64)
    if r.shape != (B.NUM_XCDS,) or not np.all(r > 0):
        raise ValueError("need 8 positive rates")
    w = np.clip(np.rint(scale * r / r.max()), 1, B.MAX_XCD_WEIGHT).astype(np.int64)
    return tuple(int(v) for v in w)
