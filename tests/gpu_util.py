"""Helpers for the GPU parity tests: run the HIP path through the C ABI, and
bring the matching slice of the inputs to the host for the oracle."""

import numpy as np
import torch

import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU (gfx950)")
    return torch.device("cuda:0")


def to_device(inp, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def config_for(w, inp):
    return lb.DecodeConfig(w.num_q_heads, w.num_kv_heads, w.kv_dtype, inp["max_blocks"],
                           inp["num_pages"], page_stride=inp["page_stride"],
                           head_stride=inp["head_stride"], rope_theta=w.rope_theta,
                           rms_eps=w.rms_eps, norm_before_rope=w.norm_before_rope,
                           k_scale=w.k_scale, v_scale=w.v_scale,
                           tokens_per_seq=w.max_new_tokens)


def run_step(w, g, sched, lse=True, cfg=None):
    """One decode step through lbsr_decode_step on device inputs ``g`` (modified in place:
    the caches receive the new tokens).  Returns q_out, out, lse, plan, error word."""
    dev = g["q"].device
    cfg = cfg or config_for(w, g)
    ws = lb.alloc_workspace(cfg, w.batch, sched, device=dev)
    q_out = torch.empty_like(g["q"])
    out = torch.empty(g["q"].shape, dtype=cfg.out_torch_dtype, device=dev)
    lse_t = (torch.empty(cfg.tokens_shape(w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
             if lse else None)
    lb.decode_step(cfg, g["q"], g["k"], g["v"], g["positions"], g["seq_lens"], g["q_norm_w"],
                   g["k_norm_w"], g["block_table"], g["k_cache"], g["v_cache"], q_out, sched, ws,
                   out, lse_t)
    torch.cuda.synchronize()
    return {"q_out": q_out, "out": out, "lse": lse_t, "ws": ws, "cfg": cfg,
            "plan": lb.read_plan(cfg, w.batch, sched, ws),
            "error": lb.read_error(cfg, w.batch, sched, ws)}


def compact_pools(g, w, seqs):
    """Host copies of only the pages that sequences ``seqs`` own, renumbered
    0..n-1, with block-table rows rewritten to match.  Returns
    (k_pool, v_pool, block_table, page_map) where page_map[orig] = new."""
    bt = g["block_table"].cpu().numpy()
    pages = []
    for b in seqs:
        n = -(-int(w.seq_lens[b]) // 64)
        pages.extend(bt[b, :n].tolist())
    pages = sorted(set(pages))
    page_map = {p: i for i, p in enumerate(pages)}
    ps = g["page_stride"]
    idx = torch.tensor(pages, dtype=torch.long, device=g["k_cache"].device)
    n_pages = g["num_pages"]
    out = []
    for key in ("k_cache", "v_cache"):
        pool = g[key].view(n_pages, ps).index_select(0, idx).reshape(-1).cpu()
        if pool.dtype == torch.bfloat16:
            out.append(pool.view(torch.int16).numpy().view(np.uint16))
        else:
            out.append(pool.numpy())
    new_bt = np.full_like(bt, -1)
    for b in seqs:
        n = -(-int(w.seq_lens[b]) // 64)
        new_bt[b, :n] = [page_map[p] for p in bt[b, :n]]
    return out[0], out[1], new_bt, page_map


def remap_slots(pro, page_map):
    pro = dict(pro)
    slots = pro["slots"].copy()
    slots[:, 0] = [page_map.get(int(p), -1) for p in slots[:, 0]]
    pro["slots"] = slots
    return pro
