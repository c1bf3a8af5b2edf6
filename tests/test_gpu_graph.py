"""The step captured in a HIP graph ([B] "Code analysis 2": the op writes a
caller-provided output and is entered directly, so it can be captured).

The library records only kernel launches (no memsets, copies or
allocations).  Each test captures a call once, replays it several times with
the program's own eager work and synchronisations between the replays, and
checks every replay against the eager result bit for bit (same kernels, same
inputs: the results are deterministic)."""

import pytest
import torch

import load_balanced_split_rope_amd as lb
from load_balanced_split_rope_amd import workloads as wl
from gpu_util import device, to_device, config_for

pytestmark = pytest.mark.gpu


def replay_and_compare(call, outputs, replays=4):
    """Run `call` eagerly, capture it, then replay it `replays` times, each
    time after clobbering the outputs and doing unrelated eager work."""
    call()
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                          # warm up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        call()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=outputs[0].device)
    for r in range(replays):
        for t in outputs:
            t.zero_()
        scratch.mul_(1.0001).add_(0.5)                   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, w in zip(outputs, want):
            assert torch.equal(t, w), f"replay {r}"


@pytest.mark.parametrize("kv_dtype,out_dtype", [("bf16", "bf16"), ("fp8", "bf16"),
                                                ("bf16", "fp8")])
def test_decode_step_in_a_graph(kv_dtype, out_dtype):
    dev = device()
    w = wl.custom([3000, 70, 5000, 1, 64], num_q_heads=64, num_kv_heads=8, kv_dtype=kv_dtype,
                  seed=960)
    g = to_device(wl.make_inputs(w), dev)
    cfg = config_for(w, g)
    cfg.out_dtype, cfg.out_scale = out_dtype, 2.0 ** -6
    sched = lb.Schedule("dynamic", num_workers=256)
    ws = lb.alloc_workspace(cfg, w.batch, sched, device=dev)
    q_out = torch.empty_like(g["q"])
    out = torch.empty(g["q"].shape, dtype=cfg.out_torch_dtype, device=dev)
    lse = torch.empty(w.batch, 64, dtype=torch.float32, device=dev)

    def call():
        lb.decode_step(cfg, g["q"], g["k"], g["v"], g["positions"], g["seq_lens"],
                       g["q_norm_w"], g["k_norm_w"], g["block_table"], g["k_cache"],
                       g["v_cache"], q_out, sched, ws, out, lse)

    replay_and_compare(call, [q_out, out, lse])
    assert lb.read_error(cfg, w.batch, sched, ws) == 0


def test_ragged_prefill_step_in_a_graph():
    """The ragged prefill records two launches besides the prologue: the plan
    that writes the work list into the workspace, then attention."""
    dev = device()
    w = wl.custom([300, 5, 700, 64], seed=961, new_tokens=[300, 0, 33, 1])
    g = to_device(wl.make_inputs(w), dev)
    cfg = config_for(w, g)
    ws = lb.alloc_prefill_workspace(cfg, w.batch, g["q"].shape[0], device=dev)
    q_out, out = torch.empty_like(g["q"]), torch.empty_like(g["q"])
    lse = torch.empty(g["q"].shape[:2], dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def call():
        lb.prefill_step_varlen(cfg, g["q_start"], g["q"], g["k"], g["v"], g["positions"],
                               g["seq_lens"], g["q_norm_w"], g["k_norm_w"], g["block_table"],
                               g["k_cache"], g["v_cache"], q_out, ws, out, lse, err)

    replay_and_compare(call, [q_out, out, lse])
    assert int(err.item()) == 0


@pytest.mark.parametrize("fold", [False, True])
def test_consecutive_steps_in_one_graph(fold):
    """Two decode steps of different batches captured in one graph, sharing one
    workspace (as a decode loop captures several steps or layers at once): the
    second step's schedule overwrites the first's in stream order, and each
    step's outputs must equal its eager run on every replay."""
    dev = device()
    wa = wl.custom([3000, 70, 5000, 1, 64], num_q_heads=64, num_kv_heads=8, seed=962)
    wb = wl.custom([129, 8000, 2, 640, 65, 4096], num_q_heads=64, num_kv_heads=8, seed=963)
    ga, gb = to_device(wl.make_inputs(wa), dev), to_device(wl.make_inputs(wb), dev)
    sched = lb.Schedule("dynamic", num_workers=256, fold_merge=fold)
    cfa, cfb = config_for(wa, ga), config_for(wb, gb)
    ws = lb.alloc_workspace(cfb if wb.batch >= wa.batch else cfa, max(wa.batch, wb.batch), sched,
                            device=dev)
    assert ws.numel() >= lb.workspace_layout(cfa, wa.batch, sched).total
    bufs = []
    for w, g in ((wa, ga), (wb, gb)):
        bufs.append((torch.empty_like(g["q"]), torch.empty_like(g["q"]),
                     torch.empty(w.batch, 64, dtype=torch.float32, device=dev)))

    def call():
        for (w, g, cf), (q_out, out, lse) in zip(((wa, ga, cfa), (wb, gb, cfb)), bufs):
            lb.decode_step(cf, g["q"], g["k"], g["v"], g["positions"], g["seq_lens"],
                           g["q_norm_w"], g["k_norm_w"], g["block_table"], g["k_cache"],
                           g["v_cache"], q_out, sched, ws, out, lse)

    replay_and_compare(call, [t for b in bufs for t in b])
