"""The streaming-read probe (lbsr_stream_read) reads every byte of its buffer
exactly once, in both forms and for any workgroup count: each workgroup
folds what it read into one XOR word, so the XOR of the sink words must equal
the XOR of the whole buffer.  With random contents a block that is skipped, or
read twice (x ^ x = 0), changes the result."""

import numpy as np
import pytest
import torch

import load_balanced_split_rope_amd as lb
from gpu_util import device

pytestmark = pytest.mark.gpu

BLOCK = 32 * 1024     # the probe's burst: a buffer is a whole number of them


def xor_all(t):
    return int(np.bitwise_xor.reduce(t.cpu().numpy().view(np.uint32).ravel()))


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("blocks,workgroups", [(1, 1), (1000, 0), (1000, 7), (1000, 256),
                                               (4099, 1000), (64, 2048)])
def test_stream_read_reads_every_byte_once(mode, blocks, workgroups):
    dev = device()
    g = torch.Generator(device="cpu").manual_seed(blocks * 31 + workgroups * 7 + mode)
    host = torch.randint(-2**31, 2**31 - 1, (blocks * BLOCK // 4,), dtype=torch.int64,
                         generator=g).to(torch.int32)
    buf = host.to(dev)
    n = workgroups or lb.device_workers(0)
    sink = torch.zeros(n, dtype=torch.int32, device=dev)
    print(f"stream_read mode {mode}: {blocks} blocks, {n} workgroups", flush=True)
    lb.stream_read(buf, sink, workgroups=workgroups, mode=mode)
    torch.cuda.synchronize()
    assert xor_all(sink) == xor_all(host)


def test_stream_read_refuses_a_short_sink():
    """One sink word per workgroup: a shorter sink is refused before any launch."""
    dev = device()
    buf = torch.zeros(BLOCK, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="one per workgroup"):
        lb.stream_read(buf, torch.zeros(7, dtype=torch.int32, device=dev), workgroups=8)
    with pytest.raises(ValueError, match="int32 or uint32"):
        lb.stream_read(buf, torch.zeros(8, dtype=torch.float32, device=dev), workgroups=8)
