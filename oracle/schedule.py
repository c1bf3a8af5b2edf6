"""The per-step tile schedule: dynamic (length-proportional) and static split-KV.

Page A, "Why does dynamic scheduling matter in attention?": a static split-KV
schedule is built for a batch of equal lengths, so with mixed lengths some
compute units idle while others still work through the long sequence; the
backend's decode scheduler instead deals 64-token tiles to the compute units
in proportion to each sequence's actual length at the current step.

Readings:

* R5 -- a sequence's length L counts the new token; it has n = ceil(L/64)
  tiles.
* R11 (dynamic) -- lay all tiles of the batch end to end in sequence order
  (T tiles in total); worker w of P owns flat tiles
  [floor(w*T/P), floor((w+1)*T/P)).  A worker's range is cut where a sequence
  ends; each piece is a *chunk* (sequence, first tile, end tile, worker), with
  tile indices local to the sequence.  Chunks are numbered in flat order.
* R11w (weighted dynamic, an MI355X refinement; the pages assume equal
  compute units) -- worker w weighs the weight of the XCD that runs it and
  owns flat tiles [floor(T*C(w)/C(P)), floor(T*C(w+1)/C(P))), C(w) being the
  summed weight of workers 0..w-1.  The attention launch deals workgroup i to
  XCD i mod 8 and gives each XCD a contiguous run of workers, XCD 0's first,
  so XCD x runs as many workers as there are i < P with i mod 8 == x.  Equal
  weights give R11 exactly.
* R12 (static) -- every sequence gets the same number of splits S
  (default max(1, floor(P/B))); split s of sequence b covers its tiles
  [floor(s*n_b/S), floor((s+1)*n_b/S)) and is worker b*S + s; empty splits
  produce no chunk.

Both produce the same arrays: per-sequence tile prefix sums, per-worker chunk
ranges, the chunk list and per-sequence chunk ranges.  The schedule is integer
arithmetic with a unique answer; products w*T use Python integers, so there
is no overflow at any size.
"""

from dataclasses import dataclass

import numpy as np

TILE_TOKENS = 64


@dataclass
class Plan:
    cu_tiles: np.ndarray      # [B+1] prefix sums of tiles per sequence
    worker_chunk: np.ndarray  # [W+1] worker w owns chunks [worker_chunk[w], worker_chunk[w+1])
    chunks: np.ndarray        # [C, 4] (sequence, first tile, end tile, worker)
    seq_chunk: np.ndarray     # [B+1] sequence b owns chunks [seq_chunk[b], seq_chunk[b+1])
    num_workers: int

    @property
    def num_chunks(self):
        return int(self.chunks.shape[0])


def tiles_per_sequence(seq_lens, tile=TILE_TOKENS):
    """n_b = ceil(L_b / 64) (R5)."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    if np.any(lens < 1):
        raise ValueError("every sequence must hold at least the new token")
    return (lens + tile - 1) // tile


def _seq_chunk(chunks, batch):
    seq_chunk = np.zeros(batch + 1, dtype=np.int64)
    for b in range(batch):
        idx = np.nonzero(chunks[:, 0] == b)[0]
        seq_chunk[b] = idx[0]
        # a sequence's chunks are consecutive in both schedules
        assert np.array_equal(idx, np.arange(idx[0], idx[0] + idx.size))
    seq_chunk[batch] = chunks.shape[0]
    return seq_chunk


NUM_XCDS = 8


def workers_per_xcd(num_workers):
    """How many of the P workgroups each XCD receives when workgroup i goes to XCD i mod 8 (R11w)."""
    return [len(range(x, int(num_workers), NUM_XCDS)) for x in range(NUM_XCDS)]


def worker_weights(num_workers, xcd_weights=None):
    """Weight of every worker: 1 each, or its XCD's weight, XCD 0's run first (R11w)."""
    P = int(num_workers)
    if xcd_weights is None:
        return [1] * P
    if len(xcd_weights) != NUM_XCDS or any(int(x) < 1 for x in xcd_weights):
        raise ValueError("xcd_weights: 8 positive integers")
    out = []
    for x, count in enumerate(workers_per_xcd(P)):
        out += [int(xcd_weights[x])] * count
    return out


def plan_dynamic(seq_lens, num_workers, xcd_weights=None):
    """Length-proportional schedule over flat 64-token tiles (R11; R11w with weights)."""
    n = tiles_per_sequence(seq_lens)
    batch = n.size
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    total = int(cu[-1])
    P = int(num_workers)
    if P < 1:
        raise ValueError("need at least one worker")
    cum = [0]
    for wt in worker_weights(P, xcd_weights):
        cum.append(cum[-1] + wt)
    chunks = []
    worker_chunk = [0]
    for w in range(P):
        start = (total * cum[w]) // cum[P]
        end = (total * cum[w + 1]) // cum[P]
        t = start
        while t < end:
            b = int(np.searchsorted(cu, t, side="right") - 1)   # sequence holding flat tile t
            stop = min(end, int(cu[b + 1]))
            chunks.append((b, t - int(cu[b]), stop - int(cu[b]), w))
            t = stop
        worker_chunk.append(len(chunks))
    chunks = np.asarray(chunks, dtype=np.int64).reshape(-1, 4)
    return Plan(cu, np.asarray(worker_chunk, dtype=np.int64), chunks,
                _seq_chunk(chunks, batch), P)


def default_static_splits(batch, num_workers):
    """S = max(1, floor(P / B)) (R12)."""
    return max(1, int(num_workers) // int(batch))


def plan_static(seq_lens, splits):
    """Static equal split-KV: S splits of every sequence's own tiles (R12)."""
    n = tiles_per_sequence(seq_lens)
    batch = n.size
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    S = int(splits)
    if S < 1:
        raise ValueError("need at least one split")
    chunks = []
    worker_chunk = [0]
    for b in range(batch):
        nb = int(n[b])
        for s in range(S):
            t0 = (s * nb) // S
            t1 = ((s + 1) * nb) // S
            if t1 > t0:
                chunks.append((b, t0, t1, b * S + s))
            worker_chunk.append(len(chunks))
    chunks = np.asarray(chunks, dtype=np.int64).reshape(-1, 4)
    return Plan(cu, np.asarray(worker_chunk, dtype=np.int64), chunks,
                _seq_chunk(chunks, batch), batch * S)
