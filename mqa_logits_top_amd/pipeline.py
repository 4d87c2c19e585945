"""The row-chunked dense indexer, serial or on two streams.

P2 Modifications: the dense logits are computed for a chunk of rows at a time
under a fixed byte budget, and each chunk's top-k goes into one shared selected
buffer.  P3 ("the bench gains a pipelined mode"): chunk n's top-k runs on a side
stream, gated by an event, while chunk n + 1's logits run on the main stream.

Each chunk runs idx_mqa_logits into one of two row-major logit buffers, then
idx_topk keeps K + 512 candidates and idx_refine_topk settles the exact
boundary into the chunk's rows of the shared output.  With a side stream, the
selection of chunk n waits for its logits (an event recorded on the main
stream), and the logits of chunk n + 2 wait for the selection of chunk n, which
last read that buffer.  Both streams keep the default priority.  Every step is
a libidx call; this module only orders them.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (Inputs, REFINE_WS, candidate_capacity, idx_mqa_logits, idx_refine_topk, idx_topk)


def rows_for_budget(W: int, budget_bytes: int) -> int:
    """Rows of fp32 logits [rows, W] that fit the budget (P2: a 2 GiB logits budget)."""
    return max(1, budget_bytes // (4 * max(W, 1)))


class RowChunkedDense:
    """Buffers and launch order of the row-chunked dense indexer for one problem."""

    def __init__(self, d: Inputs, K: int, rows: int, W: Optional[int] = None):
        self.d, self.K, self.rows = d, K, rows
        self.W = d.W if W is None else W
        self.Kc = candidate_capacity(K)
        dev = d.q.device
        nr = min(rows, d.T)
        # logits rows padded by 64 floats, so that the rows streamed together start on
        # different memory channels
        self.bufs = [torch.empty((nr, self.W + 64), dtype=torch.float32, device=dev)[:, :self.W] for _ in range(2)]
        self.cand = [(torch.empty((nr, self.Kc), dtype=torch.int32, device=dev),
                      torch.empty((nr, self.Kc), dtype=torch.float32, device=dev)) for _ in range(2)]
        self.rws = [torch.empty(REFINE_WS, dtype=torch.uint8, device=dev) for _ in range(2)]
        self.chunks = [(r0, min(rows, d.T - r0)) for r0 in range(0, d.T, rows)]

    def peak_transient_bytes(self, two_streams: bool) -> int:
        """Buffers this comparator holds beyond the [T, K] outputs."""
        n = 2 if two_streams else 1
        per = self.bufs[0].shape[0] * self.W * 4 + self.cand[0][0].numel() * 8 + REFINE_WS
        return n * per

    def _sub(self, r0: int, n: int) -> Inputs:
        d = self.d
        return Inputs(q=d.q[r0:r0 + n], q_scale=d.q_scale[r0:r0 + n], k=d.k, k_scale=d.k_scale, w=d.w[r0:r0 + n],
                      ks=d.ks[r0:r0 + n], ke=d.ke[r0:r0 + n], k_fmt=d.k_fmt, scale=d.scale)

    def _select(self, i, r0, n, sp, out_idx, out_val, st):
        lg = self.bufs[i % 2][:n]
        ci, cv = self.cand[i % 2]
        idx_topk(lg, sp.ks, sp.ke, self.Kc, W=self.W, out_idx=ci[:n], out_val=cv[:n], stream=st)
        idx_refine_topk(sp, ci[:n], cv[:n], self.K, out_idx=out_idx[r0:r0 + n],
                        out_val=None if out_val is None else out_val[r0:r0 + n], ws=self.rws[i % 2], stream=st)

    def run(self, out_idx: torch.Tensor, out_val: Optional[torch.Tensor], stream, side=None):
        """Enqueue the whole comparator on `stream` (and `side` for the selections, if given)."""
        if side is None:
            for i, (r0, n) in enumerate(self.chunks):
                sp = self._sub(r0, n)
                idx_mqa_logits(sp, self.W, out=self.bufs[i % 2][:n], stream=stream)
                self._select(i, r0, n, sp, out_idx, out_val, stream)
            return
        done = [None, None]                   # selection of the chunk that last read each buffer
        for i, (r0, n) in enumerate(self.chunks):
            sp = self._sub(r0, n)
            if done[i % 2] is not None:
                stream.wait_event(done[i % 2])
            idx_mqa_logits(sp, self.W, out=self.bufs[i % 2][:n], stream=stream)
            ready = torch.cuda.Event()
            ready.record(stream)
            side.wait_event(ready)
            self._select(i, r0, n, sp, out_idx, out_val, side)
            done[i % 2] = torch.cuda.Event()
            done[i % 2].record(side)
        last = done[(len(self.chunks) - 1) % 2]
        if last is not None:
            stream.wait_event(last)
