"""The fused indexer captured in a HIP graph (torch.cuda.graph) and replayed: the library
enqueues only kernels on the caller's stream (no allocation, memset or synchronisation), so
a captured call replays to the eager result.  Each replay follows eager work of its own
(other library calls, fills of the outputs, synchronisations) and is checked bitwise against
the eager outputs: the caller-workspace entry and the allocation-free one."""
import pytest
import torch

import mqa_logits_top_amd as idx
import synth

pytestmark = pytest.mark.gpu

K, BLOCK_K, ROW_CHUNK = 300, 8192, 256   # 3 row chunks x (block launches + slab launches)


def _problem():
    return idx.Inputs.from_host(synth.make_problem(700, 40000, 64, seed=31))


def _other():
    return idx.Inputs.from_host(synth.make_problem(90, 5000, 32, k_fmt=synth.K_MXFP4, seed=32))


def _replays_match(call, d, outs, eager, other):
    oi, ov = outs
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(d, oi, ov)                      # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call(d, oi, ov)
    for rep in range(4):
        oi.fill_(-7)
        ov.fill_(float("nan"))
        other()                              # eager library work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(oi, eager[0]), f"replay {rep}: indices"
        assert torch.equal(ov.view(torch.int32), eager[1].view(torch.int32)), f"replay {rep}: values"


def test_caller_workspace_entry_in_a_graph():
    d = _problem()
    ws = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=K, block_k=BLOCK_K,
                                            row_chunk=ROW_CHUNK), dtype=torch.uint8, device="cuda")
    eager = idx.idx_logits_topk_fused(d, K, block_k=BLOCK_K, row_chunk=ROW_CHUNK, ws=ws)
    eager = (eager[0].clone(), eager[1].clone())
    oi = torch.empty_like(eager[0])
    ov = torch.empty_like(eager[1])
    d2 = _other()
    ws2 = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d2, K=64, block_k=2048),
                      dtype=torch.uint8, device="cuda")

    def call(dd, a, b):
        idx.idx_logits_topk_fused(dd, K, block_k=BLOCK_K, row_chunk=ROW_CHUNK, out_idx=a, out_val=b, ws=ws)

    _replays_match(call, d, (oi, ov), eager, lambda: idx.idx_logits_topk_fused(d2, 64, block_k=2048, ws=ws2))


def test_allocation_free_entry_in_a_graph():
    """The static workspace is shared with the eager calls between the replays (one stream, in
    order): each replay still reproduces the eager result."""
    d = _problem()
    eager = idx.idx_logits_topk_fused_static(d, K, block_k=BLOCK_K, row_chunk=ROW_CHUNK)
    eager = (eager[0].clone(), eager[1].clone())
    oi = torch.empty_like(eager[0])
    ov = torch.empty_like(eager[1])
    d2 = _other()

    def call(dd, a, b):
        idx.idx_logits_topk_fused_static(dd, K, block_k=BLOCK_K, row_chunk=ROW_CHUNK, out_idx=a, out_val=b)

    _replays_match(call, d, (oi, ov), eager, lambda: idx.idx_logits_topk_fused_static(d2, 64, block_k=2048))
