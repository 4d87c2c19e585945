"""Launch timing: with a record on, every scoring launch of a call gets its own pair of events
on the call's stream.  A fused call's record matches its key schedule (block launches, the
slab launch, the passes over flagged row blocks), each with a positive duration; a call under
stream capture and calls after the record stops are not recorded."""
import os

import pytest
import torch

import mqa_logits_top_amd as idx
import synth

pytestmark = pytest.mark.gpu


def _fused_problem():
    # K + 512 = 576 and B_k = 8192: keys 0..16384 in two block launches (20 x 576 > 8192),
    # then keys 16384..40000 in one slab launch, whose flagged-row passes take three blocks
    return idx.Inputs.from_host(synth.make_problem(16, 40000, 64, k_fmt=synth.K_FP8, seed=12))


def test_fused_call_record_follows_its_schedule():
    d = _fused_problem()
    idx.idx_logits_topk_fused(d, 64, block_k=8192)          # warm
    torch.cuda.synchronize()
    idx.idx_launch_timing(True)
    try:
        idx.idx_logits_topk_fused(d, 64, block_k=8192)
        rec = idx.idx_launch_timing_read()
    finally:
        idx.idx_launch_timing(False)
    got = [(e["mode"], e["flagged"], e["row0"], e["nrows"], e["key0"], e["nkeys"]) for e in rec]
    if os.environ.get("IDX_EXACT", "0") not in ("", "0"):
        # exact scores: no candidate slabs, one block per launch
        want = [("block", False, 0, 16, kb, min(8192, 40000 - kb)) for kb in range(0, 40000, 8192)]
    else:
        want = [("block", False, 0, 16, 0, 8192), ("block", False, 0, 16, 8192, 8192),
                ("slab", False, 0, 16, 16384, 23616),
                ("block", True, 0, 16, 16384, 8192), ("block", True, 0, 16, 24576, 8192),
                ("block", True, 0, 16, 32768, 7232)]
    assert got == want, got
    assert all(e["ms"] > 0 for e in rec), rec


def test_dense_launch_capture_and_stop():
    d = _fused_problem()
    W = d.W
    out = torch.empty((d.T, W), dtype=torch.float32, device="cuda")
    idx.idx_mqa_logits(d, W, out=out)
    torch.cuda.synchronize()
    idx.idx_launch_timing(True)
    try:
        idx.idx_mqa_logits(d, W, out=out)
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):                          # captured: not recorded
            idx.idx_mqa_logits(d, W, out=out)
        g.replay()
        torch.cuda.synchronize()
        rec = idx.idx_launch_timing_read()                 # clears the record, recording goes on
        idx.idx_mqa_logits_block(d, 2, 5, 256, 300, out=out)
        rec2 = idx.idx_launch_timing_read()
        idx.idx_launch_timing(False)
        idx.idx_mqa_logits(d, W, out=out)                  # after the stop: not recorded
        rec3 = idx.idx_launch_timing_read()
    finally:
        idx.idx_launch_timing(False)
    assert [(e["mode"], e["row0"], e["nrows"], e["key0"], e["nkeys"]) for e in rec] == [("dense", 0, d.T, 0, d.L)]
    assert rec[0]["ms"] > 0
    assert [(e["mode"], e["row0"], e["nrows"], e["key0"], e["nkeys"]) for e in rec2] == [("block", 2, 5, 256, 300)]
    assert rec3 == []
