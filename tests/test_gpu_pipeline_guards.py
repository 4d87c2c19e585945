"""The row-chunked dense indexer on one and on two streams (P3's pipelined mode: chunk
n's top-k on a side stream while chunk n + 1's logits run) against the fp64 oracle,
and a fused call whose outputs and workspace sit between guard bands that must
come back untouched."""
import numpy as np
import pytest
import torch

import mqa_logits_top_amd as idx
from mqa_logits_top_amd.pipeline import RowChunkedDense
import oracle
import synth
from checks import topk_ok, windows_match

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k_fmt,H,rows", [(synth.K_FP8, 32, 300), (synth.K_MXFP4, 64, 257)])
def test_two_stream_pipeline_vs_oracle(k_fmt, H, rows):
    T, L, K = 1200, 20000, 256
    p = synth.make_problem(T, L, H, k_fmt=k_fmt, seed=91 + H)
    d = idx.Inputs.from_host(p)
    dq = oracle.Dequantised(p)
    windows_match(d, dq)
    rc = RowChunkedDense(d, K, rows)
    assert len(rc.chunks) >= 4
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    si = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    sv = torch.empty((T, K), dtype=torch.float32, device="cuda")
    pi = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    pv = torch.empty((T, K), dtype=torch.float32, device="cuda")
    rc.run(si, sv, stream)
    for _ in range(2):   # twice: the second run reuses buffers the first left behind
        rc.run(pi, pv, stream, side)
    torch.cuda.synchronize()
    assert torch.equal(si, pi) and torch.equal(sv.view(torch.int32), pv.view(torch.int32))
    fi, fv = idx.idx_logits_topk_fused(d, K, block_k=4096)
    assert torch.equal(fi, pi) and torch.equal(fv.view(torch.int32), pv.view(torch.int32))
    o = oracle.rows_logits(dq, range(T))
    topk_ok(pi.cpu().numpy(), pv.cpu().numpy(), o, dq.ks, K)


GUARD = 4096


def _guarded(nbytes, dtype, fill=0xA5):
    """A buffer of nbytes between two GUARD-byte bands of `fill`; returns (whole, view)."""
    whole = torch.full((GUARD + nbytes + GUARD,), fill, dtype=torch.uint8, device="cuda")
    return whole, whole[GUARD:GUARD + nbytes].view(dtype)


def _bands_intact(whole, fill=0xA5):
    w = whole.cpu().numpy()
    return (w[:GUARD] == fill).all() and (w[-GUARD:] == fill).all()


def test_fused_call_stays_inside_its_buffers():
    """Outputs and workspace surrounded by 0xA5 guard bands: several row chunks, key launches
    that take the slab path, a masked consumer and the slot transform; the bands are intact
    afterwards and the results match the oracle."""
    T, L, H, K, Bk, rc = 300, 9000, 64, 100, 2048, 128
    p = synth.make_problem(T, L, H, seed=5)
    d = idx.Inputs.from_host(p)
    dq = oracle.Dequantised(p)
    nws = idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=K, block_k=Bk, row_chunk=rc)
    wws, ws = _guarded(nws, torch.uint8, fill=0x3C)
    ws.fill_(0x3C)
    wi, oi = _guarded(T * K * 4, torch.int32)
    wv, ov = _guarded(T * K * 4, torch.float32)
    wsl, osl = _guarded(T * K * 4, torch.int32)
    oi, ov, osl = oi.view(T, K), ov.view(T, K), osl.view(T, K)
    table = torch.arange(L, dtype=torch.int32, device="cuda") * 3 + 1
    idx.idx_logits_topk_fused_paged(d, K, table, block_k=Bk, row_chunk=rc, out_idx=oi, out_val=ov, out_slot=osl, ws=ws)
    torch.cuda.synchronize()
    assert idx.overflow_count(ws) == 0
    for name, whole in (("idx", wi), ("val", wv), ("slot", wsl)):
        assert _bands_intact(whole), f"{name}: guard band overwritten"
    assert _bands_intact(wws, fill=0x3C), "workspace: guard band overwritten"
    o = oracle.rows_logits(dq, range(T))
    topk_ok(oi.cpu().numpy(), ov.cpu().numpy(), o, dq.ks, K)
    ids = oi.cpu().numpy()
    assert np.array_equal(osl.cpu().numpy(), np.where(ids >= 0, ids * 3 + 1, -1))
    # a masked consumer into the same guarded buffers
    rng = np.random.default_rng(3)
    W = d.W
    mask = torch.from_numpy((rng.random((T, W)) < 0.2).astype(np.uint8)).cuda()
    idx.idx_logits_topk_fused(d, K, block_k=Bk, row_chunk=rc, mask=mask, out_idx=oi, out_val=ov, ws=ws)
    torch.cuda.synchronize()
    for name, whole in (("idx", wi), ("val", wv)):
        assert _bands_intact(whole), f"{name}: guard band overwritten (masked)"
    assert _bands_intact(wws, fill=0x3C), "workspace: guard band overwritten (masked)"
    allowed = [mask[t, :len(o[t])].cpu().numpy().astype(bool) for t in range(T)]
    topk_ok(oi.cpu().numpy(), ov.cpu().numpy(), o, dq.ks, K, allowed=allowed)
