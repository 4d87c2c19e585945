"""The allocation-free fused indexer (library-owned static workspace) against the entry point
with a caller workspace: identical outputs on two calls in a row on one GPU, the second with a
smaller problem (the workspace keeps the first call's contents), a masked call, and the size
limit reported before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import mqa_logits_top_amd as idx
import oracle
import synth
from checks import topk_ok

pytestmark = pytest.mark.gpu


def _pair(p, K, block_k, row_chunk, mask=None):
    d = idx.Inputs.from_host(p)
    si, sv = idx.idx_logits_topk_fused_static(d, K, block_k=block_k, row_chunk=row_chunk, mask=mask)
    ws = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=K, block_k=block_k,
                                            row_chunk=row_chunk), dtype=torch.uint8, device="cuda")
    fi, fv = idx.idx_logits_topk_fused(d, K, block_k=block_k, row_chunk=row_chunk, mask=mask, ws=ws)
    torch.cuda.synchronize()
    assert idx.overflow_count(ws) == 0
    return d, (si, sv), (fi, fv)


def test_static_workspace_equals_caller_workspace():
    # first call: 3 row chunks x 3 key launches (slab path), H = 64, fp8 keys
    p1 = synth.make_problem(700, 40000, 64, seed=12)
    K1, bk1, rc1 = 300, 8192, 256
    d1, (si, sv), (fi, fv) = _pair(p1, K1, bk1, rc1)
    assert torch.equal(si, fi) and torch.equal(sv.view(torch.int32), fv.view(torch.int32))
    dq1 = oracle.Dequantised(p1)
    rows = [0, 255, 256, 511, 512, 699]
    topk_ok(si.cpu().numpy()[rows], sv.cpu().numpy()[rows], oracle.rows_logits(dq1, rows), dq1.ks[rows], K1)
    # second call, smaller: H = 32, MXFP4 keys, one row chunk, a consumer mask
    p2 = synth.make_problem(90, 5000, 32, k_fmt=synth.K_MXFP4, seed=13)
    rng = np.random.default_rng(13)
    mask = torch.from_numpy((rng.random((90, 5000)) < 0.4).astype(np.uint8)).cuda()
    d2, (si2, sv2), (fi2, fv2) = _pair(p2, 64, 2048, 0, mask=mask)
    assert torch.equal(si2, fi2) and torch.equal(sv2.view(torch.int32), fv2.view(torch.int32))
    dq2 = oracle.Dequantised(p2)
    o2 = oracle.rows_logits(dq2, range(90))
    allowed = [mask[t, :len(o2[t])].cpu().numpy().astype(bool) for t in range(90)]
    topk_ok(si2.cpu().numpy(), sv2.cpu().numpy(), o2, dq2.ks, 64, allowed=allowed)
    # the first problem again after the second: the same bits
    si3, sv3 = idx.idx_logits_topk_fused_static(d1, K1, block_k=bk1, row_chunk=rc1)
    assert torch.equal(si3, fi) and torch.equal(sv3.view(torch.int32), fv.view(torch.int32))


def test_static_workspace_size_limit():
    """A call that would need more than IDX_STATIC_WS_BYTES is refused (nothing enqueued); a
    smaller row chunk of the same problem fits."""
    p = synth.make_problem(2048, 65536, 32, seed=0)
    d = idx.Inputs.from_host(p)
    need = idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=2048, block_k=32768)
    assert need > idx.STATIC_WS_BYTES
    oi = torch.full((d.T, 2048), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(idx.IdxError) as e:
        idx.idx_logits_topk_fused_static(d, 2048, block_k=32768, out_idx=oi)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert (oi == -7).all()
    rc = 256
    assert idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=2048, block_k=32768,
                                  row_chunk=rc) <= idx.STATIC_WS_BYTES
    si, sv = idx.idx_logits_topk_fused_static(d, 2048, block_k=32768, row_chunk=rc)
    fi, fv = idx.idx_logits_topk_fused(d, 2048, block_k=32768, row_chunk=rc)
    assert torch.equal(si, fi) and torch.equal(sv.view(torch.int32), fv.view(torch.int32))
