"""The five workloads at full size, in the launch configuration the benchmark
uses, checked against the fp64 oracle: every row of the tiny and GLM-shaped
chunks, sampled rows elsewhere (first and last rows of each request, rows next
to row-chunk and key-block boundaries, and a stride), plus properties that hold
at any size: fused == dense + refine bitwise, row-count invariance over row
chunks of 128 .. 4096 rows, and the candidate mask's internal consistency."""
import numpy as np
import pytest
import torch

import mqa_logits_top_amd as idx
import oracle
import synth
from checks import dense_ref, logits_ok, topk_ok, windows_match

pytestmark = pytest.mark.gpu

_cache = {}


def prob(name):
    if name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        p = synth.make_config(name)
        d = idx.Inputs.from_host(p)
        dq = oracle.Dequantised(p)
        windows_match(d, dq)
        _cache[name] = (p, d, dq)
    return _cache[name]


def sample_rows(dq, meta, n_stride=12):
    T = dq.T
    rows = {0, T - 1}
    rows.update(range(0, T, max(1, T // n_stride)))
    for b in (128, 1024, 1100, 2048, 4096, 8192):
        for r in (b - 1, b):
            if r < T:
                rows.add(r)
    if "cu_q" in meta:
        for c in meta["cu_q"]:
            for r in (c - 1, c):
                if 0 <= r < T:
                    rows.add(r)
    return sorted(rows)


def fused(d, K, block_k, row_chunk=0, mask=None):
    ws = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=K, block_k=block_k,
                                            row_chunk=row_chunk), dtype=torch.uint8, device="cuda")
    gi, gv = idx.idx_logits_topk_fused(d, K, block_k=block_k, row_chunk=row_chunk, mask=mask, ws=ws)
    torch.cuda.synchronize()
    assert idx.overflow_count(ws) == 0
    return gi, gv


def _check_rows(d, dq, rows, gi, gv, K, lg=None, chunk=256):
    """Oracle rows in chunks (bounded host memory): fused top-K sets and values, and the dense
    logits of the same rows when lg is given."""
    rows = list(rows)
    for c0 in range(0, len(rows), chunk):
        rs = rows[c0:c0 + chunk]
        o = oracle.rows_logits(dq, rs)
        topk_ok(gi[rs], gv[rs], o, dq.ks[rs], K, what=f"rows {rs[0]}..{rs[-1]}")
        if lg is not None:
            g = lg[rs].cpu().numpy()
            logits_ok(g, dense_ref(o, g.shape[1]), what=f"logits rows {rs[0]}..{rs[-1]}")


@pytest.mark.parametrize("name", ["tiny", "glm_chunk", "dsv4_mxfp4"])
def test_config_fused_vs_oracle(name):
    """tiny and glm_chunk: every row; dsv4_mxfp4: sampled rows.  Fused top-K and dense
    logits against the oracle; the dense comparator (top-(K + 512) of the dense logits,
    then the exact boundary) equals the fused result bitwise."""
    p, d, dq = prob(name)
    K, Bk = p.meta["K"], p.meta["block_k"]
    gi, gv = fused(d, K, Bk)
    rows = range(dq.T) if name in ("tiny", "glm_chunk") else sample_rows(dq, p.meta)
    lg = idx.idx_mqa_logits(d, d.W)
    gin, gvn = gi.cpu().numpy(), gv.cpu().numpy()
    _check_rows(d, dq, rows, gin, gvn, K, lg)
    ci, cv = idx.idx_topk(lg, d.ks, d.ke, idx.candidate_capacity(K))
    del lg
    di, dv = idx.idx_refine_topk(d, ci, cv, K)
    assert torch.equal(di, gi)
    assert torch.equal(dv.view(torch.int32), gv.view(torch.int32))


def test_dsv4_row_count_invariance():
    """P2 Accuracy/equivalence: scoring all rows in one call or in row chunks of 128 .. 4096
    gives identical output (bitwise), here at the DeepSeek-V4-like MXFP4 shape."""
    p, d, dq = prob("dsv4_mxfp4")
    K, Bk = p.meta["K"], p.meta["block_k"]
    gi, gv = fused(d, K, Bk, row_chunk=0)
    for rc in (128, 256, 512, 1024, 2048, 4096):
        ci, cv = fused(d, K, Bk, row_chunk=rc)
        assert torch.equal(ci, gi) and torch.equal(cv.view(torch.int32), gv.view(torch.int32)), rc


def test_long_ctx_row_count_invariance():
    """P2 Accuracy/equivalence at its own shape: the 16384-row long-context chunk scored in one
    call and in row chunks of 128 .. 4096 gives identical output, bitwise."""
    p, d, dq = prob("long_ctx")
    K, Bk = p.meta["K"], p.meta["block_k"]
    gi, gv = fused(d, K, Bk, row_chunk=0)
    for rc in (128, 256, 512, 1024, 2048, 4096):
        ci, cv = fused(d, K, Bk, row_chunk=rc)
        assert torch.equal(ci, gi) and torch.equal(cv.view(torch.int32), gv.view(torch.int32)), rc


def test_dsv4_duplicate_keys_tie_by_index():
    p, d, dq = prob("dsv4_mxfp4")
    K = p.meta["K"]
    gi, _ = fused(d, K, p.meta["block_k"])
    gi = gi.cpu().numpy()
    dst, src = p.meta["dup_dst"], p.meta["dup_src"]
    # a duplicated key scores exactly like its source: when both are in a row's window,
    # either both are selected, or only the lower index, or neither
    bad = 0
    for t in sample_rows(dq, p.meta):
        sel = set(gi[t][gi[t] >= 0].tolist())
        ke = int(dq.ke[t])
        for a_, b_ in zip(dst, src):
            if a_ < ke and b_ < ke:
                lo, hi = min(a_, b_), max(a_, b_)
                bad += (hi in sel) and (lo not in sel)
    assert bad == 0


def test_long_ctx_fused_vs_rowchunked_dense():
    p, d, dq = prob("long_ctx")
    K, Bk = p.meta["K"], p.meta["block_k"]
    gi, gv = fused(d, K, Bk, row_chunk=4096)
    rows = sample_rows(dq, p.meta, n_stride=8)
    _check_rows(d, dq, rows, gi.cpu().numpy(), gv.cpu().numpy(), K)
    # row-count invariance: other row chunks give identical bits
    gi2, gv2 = fused(d, K, Bk, row_chunk=1024)
    assert torch.equal(gi, gi2) and torch.equal(gv.view(torch.int32), gv2.view(torch.int32))
    # the row-chunked dense comparator under a 2 GiB fp32 logits budget
    W = d.W
    chunk = (2 << 30) // (4 * W)
    buf = torch.empty((chunk, W), dtype=torch.float32, device="cuda")
    Kc = idx.candidate_capacity(K)
    ci = torch.empty((p.T, Kc), dtype=torch.int32, device="cuda")
    cv = torch.empty((p.T, Kc), dtype=torch.float32, device="cuda")
    for r0 in range(0, p.T, chunk):
        nr = min(chunk, p.T - r0)
        sub = idx.Inputs(q=d.q[r0:r0 + nr], q_scale=d.q_scale[r0:r0 + nr], k=d.k, k_scale=d.k_scale,
                         w=d.w[r0:r0 + nr], ks=d.ks[r0:r0 + nr], ke=d.ke[r0:r0 + nr], k_fmt=d.k_fmt)
        lg = idx.idx_mqa_logits(sub, W, out=buf[:nr])
        idx.idx_topk(lg, sub.ks, sub.ke, Kc, out_idx=ci[r0:r0 + nr], out_val=cv[r0:r0 + nr])
    del buf
    di, dv = idx.idx_refine_topk(d, ci, cv, K)
    assert torch.equal(di, gi) and torch.equal(dv.view(torch.int32), gv.view(torch.int32))


def test_ragged_candidates_and_masked_consumer():
    p, d, dq = prob("ragged_cand")
    c = p.meta
    W = d.W
    n_blocks, pool, K = c["n_blocks"], c["pool"], c["K"]
    blocks = torch.empty((p.T, n_blocks), dtype=torch.int32, device="cuda")
    ws = torch.empty(idx.idx_workspace_size(idx.IDX_OP_BLOCK_CANDIDATES, d, block_k=c["block_k"], row_chunk=4096,
                                            pool=pool, n_blocks=n_blocks), dtype=torch.uint8, device="cuda")
    mask, _ = idx.idx_block_candidates(d, W, pool=pool, n_blocks=n_blocks, block_k=c["block_k"], row_chunk=4096,
                                       out_blocks=blocks, ws=ws)
    torch.cuda.synchronize()
    assert idx.overflow_count(ws) == 0
    rows = sample_rows(dq, p.meta, n_stride=8)
    o = oracle.rows_logits(dq, rows)
    mk = mask[rows].cpu().numpy()
    bk = blocks[rows].cpu().numpy()
    for i, (t, v) in enumerate(zip(rows, o)):
        P = oracle.pool_row(v, pool)
        gb = bk[i][bk[i] >= 0]
        assert len(gb) == min(n_blocks, len(P))
        want = np.zeros(W, np.uint8)
        for b in gb:
            want[b * pool:min((b + 1) * pool, len(v))] = 1
        assert np.array_equal(mk[i], want), f"row {t}"
        topk_ok(np.concatenate([gb, -np.ones(n_blocks - len(gb), np.int64)])[None], None, [P], [0], n_blocks,
                what=f"blocks row {t}")
    # a later layer (fresh q, w; same keys) restricted to the published mask
    p2 = synth.consumer_layer(p)
    d2 = idx.Inputs.from_host(p2)
    gi, gv = fused(d2, K, c["block_k"], row_chunk=4096, mask=mask)
    dq2 = oracle.Dequantised(p2)
    o2 = oracle.rows_logits(dq2, rows)
    allowed = [mk[i][:len(o2[i])].astype(bool) for i in range(len(rows))]
    topk_ok(gi.cpu().numpy()[rows], gv.cpu().numpy()[rows], o2, dq.ks[rows], K, allowed=allowed)
    # the same consumer reading the block ids instead of the byte mask: identical output
    bi, bv = idx.idx_logits_topk_fused_blocks(d2, K, blocks, pool=pool, block_k=c["block_k"], row_chunk=4096)
    assert torch.equal(bi, gi) and torch.equal(bv.view(torch.int32), gv.view(torch.int32))
