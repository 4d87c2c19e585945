"""IDX_EXACT=1: every score is computed exactly from the stored codes in fp64 (no fp8 MFMA)
and rounded to fp32 once; the fused path writes no candidate slabs.  The two limits of the
default mode do not apply then: logits of rows whose head weights have both signs meet the
plain bar, and keys built to defeat the refinement band are selected exactly.  Every output
is checked against the oracle on the parity cases."""
import numpy as np
import pytest
import torch

import mqa_logits_top_amd as idx
import oracle
import synth
from checks import dense_ref, logits_ok, topk_ok
from test_gpu_parity import CASES, _aligned_truncation_problem, _case_id, _check_candidates, _make_case, dev

pytestmark = pytest.mark.gpu


@pytest.fixture
def exact(monkeypatch):
    monkeypatch.setenv("IDX_EXACT", "1")


def _within_one_ulp(g, o):
    """fp32 results of exact scores: the oracle's fp64 value rounded to fp32, up to one fp32 ulp
    (both sides round fp64 sums taken in different orders)."""
    fin = np.isfinite(o)
    g, o = np.asarray(g, np.float64)[fin], np.asarray(o, np.float64)[fin]
    ulp = np.spacing(np.abs(o).astype(np.float32)).astype(np.float64)
    bad = np.abs(g - o) > ulp
    assert not bad.any(), f"{bad.sum()} of {g.size} values more than one fp32 ulp from the oracle"


@pytest.mark.parametrize("param", CASES, ids=_case_id)
def test_exact_logits_meet_the_plain_bar(exact, param):
    """Dense logits and a key-block rectangle, head weights of either sign included."""
    c = _make_case(param)
    W = max(c.d.W, 1)
    g = idx.idx_mqa_logits(c.d, W).cpu().numpy()
    ref = dense_ref(c.o, W)
    logits_ok(g, ref)
    _within_one_ulp(g, ref)
    row0, nrows, key0, nkeys = 2, c.p.T - 3, 256, 768
    gb = idx.idx_mqa_logits_block(c.d, row0, nrows, key0, nkeys).cpu().numpy()
    for r in range(nrows):
        t = row0 + r
        ks, ke = int(c.dq.ks[t]), int(c.dq.ke[t])
        lo, hi = max(ks, key0), min(ke, key0 + nkeys, c.p.L)
        inw = np.zeros(nkeys, bool)
        if hi > lo:
            inw[lo - key0:hi - key0] = True
            assert np.array_equal(gb[r, inw].view(np.int32), g[t, lo - ks:hi - ks].view(np.int32))
        assert np.isnan(gb[r, ~inw]).all(), "wrote outside the window"


@pytest.mark.parametrize("param", CASES, ids=_case_id)
def test_exact_fused_and_candidates(exact, param):
    """Fused top-K (selected values held to the bar for every sign of weights) and the fused
    candidate source, against the oracle."""
    c = _make_case(param)
    for K, Bk in ((64, 512), (700, 32768)):
        gi, gv = idx.idx_logits_topk_fused(c.d, K, block_k=Bk, row_chunk=16)
        topk_ok(gi.cpu().numpy(), gv.cpu().numpy(), c.o, c.dq.ks, K)
    n_blocks = 64
    W = max(c.d.W, 1)
    blocks = torch.empty((c.p.T, n_blocks), dtype=torch.int32, device="cuda")
    mask, _ = idx.idx_block_candidates(c.d, W, n_blocks=n_blocks, block_k=512, row_chunk=16, out_blocks=blocks)
    _check_candidates(c.dq, c.o, mask.cpu().numpy(), blocks.cpu().numpy(), n_blocks)


def test_exact_selection_against_aligned_truncation(exact):
    """The keys that defeat the default mode's refinement band (every 8-product group cancels
    but for products the fp8 MFMA drops): with exact scores they are selected as the oracle
    selects them."""
    p, a_rows = _aligned_truncation_problem()
    K = len(a_rows)
    dq = oracle.Dequantised(p)
    o = oracle.rows_logits(dq, range(p.T))
    fi, fv = idx.idx_logits_topk_fused(dev(p), K, block_k=1024)
    topk_ok(fi.cpu().numpy(), fv.cpu().numpy(), o, dq.ks, K)
    assert (np.sort(fi.cpu().numpy(), axis=1) == a_rows[None, :]).all()


def test_default_mode_is_unchanged(monkeypatch):
    """IDX_EXACT=0 is the default mode: bitwise the results of an unset variable."""
    c = _make_case(CASES[0])
    monkeypatch.delenv("IDX_EXACT", raising=False)
    a = idx.idx_logits_topk_fused(c.d, 64, block_k=512)
    monkeypatch.setenv("IDX_EXACT", "0")
    b = idx.idx_logits_topk_fused(c.d, 64, block_k=512)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("name,row_chunk",
                         [("glm_chunk", 0), ("dsv4_mxfp4", 0), ("ragged_cand", 4096), ("long_ctx", 4096)])
def test_default_selection_equals_exact_selection_at_full_size(monkeypatch, name, row_chunk):
    """Every row of the full workloads: the default mode's fused selection (fp8 MFMA scores,
    statistical refinement band) equals the selection from exact scores.  The exact kernel is
    held to the oracle above; the oracle itself checks only sampled rows at these sizes."""
    p = synth.make_config(name)
    d = idx.Inputs.from_host(p)
    K, Bk = p.meta["K"], p.meta["block_k"]
    ws = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=K, block_k=Bk, row_chunk=row_chunk),
                     dtype=torch.uint8, device="cuda")
    sel = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("IDX_EXACT", mode)
        gi, _ = idx.idx_logits_topk_fused(d, K, block_k=Bk, row_chunk=row_chunk, ws=ws)
        torch.cuda.synchronize()
        assert idx.overflow_count(ws) == 0
        sel[mode] = gi
    diff = (sel["0"] != sel["1"]).any(dim=1)
    assert not bool(diff.any()), f"{int(diff.sum())} rows differ, first {torch.nonzero(diff)[:5].flatten().tolist()}"
