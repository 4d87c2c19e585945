"""IDX_DEBUG=1: entry points check the preconditions that live in device memory (window
bounds, window length against W, q scales, head weights, key scales) on the device before
their own kernels, and report IDX_E_DEVICE_CHECK without touching the outputs.  Valid
inputs give the same results as without the check."""
import numpy as np
import pytest
import torch

import mqa_logits_top_amd as idx
import synth

pytestmark = pytest.mark.gpu

DEVICE_CHECK = 9


def _problem(k_fmt=synth.K_FP8):
    p = synth.make_problem(40, 3000, 32, k_fmt=k_fmt, seed=4)
    return idx.Inputs.from_host(p)


def _with(d, **kw):
    f = dict(q=d.q, q_scale=d.q_scale, k=d.k, k_scale=d.k_scale, w=d.w, ks=d.ks, ke=d.ke, k_fmt=d.k_fmt,
             scale=d.scale)
    f.update(kw)
    return idx.Inputs(**f)


def _calls(d, W):
    """Every entry point that reads windows, with outputs pre-filled with a sentinel."""
    K = 16
    out = {}

    def fused():
        oi = torch.full((d.T, K), -7, dtype=torch.int32, device="cuda")
        idx.idx_logits_topk_fused(d, K, block_k=1024, out_idx=oi)
        return oi

    def logits():
        lg = torch.full((d.T, W), 7.0, dtype=torch.float32, device="cuda")
        idx.idx_mqa_logits(d, W, out=lg)
        return lg

    def block():
        return idx.idx_mqa_logits_block(d, 0, d.T, 0, 1024)

    def topk():
        lg = torch.zeros((d.T, W), dtype=torch.float32, device="cuda")
        oi = torch.full((d.T, K), -7, dtype=torch.int32, device="cuda")
        idx.idx_topk(lg, d.ks, d.ke, K, W=W, out_idx=oi)
        return oi

    def cands():
        m = torch.full((d.T, W), 7, dtype=torch.uint8, device="cuda")
        idx.idx_block_candidates(d, W, n_blocks=8, block_k=1024, mask=m)
        return m

    def refine():
        ci = torch.full((d.T, 600), -1, dtype=torch.int32, device="cuda")
        ci[:, 0] = 0
        cv = torch.zeros((d.T, 600), dtype=torch.float32, device="cuda")
        oi = torch.full((d.T, K), -7, dtype=torch.int32, device="cuda")
        idx.idx_refine_topk(d, ci, cv, K, out_idx=oi)
        return oi

    return {"fused": fused, "logits": logits, "block": block, "topk": topk, "cands": cands, "refine": refine}


def test_valid_inputs_unchanged(monkeypatch):
    d = _problem()
    W = d.W
    monkeypatch.setenv("IDX_DEBUG", "0")
    ref = {n: f() for n, f in _calls(d, W).items()}
    monkeypatch.setenv("IDX_DEBUG", "1")
    got = {n: f() for n, f in _calls(d, W).items()}
    for n in ref:
        assert torch.equal(ref[n].view(torch.uint8), got[n].view(torch.uint8)), n


@pytest.mark.parametrize("what", ["ke_past_L", "ks_after_ke", "negative_ks", "negative_q_scale", "nan_w",
                                  "negative_k_scale", "e8m0_nan", "window_longer_than_W"])
def test_device_preconditions(monkeypatch, what):
    d = _problem(synth.K_MXFP4 if what == "e8m0_nan" else synth.K_FP8)
    W = d.W
    if what == "ke_past_L":
        bad = _with(d, ke=d.ke.clone().index_fill_(0, torch.tensor([5], device="cuda"), d.L + 3))
    elif what == "ks_after_ke":
        ks = d.ks.clone()
        ks[7] = int(d.ke[7]) + 1
        bad = _with(d, ks=ks)
    elif what == "negative_ks":
        ks = d.ks.clone()
        ks[0] = -4
        bad = _with(d, ks=ks)
    elif what == "negative_q_scale":
        qs = d.q_scale.clone()
        qs[3, 2] = -0.5
        bad = _with(d, q_scale=qs)
    elif what == "nan_w":
        w = d.w.clone()
        w[1, 0] = float("nan")
        bad = _with(d, w=w)
    elif what == "negative_k_scale":
        ksc = d.k_scale.clone()
        ksc[100] = -1.0
        bad = _with(d, k_scale=ksc)
    elif what == "e8m0_nan":
        ksc = d.k_scale.clone()
        ksc[11, 2] = 255
        bad = _with(d, k_scale=ksc)
    else:
        bad = d
        W = W - 1          # the longest window no longer fits
    monkeypatch.setenv("IDX_DEBUG", "1")
    calls = _calls(bad, W)
    # which entry points see the broken precondition
    sees = {"fused", "logits", "block", "cands", "refine"}
    if what in ("ke_past_L", "ks_after_ke", "negative_ks"):
        sees |= {"topk"}
    if what == "window_longer_than_W":
        sees = {"logits", "topk", "cands"}
    for name, fn in calls.items():
        if name not in sees:
            continue
        with pytest.raises(idx.IdxError) as e:
            fn()
        assert e.value.status == DEVICE_CHECK, (name, e.value.status)
    torch.cuda.synchronize()


def test_outputs_untouched_on_failure(monkeypatch):
    d = _problem()
    ke = d.ke.clone()
    ke[2] = d.L + 1
    bad = _with(d, ke=ke)
    monkeypatch.setenv("IDX_DEBUG", "1")
    oi = torch.full((bad.T, 16), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(idx.IdxError):
        idx.idx_logits_topk_fused(bad, 16, block_k=1024, out_idx=oi)
    torch.cuda.synchronize()
    assert (oi == -7).all()
    assert np.array_equal(idx.idx_logits_topk_fused(d, 16, block_k=1024)[0].cpu().numpy().shape, (d.T, 16))
