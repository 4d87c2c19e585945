"""Comparison rules between the HIP library's outputs and the fp64 oracle.

* Logits: in-window |g - o| <= 1e-4 + 1e-3 * |o|; out-of-window entries must be
  exactly -inf.
* Top-K index sets: bit-exact, except that keys whose oracle scores lie within
  1e-6 * |v_K| of the oracle's K-th selected score v_K may be swapped (near-ties,
  which the pages report as the only residual between two implementations).
  The number of selected keys must match, indices must be ascending, unique,
  in window, allowed by the mask, and padded with -1.  Selected values obey the
  logit bar, pads are -inf.
"""
from __future__ import annotations

import numpy as np

import oracle

ATOL = 1e-4
RTOL = 1e-3
TIE_REL = 1e-6


def logits_ok(g: np.ndarray, o: np.ndarray, what: str = "logits"):
    """g: GPU fp32, o: oracle fp64 (same shape; -inf marks out-of-window)."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    inw = np.isfinite(o)
    bad_inf = ~inw & ~(np.isneginf(g))
    assert not bad_inf.any(), f"{what}: {bad_inf.sum()} out-of-window entries are not -inf"
    err = np.abs(g[inw] - o[inw])
    lim = ATOL + RTOL * np.abs(o[inw])
    worst = int(np.argmax(err - lim)) if err.size else 0
    assert (err <= lim).all(), (f"{what}: {(err > lim).sum()} entries out of tolerance; worst err "
                                f"{err[worst]:.3e} at |o|={abs(o[inw][worst]):.3e}")
    rel = err / np.maximum(np.abs(o[inw]), 1e-30)
    return float(rel.max()) if rel.size else 0.0


def topk_row_ok(g_idx, g_val, o_win64, ks: int, K: int, allowed=None, what: str = "topk"):
    """One row: GPU (idx, val) against the oracle's fp64 window logits o_win64 (index j <-> key ks+j).
    g_val None: the index set only.  Returns the number of near-tie swaps."""
    g_idx = np.asarray(g_idx, np.int64)
    n = len(o_win64)
    o_idx, _ = oracle.topk_row(o_win64, ks, K, allowed)
    o_sel = o_idx[o_idx >= 0].astype(np.int64)
    g_sel = g_idx[g_idx >= 0]
    cnt = len(g_sel)
    assert cnt == len(o_sel), f"{what}: selected {cnt} keys, oracle {len(o_sel)}"
    assert (g_idx[:cnt] >= 0).all() and (g_idx[cnt:] == -1).all(), f"{what}: padding not at the tail"
    assert (np.diff(g_sel) > 0).all(), f"{what}: indices not strictly ascending"
    assert ((g_sel >= ks) & (g_sel < ks + n)).all(), f"{what}: index outside the window"
    if allowed is not None:
        al = np.asarray(allowed, bool)
        assert al[g_sel - ks].all(), f"{what}: selected a masked-out key"
    swaps = 0
    diff = np.setxor1d(g_sel, o_sel)
    if len(diff):
        vk = float(np.min(o_win64[o_sel - ks]))
        dv = np.abs(o_win64[diff - ks] - vk)
        assert (dv <= TIE_REL * abs(vk)).all(), (
            f"{what}: {len(diff)} differing keys, worst |o - v_K|/|v_K| = {dv.max() / abs(vk):.3e} "
            f"(keys {diff[:8]})")
        swaps = len(diff) // 2
    if g_val is not None:
        g_val = np.asarray(g_val, np.float64)
        assert np.isneginf(g_val[cnt:]).all(), f"{what}: pad values are not -inf"
        o_at = o_win64[g_sel - ks]
        err = np.abs(g_val[:cnt] - o_at)
        lim = ATOL + RTOL * np.abs(o_at)
        assert (err <= lim).all(), (f"{what}: selected values out of tolerance ({(err > lim).sum()} of {cnt}, "
                                    f"worst err {err.max():.3e})")
    return swaps


def topk_ok(g_idx, g_val, o_windows, ks, K, allowed=None, what="topk"):
    swaps = 0
    for i in range(len(o_windows)):
        al = None if allowed is None else allowed[i]
        swaps += topk_row_ok(g_idx[i], None if g_val is None else g_val[i], o_windows[i], int(ks[i]),
                             K, al, what=f"{what} row {i}")
    return swaps


def dense_ref(o_windows, W):
    """Oracle windows as dense row-relative logits [rows, W] (-inf past each window)."""
    ref = np.full((len(o_windows), W), -np.inf)
    for i, v in enumerate(o_windows):
        ref[i, :len(v)] = v
    return ref


def windows_match(d, dq):
    """The device windows the library built (or was given) equal the oracle's, row by row."""
    assert np.array_equal(d.ks.cpu().numpy().astype(np.int64), dq.ks), "ks differs from the oracle's windows"
    assert np.array_equal(d.ke.cpu().numpy().astype(np.int64), dq.ke), "ke differs from the oracle's windows"
