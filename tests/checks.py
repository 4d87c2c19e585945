"""Comparison rules between the HIP library's outputs and the fp64 oracle.

* Logits: in-window |g - o| <= 1e-4 + 1e-3 * max(|o|, m); out-of-window entries must
  be exactly -inf.  m is the size of the score's head terms, sum_h |w_h| ReLU(x_h)
  (oracle.row_magnitude): it equals |o| when every head weight is >= 0, as in all of
  the pages' workloads, so there the bar is 1e-4 + 1e-3 * |o|.  With weights of both
  signs the terms can cancel and any floating-point evaluation is only accurate
  relative to m; callers that pass no m get the plain bar.
* Top-K index sets: bit-exact, except that keys whose oracle scores lie within
  1e-6 * |v_K| of the oracle's K-th selected score v_K may be swapped (near-ties,
  which the pages report as the only residual between two implementations).
  The number of selected keys must match, indices must be ascending, unique,
  in window, allowed by the mask, and padded with -1.
"""
from __future__ import annotations

import numpy as np

import oracle

ATOL = 1e-4
RTOL = 1e-3
TIE_REL = 1e-6


def logits_ok(g: np.ndarray, o: np.ndarray, what: str = "logits", mag=None):
    """g: GPU fp32, o: oracle fp64 (same shape; -inf marks out-of-window); mag: optional
    oracle head-term sizes, same shape (values outside the window are ignored)."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    inw = np.isfinite(o)
    bad_inf = ~inw & ~(np.isneginf(g))
    assert not bad_inf.any(), f"{what}: {bad_inf.sum()} out-of-window entries are not -inf"
    err = np.abs(g[inw] - o[inw])
    size = np.abs(o[inw]) if mag is None else np.maximum(np.abs(o[inw]), np.asarray(mag, np.float64)[inw])
    lim = ATOL + RTOL * size
    worst = int(np.argmax(err - lim)) if err.size else 0
    assert (err <= lim).all(), (f"{what}: {(err > lim).sum()} entries out of tolerance; worst err "
                                f"{err[worst]:.3e} at |o|={abs(o[inw][worst]):.3e}")
    rel = err / np.maximum(np.abs(o[inw]), 1e-30)
    return float(rel.max()) if rel.size else 0.0


def topk_row_ok(g_idx, g_val, o_win64, ks: int, K: int, allowed=None, what: str = "topk", mag_win=None):
    """One row: GPU (idx, val) against the oracle's fp64 window logits o_win64 (index j <-> key ks+j);
    mag_win: optional head-term sizes of the window for the value tolerance.
    Returns the number of near-tie swaps."""
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
        size = np.abs(o_at) if mag_win is None else np.maximum(np.abs(o_at), np.asarray(mag_win)[g_sel - ks])
        err = np.abs(g_val[:cnt] - o_at)
        assert (err <= ATOL + RTOL * size).all(), f"{what}: selected values out of tolerance"
    return swaps


def topk_ok(g_idx, g_val, o_windows, ks, K, allowed=None, what="topk", mags=None):
    swaps = 0
    if mags is None:
        mags = getattr(o_windows, "mag", None)   # a window list may carry its head-term sizes
    for i in range(len(o_windows)):
        al = None if allowed is None else allowed[i]
        swaps += topk_row_ok(g_idx[i], None if g_val is None else g_val[i], o_windows[i], int(ks[i]),
                             K, al, what=f"{what} row {i}", mag_win=None if mags is None else mags[i])
    return swaps


class Windows(list):
    """Per-row oracle window logits, with each row's head-term sizes in .mag."""

    def __init__(self, rows, mag=None):
        super().__init__(rows)
        self.mag = mag
