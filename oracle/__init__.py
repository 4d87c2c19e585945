"""CPU oracle of the dense prefill indexer (MQA logits + top-K) -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or call this module.  The library's product path never does: it runs
the HIP kernels or fails.  The oracle shares no code with the HIP library (no
kernels, headers, helpers, tables or constants); it reads only the arrays the
seeded generator returns.

The arithmetic is plain single-threaded C++ in fp64 (oracle.cpp, built with g++
into liboracle.so, no HIP); this module marshals numpy arrays into it.  Where
several rows are wanted at once, rows_logits() runs the single-threaded routine
on several host threads, one row per call (ctypes releases the GIL).  Sources
and readings are listed in oracle.cpp:

    I[t, s] = sum_h w[t, h] * max(0, scale * <qd[t, h, :], kd[s, :]>),  s in [ks_t, ke_t)

* P1 -- "Running CHUNKED_PREFILL_SIZE above 1024 without the long-prompt memory
  problem": section 1 (the dense indexer call and the 8-key candidate blocks),
  section 2.1 (requests on a cached prefix), section 2.3 (key blocks, per-block
  top-k and a merge).
* P2 -- "[DeepSeek-V4.1] Bound the dense prefill indexer transient: row-chunk
  logits, tail-only candidate masks": Motivation (fp8 q x fp4 k, logits [T, lc]
  fp32), Accuracy/equivalence (index sets and masks compared; ties among
  repeated keys are the only residual).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_SO = os.path.join(_HERE, "liboracle.so")
# plain fp64: no fused multiply-add contraction, no fast-math, the generic x86-64 target
CXXFLAGS = ["-O3", "-std=c++17", "-shared", "-fPIC", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = False) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (no HIP)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", *CXXFLAGS, "-o", tmp, _SRC])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _L():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_SO)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        for name in ("orc_decode_e4m3", "orc_decode_e2m1", "orc_decode_e8m0"):
            getattr(lib, name).argtypes = [vp, i64, vp]
            getattr(lib, name).restype = None
        lib.orc_dequant_q.argtypes = [vp, vp, i64, i64, i32, i32, vp]
        lib.orc_dequant_q.restype = None
        lib.orc_dequant_k.argtypes = [vp, vp, i32, i64, i32, vp]
        lib.orc_dequant_k.restype = i32
        lib.orc_row_logits.argtypes = [vp, vp, vp, i32, i32, vp, i64, i64, i64, i64, f64, vp]
        lib.orc_row_logits.restype = i32
        lib.orc_topk_row.argtypes = [vp, i64, vp, i64, i32, vp, vp]
        lib.orc_topk_row.restype = None
        lib.orc_pool_row.argtypes = [vp, i64, i32, vp]
        lib.orc_pool_row.restype = None
        lib.orc_block_candidates_row.argtypes = [vp, i64, i32, i32, i64, vp, vp]
        lib.orc_block_candidates_row.restype = i32
        lib.orc_ragged_windows.argtypes = [vp, vp, vp, i32, i32, vp, vp]
        lib.orc_ragged_windows.restype = None
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype)


# ------------------------------------------------------------------ decoders
def _decode(fn, codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    fn(_p(c), c.size, _p(out))
    return out


def decode_e4m3(codes) -> np.ndarray:
    """OCP OFP8 E4M3 ("FN") codes -> float64 (0x7F / 0xFF are NaN)."""
    return _decode(_L().orc_decode_e4m3, codes)


def decode_e2m1(nibbles) -> np.ndarray:
    """OCP MX v1.0 FP4 E2M1 codes (low 4 bits) -> float64."""
    return _decode(_L().orc_decode_e2m1, nibbles)


def decode_e8m0(codes) -> np.ndarray:
    """OCP MX v1.0 E8M0 scale codes -> 2^(c - 127) (255 is NaN)."""
    return _decode(_L().orc_decode_e8m0, codes)


def dequant_q(q8, q_scale) -> np.ndarray:
    """qd[t, h, d] = e4m3(q8[t, h, d]) * q_scale[t, h]  (fp64 [T, H, D])."""
    q8 = _c(q8, np.uint8)
    qs = _c(q_scale, np.float32)
    T, H, D = q8.shape
    out = np.empty((T, H, D), np.float64)
    _L().orc_dequant_q(_p(q8), _p(qs), 0, T, H, D, _p(out))
    return out


def dequant_k(k, k_scale, k_fmt: int) -> np.ndarray:
    """kd[s, d]: fp8 keys e4m3(k8) * k_scale[s]; MXFP4 keys e2m1(nibble) * 2^(e8m0[s, d // 32] - 127),
    element d in the low nibble of byte d // 2 when d is even."""
    k = _c(k, np.uint8)
    L = k.shape[0]
    if k_fmt == 0:
        D = k.shape[1]
        ks = _c(k_scale, np.float32)
    elif k_fmt == 1:
        D = 2 * k.shape[1]
        ks = _c(k_scale, np.uint8)
    else:
        raise ValueError("k_fmt")
    out = np.empty((L, D), np.float64)
    assert _L().orc_dequant_k(_p(k), _p(ks), int(k_fmt), L, D, _p(out)) == 0
    return out


# ------------------------------------------------------------------ windows
def ragged_windows(cu_q, cu_k, cu_c=None, ratio: int = 1):
    """Per-row key windows [ks, ke) of a varlen batch (see orc_ragged_windows).  A single
    request cu_q = [0, T], cu_k = [0, L] is a chunk at the tail of its prefix:
    ks = 0, ke = L - T + t + 1."""
    cu_q = _c(cu_q, np.int32)
    cu_k = _c(cu_k, np.int32)
    cu_c = cu_k if cu_c is None else _c(cu_c, np.int32)
    B = len(cu_q) - 1
    T = int(cu_q[-1])
    ks = np.zeros(T, np.int32)
    ke = np.zeros(T, np.int32)
    _L().orc_ragged_windows(_p(cu_q), _p(cu_k), _p(cu_c), B, int(ratio), _p(ks), _p(ke))
    return ks.astype(np.int64), ke.astype(np.int64)


# ------------------------------------------------------------------ logits
class Dequantised:
    """One indexer call's inputs as the oracle reads them: the E4M3 query codes and
    scales, the head weights, the keys dequantised to fp64 [L, D] once, and the row
    windows (the problem's own, or built from its cu_seqlens by ragged_windows)."""

    def __init__(self, p):
        self.q = _c(p.q, np.uint8)
        self.q_scale = _c(p.q_scale, np.float32)
        self.w = _c(p.w, np.float32)
        self.T, self.H, self.D = self.q.shape
        self.kd = dequant_k(p.k, p.k_scale, p.k_fmt)
        self.L = self.kd.shape[0]
        if getattr(p, "ks", None) is not None:
            self.ks = np.asarray(p.ks, np.int64)
            self.ke = np.asarray(p.ke, np.int64)
        else:
            self.ks, self.ke = ragged_windows(p.cu_q, p.cu_k)
        self.scale = float(p.scale)
        self._qd = None

    @property
    def qd(self) -> np.ndarray:
        """All rows' dequantised queries, fp64 [T, H, D] (small problems)."""
        if self._qd is None:
            self._qd = dequant_q(self.q, self.q_scale)
        return self._qd

    @property
    def W(self) -> int:
        """Longest window (max_seqlen_k)."""
        return int((self.ke - self.ks).max()) if self.T else 0

    @property
    def pairs(self) -> int:
        return int((self.ke - self.ks).sum())


def row_logits(dq: Dequantised, t: int) -> np.ndarray:
    """I[t, s] for s in [ks_t, ke_t), fp64, indexed by s - ks_t (P1 section 1)."""
    ks, ke = int(dq.ks[t]), int(dq.ke[t])
    out = np.empty(max(ke - ks, 0), np.float64)
    st = _L().orc_row_logits(_p(dq.q), _p(dq.q_scale), _p(dq.w), dq.H, dq.D, _p(dq.kd), dq.L, int(t), ks, ke,
                             dq.scale, _p(out))
    assert st == 0, f"row {t}: window [{ks}, {ke}) outside [0, {dq.L}]"
    return out


def default_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def rows_logits(dq: Dequantised, rows, workers: int = 0) -> list:
    """row_logits of several rows, each computed by the single-threaded routine, rows spread
    over `workers` host threads (0: up to 16)."""
    rows = [int(t) for t in rows]
    n = workers or default_workers()
    if n <= 1 or len(rows) <= 1:
        return [row_logits(dq, t) for t in rows]
    with ThreadPoolExecutor(max_workers=n) as ex:
        return list(ex.map(lambda t: row_logits(dq, t), rows))


def dense_logits(dq: Dequantised, rows, W: int) -> np.ndarray:
    """Row-relative dense logits [len(rows), W]: column j holds key ks_t + j; -inf outside the
    window (P1 section 1: output [T, max_seqlen_k] fp32)."""
    rows = list(rows)
    out = np.full((len(rows), W), -np.inf)
    for i, v in enumerate(rows_logits(dq, rows)):
        out[i, :len(v)] = v
    return out


# ------------------------------------------------------------------ selection
def topk_row(vals64, ks: int, K: int, allowed=None):
    """Top-K of one row's window (P1 section 2.3 / P2 Modifications).  vals64: fp64 logits,
    index j <-> key ks + j.  allowed: optional bool per j (the candidate mask).  Returns
    (idx int32 [K] ascending then -1, val float32 [K] then -inf)."""
    v = _c(vals64, np.float64)
    n = len(v)
    al = None
    if allowed is not None:
        al = _c(np.asarray(allowed, bool)[:n], np.uint8)
        assert len(al) == n
    idx = np.empty(K, np.int32)
    val = np.empty(K, np.float32)
    _L().orc_topk_row(_p(v), n, _p(al) if al is not None else None, int(ks), int(K), _p(idx), _p(val))
    return idx, val


def pool_row(vals64, pool: int) -> np.ndarray:
    """P[b] = max over keys ks + pool*b ... ks + pool*b + pool - 1 of the window (P1 section 1)."""
    v = _c(vals64, np.float64)
    out = np.empty(-(-len(v) // pool), np.float64)
    _L().orc_pool_row(_p(v), len(v), int(pool), _p(out))
    return out


def block_candidates_row(vals64, pool: int, n_blocks: int, W: int):
    """Candidate source of one row (P1 section 1): (mask uint8 [W], kept blocks ascending int64)."""
    v = _c(vals64, np.float64)
    mask = np.empty(W, np.uint8)
    chosen = np.empty(max(min(n_blocks, -(-len(v) // pool)), 0), np.int32)
    n = _L().orc_block_candidates_row(_p(v), len(v), int(pool), int(n_blocks), int(W), _p(mask),
                                      _p(chosen) if len(chosen) else None)
    return mask, chosen[:n].astype(np.int64)


def topk(dq: Dequantised, rows, K: int, masks=None):
    """(idx [len(rows), K], val, list of fp64 window logits) for the given rows."""
    rows = list(rows)
    logits = rows_logits(dq, rows)
    idx = np.empty((len(rows), K), np.int32)
    val = np.empty((len(rows), K), np.float32)
    for i, (t, v) in enumerate(zip(rows, logits)):
        allowed = None if masks is None else masks[i][:len(v)]
        idx[i], val[i] = topk_row(v, int(dq.ks[t]), K, allowed)
    return idx, val, logits
