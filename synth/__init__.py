"""Seeded synthetic inputs for the dense prefill indexer.

This module only draws random numbers and stores them in the input formats the
indexer consumes (fp8 E4M3 codes with per-row fp32 scales, MXFP4 codes with
E8M0 block scales, fp32 head weights, int32 key windows or a batch's
cu_seqlens).  It holds none of the
indexer's arithmetic; the GPU library and the CPU oracle both read the arrays
it returns.  The heavy loops live in ``gen.c`` (built with gcc + OpenMP).

Tensor sub-streams (one SplitMix64 counter stream each): q = 1, k = 2, w = 3,
duplicate-row choice = 4, second-layer q = 5, second-layer w = 6.

The workload shapes follow the pages' descriptions of the indexer's inputs:
a prefill chunk of T query rows with H heads of D = 128, a compressed prefix
of L keys, per-row windows [ks, ke) (causal for a chunk at the tail of its
prefix; ragged for a batch of requests), fp8 queries and fp8 or MXFP4 keys.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "gen.c")

K_FP8 = 0
K_MXFP4 = 1

S_Q, S_K, S_W, S_DUP, S_Q2, S_W2 = 1, 2, 3, 4, 5, 6


def build(force: bool = False) -> str:
    """Compile gen.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _L():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_SO)
        u64, u32, i64, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int32
        vp = ctypes.c_void_p
        lib.synth_uniform.argtypes = [u64, u32, i64, i64, vp]
        lib.synth_uniform_f32.argtypes = [u64, u32, i64, ctypes.c_float, ctypes.c_float, vp]
        lib.synth_normal.argtypes = [u64, u32, i64, i64, vp]
        lib.synth_u64.argtypes = [u64, u32, i64, vp]
        lib.synth_fp8_normal_rows.argtypes = [u64, u32, i64, i32, vp, vp]
        lib.synth_mxfp4_normal_rows.argtypes = [u64, u32, i64, i32, vp, vp]
        lib.synth_encode_e4m3.argtypes = [vp, i64, vp]
        lib.synth_encode_e2m1.argtypes = [vp, i64, vp]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- raw draws
def uniform(seed: int, stream: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    _L().synth_uniform(seed, stream, first, n, _p(out))
    return out


def uniform_f32(seed: int, stream: int, shape, lo=0.0, hi=1.0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _L().synth_uniform_f32(seed, stream, out.size, lo, hi, _p(out))
    return out


def normal(seed: int, stream: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    _L().synth_normal(seed, stream, first, n, _p(out))
    return out


def raw_u64(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _L().synth_u64(seed, stream, n, _p(out))
    return out


def encode_e4m3(x) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    _L().synth_encode_e4m3(_p(x), x.size, _p(out))
    return out


def encode_e2m1(x) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    _L().synth_encode_e2m1(_p(x), x.size, _p(out))
    return out


def fp8_normal_rows(seed: int, stream: int, rows: int, cols: int):
    """N(0,1) draws for [rows, cols], quantised per row: (codes u8, scale f32[rows])."""
    assert cols <= 1024
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty(rows, np.float32)
    _L().synth_fp8_normal_rows(seed, stream, rows, cols, _p(codes), _p(scales))
    return codes, scales


def mxfp4_normal_rows(seed: int, stream: int, rows: int, cols: int):
    """N(0,1) draws for [rows, cols], quantised to MXFP4: (packed u8 [rows, cols/2], e8m0 u8 [rows, cols/32])."""
    assert cols % 32 == 0
    packed = np.empty((rows, cols // 2), np.uint8)
    e8 = np.empty((rows, cols // 32), np.uint8)
    _L().synth_mxfp4_normal_rows(seed, stream, rows, cols, _p(packed), _p(e8))
    return packed, e8


# ---------------------------------------------------------------- problems
@dataclass
class Problem:
    """Host arrays of one indexer call (all C-contiguous numpy).

    Row windows are given either directly (ks, ke: explicit draws) or as the batch's
    cu_seqlens (cu_q, cu_k), from which each side derives them itself: the library with
    idx_ragged_windows, the oracle with its own row-by-row definition."""
    q: np.ndarray          # u8 [T, H, D]   E4M3 codes
    q_scale: np.ndarray    # f32 [T, H]
    k: np.ndarray          # u8 [L, D] (fp8) or [L, D/2] (MXFP4 packed)
    k_scale: np.ndarray    # f32 [L] (fp8) or u8 [L, D/32] (E8M0)
    k_fmt: int
    w: np.ndarray          # f32 [T, H]
    ks: Optional[np.ndarray] = None   # i32 [T] (or None: windows from cu_q / cu_k)
    ke: Optional[np.ndarray] = None   # i32 [T]
    scale: float = 1.0
    cu_q: Optional[np.ndarray] = None  # i32 [B + 1] query rows of each request
    cu_k: Optional[np.ndarray] = None  # i32 [B + 1] key rows of each request
    meta: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.q.shape[0]

    @property
    def H(self):
        return self.q.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def L(self):
        return self.k.shape[0]


def make_problem(T: int, L: int, H: int, D: int = 128, k_fmt: int = K_FP8, seed: int = 0,
                 ks: Optional[np.ndarray] = None, ke: Optional[np.ndarray] = None,
                 cu_q=None, cu_k=None,
                 dup_rows: int = 0, w_lo: float = 0.0, w_hi: float = 1.0,
                 q_stream: int = S_Q, w_stream: int = S_W, keys: Optional[tuple] = None,
                 scale: float = 1.0) -> Problem:
    """q, k ~ N(0,1) quantised (fp8 per-row amax/448, or MXFP4 for keys); w ~ U(w_lo, w_hi).

    Windows: explicit ks / ke, or a varlen batch's cu_q / cu_k; with neither, one request
    cu_q = [0, T], cu_k = [0, L] (the chunk is the tail of its prefix).
    ``keys`` reuses (k, k_scale) from another problem (same prefix, new layer).
    ``dup_rows`` > 0 byte-copies that many key rows (codes and scales) from
    other, non-copied rows, so those keys score exactly alike.
    """
    q8, qs = fp8_normal_rows(seed, q_stream, T * H, D)
    q8 = q8.reshape(T, H, D)
    qs = qs.reshape(T, H)
    if keys is not None:
        k, ksc = keys
    elif k_fmt == K_FP8:
        k, ksc = fp8_normal_rows(seed, S_K, L, D)
    elif k_fmt == K_MXFP4:
        k, ksc = mxfp4_normal_rows(seed, S_K, L, D)
    else:
        raise ValueError("k_fmt")
    meta = {}
    if dup_rows:
        # destinations: the dup_rows smallest of L uniform draws (a uniform subset);
        # sources: uniform over the rows that are not destinations.
        u = uniform(seed, S_DUP, L)
        dst = np.sort(np.argsort(u, kind="stable")[:dup_rows])
        is_dst = np.zeros(L, bool)
        is_dst[dst] = True
        pool = np.nonzero(~is_dst)[0]
        v = uniform(seed, S_DUP, dup_rows, first=L)
        src = pool[np.minimum((v * len(pool)).astype(np.int64), len(pool) - 1)]
        k = k.copy()
        ksc = ksc.copy()
        k[dst] = k[src]
        ksc[dst] = ksc[src]
        meta["dup_dst"] = dst
        meta["dup_src"] = src
    w = uniform_f32(seed, w_stream, (T, H), w_lo, w_hi)
    if ks is not None or ke is not None:
        assert ks is not None and ke is not None
        ks = np.ascontiguousarray(ks, np.int32)
        ke = np.ascontiguousarray(ke, np.int32)
        cu_q = cu_k = None
    else:
        if cu_q is None:
            cu_q, cu_k = [0, T], [0, L]
        cu_q = np.ascontiguousarray(cu_q, np.int32)
        cu_k = np.ascontiguousarray(cu_k, np.int32)
        assert int(cu_q[-1]) == T and int(cu_k[-1]) <= L
    return Problem(q=q8, q_scale=qs, k=np.ascontiguousarray(k), k_scale=np.ascontiguousarray(ksc),
                   k_fmt=k_fmt, w=w, ks=ks, ke=ke, scale=scale, cu_q=cu_q, cu_k=cu_k, meta=meta)


# The five workloads (shapes of the pages' indexer calls).  Seed 0 throughout.
CONFIGS = {
    # tiny: 64 rows against 4096 keys, H=32, fp8, K=512
    "tiny": dict(T=64, L=4096, H=32, k_fmt=K_FP8, K=512, block_k=4096),
    # GLM-5.1-shaped chunk: 2048 rows, 65536 keys, H=32, fp8, K=2048, B_k=32768
    "glm_chunk": dict(T=2048, L=65536, H=32, k_fmt=K_FP8, K=2048, block_k=32768),
    # DeepSeek-V4-like low-ratio chunk: 2048 x 102400, H=64, MXFP4 keys, K=512, 5% duplicated keys
    "dsv4_mxfp4": dict(T=2048, L=102400, H=64, k_fmt=K_MXFP4, K=512, block_k=32768, dup_rows=5120),
    # long context: 16384 x 487936, H=64, fp8, K=512
    "long_ctx": dict(T=16384, L=487936, H=64, k_fmt=K_FP8, K=512, block_k=32768),
    # ragged batch + candidate source: 4 x 7168 fresh + 2048 new on a 150000 cached prefix
    "ragged_cand": dict(cu_q=[0, 7168, 14336, 21504, 28672, 30720],
                        cu_k=[0, 7168, 14336, 21504, 28672, 180720],
                        H=64, k_fmt=K_FP8, K=512, block_k=32768, pool=8, n_blocks=2048),
}


def make_config(name: str, seed: int = 0) -> Problem:
    c = CONFIGS[name]
    if "cu_q" in c:
        T = int(c["cu_q"][-1])
        L = int(c["cu_k"][-1])
        p = make_problem(T, L, c["H"], k_fmt=c["k_fmt"], seed=seed, cu_q=c["cu_q"], cu_k=c["cu_k"])
    else:
        p = make_problem(c["T"], c["L"], c["H"], k_fmt=c["k_fmt"], seed=seed,
                         dup_rows=c.get("dup_rows", 0))
    p.meta.update(name=name, **{k: v for k, v in c.items() if k not in ("T", "L", "H", "k_fmt")})
    return p


def consumer_layer(p: Problem, seed: int = 0) -> Problem:
    """A later indexer layer of the same batch: fresh q and w (streams 5, 6), same keys and windows."""
    return make_problem(p.T, p.L, p.H, p.D, p.k_fmt, seed, ks=p.ks, ke=p.ke, cu_q=p.cu_q, cu_k=p.cu_k,
                        q_stream=S_Q2, w_stream=S_W2, keys=(p.k, p.k_scale), scale=p.scale)
