"""CPU oracle for the dense prefill indexer (MQA logits + top-K) -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or call this module.  The library's product path never does: it runs
the HIP kernels or fails.  This module shares no code with the HIP library
(no kernels, headers, helpers, tables or constants); it reads only the arrays
that the seeded generator returns.

Everything here is the plain definition, in float64 numpy, with a library
matmul and a library sort as its only primitives: no blocking, fusion or
reordering.  Sources (web pages, cited by title and section):

* P1 -- "Running CHUNKED_PREFILL_SIZE above 1024 without the long-prompt
  memory problem" (chunked-prefill-memory.md).  Section 1 describes the dense
  indexer call: a chunk's T query rows scored against the whole compressed
  prefix, output [T, max_seqlen_k] fp32, then a top-k; layer 20 pools 8-key
  blocks, keeps the top-2048 blocks and publishes a bool candidate mask that
  later layers apply with masked_fill_.  Section 2.3 states the key-blocked
  identity topk(union) == topk(union of per-block topk) and that pooling and
  masking decompose per block.
* P2 -- "[DeepSeek-V4.1] Bound the dense prefill indexer transient: row-chunk
  logits, tail-only candidate masks".  Motivation: fp8 queries x fp4 keys
  (fp8_fp4_mqa_logits), logits [T, lc] fp32.  Accuracy/equivalence: outputs
  are compared as index sets and masks; the only residual is top-k tie
  ordering among repeated text.

The score formula itself is not printed on the pages.  The oracle uses the
DeepSeek sparse-attention indexer score: for query row t and key s in the
row's window [ks_t, ke_t),

    I[t, s] = sum_h w[t, h] * max(0, scale * <qd[t, h, :], kd[s, :]>)

with qd, kd the dequantised fp8 / MXFP4 inputs.  Readings taken where the
pages are silent (each also listed in the design notes):

* q has one fp32 scale per (t, h) row of D values; fp8 keys one per key row;
  MXFP4 keys one E8M0 scale per 32 consecutive d.
* outside the window the logit is -inf and never selected.
* the top-k decision is taken on fp32 logits (the pages' logits dtype): the
  fp64 score is rounded to fp32, then ordered by (value desc, key index asc).
  Ties in fp32 therefore go to the lower key index.
* outputs list selected key indices (absolute rows of k) in ascending order,
  padded with -1 when the window (or the candidate set) is smaller than K.
* pooling blocks of 8 keys start at ks_t; a partial last block takes the max
  over its in-window keys.  Blocks are ordered (pooled value desc, block asc).
"""
from __future__ import annotations

import numpy as np

# ------------------------------------------------------------------ decoders
# OCP "8-bit Floating Point Specification (OFP8)" E4M3 ("FN": no infinities):
# 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
# subnormal (m * 2^-9); S.1111.111 is NaN.  Largest finite value 448.


def decode_e4m3(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


# OCP "Microscaling Formats (MX) v1.0": FP4 E2M1 element (1 sign, 2 exponent
# bits with bias 1, 1 mantissa bit; no inf/NaN), E8M0 scale (2^(e - 127),
# 0xFF is NaN).


def decode_e2m1(nibbles) -> np.ndarray:
    c = np.asarray(nibbles).astype(np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return s * mag


def decode_e8m0(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def dequant_q(q8, q_scale) -> np.ndarray:
    """qd[t, h, d] = e4m3(q8[t, h, d]) * q_scale[t, h]  (fp64 [T, H, D])."""
    return decode_e4m3(q8) * np.asarray(q_scale, np.float64)[..., None]


def dequant_k(k, k_scale, k_fmt: int) -> np.ndarray:
    """kd[s, d]: fp8 keys e4m3(k8) * k_scale[s]; MXFP4 keys e2m1(nibble) * 2^(e8m0[s, d//32] - 127),
    with element d in the low nibble of byte d//2 when d is even."""
    if k_fmt == 0:
        return decode_e4m3(k) * np.asarray(k_scale, np.float64)[:, None]
    if k_fmt == 1:
        k = np.asarray(k)
        L, half = k.shape
        D = 2 * half
        el = np.empty((L, D), np.float64)
        el[:, 0::2] = decode_e2m1(k & 0xF)
        el[:, 1::2] = decode_e2m1(k >> 4)
        blk = decode_e8m0(k_scale)                      # [L, D/32]
        return el * np.repeat(blk, 32, axis=1)
    raise ValueError("k_fmt")


# ------------------------------------------------------------------ logits
class Dequantised:
    """Dequantised inputs of one indexer call, kept in fp64."""

    def __init__(self, p):
        self.qd = dequant_q(p.q, p.q_scale)
        self.kd = dequant_k(p.k, p.k_scale, p.k_fmt)
        self.w = np.asarray(p.w, np.float64)
        self.ks = np.asarray(p.ks, np.int64)
        self.ke = np.asarray(p.ke, np.int64)
        self.scale = float(p.scale)


def row_logits(dq: Dequantised, t: int) -> np.ndarray:
    """I[t, s] for s in [ks_t, ke_t), fp64, indexed by s - ks_t (P1 section 1: the dense
    indexer scores each query row against its whole key window)."""
    ks, ke = int(dq.ks[t]), int(dq.ke[t])
    dots = dq.scale * (dq.qd[t] @ dq.kd[ks:ke].T)       # [H, ke - ks]
    return dq.w[t] @ np.maximum(dots, 0.0)              # sum over heads


def row_magnitude(dq: Dequantised, t: int) -> np.ndarray:
    """M[t, s] = sum_h |w[t, h]| * max(0, scale * <qd[t, h, :], kd[s, :]>) for s in [ks_t, ke_t):
    the size of I[t, s]'s head terms.  It equals I[t, s] when every weight of the row is
    >= 0 (all the pages' workloads draw w from U(0, 1)); with weights of both signs the
    terms can cancel, and a floating-point head sum is accurate relative to M, not to I.
    The parity checks take their relative tolerance against max(|I|, M)."""
    ks, ke = int(dq.ks[t]), int(dq.ke[t])
    dots = dq.scale * (dq.qd[t] @ dq.kd[ks:ke].T)       # [H, ke - ks]
    return np.abs(dq.w[t]) @ np.maximum(dots, 0.0)


def dense_logits(dq: Dequantised, rows, W: int) -> np.ndarray:
    """Row-relative dense logits [len(rows), W]: column j holds key ks_t + j; -inf outside the
    window (P1 section 1: output [T, max_seqlen_k] fp32)."""
    out = np.full((len(rows), W), -np.inf)
    for i, t in enumerate(rows):
        v = row_logits(dq, t)
        out[i, :len(v)] = v
    return out


# ------------------------------------------------------------------ selection
def _order(v32: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Permutation sorting by (value desc, position asc)."""
    return np.lexsort((pos, -v32.astype(np.float64)))


def topk_row(vals64: np.ndarray, ks: int, K: int, allowed=None):
    """Top-K of one row's window (P1 section 2.3 / P2 Modifications: ragged top-k per row).

    vals64: fp64 logits of the window (index j <-> key ks + j).  allowed: optional
    bool [len(vals64)]; keys with allowed == False are excluded (the candidate mask,
    equivalent to masked_fill_(-inf) followed by never selecting -inf).
    Returns (idx int32 [K] ascending then -1, val float32 [K] then -inf).
    """
    n = len(vals64)
    pos = np.arange(n)
    v32 = np.asarray(vals64).astype(np.float32)
    if allowed is not None:
        keep = np.nonzero(np.asarray(allowed, bool)[:n])[0]
        pos, v32 = pos[keep], v32[keep]
    take = pos[_order(v32, pos)[:K]] if len(pos) else pos
    take = np.sort(take)
    idx = np.full(K, -1, np.int32)
    val = np.full(K, -np.inf, np.float32)
    idx[:len(take)] = ks + take
    val[:len(take)] = np.asarray(vals64)[take].astype(np.float32)
    return idx, val


def pool_row(vals64: np.ndarray, pool: int) -> np.ndarray:
    """P[b] = max of the window's logits over keys ks + pool*b ... ks + pool*b + pool - 1
    (P1 section 1: 'pads and pools' 8-key blocks; the pad is -inf so a partial
    last block takes the max of its in-window keys)."""
    n = len(vals64)
    nb = -(-n // pool)
    padded = np.full(nb * pool, -np.inf)
    padded[:n] = vals64
    return padded.reshape(nb, pool).max(axis=1)


def block_candidates_row(vals64: np.ndarray, pool: int, n_blocks: int, W: int):
    """Candidate source (P1 section 1, select_candidate_blocks): pool, keep the top n_blocks
    blocks by (pooled fp32 value desc, block asc), expand to a bool mask over the row's W
    columns (column j <-> key ks + j; zero past the window).
    Returns (mask uint8 [W], chosen blocks ascending int64)."""
    P = pool_row(vals64, pool)
    b = np.arange(len(P))
    chosen = np.sort(b[_order(P.astype(np.float32), b)[:n_blocks]])
    mask = np.zeros(W, np.uint8)
    n = len(vals64)
    for blk in chosen:
        mask[blk * pool:min((blk + 1) * pool, n)] = 1
    return mask, chosen


# ------------------------------------------------------------------ whole calls
def topk(dq: Dequantised, rows, K: int, masks=None):
    """(idx [len(rows), K], val, list of fp64 window logits) for the given rows."""
    idx = np.empty((len(rows), K), np.int32)
    val = np.empty((len(rows), K), np.float32)
    logits = []
    for i, t in enumerate(rows):
        v = row_logits(dq, t)
        logits.append(v)
        allowed = None if masks is None else masks[i][:len(v)]
        idx[i], val[i] = topk_row(v, int(dq.ks[t]), K, allowed)
    return idx, val, logits


# ------------------------------------------------------------------ windows
def ragged_windows(cu_q, cu_k, cu_c=None, ratio: int = 1):
    """Per-row key windows [ks, ke) of a varlen batch, written out row by row.

    P1 section 1: a chunk's rows score against their request's whole compressed
    prefix (the ratio-1/2 source layers), and each new row sees keys up to its own
    position; P1 section 2.1: a request can land on a cached prefix.  Request i owns
    query rows [cu_q[i], cu_q[i+1]) and token rows [cu_k[i], cu_k[i+1]); its len_q new
    tokens are the last of its len_k tokens, so new row j is token prefix + j with
    prefix = len_k - len_q, and it has seen prefix + j + 1 tokens.  Keys are one per
    `ratio` consecutive tokens, in rows [cu_c[i], cu_c[i+1]) (cu_c = cu_k when
    ratio = 1), and the row sees the keys of its complete groups: floor(seen /
    ratio), at most the request's key count.  Reading: the pages give the
    compressed length but not how a partial group is treated; a key summarises a
    whole group, so a row sees a key only once its group is complete.
    """
    cu_c = cu_k if cu_c is None else cu_c
    T = int(cu_q[-1])
    ks = np.zeros(T, np.int64)
    ke = np.zeros(T, np.int64)
    for i in range(len(cu_q) - 1):
        len_q = int(cu_q[i + 1]) - int(cu_q[i])
        len_k = int(cu_k[i + 1]) - int(cu_k[i])
        len_c = int(cu_c[i + 1]) - int(cu_c[i])
        for j in range(len_q):
            seen = len_k - len_q + j + 1
            t = int(cu_q[i]) + j
            ks[t] = int(cu_c[i])
            ke[t] = int(cu_c[i]) + min(seen // ratio, len_c)
    return ks, ke
