"""Python binding of libidx, the MI355X dense prefill indexer (MQA logits + top-K).

Argument marshalling only: every step of the indexer runs in the HIP kernels
behind the C ABI declared in include/idx.h.  PyTorch supplies device memory
(outputs and workspace are allocated here with torch when the caller passes
none) and the current HIP stream.  There is no fallback: if libidx.so is
missing or fails to load, every call raises.

Function names match the C entry points.  Tensors must be on the GPU and
contiguous; key indices in outputs are absolute rows of k.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libidx.so")

IDX_K_FP8_E4M3 = 0
IDX_K_MXFP4 = 1
IDX_OP_MQA_LOGITS = 0
IDX_OP_TOPK = 1
IDX_OP_LOGITS_TOPK_FUSED = 2
IDX_OP_BLOCK_CANDIDATES = 3
IDX_OP_BLOCK_CANDIDATES_DENSE = 4
IDX_OP_GATHER_ROWS = 5

STATUS = {0: "IDX_OK", 1: "IDX_E_NULL", 2: "IDX_E_SHAPE", 3: "IDX_E_PARAM", 4: "IDX_E_FORMAT",
          5: "IDX_E_WORKSPACE", 6: "IDX_E_UNSUPPORTED", 7: "IDX_E_LAUNCH", 8: "IDX_E_ALIGN", 9: "IDX_E_DEVICE_CHECK"}

EXPORTS = ("idx_mqa_logits", "idx_mqa_logits_block", "idx_topk", "idx_logits_topk_fused",
           "idx_logits_topk_fused_paged", "idx_logits_topk_fused_blocks", "idx_logits_topk_fused_static",
           "idx_refine_topk",
           "idx_block_candidates", "idx_workspace_size", "idx_ragged_windows", "idx_ragged_windows_ratio",
           "idx_gather_rows", "idx_tail_rows", "idx_launch_timing", "idx_launch_timing_read", "idx_status_str")

IDX_TIMING_MAX = 1024
LAUNCH_MODES = {0: "dense", 1: "block", 2: "pool8", 4: "slab"}


class IdxError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status_str(status)})")


class idx_launch_time(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_float), ("mode", ctypes.c_int32), ("flagged", ctypes.c_int32),
                ("row0", ctypes.c_int32), ("nrows", ctypes.c_int32), ("key0", ctypes.c_int32),
                ("nkeys", ctypes.c_int32)]


class idx_problem(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("k_fmt", ctypes.c_int32), ("w", ctypes.c_void_p),
                ("ks", ctypes.c_void_p), ("ke", ctypes.c_void_p), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("L", ctypes.c_int32), ("scale", ctypes.c_float)]


_lib = None


def load_library():
    """Load libidx.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libidx is not built ({LIB_PATH} missing); run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, VP = ctypes.POINTER(idx_problem), ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.idx_mqa_logits.argtypes = [P, VP, i64, i32, VP]
    lib.idx_mqa_logits_block.argtypes = [P, i32, i32, i32, i32, VP, i64, VP]
    lib.idx_topk.argtypes = [VP, i64, i32, VP, VP, VP, i64, i32, i32, i32, VP, VP, VP, sz, VP]
    lib.idx_logits_topk_fused.argtypes = [P, i32, i32, i32, VP, i64, VP, VP, VP, sz, VP]
    lib.idx_logits_topk_fused_paged.argtypes = [P, i32, i32, i32, VP, i64, VP, VP, VP, VP, VP, sz, VP]
    lib.idx_logits_topk_fused_blocks.argtypes = [P, i32, i32, i32, VP, i64, i32, i32, VP, VP, VP, sz, VP]
    lib.idx_logits_topk_fused_static.argtypes = [P, i32, i32, i32, VP, i64, VP, VP, VP]
    lib.idx_refine_topk.argtypes = [P, VP, VP, i64, i32, i32, i32, VP, VP, VP, sz, VP]
    lib.idx_block_candidates.argtypes = [P, VP, i64, i32, i32, i32, i32, VP, i64, i32, VP, VP, sz, VP]
    lib.idx_workspace_size.argtypes = [i32, P, i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.idx_ragged_windows.argtypes = [VP, VP, i32, i32, VP, VP, VP]
    lib.idx_ragged_windows_ratio.argtypes = [VP, VP, VP, i32, i32, i32, VP, VP, VP]
    lib.idx_gather_rows.argtypes = [P, VP, i32, P, VP, sz, VP]
    lib.idx_tail_rows.argtypes = [VP, i32, i32, VP, VP]
    lib.idx_launch_timing.argtypes = [i32]
    lib.idx_launch_timing_read.argtypes = [ctypes.POINTER(idx_launch_time), i32, ctypes.POINTER(i32)]
    lib.idx_status_str.argtypes = [i32]
    lib.idx_status_str.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name != "idx_status_str":
            getattr(lib, name).restype = i32
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().idx_status_str(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise IdxError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class Inputs:
    """Device tensors of one indexer call (see include/idx.h, idx_problem)."""
    q: torch.Tensor        # uint8 [T, H, D]
    q_scale: torch.Tensor  # float32 [T, H]
    k: torch.Tensor        # uint8 [L, D] (fp8) or [L, D/2] (MXFP4)
    k_scale: torch.Tensor  # float32 [L] (fp8) or uint8 [L, D/32] (MXFP4)
    w: torch.Tensor        # float32 [T, H]
    ks: torch.Tensor       # int32 [T]
    ke: torch.Tensor       # int32 [T]
    k_fmt: int = IDX_K_FP8_E4M3
    scale: float = 1.0

    @property
    def T(self):
        return int(self.q.shape[0])

    @property
    def H(self):
        return int(self.q.shape[1])

    @property
    def L(self):
        return int(self.k.shape[0])

    def struct(self) -> idx_problem:
        return idx_problem(q=self.q.data_ptr(), q_scale=self.q_scale.data_ptr(), k=self.k.data_ptr(),
                           k_scale=self.k_scale.data_ptr(), k_fmt=self.k_fmt, w=self.w.data_ptr(),
                           ks=self.ks.data_ptr(), ke=self.ke.data_ptr(), T=self.T, H=self.H,
                           D=int(self.q.shape[2]), L=self.L, scale=self.scale)

    @property
    def W(self) -> int:
        """Longest row window (max_seqlen_k), read from the device windows."""
        return int((self.ke - self.ks).max().item()) if self.T else 0

    @property
    def pairs(self) -> int:
        """In-window (row, key) pairs, read from the device windows."""
        return int((self.ke.to(torch.int64) - self.ks).sum().item()) if self.T else 0

    @staticmethod
    def from_host(p, device="cuda") -> "Inputs":
        """Copy a host problem (numpy arrays with the same field names) to the device.  A problem
        without ks / ke gives its batch as cu_q / cu_k; the windows are then built on the device
        by idx_ragged_windows."""
        t = lambda a: torch.from_numpy(a).to(device)
        if getattr(p, "ks", None) is not None:
            ks, ke = t(p.ks), t(p.ke)
        else:
            ks, ke = idx_ragged_windows(t(p.cu_q), t(p.cu_k), int(p.q.shape[0]))
        return Inputs(q=t(p.q), q_scale=t(p.q_scale), k=t(p.k), k_scale=t(p.k_scale), w=t(p.w), ks=ks,
                      ke=ke, k_fmt=int(p.k_fmt), scale=float(p.scale))


def idx_workspace_size(op: int, p: Inputs, K: int = 0, block_k: int = 0, row_chunk: int = 0, pool: int = 0,
                       n_blocks: int = 0, W: int = 0) -> int:
    n = ctypes.c_size_t(0)
    s = p.struct()
    _check("idx_workspace_size",
           load_library().idx_workspace_size(op, ctypes.byref(s), K, block_k, row_chunk, pool, n_blocks, W,
                                             ctypes.byref(n)))
    return n.value


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def idx_mqa_logits(p: Inputs, W: Optional[int] = None, out: Optional[torch.Tensor] = None, stream=None):
    """Dense row-relative logits [T, W] fp32 (-inf past each row's window)."""
    if W is None:
        W = int((p.ke - p.ks).max().item()) if p.T else 0
    if out is None:
        out = torch.empty((p.T, W), dtype=torch.float32, device=p.q.device)
    s = p.struct()
    _check("idx_mqa_logits", load_library().idx_mqa_logits(ctypes.byref(s), _ptr(out), out.stride(0), W,
                                                           _stream(stream)))
    return out


def idx_mqa_logits_block(p: Inputs, row0: int, nrows: int, key0: int, nkeys: int,
                         out: Optional[torch.Tensor] = None, stream=None):
    """Logits of rows [row0, row0+nrows) x keys [key0, key0+nkeys) (in-window entries only)."""
    if out is None:
        out = torch.full((nrows, nkeys), float("nan"), dtype=torch.float32, device=p.q.device)
    s = p.struct()
    _check("idx_mqa_logits_block",
           load_library().idx_mqa_logits_block(ctypes.byref(s), row0, nrows, key0, nkeys, _ptr(out), out.stride(0),
                                               _stream(stream)))
    return out


def idx_topk(logits: torch.Tensor, ks: torch.Tensor, ke: torch.Tensor, K: int, W: Optional[int] = None,
             block_k: int = 0, mask: Optional[torch.Tensor] = None, out_idx: Optional[torch.Tensor] = None,
             out_val: Optional[torch.Tensor] = None, with_values: bool = True, stream=None):
    T = int(logits.shape[0])
    W = int(logits.shape[1]) if W is None else W
    dev = logits.device
    if out_idx is None:
        out_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    if out_val is None and with_values:
        out_val = torch.empty((T, K), dtype=torch.float32, device=dev)
    _check("idx_topk", load_library().idx_topk(
        _ptr(logits), logits.stride(0), W, _ptr(ks), _ptr(ke), _ptr(mask), mask.stride(0) if mask is not None else 0,
        T, K, block_k, _ptr(out_idx), _ptr(out_val), None, 0, _stream(stream)))
    return out_idx, out_val


def idx_logits_topk_fused(p: Inputs, K: int, block_k: int = 32768, row_chunk: int = 0,
                          mask: Optional[torch.Tensor] = None, out_idx: Optional[torch.Tensor] = None,
                          out_val: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                          with_values: bool = True, stream=None):
    dev = p.q.device
    if out_idx is None:
        out_idx = torch.empty((p.T, K), dtype=torch.int32, device=dev)
    if out_val is None and with_values:
        out_val = torch.empty((p.T, K), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(idx_workspace_size(IDX_OP_LOGITS_TOPK_FUSED, p, K=K, block_k=block_k, row_chunk=row_chunk),
                        dev)
    s = p.struct()
    _check("idx_logits_topk_fused", load_library().idx_logits_topk_fused(
        ctypes.byref(s), K, block_k, row_chunk, _ptr(mask), mask.stride(0) if mask is not None else 0,
        _ptr(out_idx), _ptr(out_val), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))
    return out_idx, out_val


def idx_logits_topk_fused_paged(p: Inputs, K: int, slot_of_key: torch.Tensor, block_k: int = 32768,
                                row_chunk: int = 0, mask: Optional[torch.Tensor] = None,
                                out_idx: Optional[torch.Tensor] = None, out_val: Optional[torch.Tensor] = None,
                                out_slot: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                                with_values: bool = True, stream=None):
    """idx_logits_topk_fused plus out_slot = slot_of_key[out_idx] (-1 pads), in the same final write."""
    dev = p.q.device
    if out_idx is None:
        out_idx = torch.empty((p.T, K), dtype=torch.int32, device=dev)
    if out_val is None and with_values:
        out_val = torch.empty((p.T, K), dtype=torch.float32, device=dev)
    if out_slot is None:
        out_slot = torch.empty((p.T, K), dtype=torch.int32, device=dev)
    if ws is None:
        ws = _workspace(idx_workspace_size(IDX_OP_LOGITS_TOPK_FUSED, p, K=K, block_k=block_k, row_chunk=row_chunk),
                        dev)
    s = p.struct()
    _check("idx_logits_topk_fused_paged", load_library().idx_logits_topk_fused_paged(
        ctypes.byref(s), K, block_k, row_chunk, _ptr(mask), mask.stride(0) if mask is not None else 0,
        _ptr(slot_of_key), _ptr(out_idx), _ptr(out_val), _ptr(out_slot), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))
    return out_idx, out_val, out_slot


def idx_logits_topk_fused_blocks(p: Inputs, K: int, blocks: torch.Tensor, pool: int = 8, block_k: int = 32768,
                                 row_chunk: int = 0, out_idx: Optional[torch.Tensor] = None,
                                 out_val: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                                 with_values: bool = True, stream=None):
    """idx_logits_topk_fused restricted to the candidate blocks blocks[t] ([T, n_blocks], -1 ignored)."""
    dev = p.q.device
    if out_idx is None:
        out_idx = torch.empty((p.T, K), dtype=torch.int32, device=dev)
    if out_val is None and with_values:
        out_val = torch.empty((p.T, K), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(idx_workspace_size(IDX_OP_LOGITS_TOPK_FUSED, p, K=K, block_k=block_k, row_chunk=row_chunk),
                        dev)
    s = p.struct()
    _check("idx_logits_topk_fused_blocks", load_library().idx_logits_topk_fused_blocks(
        ctypes.byref(s), K, block_k, row_chunk, _ptr(blocks), blocks.stride(0), int(blocks.shape[1]), pool,
        _ptr(out_idx), _ptr(out_val), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))
    return out_idx, out_val


STATIC_WS_BYTES = 128 << 20   # IDX_STATIC_WS_BYTES


def idx_logits_topk_fused_static(p: Inputs, K: int, block_k: int = 32768, row_chunk: int = 0,
                                 mask: Optional[torch.Tensor] = None, out_idx: Optional[torch.Tensor] = None,
                                 out_val: Optional[torch.Tensor] = None, with_values: bool = True, stream=None):
    """idx_logits_topk_fused on the library's static workspace: no workspace argument, and the
    library allocates nothing (the outputs are the caller's; they are allocated here only when
    not given)."""
    dev = p.q.device
    if out_idx is None:
        out_idx = torch.empty((p.T, K), dtype=torch.int32, device=dev)
    if out_val is None and with_values:
        out_val = torch.empty((p.T, K), dtype=torch.float32, device=dev)
    s = p.struct()
    _check("idx_logits_topk_fused_static", load_library().idx_logits_topk_fused_static(
        ctypes.byref(s), K, block_k, row_chunk, _ptr(mask), mask.stride(0) if mask is not None else 0,
        _ptr(out_idx), _ptr(out_val), _stream(stream)))
    return out_idx, out_val


RESERVE = 512   # extra candidates the exact boundary refinement keeps per row
REFINE_WS = 2304


def candidate_capacity(K: int) -> int:
    return min(K + RESERVE, 2560)


def idx_refine_topk(p: Inputs, cand_idx: torch.Tensor, cand_val: torch.Tensor, K: int, pool: int = 1,
                    out_idx: Optional[torch.Tensor] = None, out_val: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, with_values: bool = True, stream=None):
    dev = cand_idx.device
    T, Kc = int(cand_idx.shape[0]), int(cand_idx.shape[1])
    if out_idx is None:
        out_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    if out_val is None and with_values:
        out_val = torch.empty((T, K), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(REFINE_WS, dev)
    s = p.struct()
    _check("idx_refine_topk", load_library().idx_refine_topk(
        ctypes.byref(s), _ptr(cand_idx), _ptr(cand_val), cand_idx.stride(0), Kc, K, pool, _ptr(out_idx),
        _ptr(out_val), _ptr(ws), ws.numel(), _stream(stream)))
    return out_idx, out_val


def overflow_count(ws: torch.Tensor) -> int:
    """Rows of the last call on this workspace whose candidate list could not settle the boundary."""
    return int(ws[:4].view(torch.int32).item())


def idx_block_candidates(p: Inputs, W: int, pool: int = 8, n_blocks: int = 2048,
                         logits: Optional[torch.Tensor] = None, block_k: int = 32768, row_chunk: int = 0,
                         mask: Optional[torch.Tensor] = None, out_blocks: Optional[torch.Tensor] = None,
                         ws: Optional[torch.Tensor] = None, stream=None):
    dev = p.ks.device
    if mask is None:
        mask = torch.empty((p.T, W), dtype=torch.uint8, device=dev)
    op = IDX_OP_BLOCK_CANDIDATES_DENSE if logits is not None else IDX_OP_BLOCK_CANDIDATES
    if ws is None:
        ws = _workspace(idx_workspace_size(op, p, block_k=block_k, row_chunk=row_chunk, pool=pool,
                                           n_blocks=n_blocks, W=W), dev)
    s = p.struct()
    _check("idx_block_candidates", load_library().idx_block_candidates(
        ctypes.byref(s), _ptr(logits), logits.stride(0) if logits is not None else 0, pool, n_blocks, block_k,
        row_chunk, _ptr(mask), mask.stride(0), W, _ptr(out_blocks), _ptr(ws), ws.numel() if ws is not None else 0,
        _stream(stream)))
    return mask, out_blocks


def idx_ragged_windows(cu_q: torch.Tensor, cu_k: torch.Tensor, T: int, stream=None):
    B = int(cu_q.numel()) - 1
    ks = torch.empty(T, dtype=torch.int32, device=cu_q.device)
    ke = torch.empty(T, dtype=torch.int32, device=cu_q.device)
    _check("idx_ragged_windows", load_library().idx_ragged_windows(_ptr(cu_q), _ptr(cu_k), B, T, _ptr(ks), _ptr(ke),
                                                                   _stream(stream)))
    return ks, ke


def idx_ragged_windows_ratio(cu_q: torch.Tensor, cu_k: torch.Tensor, cu_c: torch.Tensor, ratio: int, T: int,
                             stream=None):
    """Windows over keys compressed `ratio` tokens to one (cu_c: key rows per request)."""
    B = int(cu_q.numel()) - 1
    ks = torch.empty(T, dtype=torch.int32, device=cu_q.device)
    ke = torch.empty(T, dtype=torch.int32, device=cu_q.device)
    _check("idx_ragged_windows_ratio", load_library().idx_ragged_windows_ratio(
        _ptr(cu_q), _ptr(cu_k), _ptr(cu_c), ratio, B, T, _ptr(ks), _ptr(ke), _stream(stream)))
    return ks, ke


def idx_gather_rows(p: Inputs, rows: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None) -> Inputs:
    """The problem restricted to rows[r] (-1: padding row).  The returned Inputs' row tensors
    are views of ws (the copies idx_gather_rows made); keys are shared with p."""
    R = int(rows.numel())
    if ws is None:
        ws = _workspace(idx_workspace_size(IDX_OP_GATHER_ROWS, p, K=R), p.q.device)
    s, out = p.struct(), idx_problem()
    _check("idx_gather_rows", load_library().idx_gather_rows(ctypes.byref(s), _ptr(rows), R, ctypes.byref(out),
                                                             _ptr(ws), ws.numel() if ws is not None else 0,
                                                             _stream(stream)))
    H, D = p.H, int(p.q.shape[2])

    def view(ptr, nbytes, dtype, shape):   # the array the C call placed at ptr inside ws
        if R == 0:
            return torch.empty(shape, dtype=dtype, device=p.q.device)
        o = ptr - ws.data_ptr()
        return ws[o:o + nbytes].view(dtype).view(shape)

    return Inputs(q=view(out.q, R * H * D, torch.uint8, (R, H, D)),
                  q_scale=view(out.q_scale, R * H * 4, torch.float32, (R, H)), k=p.k, k_scale=p.k_scale,
                  w=view(out.w, R * H * 4, torch.float32, (R, H)), ks=view(out.ks, R * 4, torch.int32, (R,)),
                  ke=view(out.ke, R * 4, torch.int32, (R,)), k_fmt=p.k_fmt, scale=p.scale)


def idx_tail_rows(cu_q: torch.Tensor, n: int, stream=None) -> torch.Tensor:
    """The last n rows of every request ([B * n], -1 where a request is shorter)."""
    B = int(cu_q.numel()) - 1
    rows = torch.empty(B * n, dtype=torch.int32, device=cu_q.device)
    _check("idx_tail_rows", load_library().idx_tail_rows(_ptr(cu_q), B, n, _ptr(rows), _stream(stream)))
    return rows


def idx_launch_timing(enable: bool) -> None:
    """Start (clearing the record) or stop recording the scoring launches' HIP event times."""
    _check("idx_launch_timing", load_library().idx_launch_timing(1 if enable else 0))


def idx_launch_timing_read() -> list:
    """The recorded launches, in launch order, as dicts (ms < 0: the launch failed); clears the
    record."""
    buf = (idx_launch_time * IDX_TIMING_MAX)()
    n = ctypes.c_int32()
    _check("idx_launch_timing_read", load_library().idx_launch_timing_read(buf, IDX_TIMING_MAX, ctypes.byref(n)))
    return [{"ms": e.ms, "mode": LAUNCH_MODES.get(e.mode, e.mode), "flagged": bool(e.flagged), "row0": e.row0,
             "nrows": e.nrows, "key0": e.key0, "nkeys": e.nkeys} for e in buf[:min(n.value, IDX_TIMING_MAX)]]


def idx_status_str(status: int) -> str:
    return status_str(status)
