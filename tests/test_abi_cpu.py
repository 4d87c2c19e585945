"""The C ABI without a GPU: the library loads, exports every entry point that
include/idx.h declares, and rejects bad arguments on the host before any HIP
call (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

import mqa_logits_top_amd as idx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return idx.load_library()


def _declared():
    src = open(os.path.join(ROOT, "include", "idx.h")).read()
    return sorted(set(re.findall(r"^(?:idx_status|const char \*)\s*(idx_\w+)\(", src, re.M)))


def test_exports_match_header(lib):
    names = _declared()
    assert set(names) == set(idx.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert idx.status_str(0) == "ok"
    for s in range(1, 10):
        assert idx.status_str(s) not in ("ok", "unknown status")
    assert idx.status_str(99) == "unknown status"


def _problem(**kw):
    fake = 1 << 20   # 16-byte aligned, never dereferenced: every call below fails host checks
    base = dict(q=fake, q_scale=fake, k=fake, k_scale=fake, k_fmt=0, w=fake, ks=fake, ke=fake,
                T=4, H=32, D=128, L=1024, scale=1.0)
    base.update(kw)
    return idx.idx_problem(**base)


def _fused(lib, p, K=64, block_k=1024, row_chunk=0, ws=1 << 20, ws_bytes=1 << 30, out_idx=1 << 20):
    return lib.idx_logits_topk_fused(ctypes.byref(p), K, block_k, row_chunk, None, 0, out_idx, None, ws, ws_bytes,
                                     None)


def test_paged_transform_needs_both_pointers(lib):
    p = _problem()
    f = 1 << 20
    paged = lambda slot, out_slot: lib.idx_logits_topk_fused_paged(
        ctypes.byref(p), 64, 1024, 0, None, 0, slot, f, None, out_slot, f, 1 << 30, None)
    assert paged(f, None) == 1      # NULL: a table without an output
    assert paged(None, f) == 1      # NULL: an output without a table
    assert paged(f + 2, f) == 8     # ALIGN: int32 table


def test_gather_and_tail_rows_checks(lib):
    p = _problem()
    f = 1 << 20
    out = idx.idx_problem()
    assert lib.idx_gather_rows(ctypes.byref(p), f, 4, None, f, 1 << 30, None) == 1       # NULL out
    assert lib.idx_gather_rows(ctypes.byref(p), None, 4, ctypes.byref(out), f, 1 << 30, None) == 1
    assert lib.idx_gather_rows(ctypes.byref(p), f, -1, ctypes.byref(out), f, 1 << 30, None) == 2
    assert lib.idx_gather_rows(ctypes.byref(p), f, 4, ctypes.byref(out), f, 16, None) == 5  # WORKSPACE
    assert lib.idx_gather_rows(ctypes.byref(p), f, 4, ctypes.byref(out), f + 16, 1 << 30, None) == 8
    assert lib.idx_tail_rows(None, 2, 3, f, None) == 1
    assert lib.idx_tail_rows(f, -1, 3, f, None) == 2
    n = ctypes.c_size_t()
    assert lib.idx_workspace_size(5, ctypes.byref(p), 10, 0, 0, 0, 0, 0, ctypes.byref(n)) == 0
    assert n.value == _r(10 * 32 * 128) + 2 * _r(10 * 32 * 4) + 2 * _r(10 * 4)
    # zero rows: nothing to copy, an empty problem over the same keys
    assert lib.idx_gather_rows(ctypes.byref(p), None, 0, ctypes.byref(out), None, 0, None) == 0
    assert out.T == 0 and out.L == p.L and out.k == p.k


def test_ratio_windows_checks(lib):
    f = 1 << 20
    assert lib.idx_ragged_windows_ratio(f, f, None, 2, 2, 4, f, f, None) == 1
    assert lib.idx_ragged_windows_ratio(f, f, f, 0, 2, 4, f, f, None) == 3     # PARAM: ratio < 1


def test_block_consumer_checks(lib):
    p = _problem()
    f = 1 << 20
    call = lambda blocks, ld, nb, pool, bk=1024: lib.idx_logits_topk_fused_blocks(
        ctypes.byref(p), 64, bk, 0, blocks, ld, nb, pool, f, None, f, 1 << 30, None)
    assert call(None, 16, 16, 8) == 1          # NULL
    assert call(f, 8, 16, 8) == 2              # SHAPE: ld_blocks < n_blocks
    assert call(f, 16, 16, 6) == 6             # UNSUPPORTED: pool not a power of two
    assert call(f, 16, 16, 1, 32768) == 6      # UNSUPPORTED: 65536 keys per launch in 1-key blocks
    assert call(f + 2, 16, 16, 8) == 8         # ALIGN


def test_problem_validation(lib):
    assert _fused(lib, _problem(D=64)) == 6            # UNSUPPORTED
    assert _fused(lib, _problem(H=48)) == 6
    assert _fused(lib, _problem(k_fmt=2)) == 4         # FORMAT
    assert _fused(lib, _problem(q=None)) == 1          # NULL
    assert _fused(lib, _problem(ks=None)) == 1
    assert _fused(lib, _problem(T=-1)) == 2            # SHAPE
    assert _fused(lib, _problem(scale=0.0)) == 3       # PARAM
    assert _fused(lib, _problem(scale=float("nan"))) == 3
    assert _fused(lib, _problem(q=(1 << 20) + 4)) == 8  # ALIGN
    assert _fused(lib, _problem(), K=0) == 3
    assert _fused(lib, _problem(), K=2049) == 3
    assert _fused(lib, _problem(), block_k=300) == 3
    assert _fused(lib, _problem(), block_k=65536) == 3
    assert _fused(lib, _problem(), out_idx=None) == 1
    assert _fused(lib, _problem(), ws=None) == 1
    assert _fused(lib, _problem(), ws_bytes=100) == 5   # WORKSPACE
    assert _fused(lib, _problem(), ws=(1 << 20) + 16) == 8


def test_other_entry_validation(lib):
    p = _problem()
    f = 1 << 20
    assert lib.idx_mqa_logits(ctypes.byref(p), None, 1024, 1024, None) == 1
    assert lib.idx_mqa_logits(ctypes.byref(p), f, 100, 1024, None) == 2          # ld < W
    assert lib.idx_mqa_logits(ctypes.byref(_problem(H=16)), f, 1024, 1024, None) == 6
    assert lib.idx_mqa_logits_block(ctypes.byref(p), 0, 5, 0, 256, f, 256, None) == 2   # rows past T
    assert lib.idx_mqa_logits_block(ctypes.byref(p), 0, 4, 100, 256, f, 256, None) == 3  # key0 % 256
    assert lib.idx_topk(f, 1024, 1024, f, f, None, 0, 4, 0, 0, f, None, None, 0, None) == 3      # K = 0
    assert lib.idx_topk(f, 1024, 1024, f, f, None, 0, 4, 2561, 0, f, None, None, 0, None) == 3   # K > 2560
    assert lib.idx_topk(f, 100, 1024, f, f, None, 0, 4, 8, 0, f, None, None, 0, None) == 2       # ld < W
    assert lib.idx_topk(f, 1024, 1024, f, f, f, 10, 4, 8, 0, f, None, None, 0, None) == 2        # ld_mask < W
    assert lib.idx_topk(None, 1024, 1024, f, f, None, 0, 4, 8, 0, f, None, None, 0, None) == 1
    assert lib.idx_topk(f, 1024, 1024, f, f, None, 0, 4, 8, 40000, f, None, None, 0, None) == 3  # block_k
    assert lib.idx_block_candidates(ctypes.byref(p), None, 0, 4, 16, 1024, 0, f, 1024, 1024, None, f,
                                    1 << 30, None) == 6    # pool != 8
    assert lib.idx_block_candidates(ctypes.byref(p), None, 0, 8, 4096, 1024, 0, f, 1024, 1024, None, f,
                                    1 << 30, None) == 3    # n_blocks > 2048
    assert lib.idx_block_candidates(ctypes.byref(p), None, 0, 8, 16, 1024, 0, None, 1024, 1024, None, f,
                                    1 << 30, None) == 1    # mask NULL
    assert lib.idx_block_candidates(ctypes.byref(p), None, 0, 8, 16, 1024, 0, f, 10, 1024, None, f,
                                    1 << 30, None) == 2    # ld_mask < W
    assert lib.idx_ragged_windows(None, f, 2, 4, f, f, None) == 1
    assert lib.idx_ragged_windows(f, f, -1, 4, f, f, None) == 2


def _r(x):
    return (x + 255) // 256 * 256


def test_workspace_sizes(lib):
    head = 2304
    kc = lambda K: min(K + 512, 2560)
    p = _problem(T=2048, L=65536)
    n = ctypes.c_size_t()
    assert lib.idx_workspace_size(2, ctypes.byref(p), 2048, 32768, 0, 0, 0, 0, ctypes.byref(n)) == 0
    # scores of one block of B_k keys ([Tc, B_k + 64] fp32; a row's (value, id) slabs of the later
    # launches, ns slabs of 512 pairs, lie in its scratch row), then the slabs' bookkeeping:
    # thresholds, overflow flags, count words (ns splits x 4 parts), the two-call top-K's row
    # words.  Here K + 512 = 2560 > 65536 / 20: both blocks are block launches and there are no
    # slabs.
    slab = lambda Tc, ns: _r(Tc * 4) + _r((Tc // 8 + 1) * 4) + _r(Tc * ns * 4 * 4) + _r(Tc * 4)
    flags = 16384 * 4   # window flags of the scoring launches, a fixed region
    shift = lambda T, Tc: _r((-(-T // Tc) + 1) * 4)   # each row chunk's first window key
    assert n.value == (head + 2 * _r(2048 * kc(2048) * 4) + 2048 * (32768 + 64) * 4 + slab(2048, 0) + flags
                       + shift(2048, 2048))
    # the row chunk and B_k bound the workspace: later launches take at most four blocks (16 splits)
    p2 = _problem(T=16384, L=487936)
    assert lib.idx_workspace_size(2, ctypes.byref(p2), 512, 32768, 4096, 0, 0, 0, ctypes.byref(n)) == 0
    assert n.value == (head + 2 * _r(4096 * kc(512) * 4) + 4096 * (32768 + 64) * 4 + slab(4096, 16) + flags
                       + shift(16384, 4096))
    m = ctypes.c_size_t()
    p3 = _problem(T=16384, L=262144)
    assert lib.idx_workspace_size(2, ctypes.byref(p3), 512, 32768, 4096, 0, 0, 0, ctypes.byref(m)) == 0
    assert m.value == n.value
    p4 = _problem(T=16384, L=65536)
    assert lib.idx_workspace_size(2, ctypes.byref(p4), 512, 32768, 4096, 0, 0, 0, ctypes.byref(m)) == 0
    assert m.value < n.value
    # a small B_k: a row's slabs (1024 floats per split) take more than B_k + 64 floats, and the
    # scratch rows widen to hold them (exactly one slab count fits the size)
    p5 = _problem(T=4096, L=200000)
    assert lib.idx_workspace_size(2, ctypes.byref(p5), 64, 2048, 512, 0, 0, 0, ctypes.byref(m)) == 0
    fits = [ns for ns in range(1, 65)
            if m.value == (head + 2 * _r(512 * kc(64) * 4) + _r(512 * max(2048 + 64, 1024 * ns) * 4)
                           + slab(512, ns) + flags + shift(4096, 512))]
    assert len(fits) == 1 and 1024 * fits[0] > 2048 + 64, fits
    assert lib.idx_workspace_size(3, ctypes.byref(p), 0, 32768, 0, 8, 2048, 0, ctypes.byref(n)) == 0
    assert n.value == head + 2 * _r(2048 * kc(2048) * 4) + 2048 * (4096 + 64) * 4 + 2048 * 2048 * 4 + flags
    assert lib.idx_workspace_size(4, ctypes.byref(p), 0, 0, 1024, 8, 2048, 65536, ctypes.byref(n)) == 0
    assert n.value == head + 2 * _r(1024 * kc(2048) * 4) + 1024 * (8192 + 64) * 4 + 1024 * 2048 * 4
    assert lib.idx_workspace_size(0, ctypes.byref(p), 0, 0, 0, 0, 0, 0, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.idx_workspace_size(2, ctypes.byref(p), 0, 32768, 0, 0, 0, 0, ctypes.byref(n)) == 3
    assert lib.idx_workspace_size(9, ctypes.byref(p), 1, 256, 0, 0, 0, 0, ctypes.byref(n)) == 3


def test_static_workspace_limit(lib):
    """The allocation-free fused entry refuses, on the host, a call whose workspace would exceed
    IDX_STATIC_WS_BYTES, and checks its arguments like the entry with a caller workspace."""
    f = 1 << 20
    big = _problem(T=2048, L=65536)
    call = lambda p, K=2048, bk=32768, rc=0, oi=f: lib.idx_logits_topk_fused_static(
        ctypes.byref(p), K, bk, rc, None, 0, oi, None, None)
    assert call(big) == 5                      # WORKSPACE: 2048 rows x 65536 keys per launch
    assert call(big, rc=256, oi=None) == 1     # NULL output, checked before the workspace lookup
    assert call(big, rc=256, K=0) == 3         # PARAM
    assert call(_problem(D=64), rc=256) == 6   # UNSUPPORTED
    n = ctypes.c_size_t()
    assert lib.idx_workspace_size(2, ctypes.byref(big), 2048, 32768, 256, 0, 0, 0, ctypes.byref(n)) == 0
    assert n.value <= idx.STATIC_WS_BYTES


def test_refine_validation(lib):
    p = _problem()
    f = 1 << 20
    assert lib.idx_refine_topk(ctypes.byref(p), None, f, 600, 600, 64, 1, f, None, f, 4096, None) == 1
    assert lib.idx_refine_topk(ctypes.byref(p), f, f, 600, 600, 700, 1, f, None, f, 4096, None) == 3   # K > Kc
    assert lib.idx_refine_topk(ctypes.byref(p), f, f, 3000, 3000, 64, 1, f, None, f, 4096, None) == 3  # Kc > 2560
    assert lib.idx_refine_topk(ctypes.byref(p), f, f, 600, 600, 64, 4, f, None, f, 4096, None) == 6   # pool
    assert lib.idx_refine_topk(ctypes.byref(p), f, f, 500, 600, 64, 1, f, None, f, 4096, None) == 2   # ld < Kc
    assert lib.idx_refine_topk(ctypes.byref(p), f, f, 600, 600, 64, 1, f, None, f, 100, None) == 5    # ws


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library every entry point raises; there is no fallback path."""
    monkeypatch.setattr(idx, "_lib", None)
    monkeypatch.setattr(idx, "LIB_PATH", str(tmp_path / "libidx.so"))
    with pytest.raises(ImportError, match="not built"):
        idx.load_library()
    with pytest.raises(ImportError, match="not built"):
        idx.idx_status_str(0)


def test_launch_timing_host_checks(lib):
    """The timing read-out checks its arguments on the host; an empty record reads as 0
    launches, and stopping a record that never started is a no-op (no device is touched)."""
    n = ctypes.c_int32(-5)
    assert lib.idx_launch_timing_read(None, 0, None) == 1          # NULL count
    assert lib.idx_launch_timing_read(None, 4, ctypes.byref(n)) == 1   # NULL output with cap > 0
    assert lib.idx_launch_timing_read(None, -1, ctypes.byref(n)) == 3  # PARAM
    assert lib.idx_launch_timing(0) == 0
    assert lib.idx_launch_timing_read(None, 0, ctypes.byref(n)) == 0 and n.value == 0
    assert ctypes.sizeof(idx.idx_launch_time) == 28
