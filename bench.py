"""Benchmark of the dense prefill indexer on one MI355X.

A step is one pass of the indexer's hot path over one batch: the per-row key
windows are built from the batch's cu_seqlens on the device, then the fused
key-blocked logits + top-K runs (scoring on fp8 MFMA with the ReLU-weighted
head sum in registers, per-block exact top-K with a running merge, exact
boundary refinement).  Headline workload: the long-context chunk, T = 16384
query rows against L = 487936 keys (P2 Motivation's 16384-row chunk at 487,936
context), H = 64, D = 128, fp8 q and k with per-row scales, causal windows,
K = 512, key blocks of 32768, row chunks of 4096.

Printed: one JSON line.  value = scored in-window (row, key) pairs per second
(inputs resident in HBM).  roofline: the scoring kernel's algorithmic fp8 FLOPs
(2 H D per in-window pair) per launch over its average launch duration (HIP
events on the launch stream, the launches the fused path makes) against the
fp8 dense MFMA peak.  cpu_baseline: the single-threaded fp64 C++ oracle on a
stratified row sample of the same workload, one row per host thread.  extra:
the other workloads, each with its own scoring roofline (the DeepSeek-V4-like
MXFP4 chunk at T = 2048, L = 102400 is the logits-stage target shape), the
row-chunked dense comparator, the two-stream pipeline and the candidate source.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mqa_logits_top_amd as idx  # noqa: E402
from mqa_logits_top_amd.pipeline import RowChunkedDense, rows_for_budget  # noqa: E402
import synth  # noqa: E402

METRIC = "indexer (row,key) pairs/s fused logits+top-K; % fp8 MFMA peak; peak bytes"
FP8_PEAK = 5.0e15      # MI355X dense fp8 MFMA, FLOP/s
HBM_PEAK = 8.0e12
HEADLINE = "long_ctx"
# Row chunks: long_ctx is fastest at 4096 (8192 and 16384: +1%); the ragged batch at 8192 (-11%
# against 4096: half as many row chunks, each planning its launches over all of L, most of them
# empty for the short requests), still under the 2 GiB logits budget (1092 MiB workspace).
ROW_CHUNK = {"tiny": 0, "glm_chunk": 0, "dsv4_mxfp4": 0, "long_ctx": 4096, "ragged_cand": 8192}
DESCRIBE = {
    "tiny": "tiny: T=64 L=4096 H=32 D=128 fp8 q/k per-row scales, causal windows, top-K=512",
    "glm_chunk": "glm_chunk: T=2048 L=65536 H=32 D=128 fp8 q/k per-row scales, causal windows, top-K=2048, "
                 "fused key blocks B_k=32768",
    "dsv4_mxfp4": "dsv4_mxfp4: T=2048 L=102400 H=64 D=128 fp8 q, MXFP4 keys (E2M1, E8M0 per 32), 5% duplicated "
                  "key rows, causal windows, top-K=512, fused key blocks B_k=32768",
    "long_ctx": "long_ctx: T=16384 L=487936 H=64 D=128 fp8 q/k per-row scales, causal windows, top-K=512, "
                "fused key blocks B_k=32768, row chunks of 4096",
    "ragged_cand": "ragged_cand: 4 x 7168 new tokens + 2048 new on a 150000-token prefix (30720 rows, 180720 keys), "
                   "H=64 fp8, top-K=512, row chunks of 8192",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the scoring kernel's code (logits.hip, the LogitsArgs struct and the key-split
    planning; comments and blank lines excluded), to tell whether committed counter figures
    were taken on the kernel and launch layout as they stand."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mqa_logits_top_amd", "csrc")
    with open(os.path.join(csrc, "logits.hip")) as fh:
        text = fh.read()
    with open(os.path.join(csrc, "kernels.h")) as fh:
        hdr = fh.read()
    a = hdr.index("struct LogitsArgs {")
    text += hdr[a:hdr.index("};", a)]
    with open(os.path.join(csrc, "api.cpp")) as fh:
        api = fh.read()
    a = api.index("void plan_splits(")
    text += api[a:api.index("\n}\n", a)]
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic(workload, mode, rect):
    """HBM bytes per scoring launch of one mode ("block", "slab") from the committed rocprofv3
    counter summary, if it was taken on the current kernel source and the same launch rectangle
    (rows, keys)."""
    path = os.path.join(ROOT, "profiles", "logits_hbm_traffic.json")
    try:
        with open(path) as f:
            e = json.load(f).get(f"{workload}/{mode}")
        if e and e.get("kernel_source_hash") == kernel_source_hash() and e.get("rect") == list(rect):
            return e["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def time_events(fn, n, stream):
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def block_launches(L, block_k, K):
    """Number of one-block launches at the start of a row chunk's key schedule."""
    kc = min(K + 512, 2560)
    if L <= block_k:
        return 1
    nb = 1
    while nb * block_k < L and kc * 20 > nb * block_k:
        nb += 1
    return nb


def key_launches(L, block_k, K):
    """(key0, keys) of the fused path's scoring launches over one row chunk: one block of B_k
    keys per launch while the keys seen stay below 20 (K + 512), then up to four blocks per
    launch, spread evenly over the keys left (the slab launches)."""
    if L <= block_k:
        return [(0, L)]
    nb = block_launches(L, block_k, K)
    out = [(i * block_k, min(block_k, L - i * block_k)) for i in range(nb) if i * block_k < L]
    rest = L - nb * block_k
    if rest <= 0:
        return out
    n2 = -(-rest // (4 * block_k))
    step = -(-(-(-rest // n2)) // 256) * 256
    return out + [(kb, min(step, L - kb)) for kb in range(nb * block_k, L, step)]


def launch_rects(d, block_k, row_chunk, K):
    """The (row0, rows, key0, keys) rectangles the fused path scores, one per launch."""
    Tc = d.T if row_chunk <= 0 else min(row_chunk, d.T)
    return [(r0, min(Tc, d.T - r0), kb, nk) for r0 in range(0, d.T, Tc) for kb, nk in key_launches(d.L, block_k, K)]


def rect_pairs(d, r0, nr, kb, nk):
    lo = torch.clamp(d.ks[r0:r0 + nr].to(torch.int64), min=kb)
    hi = torch.clamp(d.ke[r0:r0 + nr].to(torch.int64), max=kb + nk)
    return int(torch.clamp(hi - lo, min=0).sum().item())


def scoring_roofline(d, block_k, row_chunk, K, reps, stream, workload):
    """The scoring kernel over the fused path's launch rectangles (key-block store, as
    idx_mqa_logits_block launches it), reps passes back to back between one pair of events on
    `stream`; achieved = algorithmic fp8 FLOPs per launch / average launch duration."""
    rects = launch_rects(d, block_k, row_chunk, K)
    rmax = max(r[1] for r in rects)
    kmax = max(r[3] for r in rects)
    scratch = torch.empty((rmax, kmax + 64), dtype=torch.float32, device=d.q.device)[:, :kmax]

    def run():
        for _ in range(reps):
            for r0, nr, kb, nk in rects:
                idx.idx_mqa_logits_block(d, r0, nr, kb, nk, out=scratch, stream=stream)

    run()  # warm
    t = time_events(run, 3, stream)
    flops = sum(2 * d.H * 128 * rect_pairs(d, *r) for r in rects)
    del scratch
    avg_ms = float(np.median(t)) / (reps * len(rects))
    per_launch = flops / len(rects)
    achieved = per_launch / (avg_ms * 1e-3)
    main = max(rects, key=lambda r: r[1] * r[3])
    return {"bound": "mfma", "achieved": achieved / 1e12, "peak": FP8_PEAK / 1e12, "unit": "TFLOP/s",
            "frac": achieved / FP8_PEAK, "traffic": load_traffic(workload, "block", (main[1], main[3])),
            "kernel": f"logits_kernel (scoring, {'MXFP4' if d.k_fmt else 'fp8'} keys, H={d.H}, key-block store)",
            "avg_launch_ms": avg_ms, "launches_per_pass": len(rects), "flop_per_launch": per_launch,
            "rect_rows_keys": [main[1], main[3]]}


KEY_SHIFT_ALIGN = 256   # a row chunk's launches start at its first window key, rounded down to this


def chunk_shifts(d, Tc):
    """First window key of each row chunk, rounded down to KEY_SHIFT_ALIGN (the fused path shifts
    the chunk's key launches by it on the device)."""
    ks = torch.clamp(d.ks.to(torch.int64), min=0).cpu()
    ke = torch.clamp(d.ke.to(torch.int64), max=d.L).cpu()
    out = []
    for r0 in range(0, d.T, Tc):
        lo, hi = ks[r0:r0 + Tc], ke[r0:r0 + Tc]
        live = lo[hi > lo]
        out.append(int(live.min()) // KEY_SHIFT_ALIGN * KEY_SHIFT_ALIGN if live.numel() else 0)
    return out


def fused_launch_roofline(step, d, row_chunk, n_steps, stream, workload):
    """The fused step's scoring launches, timed by the library's launch-timing record (two HIP
    events on the step's stream around each launch, both dispatches of its pair) over n_steps
    steps.  The launch kind that takes the most time gives the roofline: algorithmic fp8 FLOPs
    per launch (2 H D per in-window (row, key) pair of its rectangle) / its mean duration."""
    torch.cuda.synchronize()
    idx.idx_launch_timing(True)
    try:
        for _ in range(n_steps):
            step()
        torch.cuda.synchronize()
        rec = idx.idx_launch_timing_read()
    finally:
        idx.idx_launch_timing(False)
    Tc = d.T if row_chunk <= 0 else min(row_chunk, d.T)
    shift = chunk_shifts(d, Tc)
    groups = {}
    for e in rec:
        assert e["ms"] > 0, e
        kind = e["mode"] + (" (flagged rows)" if e["flagged"] else "")
        sh = shift[e["row0"] // Tc]
        lo, hi = min(d.L, e["key0"] + sh), min(d.L, e["key0"] + e["nkeys"] + sh)
        g = groups.setdefault(kind, {"n": 0, "ms": 0.0, "flop": 0, "keys": 0, "rows": 0})
        g["n"] += 1
        g["ms"] += e["ms"]
        if not e["flagged"]:   # a flagged-rows pass scores only the row blocks the slab check flagged
            g["flop"] += 2 * d.H * 128 * rect_pairs(d, e["row0"], e["nrows"], lo, hi - lo)
        g["keys"] = max(g["keys"], e["nkeys"])
        g["rows"] = max(g["rows"], e["nrows"])
    main = max((k for k in groups if "flagged" not in k), key=lambda k: groups[k]["ms"])
    g = groups[main]
    avg_ms = g["ms"] / g["n"]
    per_launch = g["flop"] / g["n"]
    achieved = per_launch / (avg_ms * 1e-3)
    what = {"slab": "candidate-slab launches", "block": "key-block launches"}.get(main, main + " launches")
    others = {k: {"launches_per_step": v["n"] / n_steps, "mean_ms": v["ms"] / v["n"],
                  "tflops": v["flop"] / (v["ms"] * 1e-3) / 1e12 if "flagged" not in k else None}
              for k, v in groups.items() if k != main}
    return {"bound": "mfma", "achieved": achieved / 1e12, "peak": FP8_PEAK / 1e12, "unit": "TFLOP/s",
            "frac": achieved / FP8_PEAK, "traffic": load_traffic(workload, main, (g["rows"], g["keys"])),
            "kernel": f"logits_kernel (scoring, {'MXFP4' if d.k_fmt else 'fp8'} keys, H={d.H}, {what} of the fused step)",
            "launch_mode": main, "avg_launch_ms": avg_ms, "launches_per_step": g["n"] / n_steps,
            "flop_per_launch": per_launch, "rect_rows_keys": [g["rows"], g["keys"]],
            "timing": f"library launch-timing record over {n_steps} fused steps after the timed ones",
            "other_launches": others}


def fused_step(d, K, block_k, row_chunk, cu_q, cu_k, stream):
    """(step function, outputs, workspace) of one workload: windows from cu_seqlens on the device,
    then the fused indexer."""
    dev = d.q.device
    ws = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=K, block_k=block_k, row_chunk=row_chunk),
                     dtype=torch.uint8, device=dev)
    oi = torch.empty((d.T, K), dtype=torch.int32, device=dev)
    ov = torch.empty((d.T, K), dtype=torch.float32, device=dev)
    ks = torch.empty(d.T, dtype=torch.int32, device=dev)
    ke = torch.empty(d.T, dtype=torch.int32, device=dev)
    lib = idx.load_library()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    dd = idx.Inputs(q=d.q, q_scale=d.q_scale, k=d.k, k_scale=d.k_scale, w=d.w, ks=ks, ke=ke, k_fmt=d.k_fmt,
                    scale=d.scale)
    B = int(cu_q.numel()) - 1

    def step():
        st = lib.idx_ragged_windows(idx._ptr(cu_q), idx._ptr(cu_k), B, d.T, idx._ptr(ks), idx._ptr(ke), sptr)
        assert st == 0
        idx.idx_logits_topk_fused(dd, K, block_k=block_k, row_chunk=row_chunk, out_idx=oi, out_val=ov, ws=ws,
                                  stream=stream)

    return step, oi, ov, ws


def peak_check(d, K, block_k, row_chunk, stream):
    """Device memory one fused call takes beyond its inputs, from torch's allocator statistics:
    the workspace and the [T, K] outputs the binding allocates; the library allocates nothing."""
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    oi, ov = idx.idx_logits_topk_fused(d, K, block_k=block_k, row_chunk=row_chunk, stream=stream)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    ws = idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=K, block_k=block_k, row_chunk=row_chunk)
    del oi, ov
    return {"allocator_peak_bytes": int(peak), "workspace_bytes": int(ws), "outputs_bytes": int(8 * d.T * K)}


def workload(name, dev, stream, steps, warmup, roof_reps):
    """One workload's fused step, timed with events over `steps` steps, and its scoring roofline."""
    p = synth.make_config(name)
    d = idx.Inputs.from_host(p, device=dev)
    K, Bk, rc = p.meta["K"], p.meta["block_k"], ROW_CHUNK[name]
    cu_q = torch.from_numpy(p.cu_q).to(dev)
    cu_k = torch.from_numpy(p.cu_k).to(dev)
    step, oi, ov, ws = fused_step(d, K, Bk, rc, cu_q, cu_k, stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    assert idx.overflow_count(ws) == 0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / steps
    pairs = d.pairs
    flops = 2 * d.H * 128 * pairs
    line = {"workload": DESCRIBE[name], "T": d.T, "L": d.L, "H": d.H, "K": K, "block_k": Bk, "row_chunk": rc,
            "pairs": pairs, "ms": ms, "wall_ms": wall / steps * 1e3, "pairs_per_s": pairs / (ms * 1e-3),
            "tflops": flops / (ms * 1e-3) / 1e12, "fp8_peak_frac_step": flops / (ms * 1e-3) / FP8_PEAK,
            "peak_transient_bytes": int(ws.numel())}
    log(f"[bench] {name}: fused step {ms:.4f} ms -> {line['pairs_per_s']:.4e} pairs/s, {line['tflops']:.0f} TFLOP/s "
        f"({100 * line['fp8_peak_frac_step']:.1f}% of fp8 peak at step level), workspace {ws.numel() / 2**20:.0f} MiB")
    if roof_reps:
        line["roofline"] = fused_launch_roofline(step, d, rc, 3, stream, name)
        r = line["roofline"]
        log(f"[bench] {name}: scoring kernel, {r['launch_mode']} launches of the fused step, {r['avg_launch_ms']:.4f} "
            f"ms/launch -> {r['achieved']:.1f} TFLOP/s ({100 * r['frac']:.1f}% of fp8 peak)")
        line["scoring_block_store"] = scoring_roofline(d, Bk, rc, K, roof_reps, stream, name)
        r = line["scoring_block_store"]
        log(f"[bench] {name}: scoring kernel, key-block store over the step's rectangles, {r['avg_launch_ms']:.4f} "
            f"ms/launch -> {r['achieved']:.1f} TFLOP/s ({100 * r['frac']:.1f}% of fp8 peak)")
    return p, d, line, (oi, ov, ws)


def cpu_baseline(p, K, g_idx, budget_s, workers):
    """The single-threaded fp64 C++ oracle on a stratified row sample (first and last rows, every
    ceil(T/256)-th row, rows next to row-chunk and key-block boundaries; each row scored in full
    and its top-K computed), one row per host thread; then one thread alone on a few rows.  The
    sampled rows' top-K sets are checked against the GPU's (near-ties within 1e-6 may swap)."""
    import oracle

    t0 = time.perf_counter()
    dq = oracle.Dequantised(p)
    setup = time.perf_counter() - t0
    T = dq.T
    rows = {0, T - 1, *range(0, T, -(-T // 256))}
    for b in (1024, 4096, 8192, 12288):
        rows.update(r for r in (b - 1, b) if 0 <= r < T)
    rows = sorted(rows)
    rng = np.random.default_rng(0)
    rows = [rows[i] for i in rng.permutation(len(rows))]

    def one(t):
        v = oracle.row_logits(dq, t)
        i, _ = oracle.topk_row(v, int(dq.ks[t]), K)
        return t, v, i

    done, pairs, checked = [], 0, 0
    from concurrent.futures import ThreadPoolExecutor
    t1 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for b0 in range(0, len(rows), workers):
            for t, v, i in ex.map(one, rows[b0:b0 + workers]):
                pairs += len(v)
                done.append(t)
                g = g_idx[t][g_idx[t] >= 0]
                o = i[i >= 0]
                diff = np.setxor1d(g, o)
                if len(diff):
                    vk = float(np.min(v[o - dq.ks[t]]))
                    assert len(g) == len(o) and (np.abs(v[diff - dq.ks[t]] - vk) <= 1e-6 * abs(vk)).all(), \
                        f"row {t}: GPU top-K differs from the oracle"
                checked += 1
            if time.perf_counter() - t1 > budget_s:
                break
    el = time.perf_counter() - t1
    t2 = time.perf_counter()
    sp = 0
    for t in rows[:2]:
        sp += len(one(t)[1])
    single = sp / (time.perf_counter() - t2)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    rate = pairs / el
    return {"value": rate, "unit": "pairs/s", "cores": int(workers), "kind": "oracle",
            "sample": f"{len(done)} of {T} rows (stratified: first/last, every {-(-T // 256)}th, chunk boundaries), "
                      f"full windows, logits + top-{K}, {pairs} pairs in {el:.1f} s on {workers} threads, one row "
                      f"per thread (+{setup:.1f} s dequantisation, not counted); GPU top-K checked on every "
                      f"sampled row; full workload extrapolated: {dq.pairs / rate:.0f} s",
            "single_core_value": single, "rows_checked": checked, "cpu_model": model, "host_cpus": os.cpu_count()}


COPY_BYTES = 256 << 20   # calibration copy of the traffic probe
# A scoring launch is two dispatches over one grid, the f16 head-sum form, then the fp32 form
# (each workgroup works in one of them); these prefixes name both.
PROBE = {"glm_chunk": "logits_kernel<0, 32, 1, 4, ", "long_ctx": "logits_kernel<0, 64, 1, 4, ",
         "dsv4_mxfp4": "logits_kernel<1, 64, 1, 4, "}
# the candidate-slab launches of the fused calls the probe makes (every slab launch of the call)
SLAB_PROBE = {"long_ctx": "logits_kernel<0, 64, 4, 4, ", "dsv4_mxfp4": "logits_kernel<1, 64, 4, 4, "}
PROBE_CALLS = ("glm_chunk fused", "ragged_cand candidates", "long_ctx fused", "dsv4_mxfp4 fused")
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_MFMA",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "GRBM_COUNT")


def launch_pairs(values):
    """Per-launch sums of the (f16 form, fp32 form) dispatch pairs of a scoring launch, in order."""
    return [values[i] + values[i + 1] for i in range(0, len(values) - 1, 2)]


def traffic_probe(dev):
    """Launches for a rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE run: one fused glm_chunk call, the
    ragged workload's candidate source (the selection, refinement, pooling and mask kernels), one
    fused long_ctx call and one fused dsv4_mxfp4 call (their candidate-slab launches), then the
    scoring kernel on the glm_chunk, long_ctx and dsv4_mxfp4 key-block rectangles (as the fused
    path launches them) twice each, then two device-to-device copies of COPY_BYTES that calibrate
    what those counters read for a known number of bytes."""
    p = synth.make_config("glm_chunk")
    d = idx.Inputs.from_host(p, device=dev)
    idx.idx_logits_topk_fused(d, p.meta["K"], block_k=p.meta["block_k"])
    p5 = synth.make_config("ragged_cand")
    c5 = p5.meta
    d5 = idx.Inputs.from_host(p5, device=dev)
    blocks5 = torch.empty((p5.T, c5["n_blocks"]), dtype=torch.int32, device=dev)
    idx.idx_block_candidates(d5, d5.W, pool=c5["pool"], n_blocks=c5["n_blocks"], block_k=c5["block_k"],
                             row_chunk=ROW_CHUNK["ragged_cand"], out_blocks=blocks5)
    torch.cuda.synchronize()
    del d5, blocks5
    torch.cuda.empty_cache()
    for name in SLAB_PROBE:
        pw = synth.make_config(name)
        dw = idx.Inputs.from_host(pw, device=dev)
        idx.idx_logits_topk_fused(dw, pw.meta["K"], block_k=pw.meta["block_k"], row_chunk=ROW_CHUNK[name])
        torch.cuda.synchronize()
        del dw
        torch.cuda.empty_cache()
        log(f"[bench] traffic probe: {name} fused call")
    for name in PROBE:
        pw = p if name == "glm_chunk" else synth.make_config(name)
        dw = d if name == "glm_chunk" else idx.Inputs.from_host(pw, device=dev)
        r0, nr, kb, nk = max(launch_rects(dw, pw.meta["block_k"], ROW_CHUNK[name], pw.meta["K"]),
                             key=lambda r: r[1] * r[3])
        scratch = torch.empty((nr, nk + 64), dtype=torch.float32, device=dev)[:, :nk]
        for rep in range(2):
            idx.idx_mqa_logits_block(dw, r0, nr, kb, nk, out=scratch)
        torch.cuda.synchronize()
        del scratch
        log(f"[bench] traffic probe: {name} scoring rectangle {nr} rows x {nk} keys at ({r0}, {kb}), twice")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for rep in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] traffic probe: 2 copies of {COPY_BYTES} bytes")


def traffic_summary(fetch_dir, write_dir):
    """Per-launch HBM bytes of the scoring kernel (the probe's last two launches of each workload)
    from two traffic-probe counter runs, each counter scaled by what it reads for the calibration
    copy; updates profiles/logits_hbm_traffic.json and prints a markdown summary."""
    import csv
    import re

    def read(dirname, counter):
        acc = {}
        for r in csv.DictReader(open(os.path.join(dirname, "run_counter_collection.csv"))):
            if r["Counter_Name"] == counter:
                k = int(r["Dispatch_Id"])
                n, v, t0, t1 = acc.get(k, (r["Kernel_Name"], 0.0, int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
                acc[k] = (n, v + float(r["Counter_Value"]) * 1024.0, t0, t1)   # KiB -> bytes, summed over instances
        return [acc[k] for k in sorted(acc)]

    rows = {c: read(dn, c) for c, dn in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir))}
    factor = {}
    for c, rs in rows.items():
        cp = [v for n, v, _, _ in rs if "copyBuffer" in n]
        factor[c] = COPY_BYTES / max(cp[-2:])           # the probe's last two dispatches are the calibration copies
    path = os.path.join(ROOT, "profiles", "logits_hbm_traffic.json")
    try:
        with open(path) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    print("| workload | launches | rows x keys | FETCH_SIZE factor | WRITE_SIZE factor | fetched MiB per launch | "
          "written MiB per launch | HBM MiB per launch (mean) |")
    print("|---|---|---|---|---|---|---|---|")
    allrec = {k: v for k, v in allrec.items() if "/" in k}   # entries keyed workload/mode only
    cases = [(name, "block", kname, 2) for name, kname in PROBE.items()] + \
            [(name, "slab", kname, None) for name, kname in SLAB_PROBE.items()]
    for name, mode, kname, last in cases:
        f = launch_pairs([v * factor["FETCH_SIZE"] for n, v, _, _ in rows["FETCH_SIZE"] if kname in n])
        w = launch_pairs([v * factor["WRITE_SIZE"] for n, v, _, _ in rows["WRITE_SIZE"] if kname in n])
        if last:
            f, w = f[-last:], w[-last:]
        p = synth.make_config(name)
        Tc = p.T if ROW_CHUNK[name] <= 0 else min(ROW_CHUNK[name], p.T)
        kl = key_launches(p.L, p.meta["block_k"], p.meta["K"])
        nb = block_launches(p.L, p.meta["block_k"], p.meta["K"])
        rect = [Tc, max(nk for _, nk in (kl if mode == "block" else kl[nb:]))]
        rec = {"kernel_source_hash": kernel_source_hash(), "rect": rect,
               "bytes_per_launch": float(np.mean(f) + np.mean(w)), "fetch_bytes_per_launch": float(np.mean(f)),
               "write_bytes_per_launch": float(np.mean(w)), "fetch_factor": factor["FETCH_SIZE"],
               "write_factor": factor["WRITE_SIZE"], "launches": len(f)}
        allrec[f"{name}/{mode}"] = rec
        fs = ", ".join(f"{x / 2**20:.1f}" for x in f) if len(f) <= 4 else \
            f"{min(f) / 2**20:.1f}-{max(f) / 2**20:.1f} ({len(f)} launches)"
        ws_ = ", ".join(f"{x / 2**20:.1f}" for x in w) if len(w) <= 4 else \
            f"{min(w) / 2**20:.1f}-{max(w) / 2**20:.1f} ({len(w)} launches)"
        print(f"| {name} | {mode} | {rect[0]} x {rect[1]} | {factor['FETCH_SIZE']:.4f} | {factor['WRITE_SIZE']:.4f} | "
              f"{fs} | {ws_} | {rec['bytes_per_launch'] / 2**20:.1f} |")
    with open(path, "w") as fo:
        json.dump(allrec, fo, indent=1)
    print(f"\nKernel source hash {kernel_source_hash()}.")
    # the other kernels of the probe: bytes per dispatch and the rate over its (profiled) duration
    groups = {}
    nkb = 0
    # the fused calls and the candidate source end with their last refinement; the key-block
    # rectangles and the copies follow
    last_ref = max(i for i, (n, _, _, _) in enumerate(rows["FETCH_SIZE"]) if "refine_kernel" in n)
    for i, ((n, fv, t0, t1), (_, wv, _, _)) in enumerate(zip(rows["FETCH_SIZE"], rows["WRITE_SIZE"])):
        if i > last_ref:
            break
        m = re.search(r"namespace\)::(\w+(?:<[^>]*>)?)", n)
        name = m.group(1) if m else n.split("(")[0]
        if name.startswith("key_bound_kernel"):
            nkb += 1
        wl = PROBE_CALLS[min(max(nkb, 1), len(PROBE_CALLS)) - 1]
        if not (n.startswith("void idx") or n.startswith("idx::")):
            continue
        g = groups.setdefault((wl, name), [0, 0.0, 0.0, 0.0])
        g[0] += 1
        g[1] += fv * factor["FETCH_SIZE"]
        g[2] += wv * factor["WRITE_SIZE"]
        g[3] += (t1 - t0) * 1e-9
    print("\n| workload | kernel | dispatches | fetched MiB per dispatch | written MiB per dispatch | us per dispatch | GB/s |")
    print("|---|---|---|---|---|---|---|")
    for (w_, name), (cnt, fb, wb, t) in sorted(groups.items(), key=lambda x: (x[0][0], -x[1][3])):
        print(f"| {w_} | {name} | {cnt} | {fb / cnt / 2**20:.1f} | {wb / cnt / 2**20:.1f} | {t / cnt * 1e6:.1f} | "
              f"{(fb + wb) / t / 1e9:.0f} |")


def mfma_summary(pmc_dir):
    """Markdown summary of a traffic-probe run under rocprofv3 --pmc with MFMA_COUNTERS: for the
    last two key-block and candidate-slab scoring launches of each probed workload, the issued
    MFMA work, MFMA-busy cycles,
    VALU instructions and the shader clock (GRBM_COUNT over the dispatch's duration, 8 XCDs)."""
    import csv
    acc = {}
    for r in csv.DictReader(open(os.path.join(pmc_dir, "run_counter_collection.csv"))):
        k = int(r["Dispatch_Id"])
        e = acc.setdefault(k, {"name": r["Kernel_Name"], "t": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [acc[k] for k in sorted(acc)]
    cols = ("SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_VALU_MFMA_BUSY_CYCLES",
            "SQ_INSTS_VALU", "GRBM_COUNT")
    print("| workload | launches | form | duration us | " + " | ".join(cols) + " | clock GHz | MFMA busy | VALU per MFMA |")
    print("|---|---|---|---|" + "---|" * (len(cols) + 3))
    cases = [(name, "block", kname) for name, kname in PROBE.items()] + \
            [(name, "slab", kname) for name, kname in SLAB_PROBE.items()]
    for name, mode, kname in cases:
        ds = [e for e in disp if kname in e["name"]][-4:]
        for e in ds:
            cyc = e.get("GRBM_COUNT", 0.0) / 8.0                      # per XCD
            busy = e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / 1024.0    # per SIMD
            form = "f16" if "true>" in e["name"] else "fp32"
            print(f"| {name} | {mode} | {form} | {e['t'] * 1e6:.1f} | " + " | ".join(f"{e.get(c, 0.0):.4g}" for c in cols)
                  + f" | {cyc / e['t'] / 1e9 if e['t'] > 0 else 0:.2f} | {busy / cyc if cyc else 0:.3f} | "
                  f"{e.get('SQ_INSTS_VALU', 0.0) / max(1.0, e.get('SQ_INSTS_MFMA', 0.0)):.2f} |")


def _short_kernel(n):
    import re
    m = re.search(r"namespace\)::(\w+(?:<[^>]*>)?)", n)
    return m.group(1) if m else n.split("(")[0][:48]


def trace_summary(trace_dir, slab="logits_kernel<0, 64, 4, 4, ", scoring="logits_kernel<0, 64, 1, 4, "):
    """Markdown summary of a rocprofv3 --kernel-trace run of the default headline bench: each
    fused step (from its window kernel to its last refinement) by kernel, the fused steps'
    candidate-slab launches (the roofline's launches), then the block-store scoring launches
    over the step's rectangles; a launch is the pair (f16 form, fp32 form) of dispatches."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    ev = [(_short_kernel(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    ours = ("logits", "topk", "merge", "refine", "slab", "key_bound")
    steps, i = [], 0
    while i < len(ev):
        if not ev[i][0].startswith("ragged_kernel"):
            i += 1
            continue
        k = i
        while k + 1 < len(ev) and ev[k + 1][0].startswith(ours):
            k += 1
        if any(n.startswith("refine_kernel") for n, _, _ in ev[i:k + 1]):   # a whole fused step
            steps.append(ev[i:k + 1])
        i = k + 1
    if len(steps) > 1:
        steps = steps[1:]   # the warm-up step
    print(f"{len(steps)} fused steps after the warm-up (each from its window kernel to its last refinement)\n")
    if steps:
        names = []
        for st in steps:
            for n, _, _ in st:
                if n not in names:
                    names.append(n)
        print("| kernel | dispatches per step | mean us per dispatch | us per step |")
        print("|---|---|---|---|")
        for n in names:
            per = [[(b - a) / 1e3 for m, a, b in st if m == n] for st in steps]
            allv = [x for v in per for x in v]
            print(f"| `{n}` | {len(allv) / len(steps):.0f} | {np.mean(allv):.1f} | {np.mean([sum(v) for v in per]):.0f} |")
        spans = [(st[-1][2] - st[0][1]) / 1e3 for st in steps]
        busy = [sum(b - a for _, a, b in st) / 1e3 for st in steps]
        print("\nstep spans (us): " + ", ".join(f"{x:.0f}" for x in spans)
              + "; kernel time per step (us): " + ", ".join(f"{x:.0f}" for x in busy))
        sp = [(st[j + 1][2] - st[j][1]) / 1e3 for st in steps for j in range(len(st) - 1)
              if st[j][0] == slab + "true>" and st[j + 1][0] == slab + "false>"]
        f16 = [(b - a) / 1e3 for st in steps for n, a, b in st if n == slab + "true>"]
        if sp:
            print(f"\nslab launches of the fused steps: {len(sp)} launches of `{slab}...>`: f16 form mean "
                  f"{np.mean(f16):.1f} us, launch (first start to second end) mean {np.mean(sp):.1f} us, "
                  f"median {np.median(sp):.1f} us")
    # roofline: runs of consecutive block-store scoring dispatches
    runs, cur = [], []
    for n, a, b in ev:
        if n.startswith(scoring):
            cur.append((n, a, b))
        else:
            if len(cur) >= 16:
                runs.append(cur)
            cur = []
    if len(cur) >= 16:
        runs.append(cur)
    for r in runs:
        f16 = [(b - a) / 1e3 for n, a, b in r if n.endswith("true>")]
        f32 = [(b - a) / 1e3 for n, a, b in r if n.endswith("false>")]
        pairs = [(r[j + 1][2] - r[j][1]) / 1e3 for j in range(0, len(r) - 1, 2)
                 if r[j][0].endswith("true>") and r[j + 1][0].endswith("false>")]
        print(f"\nblock-store run: {len(pairs)} launches of `{scoring}...>`: f16 form mean {np.mean(f16):.1f} us "
              f"(median {np.median(f16):.1f}), fp32 form mean {np.mean(f32):.1f} us, launch (first start to "
              f"second end) mean {np.mean(pairs):.1f} us, median {np.median(pairs):.1f} us")


def extras(dev, stream, glm, dsv4):
    """Measurements beside the headline: logits-stage variants at the DeepSeek-V4-like shape, the
    row-chunked dense comparator at long context (and on two streams at glm_chunk), the workspace
    against L, the index -> slot transform and the ragged candidate source with its consumers."""
    ex = {}
    p3, d3, _, _ = dsv4
    # the logits stage at T=2048, L=102400 scored in one launch over all keys (the dense path's stage)
    scratch = torch.empty((d3.T, d3.L), dtype=torch.float32, device=dev)
    run = lambda: idx.idx_mqa_logits_block(d3, 0, d3.T, 0, d3.L, out=scratch, stream=stream)
    run()
    ms = float(np.median(time_events(run, 5, stream)))
    fl = 2 * d3.H * 128 * d3.pairs
    ex["dsv4_mxfp4_logits_one_launch"] = {"ms": ms, "tflops": fl / (ms * 1e-3) / 1e12,
                                          "fp8_peak_frac": fl / (ms * 1e-3) / FP8_PEAK}
    log(f"[bench] dsv4_mxfp4 logits in one launch: {ms:.4f} ms, {100 * fl / (ms * 1e-3) / FP8_PEAK:.1f}% of fp8 peak")
    del scratch
    # the same shape with fp8 keys
    p4 = synth.make_problem(2048, 102400, 64, k_fmt=synth.K_FP8)
    d4 = idx.Inputs.from_host(p4, device=dev)
    ex["c3_shape_fp8_logits_stage"] = scoring_roofline(d4, 32768, 0, 512, 3, stream, "c3_shape_fp8")
    log(f"[bench] T=2048 L=102400 H=64 fp8 scoring {ex['c3_shape_fp8_logits_stage']['achieved']:.1f} TFLOP/s")
    del d4
    # workspace of the fused path at the long-context shape, against L: flat
    lib = idx.load_library()
    flat = {}
    for L in (65536, 131072, 262144, 487936):
        s_ = idx.idx_problem(q=1 << 20, q_scale=1 << 20, k=1 << 20, k_scale=1 << 20, k_fmt=0, w=1 << 20,
                             ks=1 << 20, ke=1 << 20, T=16384, H=64, D=128, L=L, scale=1.0)
        n_ = ctypes.c_size_t(0)
        lib.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, ctypes.byref(s_), 512, 32768, 4096, 0, 0, 0,
                               ctypes.byref(n_))
        flat[str(L)] = int(n_.value)
    ex["long_ctx_workspace_bytes_by_L"] = flat
    # two-stream overlap of the dense row-chunked comparator (glm_chunk shapes, 512-row chunks)
    pg, dg, lg, (goi, gov, gws) = glm
    Kg = pg.meta["K"]
    rc = RowChunkedDense(dg, Kg, 512)
    outs = {m: (torch.empty((dg.T, Kg), dtype=torch.int32, device=dev),
                torch.empty((dg.T, Kg), dtype=torch.float32, device=dev)) for m in ("serial", "piped")}
    side = torch.cuda.Stream()
    rc.run(*outs["serial"], stream)
    rc.run(*outs["piped"], stream, side)
    torch.cuda.synchronize()
    assert torch.equal(outs["serial"][0], outs["piped"][0]) and torch.equal(outs["serial"][0], goi)
    ts = float(np.median(time_events(lambda: rc.run(*outs["serial"], stream), 3, stream)))
    tp = float(np.median(time_events(lambda: rc.run(*outs["piped"], stream, side), 3, stream)))
    ex["dense_rowchunk_overlap"] = {"rows_per_chunk": 512, "serial_ms": ts, "two_stream_ms": tp, "gain": ts / tp - 1.0}
    log(f"[bench] glm_chunk dense row-chunked comparator: serial {ts:.3f} ms, two streams {tp:.3f} ms")
    del rc, outs
    # index -> KV-slot transform in the final write (glm_chunk)
    table = torch.randperm(2 * dg.L, device=dev)[:dg.L].to(torch.int32)
    tf = time_events(lambda: idx.idx_logits_topk_fused(dg, Kg, block_k=32768, out_idx=goi, out_val=gov, ws=gws,
                                                       stream=stream), 5, stream)
    tpg = time_events(lambda: idx.idx_logits_topk_fused_paged(dg, Kg, table, block_k=32768, out_idx=goi,
                                                              out_val=gov, ws=gws, stream=stream), 5, stream)
    ex["paged_transform"] = {"fused_ms": float(np.median(tf)), "fused_paged_ms": float(np.median(tpg))}
    return ex


def ragged_extras(dev, stream, rag):
    """Candidate source and its consumers on the ragged batch: every row vs each request's tail rows,
    byte-mask consumer vs block-list consumer."""
    p5, d5, _, _ = rag
    c5 = p5.meta
    W5, nb5, pool5, K5, bk5 = d5.W, c5["n_blocks"], c5["pool"], c5["K"], c5["block_k"]
    RC5 = ROW_CHUNK["ragged_cand"]
    blocks5 = torch.empty((d5.T, nb5), dtype=torch.int32, device=dev)
    ws5 = torch.empty(idx.idx_workspace_size(idx.IDX_OP_BLOCK_CANDIDATES, d5, block_k=bk5, row_chunk=RC5,
                                             pool=pool5, n_blocks=nb5), dtype=torch.uint8, device=dev)
    mask5 = torch.empty((d5.T, W5), dtype=torch.uint8, device=dev)
    cand_all = time_events(lambda: idx.idx_block_candidates(d5, W5, pool=pool5, n_blocks=nb5, block_k=bk5,
                                                            row_chunk=RC5, mask=mask5, out_blocks=blocks5,
                                                            ws=ws5, stream=stream), 3, stream)
    tail = idx.idx_tail_rows(torch.from_numpy(p5.cu_q).to(dev), 512)
    d5t = idx.idx_gather_rows(d5, tail)
    mask5t = torch.empty((d5t.T, W5), dtype=torch.uint8, device=dev)
    cand_tail = time_events(lambda: idx.idx_block_candidates(d5t, W5, pool=pool5, n_blocks=nb5, block_k=bk5,
                                                             row_chunk=RC5, mask=mask5t, ws=ws5, stream=stream),
                            3, stream)
    p5c = synth.consumer_layer(p5)
    d5c = idx.Inputs.from_host(p5c, device=dev)
    wsc = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d5c, K=K5, block_k=bk5, row_chunk=RC5),
                      dtype=torch.uint8, device=dev)
    cons_mask = time_events(lambda: idx.idx_logits_topk_fused(d5c, K5, block_k=bk5, row_chunk=RC5, mask=mask5,
                                                              ws=wsc, stream=stream), 3, stream)
    cons_blocks = time_events(lambda: idx.idx_logits_topk_fused_blocks(d5c, K5, blocks5, pool=pool5, block_k=bk5,
                                                                       row_chunk=RC5, ws=wsc, stream=stream),
                              3, stream)
    out = {"all_rows": {"rows": d5.T, "ms": float(np.median(cand_all)), "mask_bytes": int(mask5.numel())},
           "tail_rows_512": {"rows": int(d5t.T), "ms": float(np.median(cand_tail)), "mask_bytes": int(mask5t.numel())},
           "consumer_byte_mask_ms": float(np.median(cons_mask)),
           "consumer_block_ids_ms": float(np.median(cons_blocks)), "block_ids_bytes": int(blocks5.numel() * 4)}
    log(f"[bench] ragged candidates: all rows {np.median(cand_all):.2f} ms, tail rows {np.median(cand_tail):.2f} ms; "
        f"consumer: byte mask {np.median(cons_mask):.2f} ms, block ids {np.median(cons_blocks):.2f} ms")
    return out


def long_ctx_dense(dev, stream, line, p, d, oi, ov):
    """The row-chunked dense comparator under a 2 GiB fp32 logits budget at long context."""
    K = p.meta["K"]
    rows = rows_for_budget(d.W, 2 << 30)
    rc = RowChunkedDense(d, K, rows)
    di = torch.empty((d.T, K), dtype=torch.int32, device=dev)
    dv = torch.empty((d.T, K), dtype=torch.float32, device=dev)
    ms = float(np.median(time_events(lambda: rc.run(di, dv, stream), 1, stream)))
    assert torch.equal(di, oi) and torch.equal(dv.view(torch.int32), ov.view(torch.int32))
    out = {"rows_per_chunk": int(rows), "chunks": len(rc.chunks), "ms": ms, "pairs_per_s": d.pairs / (ms * 1e-3),
           "peak_transient_bytes": rc.peak_transient_bytes(False), "equal_to_fused": True}
    log(f"[bench] long_ctx row-chunked dense comparator ({rows} rows x {d.W} fp32 per chunk): {ms:.1f} ms, "
        f"equal to the fused result")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle wall time for cpu_baseline")
    ap.add_argument("--cpu-workers", type=int, default=0, help="host threads for cpu_baseline (0: up to 16)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", default="", help="comma-separated workloads to time (skips the rest)")
    ap.add_argument("--traffic-probe", action="store_true", help="only the launches for a counter run")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two traffic-probe counter runs (no GPU)")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="summarise a traffic-probe run with the MFMA counters (no GPU)")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="summarise a rocprofv3 --kernel-trace run of the headline bench (no GPU)")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the indexer shards by "
              f"query rows with no exchange, see the design notes)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    for var in ("IDX_EXACT", "IDX_DEBUG"):   # the benchmark times the default path
        if os.environ.pop(var, None) not in (None, "", "0"):
            log(f"[bench] {var} ignored: the benchmark times the default path")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.traffic_probe:
        traffic_probe(dev)
        return
    only = set(filter(None, args.only.split(",")))

    p, d, line, (oi, ov, ws) = workload(HEADLINE, dev, stream, args.steps, args.warmup, 1)
    roof = line.pop("roofline")
    out = {"metric": METRIC, "value": line["pairs_per_s"], "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": line["ms"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8", "data": "synthetic (seeded N(0,1) q/k quantised to fp8, w U(0,1))",
           "config": {"workload": DESCRIBE[HEADLINE], "T": d.T, "L": d.L, "H": d.H, "D": 128, "K": line["K"],
                      "block_k": line["block_k"], "row_chunk": line["row_chunk"], "pairs_per_step": line["pairs"]},
           "tflops": line["tflops"], "fp8_peak_frac_step": line["fp8_peak_frac_step"],
           "peak_transient_bytes": line["peak_transient_bytes"], "roofline": roof}
    out["peak_transient_check"] = peak_check(d, line["K"], line["block_k"], line["row_chunk"], stream)
    extra = {"workloads": {HEADLINE: line}}
    if not args.no_extra:
        extra["long_ctx_dense_rowchunked"] = long_ctx_dense(dev, stream, line, p, d, oi, ov)
    g_idx = oi.cpu().numpy()
    del d, oi, ov, ws
    torch.cuda.empty_cache()

    if not args.no_extra:
        keep = {}
        for name in ("tiny", "glm_chunk", "dsv4_mxfp4", "ragged_cand"):
            if only and name not in only:
                continue
            reps = 0 if name == "tiny" else (3 if name != "ragged_cand" else 1)
            res = workload(name, dev, stream, 10 if name != "ragged_cand" else 3, 2, reps)
            extra["workloads"][name] = res[2]
            keep[name] = res
            if name == "ragged_cand":
                extra["ragged_candidates"] = ragged_extras(dev, stream, res)
                del keep[name]
                torch.cuda.empty_cache()
        if "glm_chunk" in keep and "dsv4_mxfp4" in keep:
            extra.update(extras(dev, stream, keep["glm_chunk"], keep["dsv4_mxfp4"]))
        if "dsv4_mxfp4" in keep:
            r = keep["dsv4_mxfp4"][2]["roofline"]
            extra["logits_stage_target"] = {
                "shape": "T=2048 L=102400 H=64 MXFP4 keys (dsv4_mxfp4), the fused path's scoring launches",
                "tflops": r["achieved"], "fp8_peak_frac": r["frac"], "target_frac": 0.5}
        del keep
        torch.cuda.empty_cache()
    out["extra"] = extra

    if not args.no_cpu:
        workers = args.cpu_workers or max(1, min(16, os.cpu_count() or 1))
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_budget:.0f} s on {workers} threads)")
        out["cpu_baseline"] = cpu_baseline(p, line["K"], g_idx, args.cpu_budget, workers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
