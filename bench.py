"""Benchmark of the dense prefill indexer on one MI355X.

A step is one pass of the indexer's hot path over one batch: the per-row key
windows are built from the batch's cu_seqlens on the device, then the fused
key-blocked logits + top-K runs (scoring on fp8 MFMA with the ReLU-weighted
head sum in registers, per-block exact top-K with a running merge, exact
boundary refinement).  Workload: the GLM-5.1-shaped chunk, T = 2048 query rows
against L = 65536 keys, H = 32, D = 128, fp8 q and k with per-row scales, causal
windows, K = 2048, key blocks of 32768 (the pages' H200 microbenchmark shape).

Printed: one JSON line.  value = scored in-window (row, key) pairs per second
(inputs resident in HBM).  roofline: the scoring kernel's algorithmic fp8
FLOPs (2 H D per in-window pair) per launch over its average launch duration
(HIP events on the launch stream) against the fp8 dense MFMA peak.
cpu_baseline: the fp64 CPU oracle on a bounded row sample of the same
workload.  Extra fields: the MXFP4 logits stage at T = 2048, L = 102400, H = 64
and the ragged candidate-source pipeline.
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
import synth  # noqa: E402

METRIC = "indexer (row,key) pairs/s fused logits+top-K; % fp8 MFMA peak; peak bytes"
FP8_PEAK = 5.0e15      # MI355X dense fp8 MFMA, FLOP/s
HBM_PEAK = 8.0e12


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def block_pairs(p, kb, nk):
    lo = np.maximum(p.ks.astype(np.int64), kb)
    hi = np.minimum(p.ke.astype(np.int64), kb + nk)
    return int(np.maximum(hi - lo, 0).sum())


def kernel_source_hash():
    """Hash of the scoring kernel's code (logits.hip and the LogitsArgs struct; comments and
    blank lines excluded), to tell whether committed counter figures were taken on the kernel
    as it stands."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mqa_logits_top_amd", "csrc")
    with open(os.path.join(csrc, "logits.hip")) as fh:
        text = fh.read()
    with open(os.path.join(csrc, "kernels.h")) as fh:
        hdr = fh.read()
    a = hdr.index("struct LogitsArgs {")
    text += hdr[a:hdr.index("};", a)]
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic(workload, keys_per_launch):
    """HBM bytes per scoring launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source and launch size."""
    path = os.path.join(ROOT, "profiles", "logits_hbm_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
        e = d.get(workload)
        if e and e.get("kernel_source_hash") == kernel_source_hash() and e.get("keys_per_launch") == keys_per_launch:
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


def launch_keys(L, block_k):
    """Keys per scoring launch of the fused path: key blocks go in pairs."""
    return max(block_k, min(2 * block_k, (L + 255) // 256 * 256))


def launch_scratch(T, nkeys):
    """A [T, nkeys] view with the fused path's row pitch (64 floats past the row)."""
    return torch.empty((T, nkeys + 64), dtype=torch.float32, device="cuda")[:, :nkeys]


def scoring_launch_ms(p, d, block_k, reps, stream):
    """Average duration of the scoring kernel as the fused path launches it (key-block layout,
    two key blocks per launch): reps x (one launch per key range), back to back on `stream`
    between one pair of events."""
    lk = launch_keys(p.L, block_k)
    scratch = launch_scratch(p.T, lk)
    blocks = [(kb, min(lk, p.L - kb)) for kb in range(0, p.L, lk)]

    def run():
        for _ in range(reps):
            for kb, nk in blocks:
                idx.idx_mqa_logits_block(d, 0, p.T, kb, nk, out=scratch, stream=stream)

    run()  # warm
    t = time_events(run, 3, stream)
    flops = sum(2 * p.H * p.D * block_pairs(p, kb, nk) for kb, nk in blocks)
    del scratch
    avg_ms = float(np.median(t)) / (reps * len(blocks))
    return avg_ms, flops / len(blocks), len(blocks)


def dense_rowchunk_overlap(p, d, K, rows, stream):
    """The dense row-chunked comparator (logits of `rows` rows, then top-(K + 512) and the exact
    boundary) run serially on one stream and pipelined on two: chunk n + 1's logits on the main
    stream while chunk n's selection runs on a side stream (both default priority), logits
    double buffered and event-gated.  Returns (serial ms, pipelined ms); outputs must agree."""
    W = p.W
    Kc = idx.candidate_capacity(K)
    side = torch.cuda.Stream()
    bufs = [launch_scratch(rows, W) for _ in range(2)]
    chunks = [(r0, min(rows, p.T - r0)) for r0 in range(0, p.T, rows)]
    sub = lambda r0, n: idx.Inputs(q=d.q[r0:r0 + n], q_scale=d.q_scale[r0:r0 + n], k=d.k, k_scale=d.k_scale,
                                   w=d.w[r0:r0 + n], ks=d.ks[r0:r0 + n], ke=d.ke[r0:r0 + n], k_fmt=d.k_fmt)
    outs = {m: (torch.empty((p.T, K), dtype=torch.int32, device="cuda"),
                torch.empty((p.T, K), dtype=torch.float32, device="cuda")) for m in ("serial", "piped")}
    cand = [(torch.empty((rows, Kc), dtype=torch.int32, device="cuda"),
             torch.empty((rows, Kc), dtype=torch.float32, device="cuda")) for _ in range(2)]
    rws = [torch.empty(idx.REFINE_WS, dtype=torch.uint8, device="cuda") for _ in range(2)]

    def select(i, r0, n, sp, st):
        lg = bufs[i % 2][:n]
        ci, cv = cand[i % 2]
        idx.idx_topk(lg, sp.ks, sp.ke, Kc, W=W, out_idx=ci[:n], out_val=cv[:n], stream=st)
        oi, ov = outs["piped" if st is side else "serial"]
        idx.idx_refine_topk(sp, ci[:n], cv[:n], K, out_idx=oi[r0:r0 + n], out_val=ov[r0:r0 + n], ws=rws[i % 2],
                            stream=st)

    def serial():
        for i, (r0, n) in enumerate(chunks):
            sp = sub(r0, n)
            idx.idx_mqa_logits(sp, W, out=bufs[i % 2][:n], stream=stream)
            select(i, r0, n, sp, stream)

    def piped():
        done = [None, None]                   # selection of the chunk that last used each buffer
        for i, (r0, n) in enumerate(chunks):
            sp = sub(r0, n)
            if done[i % 2] is not None:
                stream.wait_event(done[i % 2])
            idx.idx_mqa_logits(sp, W, out=bufs[i % 2][:n], stream=stream)
            ready = torch.cuda.Event()
            ready.record(stream)
            side.wait_event(ready)
            select(i, r0, n, sp, side)
            done[i % 2] = torch.cuda.Event()
            done[i % 2].record(side)
        stream.wait_event(done[(len(chunks) - 1) % 2])

    serial(); piped()
    torch.cuda.synchronize()
    ts = float(np.median(time_events(serial, 3, stream)))
    tp = float(np.median(time_events(piped, 3, stream)))
    assert torch.equal(outs["serial"][0], outs["piped"][0])
    return ts, tp


def cpu_baseline(p, K, budget_s):
    """The fp64 oracle (numpy, BLAS threads as configured) on a bounded row sample."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    t0 = time.perf_counter()
    dq = oracle.Dequantised(p)
    setup = time.perf_counter() - t0
    order = np.random.default_rng(0).permutation(p.T)
    pairs = 0
    rows = 0
    t1 = time.perf_counter()
    for t in order:
        v = oracle.row_logits(dq, int(t))
        oracle.topk_row(v, int(p.ks[t]), K)
        pairs += len(v)
        rows += 1
        if time.perf_counter() - t1 > budget_s and rows >= 4:
            break
    el = time.perf_counter() - t1
    single = None
    try:  # one BLAS thread, a few rows
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t2 = time.perf_counter()
            sp = 0
            sel = order[rows:rows + 4] if rows + 4 <= len(order) else order[:4]   # whole sample done: reuse rows
            for t in sel:
                v = oracle.row_logits(dq, int(t))
                oracle.topk_row(v, int(p.ks[t]), K)
                sp += len(v)
            single = sp / (time.perf_counter() - t2)
    except Exception:  # pragma: no cover
        pass
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": pairs / el, "unit": "pairs/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {p.T} rows (random order, seed 0), full windows, logits + top-{K}; "
                      f"{pairs} pairs in {el:.1f} s (+{setup:.1f} s dequantisation, not counted)",
            "single_core_value": single, "cpu_model": model, "host_cpus": os.cpu_count()}


COPY_BYTES = 256 << 20   # calibration copy of the traffic probe


def traffic_probe(dev):
    """Launches for a rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE run: one fused glm_chunk call and
    the ragged workload's candidate source (the selection, refinement, pooling and mask kernels),
    then the scoring kernel on the glm_chunk key blocks (as the fused path launches it) twice, then
    two device-to-device copies of COPY_BYTES that calibrate what those counters read for a known
    number of bytes."""
    p = synth.make_config("glm_chunk")
    d = idx.Inputs.from_host(p, device=dev)
    K, Bk = p.meta["K"], p.meta["block_k"]
    idx.idx_logits_topk_fused(d, K, block_k=Bk)
    p5 = synth.make_config("ragged_cand")
    c5 = p5.meta
    d5 = idx.Inputs.from_host(p5, device=dev)
    blocks5 = torch.empty((p5.T, c5["n_blocks"]), dtype=torch.int32, device=dev)
    idx.idx_block_candidates(d5, p5.W, pool=c5["pool"], n_blocks=c5["n_blocks"], block_k=c5["block_k"],
                             row_chunk=4096, out_blocks=blocks5)
    torch.cuda.synchronize()
    del d5, blocks5
    torch.cuda.empty_cache()
    lk = launch_keys(p.L, p.meta["block_k"])
    scratch = launch_scratch(p.T, lk)
    for rep in range(2):
        for kb in range(0, p.L, lk):
            idx.idx_mqa_logits_block(d, 0, p.T, kb, min(lk, p.L - kb), out=scratch)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for rep in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] traffic probe: {2 * ((p.L + lk - 1) // lk)} scoring launches, 2 copies of {COPY_BYTES} bytes")


def traffic_summary(fetch_dir, write_dir):
    """Per-launch HBM bytes of the glm_chunk scoring kernel from two traffic-probe counter runs,
    each scaled by what the same counter reads for the calibration copy; writes
    profiles/logits_hbm_traffic.json and prints a markdown summary."""
    import csv

    def read(dirname, counter):
        acc = {}
        for r in csv.DictReader(open(os.path.join(dirname, "run_counter_collection.csv"))):
            if r["Counter_Name"] == counter:
                k = int(r["Dispatch_Id"])
                n, v, t0, t1 = acc.get(k, (r["Kernel_Name"], 0.0, int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
                acc[k] = (n, v + float(r["Counter_Value"]) * 1024.0, t0, t1)   # KiB -> bytes, summed over instances
        return [acc[k] for k in sorted(acc)]

    out = {}
    per_dispatch = {}
    for counter, dirname in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = read(dirname, counter)
        per_dispatch[counter] = rows
        lk = [v for n, v, _, _ in rows if "logits_kernel<0, 32, 1, 4>" in n]
        cp = [v for n, v, _, _ in rows if "copyBuffer" in n]
        calib = max(cp[-2:])                 # the probe's last two dispatches are the 256 MiB calibration copies
        factor = COPY_BYTES / calib
        out[counter] = {"raw_per_launch": lk, "copy_raw": calib, "factor": factor,
                        "bytes_per_launch": [v * factor for v in lk]}
    fetch, write = out["FETCH_SIZE"], out["WRITE_SIZE"]
    nl = min(len(fetch["bytes_per_launch"]), len(write["bytes_per_launch"]))
    per_launch = [fetch["bytes_per_launch"][i] + write["bytes_per_launch"][i] for i in range(nl)]
    avg = float(np.mean(per_launch))
    p = synth.make_config("glm_chunk")
    rec = {"kernel_source_hash": kernel_source_hash(), "keys_per_launch": launch_keys(p.L, p.meta["block_k"]),
           "bytes_per_launch": avg,
           "fetch_bytes_per_launch": float(np.mean(fetch["bytes_per_launch"])),
           "write_bytes_per_launch": float(np.mean(write["bytes_per_launch"])),
           "fetch_factor": fetch["factor"], "write_factor": write["factor"], "launches": nl}
    path = os.path.join(ROOT, "profiles", "logits_hbm_traffic.json")
    try:
        with open(path) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    allrec["glm_chunk"] = rec
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1)
    print("| counter | calibration copy read (bytes) | factor | scaled bytes per launch |")
    print("|---|---|---|---|")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        v = out[c]
        print(f"| {c} | {v['copy_raw']:.4g} | {v['factor']:.4f} | "
              + ", ".join(f"{x / 2**20:.1f} MiB" for x in v["bytes_per_launch"]) + " |")
    print(f"\nAverage HBM traffic per scoring launch: {avg / 2**20:.1f} MiB "
          f"(kernel source hash {rec['kernel_source_hash']}).")
    # the other kernels of the probe: bytes per dispatch and the rate over its (profiled) duration
    import re
    f_rows, w_rows = per_dispatch["FETCH_SIZE"], per_dispatch["WRITE_SIZE"]
    groups = {}
    workload = "glm_chunk fused"      # the probe's first call; the second key-bound launch starts the ragged one
    nkb = 0
    for (n, fv, t0, t1), (_, wv, _, _) in zip(f_rows, w_rows):
        m = re.search(r"namespace\)::(\w+(?:<[^>]*>)?)", n)
        name = m.group(1) if m else n.split("(")[0]
        if name.startswith("key_bound_kernel"):
            nkb += 1
            if nkb == 2:
                workload = "ragged_cand candidates"
        if name.startswith("logits_kernel<0, 32, 1, 4>") or "copyBuffer" in n or not n.startswith("void idx") and \
                not n.startswith("idx::"):
            continue
        g = groups.setdefault((workload, name), [0, 0.0, 0.0, 0.0])
        g[0] += 1
        g[1] += fv * out["FETCH_SIZE"]["factor"]
        g[2] += wv * out["WRITE_SIZE"]["factor"]
        g[3] += (t1 - t0) * 1e-9
    print("\n| workload | kernel | dispatches | fetched MiB per dispatch | written MiB per dispatch | us per dispatch | GB/s |")
    print("|---|---|---|---|---|---|---|")
    for (wl, name), (cnt, fb, wb, t) in sorted(groups.items(), key=lambda x: (x[0][0], -x[1][3])):
        print(f"| {wl} | {name} | {cnt} | {fb / cnt / 2**20:.1f} | {wb / cnt / 2**20:.1f} | {t / cnt * 1e6:.1f} | "
              f"{(fb + wb) / t / 1e9:.0f} |")


def fused_line(p, d, K, block_k, row_chunk, reps, stream):
    """One workload's fused call, timed with HIP events on `stream` after a warm-up call."""
    ws = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=K, block_k=block_k, row_chunk=row_chunk),
                     dtype=torch.uint8, device="cuda")
    oi = torch.empty((p.T, K), dtype=torch.int32, device="cuda")
    ov = torch.empty((p.T, K), dtype=torch.float32, device="cuda")
    run = lambda: idx.idx_logits_topk_fused(d, K, block_k=block_k, row_chunk=row_chunk, out_idx=oi, out_val=ov,
                                            ws=ws, stream=stream)
    run()
    ms = float(np.median(time_events(run, reps, stream)))
    flops = 2 * p.H * p.D * p.pairs
    assert idx.overflow_count(ws) == 0
    line = {"T": p.T, "L": p.L, "H": p.H, "K": K, "block_k": block_k, "row_chunk": row_chunk, "pairs": int(p.pairs),
            "ms": ms, "pairs_per_s": p.pairs / (ms * 1e-3), "tflops": flops / (ms * 1e-3) / 1e12,
            "fp8_peak_frac": flops / (ms * 1e-3) / FP8_PEAK, "peak_transient_bytes": int(ws.numel())}
    return line, oi, ov


def workload_lines(dev, stream):
    """The fused indexer on the tiny, long-context and ragged workloads (glm_chunk is the headline line,
    dsv4_mxfp4 is timed above), and on the long-context workload the row-chunked dense comparator under a
    2 GiB fp32 logits budget: logits of as many rows as fit, their top-(K + 512), then the exact boundary."""
    out = {}
    for name, row_chunk, reps in (("tiny", 0, 10), ("long_ctx", 4096, 3), ("ragged_cand", 4096, 3)):
        p = synth.make_config(name)
        d = idx.Inputs.from_host(p, device=dev)
        K, Bk = p.meta["K"], p.meta["block_k"]
        line, oi, ov = fused_line(p, d, K, Bk, row_chunk, reps, stream)
        out[name] = line
        log(f"[bench] {name}: fused {line['ms']:.3f} ms -> {line['pairs_per_s']:.3e} pairs/s, "
            f"{line['tflops']:.0f} TFLOP/s ({100 * line['fp8_peak_frac']:.1f}% of fp8 peak), "
            f"workspace {line['peak_transient_bytes'] / 2**20:.0f} MiB")
        if name == "long_ctx":
            W = p.W
            chunk = (2 << 30) // (4 * W)
            buf = torch.empty((chunk, W), dtype=torch.float32, device=dev)
            Kc = idx.candidate_capacity(K)
            ci = torch.empty((p.T, Kc), dtype=torch.int32, device=dev)
            cv = torch.empty((p.T, Kc), dtype=torch.float32, device=dev)
            rws = torch.empty(idx.REFINE_WS, dtype=torch.uint8, device=dev)
            di = torch.empty((p.T, K), dtype=torch.int32, device=dev)
            dv = torch.empty((p.T, K), dtype=torch.float32, device=dev)

            def dense():
                for r0 in range(0, p.T, chunk):
                    nr = min(chunk, p.T - r0)
                    sub = idx.Inputs(q=d.q[r0:r0 + nr], q_scale=d.q_scale[r0:r0 + nr], k=d.k, k_scale=d.k_scale,
                                     w=d.w[r0:r0 + nr], ks=d.ks[r0:r0 + nr], ke=d.ke[r0:r0 + nr], k_fmt=d.k_fmt)
                    lg = idx.idx_mqa_logits(sub, W, out=buf[:nr], stream=stream)
                    idx.idx_topk(lg, sub.ks, sub.ke, Kc, out_idx=ci[r0:r0 + nr], out_val=cv[r0:r0 + nr],
                                 stream=stream)
                idx.idx_refine_topk(d, ci, cv, K, out_idx=di, out_val=dv, ws=rws, stream=stream)

            ms = float(np.median(time_events(dense, 1, stream)))
            assert torch.equal(di, oi) and torch.equal(dv.view(torch.int32), ov.view(torch.int32))
            out[name]["dense_rowchunked"] = {"rows_per_chunk": int(chunk), "chunks": -(-p.T // chunk), "ms": ms,
                                             "pairs_per_s": p.pairs / (ms * 1e-3),
                                             "peak_transient_bytes": int(buf.numel() * 4 + 8 * p.T * Kc)}
            log(f"[bench] long_ctx: row-chunked dense comparator ({chunk} rows x {W} fp32 per chunk) {ms:.1f} ms, "
                f"equal to the fused result")
            del buf, ci, cv, rws, di, dv
        del d, oi, ov
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true", help="only the launches for a counter run")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two traffic-probe counter runs (no GPU)")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the indexer shards by "
              f"query rows with no exchange, see the design notes)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.traffic_probe:
        traffic_probe(dev)
        return

    name = "glm_chunk"
    p = synth.make_config(name)
    c = p.meta
    K, Bk = c["K"], c["block_k"]
    d = idx.Inputs.from_host(p, device=dev)
    cu_q = torch.tensor([0, p.T], dtype=torch.int32, device=dev)
    cu_k = torch.tensor([0, p.L], dtype=torch.int32, device=dev)
    ws = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=K, block_k=Bk), dtype=torch.uint8,
                     device=dev)
    out_idx = torch.empty((p.T, K), dtype=torch.int32, device=dev)
    out_val = torch.empty((p.T, K), dtype=torch.float32, device=dev)
    ks = torch.empty(p.T, dtype=torch.int32, device=dev)
    ke = torch.empty(p.T, dtype=torch.int32, device=dev)
    lib = idx.load_library()
    import ctypes
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step():
        # windows from cu_seqlens (one request: the chunk is the tail of its prefix), then the fused indexer
        st = lib.idx_ragged_windows(idx._ptr(cu_q), idx._ptr(cu_k), 1, p.T, idx._ptr(ks), idx._ptr(ke), sptr)
        assert st == 0
        dd = idx.Inputs(q=d.q, q_scale=d.q_scale, k=d.k, k_scale=d.k_scale, w=d.w, ks=ks, ke=ke, k_fmt=d.k_fmt)
        idx.idx_logits_topk_fused(dd, K, block_k=Bk, out_idx=out_idx, out_val=out_val, ws=ws, stream=stream)

    log(f"[bench] {name}: T={p.T} L={p.L} H={p.H} K={K} B_k={Bk} pairs={p.pairs}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert torch.equal(ks.cpu(), torch.from_numpy(p.ks)) and torch.equal(ke.cpu(), torch.from_numpy(p.ke))
    assert idx.overflow_count(ws) == 0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / args.steps
    value = p.pairs / (ms * 1e-3)
    log(f"[bench] fused step {ms:.4f} ms ({wall / args.steps * 1e3:.4f} ms wall) -> {value:.4e} pairs/s")

    # roofline of the dominant kernel (scoring), timed per launch on the launch stream
    avg_ms, flops_per_launch, nblk = scoring_launch_ms(p, d, Bk, max(args.steps // 2, 3), stream)
    achieved = flops_per_launch / (avg_ms * 1e-3)
    traffic = load_traffic(name, launch_keys(p.L, Bk))
    roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": FP8_PEAK / 1e12, "unit": "TFLOP/s",
            "frac": achieved / FP8_PEAK, "traffic": traffic,
            "kernel": "logits_kernel (fp8 keys, H=32, key-block store, two 32768-key blocks per launch)", "avg_launch_ms": avg_ms,
            "launches_per_step": nblk, "flop_per_launch": flops_per_launch}
    log(f"[bench] scoring kernel {avg_ms:.4f} ms/launch -> {achieved / 1e12:.1f} TFLOP/s "
        f"({100 * achieved / FP8_PEAK:.1f}% of fp8 peak)")

    peak_bytes = int(ws.numel())
    out = {"metric": METRIC, "value": value, "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8", "data": "synthetic (seeded N(0,1) q/k quantised to fp8, w U(0,1))",
           "config": {"workload": "glm_chunk: T=2048 L=65536 H=32 D=128 fp8 q/k per-row scales, causal windows, "
                                  "top-K=2048, fused key blocks B_k=32768",
                      "T": p.T, "L": p.L, "H": p.H, "D": p.D, "K": K, "block_k": Bk, "pairs_per_step": p.pairs},
           "tflops": 2 * p.H * p.D * p.pairs / (ms * 1e-3) / 1e12,
           "fp8_peak_frac_step": 2 * p.H * p.D * p.pairs / (ms * 1e-3) / FP8_PEAK,
           "peak_transient_bytes": peak_bytes,
           "roofline": roof}
    del ws

    if not args.no_extra:
        extra = {}
        # MXFP4-key logits stage at the DeepSeek-V4-like shape (T=2048, L=102400, H=64)
        p3 = synth.make_config("dsv4_mxfp4")
        d3 = idx.Inputs.from_host(p3, device=dev)
        a3, f3, n3 = scoring_launch_ms(p3, d3, p3.meta["block_k"], 3, stream)
        extra["dsv4_mxfp4_logits_stage"] = {"avg_launch_ms": a3, "tflops": f3 / (a3 * 1e-3) / 1e12,
                                            "fp8_peak_frac": f3 / (a3 * 1e-3) / FP8_PEAK}
        K3 = p3.meta["K"]
        ws3 = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d3, K=K3, block_k=p3.meta["block_k"]),
                          dtype=torch.uint8, device=dev)
        ft = time_events(lambda: idx.idx_logits_topk_fused(d3, K3, block_k=p3.meta["block_k"], ws=ws3,
                                                           stream=stream), 5, stream)
        extra["dsv4_mxfp4_fused"] = {"ms": float(np.median(ft)), "pairs_per_s": p3.pairs / (np.median(ft) * 1e-3),
                                     "peak_transient_bytes": int(ws3.numel())}
        log(f"[bench] dsv4_mxfp4 scoring {extra['dsv4_mxfp4_logits_stage']['tflops']:.1f} TFLOP/s, fused "
            f"{np.median(ft):.3f} ms")
        del d3, ws3
        # the same logits stage with fp8 keys (T=2048, L=102400, H=64)
        p4 = synth.make_problem(2048, 102400, 64, k_fmt=synth.K_FP8)
        d4 = idx.Inputs.from_host(p4, device=dev)
        a4, f4, _ = scoring_launch_ms(p4, d4, 32768, 3, stream)
        extra["c3_shape_fp8_logits_stage"] = {"avg_launch_ms": a4, "tflops": f4 / (a4 * 1e-3) / 1e12,
                                              "fp8_peak_frac": f4 / (a4 * 1e-3) / FP8_PEAK}
        log(f"[bench] T=2048 L=102400 H=64 fp8 scoring {extra['c3_shape_fp8_logits_stage']['tflops']:.1f} TFLOP/s")
        del d4
        # peak transient of the fused path at the long-context shape: flat in L
        flat = {}
        for L in (65536, 131072, 262144, 487936):
            s_ = idx.idx_problem(q=1 << 20, q_scale=1 << 20, k=1 << 20, k_scale=1 << 20, k_fmt=0, w=1 << 20,
                                 ks=1 << 20, ke=1 << 20, T=16384, H=64, D=128, L=L, scale=1.0)
            n_ = ctypes.c_size_t(0)
            lib.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, ctypes.byref(s_), 512, 32768, 4096,
                                   0, 0, 0, ctypes.byref(n_))
            flat[str(L)] = int(n_.value)
        extra["long_ctx_peak_transient_bytes_by_L"] = flat
        # two-stream overlap of the dense row-chunked comparator (glm_chunk shapes, 512-row chunks)
        ts, tp = dense_rowchunk_overlap(p, d, K, 512, stream)
        extra["dense_rowchunk_overlap"] = {"rows_per_chunk": 512, "serial_ms": ts, "two_stream_ms": tp,
                                           "gain": ts / tp - 1.0}
        log(f"[bench] dense row-chunked comparator: serial {ts:.3f} ms, two streams {tp:.3f} ms")
        # index -> KV-slot transform in the final write (glm_chunk)
        table = torch.randperm(2 * p.L, device=dev)[:p.L].to(torch.int32)
        wsg = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d, K=K, block_k=Bk), dtype=torch.uint8,
                          device=dev)
        tf = time_events(lambda: idx.idx_logits_topk_fused(d, K, block_k=Bk, out_idx=out_idx, out_val=out_val,
                                                           ws=wsg, stream=stream), 5, stream)
        tpg = time_events(lambda: idx.idx_logits_topk_fused_paged(d, K, table, block_k=Bk, out_idx=out_idx,
                                                                  out_val=out_val, ws=wsg, stream=stream), 5, stream)
        del wsg
        extra["paged_transform"] = {"fused_ms": float(np.median(tf)), "fused_paged_ms": float(np.median(tpg))}
        # candidate source and its consumers on the ragged batch: every row vs each request's tail rows,
        # byte-mask consumer vs block-list consumer
        p5 = synth.make_config("ragged_cand")
        c5 = p5.meta
        d5 = idx.Inputs.from_host(p5, device=dev)
        W5, nb5, pool5, K5, bk5 = p5.W, c5["n_blocks"], c5["pool"], c5["K"], c5["block_k"]
        blocks5 = torch.empty((p5.T, nb5), dtype=torch.int32, device=dev)
        ws5 = torch.empty(idx.idx_workspace_size(idx.IDX_OP_BLOCK_CANDIDATES, d5, block_k=bk5, row_chunk=4096,
                                                 pool=pool5, n_blocks=nb5), dtype=torch.uint8, device=dev)
        mask5 = torch.empty((p5.T, W5), dtype=torch.uint8, device=dev)
        cand_all = time_events(lambda: idx.idx_block_candidates(d5, W5, pool=pool5, n_blocks=nb5, block_k=bk5,
                                                                row_chunk=4096, mask=mask5, out_blocks=blocks5,
                                                                ws=ws5, stream=stream), 3, stream)
        tail = idx.idx_tail_rows(torch.tensor(c5["cu_q"], dtype=torch.int32, device=dev), 512)
        d5t = idx.idx_gather_rows(d5, tail)
        mask5t = torch.empty((d5t.T, W5), dtype=torch.uint8, device=dev)
        cand_tail = time_events(lambda: idx.idx_block_candidates(d5t, W5, pool=pool5, n_blocks=nb5, block_k=bk5,
                                                                 row_chunk=4096, mask=mask5t, ws=ws5, stream=stream),
                                3, stream)
        p5c = synth.consumer_layer(p5)
        d5c = idx.Inputs.from_host(p5c, device=dev)
        wsc = torch.empty(idx.idx_workspace_size(idx.IDX_OP_LOGITS_TOPK_FUSED, d5c, K=K5, block_k=bk5, row_chunk=4096),
                          dtype=torch.uint8, device=dev)
        cons_mask = time_events(lambda: idx.idx_logits_topk_fused(d5c, K5, block_k=bk5, row_chunk=4096, mask=mask5,
                                                                  ws=wsc, stream=stream), 3, stream)
        cons_blocks = time_events(lambda: idx.idx_logits_topk_fused_blocks(d5c, K5, blocks5, pool=pool5, block_k=bk5,
                                                                           row_chunk=4096, ws=wsc, stream=stream),
                                  3, stream)
        extra["ragged_candidates"] = {
            "all_rows": {"rows": p5.T, "ms": float(np.median(cand_all)), "mask_bytes": int(mask5.numel())},
            "tail_rows_512": {"rows": int(d5t.T), "ms": float(np.median(cand_tail)), "mask_bytes": int(mask5t.numel())},
            "consumer_byte_mask_ms": float(np.median(cons_mask)),
            "consumer_block_ids_ms": float(np.median(cons_blocks)), "block_ids_bytes": int(blocks5.numel() * 4)}
        log(f"[bench] ragged candidates: all rows {np.median(cand_all):.2f} ms, tail rows {np.median(cand_tail):.2f} ms;"
            f" consumer: byte mask {np.median(cons_mask):.2f} ms, block ids {np.median(cons_blocks):.2f} ms")
        del d5, d5t, d5c, mask5, mask5t, ws5, wsc
        extra["workloads"] = workload_lines(dev, stream)
        out["extra"] = extra

    if not args.no_cpu:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_budget:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(p, K, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
