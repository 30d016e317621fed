"""Benchmark: dynamic block-sparse attention on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input that is
already resident in HBM: bsa_select (block means, block scores, top-k) followed by
bsa_forward (attention over the kept blocks), both through the C ABI. The workload is the
720p-shaped video-DiT attention: B=1, H=40, S=75600 (21x45x80 latent), D=128, block 128,
keep_ratio 0.15 (89 of 591 key blocks per query block).

Prints one JSON line. `value` is milliseconds per step (lower is better). The line also
carries the attention kernel's own time, its kept-block TFLOP/s against the bf16 MFMA
peak (`roofline`), the fp8-QK variant, the full fp8 path (E4M3 Q, K, V and weights), a
dense (keep_ratio 1) forward for context, and the CPU oracle timed on a bounded sample on
this host (`cpu_baseline`).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
ATTN_SRC = os.path.join(ROOT, "dynamic_block_sparse_bsa_amd", "csrc", "attention.hip")


def kept_flops(row_ptr, col_idx, S, block):
    """4 * D-free part: sum over rows of (valid queries) x (valid keys in kept blocks).
    Multiply by 4*D for QK^T and PV multiply-adds (2 flops each)."""
    n = (S + block - 1) // block
    sizes = np.full(n, block, dtype=np.int64)
    sizes[-1] = S - (n - 1) * block
    rp = np.asarray(row_ptr, np.int64)
    csum = np.concatenate([[0], np.cumsum(sizes[np.asarray(col_idx, np.int64)[:rp[-1]]])])
    keys = csum[rp[1:]] - csum[rp[:-1]]  # keys kept by each row (empty rows included)
    qsz = np.tile(sizes, (rp.size - 1) // n)
    return int(np.sum(qsz * keys))


def traffic_from_profile(kernel_sha):
    """HBM bytes per attention launch from the committed PMC summary, if it was taken on
    the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, "attn_bf16_720p_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b) or m_sha.group(1) != kernel_sha:
        return None
    return float(m_b.group(1))


def cpu_baseline(q, k, v, cfg, budget_tokens):
    """Time the CPU oracle on this host: full selection, attention on a token sample,
    scaled to one whole call."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    B, H, S, D = q.shape
    t0 = time.perf_counter()
    ref = oracle.select(q, k, cfg["block"], cfg["keep_ratio"])
    t_sel = time.perf_counter() - t0
    budget_tokens = min(budget_tokens, B * H * S)
    tok = np.random.default_rng(0).choice(B * H * S, size=budget_tokens, replace=False)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, cfg["block"], ref["row_ptr"], ref["col_idx"], tokens=tok)
    t_att = time.perf_counter() - t0
    total_s = t_sel + t_att * (B * H * S) / budget_tokens
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {
        "value": round(total_s * 1e3, 1), "unit": "ms/step", "cores": int(os.environ["OMP_NUM_THREADS"]),
        "kind": "oracle", "cpu_model": model,
        "sample": "full selection (%.2f s) + attention for %d of %d query rows (%.2f s), scaled to all rows"
                  % (t_sel, budget_tokens, B * H * S, t_att),
    }


SWEEP_RATIOS = (0.10, 0.125, 0.15, 0.175, 0.20)


def sweep(args):
    """keep_ratio sweep over the pages' 10-20 % range on each shape: the same select and forward
    kernels, timed per call, with the output compared against dense attention (keep_ratio 1,
    every key block) computed by the same forward kernel on the same inputs."""
    import torch

    import dynamic_block_sparse_bsa_amd as bsa
    import gen

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    reps = max(2, args.steps // 4)
    for name in ("480p", "720p", "long"):
        q, k, v, cfg = gen.make_config(name)
        B, H, S, D = q.shape
        block = cfg["block"]
        to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        del q, k, v
        n = bsa.bsa_num_blocks(S, block)
        rows = B * H * n
        rp1 = torch.arange(rows + 1, dtype=torch.int32, device=dev) * n
        ci1 = torch.arange(n, dtype=torch.int32, device=dev).repeat(rows)
        dense = bsa.bsa_forward(qd, kd, vd, block, rp1, ci1)
        del rp1, ci1
        dense_f = dense.float()
        dense_norm = float(torch.linalg.vector_norm(dense_f))
        out = torch.empty_like(qd)
        for r in SWEEP_RATIOS:
            kept = bsa.bsa_num_kept(n, r)
            rp, ci = bsa.bsa_select(qd, kd, block, r)
            for _ in range(args.warmup):
                bsa.bsa_select(qd, kd, block, r, row_ptr=rp, col_idx=ci)
                bsa.bsa_forward(qd, kd, vd, block, rp, ci, out=out)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record()
            for _ in range(reps):
                bsa.bsa_select(qd, kd, block, r, row_ptr=rp, col_idx=ci)
            ev[1].record()
            for _ in range(reps):
                bsa.bsa_forward(qd, kd, vd, block, rp, ci, out=out)
            ev[2].record()
            torch.cuda.synchronize()
            sel_ms = ev[0].elapsed_time(ev[1]) / reps
            fwd_ms = ev[1].elapsed_time(ev[2]) / reps
            flop = 4.0 * D * kept_flops(rp.cpu().numpy(), ci.cpu().numpy(), S, block)
            diff = out.float() - dense_f
            line = {
                "workload": "%s: B=%d H=%d S=%d D=%d block=%d" % (name, B, H, S, D, block),
                "keep_ratio": r, "kept_blocks": kept, "n_blocks": n,
                "select_ms": round(sel_ms, 4), "attention_ms": round(fwd_ms, 4),
                "kept_tflops": round(flop / (fwd_ms * 1e-3) / 1e12, 1),
                "frac_bf16_mfma_peak": round(flop / (fwd_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "vs_dense_max_abs": round(float(diff.abs().max()), 5),
                "vs_dense_mean_abs": round(float(diff.abs().mean()), 6),
                "vs_dense_rel_l2": round(float(torch.linalg.vector_norm(diff)) / dense_norm, 5),
            }
            print(json.dumps(line), flush=True)
            del diff, rp, ci
        del qd, kd, vd, dense, dense_f, out
        torch.cuda.empty_cache()


def norm_rope_cpu_baseline(cfg, frames=2):
    """The oracle's RMSNorm + 3D RoPE and block means of one projection on this host, on the
    first `frames` latent frames of the shape, scaled to the whole sequence."""
    import gen
    import oracle

    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    B, H, D, block = cfg["B"], cfg["H"], cfg["D"], cfg["block"]
    grid = (frames,) + tuple(cfg["grid"][1:])
    S = int(np.prod(grid))
    xq, _ = gen.make_projections(B, S, H, D, cfg["seed"], grid, cfg["alpha"])
    w = gen.make_norm_weight(H * D, 1)
    t0 = time.perf_counter()
    _, y16 = oracle.norm_rope(xq, w, grid, exact=False)
    oracle.pool(y16, block)
    dt = time.perf_counter() - t0
    return {
        "value": round(dt * cfg["S"] / S * 1e3, 1), "unit": "ms/projection", "cores": int(os.environ["OMP_NUM_THREADS"]),
        "kind": "oracle",
        "sample": "%d of %d frames (%d tokens, %.2f s), scaled to the whole sequence" % (frames, cfg["grid"][0], S, dt),
    }


def norm_rope(args):
    """The fused RMSNorm + 3D RoPE + block means call on each shape's Q/K projections (the
    pages' fused-kernel item): ms per call and HBM GB/s against the 8 TB/s peak for one
    projection (bsa_norm_rope), and ms for both projections plus the selection
    (bsa_norm_rope_select). Algorithmic bytes per projection: x read once and out written
    once (2 * B*S*H*D * 2), plus the weights and the fp32 block means."""
    import torch

    import dynamic_block_sparse_bsa_amd as bsa
    import gen

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    reps = max(2, args.steps)
    for name in ("480p", "720p", "long"):
        cfg = gen.CONFIGS[name]
        B, H, S, D, block, grid = cfg["B"], cfg["H"], cfg["S"], cfg["D"], cfg["block"], cfg["grid"]
        xq, xk = gen.make_projections(B, S, H, D, cfg["seed"], grid, cfg["alpha"])
        to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        xqd, xkd = to_dev(xq), to_dev(xk)
        del xq, xk
        wq, wk = to_dev(gen.make_norm_weight(H * D, 1)), to_dev(gen.make_norm_weight(H * D, 2))
        n = bsa.bsa_num_blocks(S, block)
        out = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=dev)
        xbar = torch.empty((B, H, n, D), dtype=torch.float32, device=dev)
        ws = torch.empty(bsa.bsa_norm_rope_workspace_bytes(B, H, S, D), dtype=torch.uint8, device=dev)
        ws2 = torch.empty(bsa.bsa_norm_rope_select_workspace_bytes(B, H, S, D, block), dtype=torch.uint8, device=dev)
        one = lambda: bsa.bsa_norm_rope(xqd, wq, block, grid, out=out, xbar=xbar, workspace=ws)
        both = lambda: bsa.bsa_norm_rope_select(xqd, xkd, wq, wk, block, grid, cfg["keep_ratio"], workspace=ws2)
        for _ in range(args.warmup):
            one()
            both()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        for _ in range(reps):
            one()
        ev[1].record(stream)
        for _ in range(reps):
            both()
        ev[2].record(stream)
        torch.cuda.synchronize()
        one_ms = ev[0].elapsed_time(ev[1]) / reps
        both_ms = ev[1].elapsed_time(ev[2]) / reps
        nbytes = 2 * B * S * H * D * 2 + H * D * 2 + B * H * n * D * 4
        gbs = nbytes / (one_ms * 1e-3) / 1e9
        cpu = None
        if not args.no_cpu_baseline and name == "720p":
            cpu = norm_rope_cpu_baseline(cfg)
        line = {
            "workload": "norm_rope %s: B=%d H=%d S=%d D=%d grid=%dx%dx%d block=%d" % ((name, B, H, S, D) + tuple(grid) + (block,)),
            "norm_rope_ms": round(one_ms, 4), "bytes": nbytes, "gb_per_s": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "norm_rope_select_ms": round(both_ms, 4), "keep_ratio": cfg["keep_ratio"],
        }
        if cpu is not None:
            line["cpu_baseline"] = cpu
        print(json.dumps(line), flush=True)
        del xqd, xkd, out, xbar, ws, ws2
        torch.cuda.empty_cache()
    if args.calib_copy_mib:
        x = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(x).copy_(x)
        torch.cuda.synchronize()


def sample_power(stop, samples):
    """Append (time, socket watts, GFX clock MHz) from amd-smi about once a second until stop is set."""
    import re
    import subprocess

    while not stop.is_set():
        t = time.time()
        try:
            r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True, timeout=10).stdout
        except (OSError, subprocess.TimeoutExpired):
            return
        pw = re.search(r"SOCKET_POWER:\s*(\d+)", r)
        ck = re.search(r"GFX_0:\s*\n\s*CLK:\s*(\d+)", r)
        if pw and ck:
            samples.append((t, int(pw.group(1)), int(ck.group(1))))
        stop.wait(max(0.0, 0.7 - (time.time() - t)))


def power(args):
    """Each attention kernel on the workload back to back for a few seconds while amd-smi is
    sampled: socket power and shader clock under that kernel's load."""
    import threading

    import torch

    import dynamic_block_sparse_bsa_amd as bsa
    import gen

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    q, k, v, cfg = gen.make_config(args.config)
    B, H, S, D = q.shape
    block, r = cfg["block"], cfg["keep_ratio"]
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    n = bsa.bsa_num_blocks(S, block)
    rows = B * H * n
    rp, ci = bsa.bsa_select(qd, kd, block, r)
    q8, qs = bsa.bsa_quantize_fp8(qd, block)
    k8, ks = bsa.bsa_quantize_fp8(kd, block)
    rpf, cif, qf8, qfs, kf8, kfs = bsa.bsa_select_quantize(qd, kd, block, r)
    vt8, vts = bsa.bsa_quantize_v_fp8(vd, block)
    rp1 = torch.arange(rows + 1, dtype=torch.int32, device=dev) * n
    ci1 = torch.arange(n, dtype=torch.int32, device=dev).repeat(rows)
    out = torch.empty_like(qd)
    flop = 4.0 * D * kept_flops(rp.cpu().numpy(), ci.cpu().numpy(), S, block)
    flop1 = 4.0 * D * kept_flops(rp1.cpu().numpy(), ci1.cpu().numpy(), S, block)
    runs = [
        ("bf16", flop, lambda: bsa.bsa_forward(qd, kd, vd, block, rp, ci, out=out)),
        ("fp8_qk", flop, lambda: bsa.bsa_forward_fp8(q8, qs, k8, ks, vd, block, rp, ci, out=out)),
        ("fp8_full", flop, lambda: bsa.bsa_forward_fp8_full(qf8, qfs, kf8, kfs, vt8, vts, block, rpf, cif, out=out)),
        ("bf16_dense", flop1, lambda: bsa.bsa_forward(qd, kd, vd, block, rp1, ci1, out=out)),
    ]
    torch.cuda.synchronize()
    samples, stop = [], threading.Event()
    th = threading.Thread(target=sample_power, args=(stop, samples), daemon=True)
    th.start()
    time.sleep(2.0)
    idle = [(p, c) for _, p, c in samples]
    for name, fl, f in runs:
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0, calls = time.time(), 0
        e0.record()
        while time.time() - t0 < args.power_seconds:
            for _ in range(5):
                f()
            calls += 5
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.time()
        ms = e0.elapsed_time(e1) / calls
        load = [(p, c) for t, p, c in samples if t0 + 1.0 < t < t1]  # skip the ramp
        line = {
            "workload": "%s: B=%d H=%d S=%d D=%d block=%d keep=%g" % (args.config, B, H, S, D, block,
                                                                     1.0 if name == "bf16_dense" else r),
            "kernel": name, "calls": calls, "attention_ms": round(ms, 4),
            "kept_tflops": round(fl / (ms * 1e-3) / 1e12, 1),
            "socket_power_w": round(sum(p for p, _ in load) / len(load), 1) if load else None,
            "gfx_clock_mhz": round(sum(c for _, c in load) / len(load), 1) if load else None,
            "samples": len(load),
        }
        print(json.dumps(line), flush=True)
        time.sleep(2.0)
    stop.set()
    th.join(timeout=15)
    if idle:
        print(json.dumps({"idle_socket_power_w": round(sum(p for p, _ in idle) / len(idle), 1),
                          "idle_gfx_clock_mhz": round(sum(c for _, c in idle) / len(idle), 1)}), flush=True)


PEAK_LIB = os.path.join(ROOT, "dynamic_block_sparse_bsa_amd", "libbsa_peak.so")


def mfma_peak(dev, seconds=0.25):
    """Measured dense MFMA throughput (TFLOP/s) of this card, bf16 and fp8: every SIMD issues
    independent MFMAs with register operands (dynamic_block_sparse_bsa_amd/csrc/peak.hip).
    The attention kernels' rates are also given as fractions of these ceilings."""
    import ctypes

    import torch

    lib = ctypes.CDLL(PEAK_LIB)
    lib.bsa_peak_run.restype = ctypes.c_int
    lib.bsa_peak_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.bsa_peak_flops.restype = ctypes.c_double
    lib.bsa_peak_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    wgs = 256 * 8
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, fp8 in (("bf16", 0), ("fp8", 1)):
        iters = 64
        while True:  # grow the launch until it runs for about `seconds`
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if lib.bsa_peak_run(fp8, wgs, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream)):
                raise RuntimeError("peak probe launch failed")
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            if ms >= seconds * 1e3 or iters >= 1 << 20:
                break
            iters *= 2
        out[name + "_tflops"] = round(lib.bsa_peak_flops(fp8, wgs, iters) / (ms * 1e-3) / 1e12, 1)
    return out


def time_calls(fns, steps, warmup):
    """Times each callable of fns (run in turn, as one step) with HIP events on torch's current
    stream, the stream every call is enqueued on; returns per-callable lists of ms."""
    import torch

    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        for j, f in enumerate(fns):
            f()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    return [[ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)] for j in range(len(fns))]


def stats(ms):
    return {"mean": round(float(np.mean(ms)), 4), "median": round(float(np.median(ms)), 4),
            "min": round(float(np.min(ms)), 4)}


def workload_name(config, heads, seed, B, H, S, D, block, keep_ratio, kept, n):
    """The bench line's config.workload string."""
    name = config
    if heads:
        name += " (first %d heads: one rank's share)" % H
    if seed is not None:
        name += " (seed %d)" % seed
    return "%s: B=%d H=%d S=%d D=%d block=%d keep_ratio=%g (%d of %d key blocks kept)" % (
        name, B, H, S, D, block, keep_ratio, kept, n)


def head_slice(q, k, v, heads):
    """The first `heads` heads of each tensor: one rank's share when heads are sharded."""
    if not heads:
        return q, k, v
    return tuple(np.ascontiguousarray(x[:, :heads]) for x in (q, k, v))


def all_configs(args):
    """One JSON line per configuration: tiny, 480p, 720p, 720p dense (keep_ratio 1), long and
    fp8-QK on the 720p tensors. Each line carries the GPU select and forward times (mean,
    median, min), the kept-block TFLOP/s and its fractions of the published and the measured
    MFMA peak, the selection's HBM rate, and the oracle on this host's cores: its whole
    selection, and its attention on a stated sample of query rows scaled to the whole call
    (all rows for tiny; not run for the dense line)."""
    import torch

    import dynamic_block_sparse_bsa_amd as bsa
    import gen
    import oracle

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    peak = mfma_peak(dev)
    print(json.dumps({"mfma_peak_measured": peak}), flush=True)
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    for name in ("tiny", "480p", "720p", "long"):
        q, k, v, cfg = gen.make_config(name)
        q, k, v = head_slice(q, k, v, args.heads)
        B, H, S, D = q.shape
        block, r = cfg["block"], cfg["keep_ratio"]
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        n = bsa.bsa_num_blocks(S, block)
        rows = B * H * n
        runs = [(r, False)] + ([(1.0, True)] if name == "720p" else []) + ([(r, "fp8")] if name == "720p" else [])
        for ratio, kind in runs:
            kept = bsa.bsa_num_kept(n, ratio)
            out = torch.empty_like(qd)
            if kind is True:  # dense: every key block, no selection
                rp = torch.arange(rows + 1, dtype=torch.int32, device=dev) * n
                ci = torch.arange(n, dtype=torch.int32, device=dev).repeat(rows)
                fwd, = time_calls([lambda: bsa.bsa_forward(qd, kd, vd, block, rp, ci, out=out)], 3, 1)
                sel = None
            else:
                ws = torch.empty(bsa.bsa_select_workspace_bytes(B, H, S, D, block), dtype=torch.uint8, device=dev)
                rp = torch.empty(rows + 1, dtype=torch.int32, device=dev)
                ci = torch.empty(rows * kept, dtype=torch.int32, device=dev)
                select = lambda: bsa.bsa_select(qd, kd, block, ratio, workspace=ws, row_ptr=rp, col_idx=ci)
                if kind == "fp8":
                    q8, qs = bsa.bsa_quantize_fp8(qd, block)
                    k8, ks = bsa.bsa_quantize_fp8(kd, block)
                    quant = lambda: (bsa.bsa_quantize_fp8(qd, block, codes=q8, scale=qs),
                                     bsa.bsa_quantize_fp8(kd, block, codes=k8, scale=ks))
                    sel, qt, fwd = time_calls([select, quant, lambda: bsa.bsa_forward_fp8(q8, qs, k8, ks, vd, block, rp, ci,
                                                                                           out=out)],
                                              args.steps, args.warmup)
                else:
                    sel, fwd = time_calls([select, lambda: bsa.bsa_forward(qd, kd, vd, block, rp, ci, out=out)],
                                          args.steps, args.warmup)
            flop = 4.0 * D * kept_flops(rp.cpu().numpy(), ci.cpu().numpy(), S, block)
            tf = flop / (np.mean(fwd) * 1e-3) / 1e12
            label = name + (" dense" if kind is True else " fp8-QK" if kind == "fp8" else "")
            line = {"workload": "%s: B=%d H=%d S=%d D=%d block=%d keep_ratio=%g (%d of %d key blocks kept)"
                                % (label, B, H, S, D, block, ratio, kept, n),
                    "attention_ms": stats(fwd), "kept_tflop_per_call": round(flop / 1e12, 4),
                    "kept_tflops": round(tf, 1), "frac_bf16_mfma_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                    "frac_measured_bf16_peak": round(tf / peak["bf16_tflops"], 4)}
            if kind == "fp8":
                mixed = 2 / (1 / FP8_PEAK_TFLOPS + 1 / BF16_PEAK_TFLOPS)
                line["quantize_ms"] = stats(qt)
                line["frac_mixed_fp8_bf16_peak"] = round(tf / mixed, 4)
            if sel is not None:
                line["select_ms"] = stats(sel)
                line["select_hbm_gbs"] = round(2 * B * H * S * D * 2 / (np.mean(sel) * 1e-3) / 1e9, 1)
            if not args.no_cpu_baseline and kind is not True:
                t0 = time.perf_counter()
                ref = oracle.select(q, k, block, ratio)
                t_sel = time.perf_counter() - t0
                sample = B * H * S if name == "tiny" else min(B * H * S, args.cpu_sample)
                tok = np.sort(np.random.default_rng(0).choice(B * H * S, size=sample, replace=False))
                t0 = time.perf_counter()
                if kind == "fp8":
                    oq8, oqs = oracle.quantize_fp8(q, block)
                    ok8, oks = oracle.quantize_fp8(k, block)
                    oracle.attention_fp8(oq8, oqs, ok8, oks, v, block, ref["row_ptr"], ref["col_idx"], tokens=tok)
                else:
                    oracle.attention(q, k, v, block, ref["row_ptr"], ref["col_idx"], tokens=tok)
                t_att = (time.perf_counter() - t0) * (B * H * S) / sample
                line["cpu_baseline"] = {"kind": "oracle", "cores": int(os.environ["OMP_NUM_THREADS"]),
                                        "select_s": round(t_sel, 3), "attention_s": round(t_att, 2),
                                        "sample": "whole selection; attention on %d of %d query rows%s"
                                                  % (sample, B * H * S, "" if sample == B * H * S else ", scaled")}
            print(json.dumps(line), flush=True)
            del rp, ci, out
        del qd, kd, vd, q, k, v
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="720p", choices=["tiny", "480p", "720p", "long"])
    ap.add_argument("--seed", type=int, default=None,
                    help="draw the workload from this seed instead of its own (same shapes and recipe)")
    ap.add_argument("--heads", type=int, default=0,
                    help="run only the first HEADS heads of the workload: one rank's share when the "
                         "heads are sharded across GPUs (5 of 40 on eight GPUs)")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead: one JSON line per configuration (tiny, 480p, 720p, 720p dense, long, "
                         "fp8-QK) with the oracle timed beside each")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="instead: print the card's measured dense bf16 and fp8 MFMA throughput")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=8192, help="query rows the CPU oracle computes")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (PMC calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="keep_ratio sweep 0.10-0.20 on the 480p, 720p and long shapes instead: one "
                         "JSON line per point with ms, kept TFLOP/s and the error against dense attention")
    ap.add_argument("--power", action="store_true",
                    help="instead: run each attention kernel for a few seconds while amd-smi samples "
                         "socket power and shader clock; one JSON line per kernel")
    ap.add_argument("--power-seconds", type=float, default=6.0)
    ap.add_argument("--norm-rope", action="store_true",
                    help="instead: time the fused RMSNorm + 3D RoPE + block-means call (one projection, "
                         "and both plus the selection) on the 480p, 720p and long shapes")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the design notes "
              "describe how the work would shard by head).", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    if args.power:
        power(args)
        return
    if args.norm_rope:
        norm_rope(args)
        return
    if args.all_configs:
        all_configs(args)
        return
    if args.mfma_peak:
        import torch

        print(json.dumps({"mfma_peak_measured": mfma_peak(torch.device("cuda:0"), seconds=1.0)}), flush=True)
        return

    import torch

    import dynamic_block_sparse_bsa_amd as bsa
    import gen

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    q, k, v, cfg = gen.make_config(args.config, seed=args.seed)
    q, k, v = head_slice(q, k, v, args.heads)
    B, H, S, D = q.shape
    block, r = cfg["block"], cfg["keep_ratio"]
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    n = bsa.bsa_num_blocks(S, block)
    kept = bsa.bsa_num_kept(n, r)
    rows = B * H * n
    peak = mfma_peak(dev)
    ws = torch.empty(bsa.bsa_select_workspace_bytes(B, H, S, D, block), dtype=torch.uint8, device=dev)
    rp = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(rows * kept, dtype=torch.int32, device=dev)
    out = torch.empty_like(qd)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        bsa.bsa_select(qd, kd, block, r, workspace=ws, row_ptr=rp, col_idx=ci)
        if ev is not None:
            ev[1].record()
        bsa.bsa_forward(qd, kd, vd, block, rp, ci, out=out)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    sel_each = [e[0].elapsed_time(e[1]) for e in events]
    fwd_each = [e[1].elapsed_time(e[2]) for e in events]
    sel_ms = float(np.mean(sel_each))
    fwd_ms = float(np.mean(fwd_each))
    step_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in events]))

    flop = 4.0 * D * kept_flops(rp.cpu().numpy(), ci.cpu().numpy(), S, block)
    fwd_tflops = flop / (fwd_ms * 1e-3) / 1e12
    kernel_sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    pool_bytes = 2 * B * H * S * D * 2

    # fp8-QK variant: quantise Q and K, then attention with fp8 QK^T.
    q8, qs = bsa.bsa_quantize_fp8(qd, block)
    k8, ks = bsa.bsa_quantize_fp8(kd, block)
    out8 = torch.empty_like(qd)
    for _ in range(2):
        bsa.bsa_forward_fp8(q8, qs, k8, ks, vd, block, rp, ci, out=out8)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    reps = max(3, args.steps // 2)
    e[0].record()
    for _ in range(reps):
        bsa.bsa_quantize_fp8(qd, block, codes=q8, scale=qs)
        bsa.bsa_quantize_fp8(kd, block, codes=k8, scale=ks)
    e[1].record()
    for _ in range(reps):
        bsa.bsa_forward_fp8(q8, qs, k8, ks, vd, block, rp, ci, out=out8)
    e[2].record()
    torch.cuda.synchronize()
    quant_ms = e[0].elapsed_time(e[1]) / reps
    fwd8_ms = e[1].elapsed_time(e[2]) / reps

    # Full fp8 path: lists + Q/K codes from one pass, per-channel V codes, fp8 QK^T and PV.
    rpf, cif, qf8, qfs, kf8, kfs = bsa.bsa_select_quantize(qd, kd, block, r, workspace=ws)
    vt8, vts = bsa.bsa_quantize_v_fp8(vd, block)
    outf = torch.empty_like(qd)
    for _ in range(2):
        bsa.bsa_forward_fp8_full(qf8, qfs, kf8, kfs, vt8, vts, block, rpf, cif, out=outf)
    torch.cuda.synchronize()
    ef = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ef[0].record()
    for _ in range(reps):
        bsa.bsa_select_quantize(qd, kd, block, r, workspace=ws, row_ptr=rpf, col_idx=cif)
    ef[1].record()
    for _ in range(reps):
        bsa.bsa_quantize_v_fp8(vd, block, vt=vt8, scale=vts)
    ef[2].record()
    for _ in range(reps):
        bsa.bsa_forward_fp8_full(qf8, qfs, kf8, kfs, vt8, vts, block, rpf, cif, out=outf)
    ef[3].record()
    torch.cuda.synchronize()
    selq_ms = ef[0].elapsed_time(ef[1]) / reps
    vq_ms = ef[1].elapsed_time(ef[2]) / reps
    fwdf_ms = ef[2].elapsed_time(ef[3]) / reps
    del rpf, cif, qf8, qfs, kf8, kfs, vt8, vts, outf

    dense = None
    if not args.no_dense:
        rp1 = torch.arange(rows + 1, dtype=torch.int32, device=dev) * n
        ci1 = torch.arange(n, dtype=torch.int32, device=dev).repeat(rows)
        bsa.bsa_forward(qd, kd, vd, block, rp1, ci1, out=out)
        torch.cuda.synchronize()
        e2 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e2[0].record()
        for _ in range(2):
            bsa.bsa_forward(qd, kd, vd, block, rp1, ci1, out=out)
        e2[1].record()
        torch.cuda.synchronize()
        dms = e2[0].elapsed_time(e2[1]) / 2
        dflop = 4.0 * D * (B * H) * S * S
        dense = {"forward_ms": round(dms, 3), "tflops": round(dflop / dms / 1e9, 1),
                 "frac_bf16_peak": round(dflop / dms / 1e9 / BF16_PEAK_TFLOPS, 4)}
        del rp1, ci1

    if args.calib_copy_mib:
        x = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(q, k, v, cfg, args.cpu_sample)

    result = {
        "metric": "ms/attention call + kept-block TFLOP/s (% MFMA peak), 720p-shaped S=75600",
        "value": round(step_ms, 4),
        "unit": "ms/step (bsa_select + bsa_forward)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded noise + smooth (t,h,w) locality term, bf16)",
        "config": {"workload": workload_name(args.config, args.heads, args.seed, B, H, S, D, block, r, kept, n),
                   "global_batch": B, "seq_len": S, "heads": H, "head_dim": D, "block": block,
                   "keep_ratio": r, "parallelism": "single GPU"},
        "attention_ms": round(fwd_ms, 4),
        "attention_ms_median": round(float(np.median(fwd_each)), 4),
        "attention_ms_min": round(float(np.min(fwd_each)), 4),
        "select_ms": round(sel_ms, 4),
        "select_ms_median": round(float(np.median(sel_each)), 4),
        "select_ms_min": round(float(np.min(sel_each)), 4),
        "wall_ms_per_step": round(wall_ms, 4),
        "kept_tflop_per_call": round(flop / 1e12, 4),
        "kept_tflops": round(fwd_tflops, 1),
        "kept_tflops_per_step": round(flop / (step_ms * 1e-3) / 1e12, 1),
        "frac_bf16_mfma_peak": round(fwd_tflops / BF16_PEAK_TFLOPS, 4),
        "select_hbm_gbs": round(pool_bytes / (sel_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / BF16_PEAK_TFLOPS, 4),
                     # the committed counters cover the whole default 720p call only
                     "traffic": (traffic_from_profile(kernel_sha)
                                 if not args.heads and args.config == "720p" and args.seed is None else None),
                     "kernel": "attn_kernel<%d,%d,bf16>" % (D, block),
                     "measured_peak": peak["bf16_tflops"],
                     "frac_measured_peak": round(fwd_tflops / peak["bf16_tflops"], 4)},
        "mfma_peak_measured": peak,
        "fp8_qk": {"quantize_ms": round(quant_ms, 4), "attention_ms": round(fwd8_ms, 4),
                   "kept_tflops": round(flop / (fwd8_ms * 1e-3) / 1e12, 1),
                   "frac_mixed_peak": round(flop / (fwd8_ms * 1e-3) / 1e12 / (2 / (1 / FP8_PEAK_TFLOPS + 1 / BF16_PEAK_TFLOPS)), 4),
                   "frac_bf16_peak": round(flop / (fwd8_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "fp8_full": {"select_quantize_ms": round(selq_ms, 4), "quantize_v_ms": round(vq_ms, 4),
                     "attention_ms": round(fwdf_ms, 4),
                     "kept_tflops": round(flop / (fwdf_ms * 1e-3) / 1e12, 1),
                     "frac_fp8_mfma_peak": round(flop / (fwdf_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                     "frac_measured_fp8_peak": round(flop / (fwdf_ms * 1e-3) / 1e12 / peak["fp8_tflops"], 4),
                     "step_ms": round(selq_ms + vq_ms + fwdf_ms, 4)},
        "dense_keep_ratio_1": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
