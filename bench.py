#!/usr/bin/env python3
"""Benchmark: FlashSwin window attention, one training-step pass (forward + backward) on one GPU.

Workload (default): FlashSwin-T stage 1 with p=2, M=32: q/k/v/dO [128, 128, 128, 3, 32] bf16,
no shift, seeded synthetic N(0,1) inputs (no dataset), RoPE theta from the geometric schedule plus
N(0, 0.01^2) noise.  One step = the whole hot path over the batch: the forward (RoPE, exact-softmax
attention, LSE, and a 16-byte operand summary per window-head) then the backward (Delta, recomputed P,
dQ/dK/dV, dtheta; its prologue reads O and dO and takes the q/k/v maxima from the summary, as the
autograd wrapper does).  FLOPs per window-head:
4 N^2 d forward + 10 N^2 d backward (N = M^2), the dense convention of the workload's metric.

Prints ONE JSON line.  `roofline` describes the forward kernel of the workload (one launch of
fwd_mfma_kernel per forward call at M=32), the configuration the metric is quoted on, against the
dense bf16 MFMA peak; `bwd_roofline` describes the backward call (`launches` names the four
kernels it enqueues; together they take most of the step).  Both are timed with HIP events on the
stream the library launches on.  `traffic` is taken from the committed rocprofv3 counter summary
in profiles/ when that summary was measured on the current kernel source (sha256 match), else
null.  `m8_fwd_roofline` times the forward on the M=8 Swin-T stage-1 workload (memory-bound)
against the HBM peak, with its own `traffic` read the same way.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same workload (rank 0, N=1
only).

Modes for profiling runs: --only fwd|bwd runs just that call per step; --copy-calibration runs a
plain streaming kernel of known traffic, b = -a over 1 GiB (for scaling HBM counters);
--lowrank-only prints the rank-16 bias line alone.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
# the forward kernel instance the step launches at each window size (the instances that write the
# operand summary; M = 8: one wave per window-head)
FWD_KERNEL = {32: "fwd_mfma_kernel<16, 32, 1024, 32, false, 0, true>", 16: "fwd_mfma_kernel<8, 16, 256, 32, false, 0, true>",
              8: "fwd_m8_kernel"}
# kernels each C-ABI call launches, in order
CALL_LAUNCHES = {"wattn_fwd": ["fwd_mfma_kernel"],
                 "wattn_bwd": ["bwd_pre_kernel", "bwd_dkdv_mfma_kernel", "bwd_dq_mfma_kernel", "dtheta_reduce_kernel"]}


def kernel_source_sha():
    """Hash of every kernel source file: a traffic summary measured on other sources is not used."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "vision_transformer_windowed_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag, workload, sha):
    """HBM bytes per launch from profiles/traffic_<kernel_tag>_<workload>.md if its sha matches."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}_{workload}.md")
    if not os.path.exists(p):
        return None
    text = open(p).read()
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    m_rd = re.search(r"hbm_read_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_wr = re.search(r"hbm_write_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_rd and m_wr) or m_sha.group(1) != sha:
        return None
    return float(m_rd.group(1)) + float(m_wr.group(1))


def cpu_baseline(x, w, shift, images, gpu_out=None):
    """Time the fp64 oracle (forward + backward) on the first `images` images, one image per call."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    tr, tc = x["theta_row"].double().numpy(), x["theta_col"].double().numpy()
    dt = 0.0
    parity = {} if gpu_out is not None else None
    acc = {}
    for b in range(images):
        sl = slice(b, b + 1)
        args = [x[n][sl].double().numpy() for n in ("q", "k", "v")]
        dout = x["dout"][sl].double().numpy()
        t0 = time.perf_counter()
        ro, rl = oracle.wattn_fwd_ref(*args, tr, tc, w["M"], shift)
        g = oracle.wattn_bwd_ref(*args, dout, tr, tc, w["M"], shift)
        dt += time.perf_counter() - t0
        if gpu_out is not None:
            for name, ref, got in (("O", ro, gpu_out["out"]), ("LSE", rl, gpu_out["lse"]), ("dQ", g[0], gpu_out["dq"]),
                                   ("dK", g[1], gpu_out["dk"]), ("dV", g[2], gpu_out["dv"])):
                got = got[sl].double().cpu().numpy()
                a = acc.setdefault(name, [0.0, 0.0, 0.0])
                a[0] = max(a[0], float(np.abs(got - ref).max()))
                a[1] += float(((got - ref) ** 2).sum())
                a[2] += float((ref ** 2).sum())
    N = w["M"] ** 2
    nwh = images * (w["Hg"] // w["M"]) * (w["Wg"] // w["M"]) * w["heads"]
    flops = 14.0 * N * N * w["d"] * nwh
    res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": f"first {images} of {w['B']} images, one image per oracle call (forward + backward, fp64 "
                     f"NumPy), {dt:.1f} s of oracle time"}
    if gpu_out is not None:
        for name, (ma, se, sr) in acc.items():
            parity[name] = {"max_abs": ma, "rel_l2": (se / sr) ** 0.5}
    return res, parity


def warm_clocks(fn, seconds=0.3):
    """Call fn for about `seconds` (synchronizing every few calls) before a short timed region.  Each
    secondary line generates its inputs on the host first, which leaves the GPU idle for seconds; its
    clocks then need some 0.1 s of load to come back, longer than a few warmup calls of a sub-ms
    kernel (an M = 16 forward timed right after its input generation read 0.70 ms, 0.55 warm)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def m8_forward_roofline(dev, steps, warmup):
    """Forward on the M=8 Swin-T stage-1 workload (HBM-bound): achieved GB/s of algorithmic bytes."""
    import torch
    import vision_transformer_windowed_amd as F
    from vision_transformer_windowed_amd.inputs import WORKLOADS, workload_inputs
    name = "swin_t_s1_p4_m8"
    w = WORKLOADS[name]
    x = {k: v.to(dev) for k, v in workload_inputs(name, with_dout=False).items()}
    q, k, v = x["q"], x["k"], x["v"]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:4], device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        F.wattn_fwd(q, k, v, x["theta_row"], x["theta_col"], w["M"], 0, out=out, lse=lse)
    warm_clocks(lambda: F.wattn_fwd(q, k, v, x["theta_row"], x["theta_col"], w["M"], 0, out=out, lse=lse))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        F.wattn_fwd(q, k, v, x["theta_row"], x["theta_col"], w["M"], 0, out=out, lse=lse)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = 4 * q.numel() * q.element_size() + lse.numel() * 4  # q, k, v read; out written; lse written
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": name, "kernel": "wattn_fwd", "bound": "hbm", "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "launch_ms": round(ms, 4),
            "traffic": read_traffic("wattn_fwd", name, kernel_source_sha())}


def live_fraction(Hg, Wg, M, shift):
    """Fraction of a window's (query, key) pairs that share a Swin region label, averaged over the
    windows of the grid.  Labels combine a row region and a column region, so a window's fraction is
    the product of its row-axis and column-axis fractions, and the grid average factors the same way."""
    def axis(size):
        fr = []
        for wi in range(size // M):
            counts = {}
            for r in range(M):
                Y = wi * M + r  # shifted-frame coordinate
                lab = int(Y >= size - M) + int(Y >= size - shift) if shift else 0
                counts[lab] = counts.get(lab, 0) + 1
            fr.append(sum(c * c for c in counts.values()) / (M * M))
        return sum(fr) / len(fr)
    return axis(Hg) * axis(Wg)


def config_timing(dev, name, shift, passes, steps, warmup):
    """Time the forward and/or backward call of a named workload at one shift.  TFLOP/s under the dense
    4 N^2 d (forward) / 10 N^2 d (backward) conventions, and with a shift also over live (same-region)
    pairs only; the dense figure's fraction of the bf16 MFMA peak."""
    import torch
    import vision_transformer_windowed_amd as F
    from vision_transformer_windowed_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS[name]
    M = w["M"]
    x = {k: v.to(dev) for k, v in workload_inputs(name, with_dout="bwd" in passes).items()}
    q, k, v, tr, tc = x["q"], x["k"], x["v"], x["theta_row"], x["theta_col"]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:4], device=dev, dtype=torch.float32)
    # with a backward, the forward also writes the operand summary the backward's prologue takes
    stats = F.new_stats(q, M, shift) if "bwd" in passes else None
    fns = {"fwd": lambda: F.wattn_fwd(q, k, v, tr, tc, M, shift, out=out, lse=lse, stats=stats)}
    if "bwd" in passes:
        dout = x["dout"]
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(tr),
                 torch.empty_like(tc))
        ws = torch.empty(max(F.bwd_workspace_bytes(q, M, shift), 1), device=dev, dtype=torch.uint8)
        fns["bwd"] = lambda: F.wattn_bwd(q, k, v, out, dout, lse, tr, tc, M, shift, workspace=ws, grads=grads,
                                         stats=stats)
        fns["fwd"]()  # out and lse for the backward
    stream = torch.cuda.current_stream(dev)
    N = M * M
    nwh = w["B"] * (w["Hg"] // M) * (w["Wg"] // M) * w["heads"]
    live = live_fraction(w["Hg"], w["Wg"], M, shift)
    res = {"workload": name, "shift": shift}
    if shift:
        res["live_pair_fraction"] = round(live, 6)
    for tag in passes:
        fn = fns[tag]
        for _ in range(warmup):
            fn()
        warm_clocks(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = (4.0 if tag == "fwd" else 10.0) * N * N * w["d"] * nwh / (ms * 1e-3) / 1e12
        res[tag + "_ms"] = round(ms, 4)
        res[tag + "_tflops"] = round(tf, 2)
        res[tag + "_mfma_frac"] = round(tf / BF16_MFMA_PEAK_TFLOPS, 4)
        if tag == "fwd":  # q, k, v read and out written once, lse written: the forward's HBM floor
            nbytes = 4 * q.numel() * q.element_size() + lse.numel() * 4
            res["fwd_hbm_frac"] = round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        if shift:
            res[tag + "_tflops_live"] = round(tf * live, 2)
    return res


LOWRANK_SEED = 2024  # factors of the rank-16 bias line (inputs.lowrank_factors)


def lowrank_step(dev, steps, warmup, rank=16):
    """Forward and backward with a rank-16 additive bias (factors U, W [heads, M*M, 16], N(0, 0.5^2)) on
    the M = 16 stage-1 workload at s = 0, beside the same calls without the bias.  FLOP conventions: the
    bias adds r channels to the score contraction, so the forward is 4 N^2 d + 2 N^2 r and the backward
    10 N^2 d + 6 N^2 r (S recomputed with the r channels, dU = dS W and dW = dS^T U)."""
    import torch
    import vision_transformer_windowed_amd as F
    from vision_transformer_windowed_amd.inputs import WORKLOADS, lowrank_factors, workload_inputs
    name = "flashswin_t_s1_p2_m16"
    w = WORKLOADS[name]
    M, d = w["M"], w["d"]
    x = {k: v.to(dev) for k, v in workload_inputs(name, with_dout=True).items()}
    q, k, v, tr, tc, dout = x["q"], x["k"], x["v"], x["theta_row"], x["theta_col"], x["dout"]
    U, W = (t.to(dev) for t in lowrank_factors(w["heads"], M, rank, seed=LOWRANK_SEED))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:4], device=dev, dtype=torch.float32)
    ws = torch.empty(max(F.flashswin_wattn_bwd_lowrank_workspace_size(*q.shape, M, 0, F.FSW_BF16, rank), 1),
                     device=dev, dtype=torch.uint8)
    stats = F.new_stats(q, M, 0)
    fns = {"fwd": lambda: F.wattn_fwd_lowrank(q, k, v, tr, tc, U, W, M, 0, out=out, lse=lse, stats=stats),
           "bwd": lambda: F.wattn_bwd_lowrank(q, k, v, out, dout, lse, tr, tc, U, W, M, 0, workspace=ws, stats=stats)}
    fns["fwd"]()
    stream = torch.cuda.current_stream(dev)
    N = M * M
    nwh = w["B"] * (w["Hg"] // M) * (w["Wg"] // M) * w["heads"]
    flops = {"fwd": (4.0 * N * N * d + 2.0 * N * N * rank) * nwh, "bwd": (10.0 * N * N * d + 6.0 * N * N * rank) * nwh}
    res = {"workload": name, "shift": 0, "rank": rank}
    for tag in ("fwd", "bwd"):
        fn = fns[tag]
        for _ in range(warmup):
            fn()
        warm_clocks(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = flops[tag] / (ms * 1e-3) / 1e12
        res[tag + "_ms"] = round(ms, 4)
        res[tag + "_tflops"] = round(tf, 2)
        res[tag + "_mfma_frac"] = round(tf / BF16_MFMA_PEAK_TFLOPS, 4)
    return res


def materialized_vs_fused(dev, steps, warmup):
    """The forward computed the standard Swin way, with every window's score matrix in HBM (the
    materialized comparison path), against the fused forward, at M = 8, 16 and 32 on the stage-1 grids:
    milliseconds per call and the bytes of score workspace the materialized path needs (the fused path
    needs none)."""
    import torch
    import vision_transformer_windowed_amd as F
    from vision_transformer_windowed_amd.inputs import WORKLOADS, workload_inputs
    res = []
    for name in ("swin_t_s1_p4_m8", "flashswin_t_s1_p2_m16", "flashswin_t_s1_p2_m32"):
        w = WORKLOADS[name]
        x = {k: v.to(dev) for k, v in workload_inputs(name, with_dout=False).items()}
        q, k, v, tr, tc = x["q"], x["k"], x["v"], x["theta_row"], x["theta_col"]
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:4], device=dev, dtype=torch.float32)
        nbytes = F.flashswin_wattn_fwd_materialized_workspace_size(*q.shape, w["M"], 0, F.FSW_BF16)
        stream = torch.cuda.current_stream(dev)
        row = {"workload": name, "M": w["M"], "materialized_workspace_bytes": nbytes}
        ws = None
        for tag, fn in (("fused_ms", lambda: F.wattn_fwd(q, k, v, tr, tc, w["M"], 0, out=out, lse=lse)),
                        ("materialized_ms", lambda: F.wattn_fwd_materialized(q, k, v, tr, tc, w["M"], 0, out=out,
                                                                             lse=lse, workspace=ws))):
            if tag == "materialized_ms":  # the fused call is timed before the score workspace exists
                ws = torch.empty(nbytes, device=dev, dtype=torch.uint8)
            n_steps, n_warm = (steps, warmup) if tag == "materialized_ms" else (4 * steps, 4 * warmup + 2)
            for _ in range(n_warm):
                fn()
            warm_clocks(fn, 0.3 if tag == "fused_ms" else 0.1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n_steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            row[tag] = round(e0.elapsed_time(e1) / n_steps, 4)
        row["materialized_over_fused"] = round(row["materialized_ms"] / row["fused_ms"], 3)
        res.append(row)
        del ws
        torch.cuda.empty_cache()
    return res


def m16_step(dev, steps, warmup):
    """Forward and backward at M = 16 (the pages' comparison-table window) on the stage-1 grid."""
    return config_timing(dev, "flashswin_t_s1_p2_m16", 0, ("fwd", "bwd"), steps, warmup)


def packed_forward(dev, steps, warmup):
    """M=8 Swin-T stage-1 forward (HBM-bound) from packed qkv [B, Hg, Wg, 3, heads, d]: read in place by
    the packed entry point, against splitting it into contiguous q, k, v first (three copies) and calling
    the separate-tensor entry point."""
    import torch
    import vision_transformer_windowed_amd as F
    from vision_transformer_windowed_amd.inputs import WORKLOADS, workload_inputs
    name = "swin_t_s1_p4_m8"
    w = WORKLOADS[name]
    x = workload_inputs(name, with_dout=False)
    qkv = torch.stack([x["q"], x["k"], x["v"]], dim=3).contiguous().to(dev)
    tr, tc = x["theta_row"].to(dev), x["theta_col"].to(dev)
    out = torch.empty(qkv.shape[:3] + qkv.shape[4:], device=dev, dtype=qkv.dtype)
    lse = torch.empty(qkv.shape[:3] + qkv.shape[4:5], device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)

    def packed():
        F.wattn_fwd_packed(qkv, tr, tc, w["M"], 0, out=out, lse=lse)

    def split():
        q, k, v = (t.contiguous() for t in qkv.unbind(3))
        F.wattn_fwd(q, k, v, tr, tc, w["M"], 0, out=out, lse=lse)

    res = {"workload": name, "layout": "qkv [B, Hg, Wg, 3, heads, d]"}
    for tag, fn in (("packed_ms", packed), ("split_then_call_ms", split)):
        for _ in range(warmup):
            fn()
        warm_clocks(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[tag] = round(e0.elapsed_time(e1) / steps, 4)
    nbytes = 4 * out.numel() * out.element_size() + lse.numel() * 4
    res["packed_GBps"] = round(nbytes / (res["packed_ms"] * 1e-3) / 1e9, 1)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="flashswin_t_s1_p2_m32")
    ap.add_argument("--shift", type=int, default=None)
    ap.add_argument("--only", choices=["step", "fwd", "bwd"], default="step")
    ap.add_argument("--cpu-images", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--lowrank-only", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the batch would shard across GPUs, with one all-reduce of dtheta in the backward).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import vision_transformer_windowed_amd as F
    from vision_transformer_windowed_amd.inputs import WORKLOADS, workload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration:
        # a plain streaming kernel of known traffic: b = -a over 1 GiB of float32 (1 GiB read, 1 GiB written)
        n = 1 << 28
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.warmup + args.steps):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "kernel": "neg", "launches": args.warmup + args.steps}))
        return
    if args.lowrank_only:  # the rank-16 bias line alone (profiling runs)
        print(json.dumps(lowrank_step(dev, args.steps, args.warmup)), flush=True)
        return

    w = WORKLOADS[args.workload]
    shift = w["shifts"][0] if args.shift is None else args.shift
    M = w["M"]
    t_gen = time.perf_counter()
    x = workload_inputs(args.workload, with_dout=True)
    xd = {k: v.to(dev) for k, v in x.items()}
    gen_s = time.perf_counter() - t_gen
    q, k, v, dout = xd["q"], xd["k"], xd["v"], xd["dout"]
    tr, tc = xd["theta_row"], xd["theta_col"]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:4], device=dev, dtype=torch.float32)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(tr),
             torch.empty_like(tc))
    ws = torch.empty(max(F.bwd_workspace_bytes(q, M, shift), 1), device=dev, dtype=torch.uint8)
    # the forward's operand summary (16 bytes per window-head): the backward's prologue reads O and dO only
    stats = F.new_stats(q, M, shift)

    def fwd():
        F.wattn_fwd(q, k, v, tr, tc, M, shift, out=out, lse=lse, stats=stats)

    def bwd():
        F.wattn_bwd(q, k, v, out, dout, lse, tr, tc, M, shift, workspace=ws, grads=grads, stats=stats)

    fwd()  # the backward needs a valid LSE even in --only bwd mode
    for _ in range(args.warmup):
        if args.only in ("step", "fwd"):
            fwd()
        if args.only in ("step", "bwd"):
            bwd()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        if args.only in ("step", "fwd"):
            fwd()
        ev[i][1].record(stream)
        if args.only in ("step", "bwd"):
            bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_each = sorted(e[0].elapsed_time(e[1]) for e in ev)
    bwd_each = sorted(e[1].elapsed_time(e[2]) for e in ev)
    step_each = sorted(e[0].elapsed_time(e[2]) for e in ev)
    fwd_ms = sum(fwd_each) / K
    bwd_ms = sum(bwd_each) / K

    N = M * M
    nwh = w["B"] * (w["Hg"] // M) * (w["Wg"] // M) * w["heads"]
    fwd_flops = 4.0 * N * N * w["d"] * nwh
    bwd_flops = 10.0 * N * N * w["d"] * nwh
    step_flops = (fwd_flops if args.only != "bwd" else 0) + (bwd_flops if args.only != "fwd" else 0)
    ms_per_step = wall / K * 1e3
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    sha = kernel_source_sha()
    fwd_roofline = bwd_roofline = None
    if args.only != "bwd":
        fwd_tf = fwd_flops / (fwd_ms * 1e-3) / 1e12
        fwd_roofline = {"bound": "mfma", "achieved": round(fwd_tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(fwd_tf / BF16_MFMA_PEAK_TFLOPS, 4),
                        "traffic": read_traffic("wattn_fwd", args.workload, sha), "kernel": FWD_KERNEL.get(M),
                        "call": "wattn_fwd", "launches": CALL_LAUNCHES["wattn_fwd"], "launch_ms": round(fwd_ms, 4),
                        "flops_per_launch": fwd_flops, "kernel_source_sha": sha}
    if args.only != "fwd":
        bwd_tf = bwd_flops / (bwd_ms * 1e-3) / 1e12
        bwd_roofline = {"bound": "mfma", "achieved": round(bwd_tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(bwd_tf / BF16_MFMA_PEAK_TFLOPS, 4),
                        "traffic": read_traffic("wattn_bwd", args.workload, sha), "call": "wattn_bwd",
                        "launches": CALL_LAUNCHES["wattn_bwd"], "launch_ms": round(bwd_ms, 4),
                        "flops_per_call": bwd_flops, "kernel_source_sha": sha}
    roofline = fwd_roofline if fwd_roofline is not None else bwd_roofline
    m8 = packed = m16 = masked = bwd32 = mat = d64 = lowrank = None
    if not args.no_secondary and args.only == "step":
        m8 = m8_forward_roofline(dev, max(args.steps, 10), max(args.warmup, 2))
        packed = packed_forward(dev, max(args.steps, 10), max(args.warmup, 2))
        m16 = m16_step(dev, max(args.steps, 10), max(args.warmup, 2))
        masked = config_timing(dev, "flashswin_t_s2_shift16_m32", 16, ("fwd",), max(args.steps, 10),
                               max(args.warmup, 2))
        bwd32 = [config_timing(dev, "flashswin_t_s1_p2_m32_bwd", s, ("bwd",), max(args.steps, 10),
                               max(args.warmup, 2)) for s in WORKLOADS["flashswin_t_s1_p2_m32_bwd"]["shifts"]]
        d64 = [config_timing(dev, "wide_heads_s1_p2_m16_d64", s, ("fwd", "bwd"), max(args.steps, 10),
                             max(args.warmup, 2)) for s in WORKLOADS["wide_heads_s1_p2_m16_d64"]["shifts"]]
        mat = materialized_vs_fused(dev, 5, 1)
        lowrank = lowrank_step(dev, max(args.steps // 4, 3), 1)

    gpu_out = {"out": out, "lse": lse, "dq": grads[0], "dk": grads[1], "dv": grads[2]}
    cpu, parity = (None, None)
    if not args.no_cpu_baseline and args.only == "step":
        cpu, parity = cpu_baseline(x, w, shift, args.cpu_images, gpu_out)

    line = {
        "metric": "window-attn TFLOP/s + % MFMA/HBM roofline, FlashSwin-T stage-1 p=2 M=32",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w["dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": w["B"], "grid": [w["Hg"], w["Wg"]], "heads": w["heads"],
                   "d": w["d"], "M": M, "shift": shift, "pass": args.only,
                   "flops_per_step": step_flops},
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        # per-step event times of the timed steps: median and minimum (the means are above)
        "step_ms_median_min": [round(step_each[K // 2], 4), round(step_each[0], 4)],
        "fwd_ms_median_min": [round(fwd_each[K // 2], 4), round(fwd_each[0], 4)],
        "bwd_ms_median_min": [round(bwd_each[K // 2], 4), round(bwd_each[0], 4)],
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2) if args.only != "bwd" else None,
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2) if args.only != "fwd" else None,
        "window_heads_per_s": round(nwh / (ms_per_step * 1e-3), 1),
        "roofline": roofline,
        "bwd_roofline": bwd_roofline,
        "m8_fwd_roofline": m8,
        "m8_fwd_packed_qkv": packed,
        "m16_step": m16,
        "m32_shift16_fwd": masked,
        "m32_bwd_b32": bwd32,
        "materialized_vs_fused": mat,
        "d64_m16_step": d64,
        "lowrank_r16_m16_step": lowrank,
        "cpu_baseline": cpu,
        "parity_sample": parity,
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
