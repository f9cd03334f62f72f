#!/usr/bin/env python3
"""Throughput of the QLoRA hot path on one MI355X.

A step is one forward + backward pass of the Llama-3-8B-shaped QLoRA SwiGLU
MLP block (M = 8192 tokens, i.e. batch 2 x sequence 4096, hidden 4096,
intermediate 14336, LoRA rank 16, alpha 16, NF4 block 64 with fp32 absmax):
three QLoRA linears with the SwiGLU activation fused into the GEMM epilogues
and recomputed in the backward pass, plus every LoRA gradient.  Inputs are
seeded synthetic data of that shape, resident in HBM before timing starts.

Prints ONE JSON line: fwd+bwd TFLOP/s (model FLOPs 12 M D I + 18 M r (D+I)),
tokens/s, the roofline of the dominant GEMM kernel (timed with HIP events on
the library's stream through qlora_trace_install), the CPU oracle timed on a
bounded token sample of the same workload, and secondary lines for the
single-linear workloads (Llama-3-8B q_proj, and the skinny M=64 gate_proj
against the HBM roofline with its NF4 weights rotated to defeat the 256 MB
last-level cache), the 16-bit merge, the packed q/k/v adapters, RMSNorm and
the fused output head + cross-entropy.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="target oracle work for the CPU baseline")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (the known-size kernel "
                         "that calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--only", default=None, metavar="IDX|merge|rmsnorm|qkv|ce|rmsmlp",
                    help="profiling aid: time only workload config IDX (0-4; the skinny linear with 4 rotated "
                         "weight copies), the 16-bit merge, RMSNorm, the packed q/k/v adapters, the fused head + "
                         "cross-entropy or the RMSNorm + MLP forward (fused against two calls), and print its "
                         "own JSON line instead of the metric line")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_MIB"),
                    help="no GPU: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --copy-probe-mib run into profiles/traffic_<kernel>.txt")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(u16):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


# the sources a kernel kind's code and launch arguments come from (besides
# every header and the C ABI's launch code)
KERNEL_SOURCES = {"bgemm": ("qlora_bgemm.hip",), "qgemm": ("qlora_kernels.hip",),
                  "skinny": ("qlora_skinny.hip", "qlora_skinny2.hip")}


def kernel_source_sha(key=None):
    """Hash of the kernel sources: all of them, or those that build the kernel
    kind of a traffic key ('bgemm_fwd_swiglu', 'skinny_fwd', ...)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "qlora_fine_tuning_linear_amd", "csrc")
    own = KERNEL_SOURCES.get(key.split("_")[0]) if key else None
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".h", ".cpp")):
            continue
        if own is not None and not (f.endswith(".h") or f == "qlora_api.hip" or f in own):
            continue
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % key)
    if not os.path.exists(path):
        return None
    try:
        rec = json.loads("".join(l for l in open(path) if not l.startswith("#")))
    except ValueError:
        return None
    if rec.get("source_sha") != kernel_source_sha(key):
        return None
    return rec.get("hbm_bytes_per_launch")


KIND_OF_MODE = {0: "fwd", 1: "fwd_swiglu", 2: "bwd_dx", 3: "bwd_dh_swiglu", 4: "bwd_dx_dual"}
# committed rocprofv3 kernel statistics of each workload's bench command
PROFILE_OF_WORKLOAD = {"llama3_8b_mlp_m8192_r16": "kernel_stats_mlp_llama3_8b_m8192.md",
                       "llama3_70b_mlp_m4096_r64_dq": "kernel_stats_mlp_llama3_70b_m4096_dq.md"}


def kernel_key(csv_name):
    """'void qk::bgemm_kernel<1>(GemmArgs)' -> 'bgemm_fwd_swiglu', the skinny
    GEMMs -> 'skinny_fwd' / 'skinny_bwd' (None for other kernels)."""
    import re
    m = re.search(r"\b([qb]gemm)_kernel<(\d+)", csv_name)
    if m:
        return "%s_%s" % (m.group(1), KIND_OF_MODE[int(m.group(2))])
    m = re.search(r"\bskinny_(fwd2?|bwd)_kernel<", csv_name)
    if m:
        return "skinny_%s" % m.group(1).rstrip("2")
    return None


def summarize_traffic(fetch_csv, write_csv, copy_mib, command):
    """Per-launch HBM bytes of every GEMM kernel in a profiled bench run.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read
    for the plain copy of copy_mib MiB in the same run (the copy moves exactly
    that many bytes each way); the factors are recorded with the result."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return vals

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0

    def calib(vals):
        c = [v for k, vs in vals.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs
             if v > 0.5 * copy_kib]
        if not c:
            raise SystemExit("no copy dispatch of about %d MiB in the counter file" % copy_mib)
        return copy_kib / statistics.median(c)

    cf, cw = calib(f), calib(w)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    written = []
    for name in sorted(set(f) & set(w)):
        key = kernel_key(name)
        if key is None:
            continue
        fk, wk = statistics.median(f[name]), statistics.median(w[name])
        rec = {"kernel": name, "launches": len(f[name]), "fetch_kib_per_launch": fk, "write_kib_per_launch": wk,
               "copy_probe_mib": copy_mib, "calib_fetch": cf, "calib_write": cw,
               "hbm_bytes_per_launch": int(round((fk * cf + wk * cw) * 1024)), "source_sha": kernel_source_sha(key)}
        path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % key)
        with open(path, "w") as fh:
            fh.write("# HBM traffic per launch of %s (median over launches), from two rocprofv3 --pmc runs\n" % name)
            fh.write("# of the command below (FETCH_SIZE, then WRITE_SIZE), each scaled by the counter value\n")
            fh.write("# of the %d MiB plain copy in the same run.\n# command: %s\n" % (copy_mib, command))
            fh.write(json.dumps(rec, indent=1) + "\n")
        written.append(path)
    return written


def step_spread(fwd, bwd, n):
    """Median and p10 / p90 of n steps, each timed on its own with HIP events
    around the forward and the backward (after the K steps of the headline,
    which are timed as one block)."""
    import statistics
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n + 1)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[2 * i].record()
        fwd()
        ev[2 * i + 1].record()
        bwd()
    ev[2 * n].record()
    torch.cuda.synchronize()
    f = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)]
    b = [ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(n)]
    t = [x + y for x, y in zip(f, b)]

    def pct(v):
        q = statistics.quantiles(v, n=10, method="inclusive")
        return {"median": round(statistics.median(v), 4), "p10": round(q[0], 4), "p90": round(q[-1], 4)}

    return {"steps": n, "fwd_bwd_ms": pct(t), "fwd_ms": pct(f), "bwd_ms": pct(b)}


def profiled_avg_ms(profile, kernel_prefix):
    """Average duration (ms) of the kernel whose name starts with kernel_prefix
    in a committed rocprofv3 kernel-statistics summary (profiles/*.md), or None."""
    import re
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    for line in open(path):
        m = re.match(r"\|\s*`([^`]*)`\s*\|\s*(\d+)\s*\|\s*([0-9.]+)\s*\|", line)
        if m and re.sub(r"^\w+::", "", m.group(1)).startswith(kernel_prefix):
            return float(m.group(3)) / 1000.0
    return None


MODE_OF_KIND = {v: k for k, v in KIND_OF_MODE.items()}


def gemm_flops(kind, M, D, I, r):
    """Algorithmic FLOPs of one launch of each GEMM kind of the MLP step
    (main product + the rank-r LoRA epilogue product)."""
    return {
        "fwd_swiglu": 2 * M * D * (2 * I) + 2 * M * (2 * I) * r,
        "fwd": 2 * M * I * D + 2 * M * D * r,
        "bwd_dh_swiglu": 2 * M * D * I + 2 * M * I * r,
        "bwd_dx_dual": 2 * M * (2 * I) * D + 2 * M * D * (2 * r),
    }[kind]


def mlp_step_bench(q, synth, steps, warmup, idx=2):
    import torch
    cfg = synth.CONFIGS[idx]
    M, D, I, r = cfg.M, cfg.D, cfg.I, cfg.r
    log("building %s inputs" % cfg.name)
    inp = synth.mlp_inputs(cfg, synth.seed_of(idx))
    cb = torch.from_numpy(synth.nf4_codebook()).cuda()

    def lin(W, A, B):
        Wd = torch.from_numpy(W).cuda()
        w = q.nf4_quantize(Wd, cb, dq_group=cfg.dq_group)
        del Wd
        return q.QLoraLinear(w, dev_bf16(A), dev_bf16(B), cfg.alpha)

    P = q.QLoraMlp(lin(inp["Wg"], inp["Ag"], inp["Bg"]), lin(inp["Wu"], inp["Au"], inp["Bu"]),
                   lin(inp["Wd"], inp["Ad"], inp["Bd"]))
    X, dY = dev_bf16(inp["X"]), dev_bf16(inp["dY"])
    del inp
    Y = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty_like(Y)
    S = q.alloc_mlp_saved(P, M, "cuda")
    grads = dict(dA_g=torch.empty_like(P.gate.A), dB_g=torch.empty_like(P.gate.B),
                 dA_u=torch.empty_like(P.up.A), dB_u=torch.empty_like(P.up.B),
                 dA_d=torch.empty_like(P.down.A), dB_d=torch.empty_like(P.down.B))
    ws = torch.empty(q.qlora_mlp_workspace_bytes(P, M), dtype=torch.uint8, device="cuda")

    def step():
        q.qlora_mlp_fwd(P, X, Y=Y, saved=S, ws=ws)
        q.qlora_mlp_bwd(P, dY, X, S, dX=dX, grads=grads, ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    trace = q.LaunchTrace(capacity=8 * steps + 8)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with trace:
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    spread = step_spread(lambda: q.qlora_mlp_fwd(P, X, Y=Y, saved=S, ws=ws),
                         lambda: q.qlora_mlp_bwd(P, dY, X, S, dX=dX, grads=grads, ws=ws), max(100, steps))
    per_kind, kname = {}, {}
    for kind, kernel, d in trace.launches():
        per_kind.setdefault(kind, []).append(d)
        kname[kind] = kernel
    trace.close()
    flops = 12 * M * D * I + 18 * M * r * (D + I)
    dom = max(per_kind, key=lambda k: sum(per_kind[k]))
    dom_ms = sum(per_kind[dom]) / len(per_kind[dom])
    dom_flops = gemm_flops(dom, M, D, I, r)
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    dom_kernel = "%s<%s>" % (kname[dom], dom)
    traffic = stored_traffic("%s_%s" % (kname[dom].split("_")[0], dom))
    kernels = {"%s<%s>" % (kname[k], k): {"launches_per_step": len(v) / steps, "avg_ms": sum(v) / len(v),
                                          "tflops": gemm_flops(k, M, D, I, r) / (sum(v) / len(v) * 1e-3) / 1e12}
               for k, v in per_kind.items()}
    return dict(cfg=cfg, ms=ms, wall=wall, flops=flops, dom=dom, dom_kernel=dom_kernel, dom_ms=dom_ms,
                dom_flops=dom_flops, achieved=achieved, traffic=traffic, kernels=kernels, spread=spread)


def linear_bench(q, synth, idx, steps, warmup, rotate=1):
    """fwd+bwd of one QLoRA linear; with rotate > 1 the NF4 weight is cycled
    over that many copies so that it streams from HBM every step."""
    import torch
    cfg = synth.CONFIGS[idx]
    M, K, N, r = cfg.M, cfg.K, cfg.N, cfg.r
    inp = synth.linear_inputs(cfg, synth.seed_of(idx))
    cb = torch.from_numpy(synth.nf4_codebook()).cuda()
    Wd = torch.from_numpy(inp["W0"]).cuda()
    w = q.nf4_quantize(Wd, cb, dq_group=cfg.dq_group)
    del Wd
    A, B = dev_bf16(inp["A"]), dev_bf16(inp["B"])
    Ls = [q.QLoraLinear(w, A, B, cfg.alpha)]
    for _ in range(rotate - 1):
        w2 = q.Nf4Weight(w.codes.clone(), None if w.absmax is None else w.absmax.clone(),
                         None if w.absmax_q is None else w.absmax_q.clone(),
                         None if w.absmax_scale is None else w.absmax_scale.clone(), cb, N, K, cfg.dq_group)
        Ls.append(q.QLoraLinear(w2, A, B, cfg.alpha))
    X, dY = dev_bf16(inp["X"]), dev_bf16(inp["dY"])
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    XA = torch.empty(M, r, dtype=torch.float32, device="cuda")
    dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dA, dB = torch.empty_like(A), torch.empty_like(B)
    ws = torch.empty(q.qlora_linear_workspace_bytes(Ls[0], M), dtype=torch.uint8, device="cuda")

    def step(i):
        # With several weight copies the forward and the backward of a step use
        # different ones, and a copy comes back only after the others have
        # streamed: nothing of it is left in the 256 MB last-level cache, as in
        # training, where every other layer runs between a layer's forward and
        # its backward.  The copies hold the same values.
        Lf, Lb = Ls[(2 * i) % len(Ls)], Ls[(2 * i + 1) % len(Ls)]
        q.qlora_linear_fwd(Lf, X, Y=Y, XA=XA, ws=ws)
        q.qlora_linear_bwd(Lb, dY, X, XA, dX=dX, dA=dA, dB=dB, ws=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 4 * M * N * K + 6 * M * r * (N + K)
    wbytes = N * K // 2 + (N * K // 64) * (1 if cfg.dq_group else 4) + \
        (4 * (-(-(N * K // 64) // cfg.dq_group)) if cfg.dq_group else 0)
    # algorithmic bytes: the NF4 weight once per pass; activations, LoRA
    # parameters and gradients read or written once
    fwd_bytes = wbytes + 2 * M * K + 2 * r * K + 2 * N * r + 2 * M * N + 4 * M * r
    bwd_bytes = wbytes + 2 * M * N + 2 * M * K + 4 * M * r + 2 * r * K + 2 * N * r + \
        2 * M * K + 2 * r * K + 2 * N * r
    total_bytes = fwd_bytes + bwd_bytes
    return dict(workload=cfg.name, ms_per_step=ms, tflops=flops / (ms * 1e-3) / 1e12,
                frac_bf16_peak=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                tokens_per_s=M / (ms * 1e-3), algorithmic_bytes=total_bytes,
                hbm_gbs=total_bytes / (ms * 1e-3) / 1e9,
                frac_hbm_peak=total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, weight_copies=rotate,
                mall_defeated=("forward and backward on different weight copies, each reused after %d others"
                               % (rotate - 1)) if rotate > 1 else None)


def merge_bench(q, synth, steps, warmup, copies=3):
    """qlora_merge of the Llama-3-8B gate weight (14336 x 4096, r = 16) into
    bf16, cycled over `copies` weights and outputs (more bytes than the 256 MB
    last-level cache); HBM-bound: algorithmic bytes = codes + absmax + A + B
    read once, the 16-bit weight written once."""
    import torch
    idx = 2
    cfg = synth.CONFIGS[idx]
    inp = synth.mlp_inputs(cfg, synth.seed_of(idx), M=1)
    N, K, r = cfg.I, cfg.D, cfg.r
    cb = torch.from_numpy(synth.nf4_codebook()).cuda()
    Wd = torch.from_numpy(inp["Wg"]).cuda()
    w = q.nf4_quantize(Wd, cb, dq_group=cfg.dq_group)
    del Wd
    A, B = dev_bf16(inp["Ag"]), dev_bf16(inp["Bg"])
    del inp
    Ls = [q.QLoraLinear(w, A, B, cfg.alpha)]
    for _ in range(copies - 1):
        w2 = q.Nf4Weight(w.codes.clone(), None if w.absmax is None else w.absmax.clone(),
                         None if w.absmax_q is None else w.absmax_q.clone(),
                         None if w.absmax_scale is None else w.absmax_scale.clone(), cb, N, K, cfg.dq_group)
        Ls.append(q.QLoraLinear(w2, A, B, cfg.alpha))
    outs = [torch.empty(N, K, dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    for i in range(warmup):
        q.qlora_merge(Ls[i % copies], out=outs[i % copies])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        q.qlora_merge(Ls[i % copies], out=outs[i % copies])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = N * K // 2 + (N * K // 64) * (1 if cfg.dq_group else 4) + 2 * r * K + 2 * N * r + 2 * N * K
    return dict(workload="merge_16bit_llama3_8b_gate_14336x4096_r16", ms_per_call=ms, algorithmic_bytes=nbytes,
                hbm_gbs=nbytes / (ms * 1e-3) / 1e9, frac_hbm_peak=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                weight_copies=copies)


def grouped_bench(q, synth, steps, warmup, M=4096, K=4096, Ns=(4096, 1024, 1024), r=16, alpha=16.0):
    """Packed q/k/v adapters of Llama-3-8B (K=4096; q 4096, k and v 1024 rows
    each, r=16) at 4096 tokens, fwd+bwd through qlora_grouped_fwd/_bwd; the
    same work as three separate linear calls is timed beside it for context."""
    import torch
    cb = torch.from_numpy(synth.nf4_codebook()).cuda()
    Nt, G = sum(Ns), len(Ns)
    Wd = torch.from_numpy(synth.weight_rows(7, 2, K, 0, Nt)).cuda()
    w = q.nf4_quantize(Wd, cb)
    bound = 1.0 / K ** 0.5
    A = dev_bf16(synth.uniform_bf16(7, 3, G * r * K, -bound, bound).reshape(G * r, K))
    Bs = [dev_bf16(synth.normal_bf16(7, 10 + g, Ns[g] * r, 0.0, 0.01).reshape(Ns[g], r)) for g in range(G)]
    X = dev_bf16(synth.normal_bf16(7, 4, M * K).reshape(M, K))
    dY = dev_bf16(synth.normal_bf16(7, 5, M * Nt).reshape(M, Nt))
    Q = q.QLoraGrouped(w, A, Bs, [alpha] * G)
    ws = torch.empty(q.qlora_grouped_workspace_bytes(Q, M), dtype=torch.uint8, device="cuda")
    # the separate layers: each group's rows quantized on their own (same codes)
    Ls, off = [], 0
    for g in range(G):
        wg = q.nf4_quantize(Wd[off:off + Ns[g]].contiguous(), cb)
        Ls.append(q.QLoraLinear(wg, A[g * r:(g + 1) * r].contiguous(), Bs[g], alpha))
        off += Ns[g]
    del Wd
    dYs = [dY[:, sum(Ns[:g]):sum(Ns[:g + 1])].contiguous() for g in range(G)]
    wss = [torch.empty(q.qlora_linear_workspace_bytes(L, M), dtype=torch.uint8, device="cuda") for L in Ls]

    def grouped_step():
        Y, XA = q.qlora_grouped_fwd(Q, X, ws=ws)
        q.qlora_grouped_bwd(Q, dY, X, XA, ws=ws)

    def separate_step():
        for g in range(G):
            Y, XA = q.qlora_linear_fwd(Ls[g], X, ws=wss[g])
            q.qlora_linear_bwd(Ls[g], dYs[g], X, XA, ws=wss[g])

    def timed(f):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    g_ms, s_ms = timed(grouped_step), timed(separate_step)
    flops = sum(4 * M * n * K + 6 * M * r * (n + K) for n in Ns)
    return dict(workload="grouped_qkv_llama3_8b_m%d_r%d" % (M, r), ms_per_step=g_ms,
                tflops=flops / (g_ms * 1e-3) / 1e12, frac_bf16_peak=flops / (g_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                separate_layers_ms=s_ms)


def rmsnorm_bench(q, synth, steps, warmup, M=8192, D=4096, eps=1e-5):
    """rmsnorm_fwd and rmsnorm_bwd (with dw) at the Llama-3-8B hidden size and
    the MLP workload's token count; HBM-bound.  Algorithmic bytes: forward
    reads X and writes Y (+ rstd); backward reads dY and X and writes dX (+ rstd,
    w, dw)."""
    import torch
    X = dev_bf16(synth.normal_bf16(1, 40, M * D).reshape(M, D))
    dY = dev_bf16(synth.normal_bf16(1, 41, M * D).reshape(M, D))
    w = dev_bf16(synth.normal_bf16(1, 42, D, 1.0, 0.1))
    Y, rstd = torch.empty_like(X), torch.empty(M, dtype=torch.float32, device="cuda")
    dX, dw = torch.empty_like(X), torch.empty(D, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(int(q.load_library().rmsnorm_bwd_workspace_bytes(M, D)), 256), dtype=torch.uint8,
                     device="cuda")

    def timed(f):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    f_ms = timed(lambda: q.rmsnorm_fwd(X, w, eps, Y=Y, rstd=rstd))
    b_ms = timed(lambda: q.rmsnorm_bwd(dY, X, w, rstd, dX=dX, dw=dw, ws=ws))
    fb = 2 * M * D * 2 + 4 * M + 2 * D
    bb = 3 * M * D * 2 + 4 * M + 2 * D + 4 * D
    return dict(workload="rmsnorm_m%d_d%d" % (M, D), fwd_ms=f_ms, bwd_ms=b_ms,
                fwd_hbm_gbs=fb / (f_ms * 1e-3) / 1e9, bwd_hbm_gbs=bb / (b_ms * 1e-3) / 1e9,
                fwd_frac_hbm_peak=fb / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                bwd_frac_hbm_peak=bb / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)


def rms_mlp_bench(q, synth, steps, warmup, idx=2, eps=1e-5):
    """RMSNorm + MLP forward of the Llama-3-8B-shaped block: the two-call path
    (rmsnorm_fwd writes the normalised input, qlora_mlp_fwd reads it) against
    qlora_mlp_fwd_rmsnorm, with and without the normalised input kept."""
    import torch
    cfg = synth.CONFIGS[idx]
    M, D = cfg.M, cfg.D
    inp = synth.mlp_inputs(cfg, synth.seed_of(idx))
    cb = torch.from_numpy(synth.nf4_codebook()).cuda()

    def lin(W, A, B):
        Wd = torch.from_numpy(W).cuda()
        w = q.nf4_quantize(Wd, cb, dq_group=cfg.dq_group)
        del Wd
        return q.QLoraLinear(w, dev_bf16(A), dev_bf16(B), cfg.alpha)

    P = q.QLoraMlp(lin(inp["Wg"], inp["Ag"], inp["Bg"]), lin(inp["Wu"], inp["Au"], inp["Bu"]),
                   lin(inp["Wd"], inp["Ad"], inp["Bd"]))
    X = dev_bf16(inp["X"])
    del inp
    w = dev_bf16(synth.normal_bf16(1, 42, D, 1.0, 0.1))
    Y, Xn = torch.empty(M, D, dtype=torch.bfloat16, device="cuda"), torch.empty(M, D, dtype=torch.bfloat16,
                                                                                device="cuda")
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    S = q.alloc_mlp_saved(P, M, "cuda")
    ws = torch.empty(max(q.qlora_mlp_workspace_bytes(P, M), q.qlora_mlp_rmsnorm_workspace_bytes(P, M)),
                     dtype=torch.uint8, device="cuda")

    def timed(f):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def two_call():
        q.rmsnorm_fwd(X, w, eps, Y=Xn, rstd=rstd)
        q.qlora_mlp_fwd(P, Xn, Y=Y, saved=S, ws=ws)

    t2 = timed(two_call)
    tf = timed(lambda: q.qlora_mlp_fwd_rmsnorm(P, X, w, eps, Y=Y, saved=S, rstd=rstd, ws=ws))
    tx = timed(lambda: q.qlora_mlp_fwd_rmsnorm(P, X, w, eps, Y=Y, saved=S, rstd=rstd, Xn=Xn, ws=ws))
    return dict(workload="rmsnorm_mlp_fwd_%s" % cfg.name, two_call_ms=t2, fused_ms=tf, fused_keep_xn_ms=tx)


def ce_bench(q, synth, steps, warmup, T=4096, D=4096, V=128256, chunk=1024):
    """qlora_linear_ce at the page's example (4096 tokens, hidden 4096, a 128256
    class vocabulary): loss and dX in token chunks.  FLOPs: the logits and the
    dX product, 2 T D V each.  Also reported: the call's workspace (one chunk of
    bf16 logits, the transposed head, dX partials) against the [T, V] fp32 logit
    matrix an unfused loss would hold."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    X = torch.randn(T, D, device="cuda", generator=g).bfloat16()
    W = (torch.randn(V, D, device="cuda", generator=g) * (2.0 / D ** 0.5)).bfloat16()
    t = torch.randint(0, V, (T,), device="cuda", generator=g, dtype=torch.int32)
    dX = torch.empty_like(X)
    nbytes = q.qlora_linear_ce_workspace_bytes(T, D, V, chunk, True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    f = lambda: q.qlora_linear_ce(X, W, t, chunk=chunk, dX=dX, ws=ws)
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        f()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 4.0 * T * D * V
    return dict(workload="linear_ce_t%d_d%d_v%d_chunk%d" % (T, D, V, chunk), ms_per_call=ms,
                tflops=flops / (ms * 1e-3) / 1e12, frac_bf16_peak=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                tokens_per_s=T / (ms * 1e-3), workspace_gb=nbytes / 1e9, unfused_fp32_logits_gb=T * V * 4 / 1e9)


def cpu_baseline(synth, target_s):
    """The oracle (fp64 numpy) on the first tokens of the same MLP workload."""
    import numpy as np
    from oracle import nf4 as onf4
    from oracle import qlora as oq
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    cfg = synth.CONFIGS[2]
    cb = synth.nf4_codebook()
    log("cpu baseline: oracle quantization of the three weights")
    inp = synth.mlp_inputs(cfg, synth.seed_of(2), M=256)
    W = {}
    for k in ("Wg", "Wu", "Wd"):
        W[k] = onf4.dequantize(onf4.quantize(inp[k], cb, dq_group=cfg.dq_group), cb).astype(np.float64)
        del inp[k]
    args = (W["Wg"], W["Wu"], W["Wd"], inp["Ag"], inp["Bg"], inp["Au"], inp["Bu"], inp["Ad"], inp["Bd"])

    def run(m):
        x, dy = inp_rows["X"][:m], inp_rows["dY"][:m]
        t = time.perf_counter()
        f = oq.mlp_forward(x, *args, cfg.alpha)
        oq.mlp_backward(dy, x, f["G"], f["U"], *args, cfg.alpha)
        return time.perf_counter() - t

    probe_m = 128
    inp_rows = synth.mlp_inputs(cfg, synth.seed_of(2), M=probe_m, with_weights=False)
    t_probe = run(probe_m)
    m = int(min(cfg.M, max(probe_m, probe_m * target_s / max(t_probe, 1e-3))))
    m = max(64, (m // 64) * 64)
    inp_rows = synth.mlp_inputs(cfg, synth.seed_of(2), M=m, with_weights=False)
    t = run(m)
    flops = 12 * m * cfg.D * cfg.I + 18 * m * cfg.r * (cfg.D + cfg.I)
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": "first %d of %d tokens of %s, fwd+bwd, fp64 numpy oracle (weights dequantized by the "
                      "oracle), %.1f s" % (m, cfg.M, cfg.name, t),
            "tokens_per_s": m / t}


def mlp_line(cfg, r):
    """Secondary line of an MLP workload: fwd+bwd time, TFLOP/s, fraction of
    the bf16 peak, tokens/s, and its dominant GEMM kernel."""
    return {"workload": cfg.name, "ms_per_step": round(r["ms"], 4),
            "tflops": round(r["flops"] / (r["ms"] * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(r["flops"] / (r["ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "tokens_per_s": round(cfg.M / (r["ms"] * 1e-3), 1),
            "dominant_kernel": r["dom_kernel"], "dominant_avg_ms": round(r["dom_ms"], 4),
            "dominant_frac_bf16_peak": round(r["achieved"] / BF16_PEAK_TFLOPS, 4),
            "spread": r["spread"],
            "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in r["kernels"].items()}}


def main():
    a = parse()
    if a.summarize_traffic:
        fetch_csv, write_csv, mib = a.summarize_traffic
        cmd = os.environ.get("TRAFFIC_COMMAND", "(see the profiles README)")
        for p in summarize_traffic(fetch_csv, write_csv, int(mib), cmd):
            print(p)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the QLoRA linear / MLP path here runs on a single GPU "
              "(data-parallel sharding over tokens is a design note of the repository, not launched). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import qlora_fine_tuning_linear_amd as q
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    q.load_library()
    if a.copy_probe_mib > 0:
        n = a.copy_probe_mib * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if a.only in ("merge", "rmsnorm", "qkv", "ce", "rmsmlp"):
        fn = {"merge": merge_bench, "rmsnorm": rmsnorm_bench, "qkv": grouped_bench, "ce": ce_bench,
              "rmsmlp": rms_mlp_bench}[a.only]
        s = fn(q, synth, max(10, a.steps), a.warmup)
        print(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()}), flush=True)
        return
    if a.only is not None:
        a.only = int(a.only)
        cfg = synth.CONFIGS[a.only]
        if cfg.kind == "mlp":
            line = mlp_line(cfg, mlp_step_bench(q, synth, a.steps, a.warmup, idx=a.only))
        else:
            s = linear_bench(q, synth, a.only, a.steps, a.warmup, rotate=4 if a.only == 4 else 1)
            line = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()}
        print(json.dumps(line), flush=True)
        return
    r = mlp_step_bench(q, synth, a.steps, a.warmup)
    cfg = r["cfg"]
    value = r["flops"] / (r["ms"] * 1e-3) / 1e12
    out = {
        "metric": "QLoRA fwd+bwd TFLOP/s (SwiGLU MLP block, all three projections QLoRA)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.M, "hidden": cfg.D, "intermediate": cfg.I,
                   "lora_rank": cfg.r, "lora_alpha": cfg.alpha, "nf4_block": cfg.blocksize,
                   "double_quant": bool(cfg.dq_group), "parallelism": "single-gpu"},
        "tokens_per_s": round(cfg.M / (r["ms"] * 1e-3), 1),
        "frac_bf16_peak": round(value / BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": r["dom_kernel"],
                     "achieved": round(r["achieved"], 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(r["achieved"] / BF16_PEAK_TFLOPS, 4), "traffic": r["traffic"],
                     "flops_per_launch": r["dom_flops"], "avg_launch_ms": round(r["dom_ms"], 4)},
        "spread": r["spread"],
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in r["kernels"].items()},
    }
    # the same kernel's average in the committed rocprofv3 kernel statistics of
    # this workload, and the fraction it gives
    prof = profiled_avg_ms(PROFILE_OF_WORKLOAD.get(cfg.name, ""),
                           "bgemm_kernel<%d," % MODE_OF_KIND[r["dom"]])
    if prof:
        out["roofline"]["profiled_avg_launch_ms"] = round(prof, 4)
        out["roofline"]["profiled_frac"] = round(r["dom_flops"] / (prof * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
        out["roofline"]["profile"] = "profiles/" + PROFILE_OF_WORKLOAD[cfg.name]
    if not a.no_secondary:
        sec = []
        log("secondary: %s" % synth.CONFIGS[3].name)
        sec.append(mlp_line(synth.CONFIGS[3], mlp_step_bench(q, synth, max(5, a.steps // 2), min(a.warmup, 3),
                                                             idx=3)))
        for idx, steps, rot in ((0, max(20, a.steps), 1), (1, max(5, a.steps), 1), (4, max(10, a.steps), 4)):
            log("secondary: %s" % synth.CONFIGS[idx].name)
            s = linear_bench(q, synth, idx, steps, a.warmup, rotate=rot)
            sec.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()})
        log("secondary: merge")
        s = merge_bench(q, synth, max(10, a.steps), a.warmup)
        sec.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()})
        log("secondary: grouped q/k/v")
        s = grouped_bench(q, synth, max(5, a.steps), a.warmup)
        sec.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()})
        log("secondary: rmsnorm")
        s = rmsnorm_bench(q, synth, max(20, a.steps), a.warmup)
        sec.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()})
        log("secondary: rmsnorm + MLP forward, fused and two-call")
        s = rms_mlp_bench(q, synth, max(10, a.steps), a.warmup)
        sec.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()})
        log("secondary: linear + cross-entropy")
        s = ce_bench(q, synth, max(3, a.steps // 3), min(a.warmup, 2))
        sec.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()})
        out["secondary"] = sec
    out["cpu_baseline"] = None if a.no_cpu_baseline else cpu_baseline(synth, a.cpu_seconds)
    if out["cpu_baseline"]:
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 5)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
