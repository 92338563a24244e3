#!/usr/bin/env python3
"""Benchmark of the LittleBit layer's decode path on one MI355X.

Workload (the headline configuration): the Llama2-7B-shaped MLP
up-projection, 4096 -> 11008, two branches of rank 1472 (about 1.0 bit per
weight), fp16 scales ~U[0.5, 1.5], one fp16 token ~N(0, 1) per call (batch-1
decode GEMV).  Inputs are synthetic and seeded (binary_rank_gemv_amd.synth for
the first copy of the layer, torch's seeded GPU generator for the others).

One step = one littlebit_linear_fwd call (every step of the layer for one
token).  To measure HBM rather than the 256 MB last-level cache, the timed
loop cycles through distinct copies of the layer totalling >= 1 GB; the calls
are captured once in a HIP graph and replayed.

Prints one JSON line (see the keys below), including a roofline object for the
decode kernel and a cpu_baseline object for the float64 CPU oracle timed on
a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix-core peak


def algorithmic_bytes(m, n, ranks, batch):
    """Unpadded sign bits + fp16 scales + fp16 x + fp16 y for one call."""
    bits = sum(r * (m + n) for r in ranks)
    scales = sum(m + n + r for r in ranks) * 2
    return bits // 8 + scales + 2 * batch * n + 2 * batch * m


def time_eager(torch, call, steps, warmup):
    """Milliseconds per call of `call` launched back to back (no graph)."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        call()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def time_graph(torch, calls, steps, warmup):
    """Capture a HIP graph over one cycle of `calls` (plus remainders) and
    return milliseconds per call over `steps` timed calls."""
    n = len(calls)

    def capture(k):
        gr = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in calls[:k]:
                c()
            torch.cuda.synchronize()
            with torch.cuda.graph(gr, stream=s):
                for c in calls[:k]:
                    c()
        torch.cuda.current_stream().wait_stream(s)
        return gr

    graphs = {n: capture(n)}
    for k in {steps % n, warmup % n} - {0}:
        graphs[k] = capture(k)

    def run(k_steps):
        reps, rem = divmod(k_steps, n)
        for _ in range(reps):
            graphs[n].replay()
        if rem:
            graphs[rem].replay()

    run(warmup)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    run(steps)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def copies_for(bytes_per_copy, total_bytes):
    return max(1, int(np.ceil(total_bytes / bytes_per_copy)))


def layer_bytes(layer):
    return sum(b.v_bits.numel() + b.u_bits.numel() + 2 * (b.h.numel() + b.l.numel() + b.g.numel())
               for b in layer.branches)


def extra_measurements(lb, torch, synth, args):
    """The other configurations of the metric: the 13B block at batch 1 (time
    per block), the 70B up-projection at batch 1 and 16, and the 2048-token
    prefill of the 7B up-projection (matrix-core utilisation)."""
    out = {}
    # 13B-shaped block, one call = the 7 projections for one token
    for setting in ("0.55", "0.1"):
        shapes = synth.block13b_shapes(setting)
        one = [make_copy(lb, torch, sh, 5000 + i) for i, sh in enumerate(shapes)]
        per_block = sum(layer_bytes(l) for l in one)
        nb = copies_for(per_block, args.copies_gb * 1e9)
        blocks = [one] + [[make_copy(lb, torch, sh, 6000 + 7 * j + i) for i, sh in enumerate(shapes)]
                          for j in range(nb - 1)]
        xs = [torch.randn((1, n), device="cuda").half() for n in (5120, 5120, 5120, 13824)]
        ys = [torch.empty((1, sh.m), dtype=torch.float16, device="cuda") for sh in shapes]
        ws = torch.zeros(lb.littlebit_block_workspace_bytes(one, 1), dtype=torch.uint8, device="cuda")
        calls = [lambda b=b: lb.littlebit_block_fwd(b, *xs, outs=ys, workspace=ws) for b in blocks]
        ms = time_graph(torch, calls, max(4 * nb, 400), 2 * nb)
        abytes = sum(algorithmic_bytes(sh.m, sh.n, sh.ranks, 1) for sh in shapes)
        out[f"block13b_{setting}bpw_b1"] = {"us_per_block": round(ms * 1e3, 3), "tokens_per_s": round(1e3 / ms, 1),
                                             "algorithmic_bytes": abytes,
                                             "hbm_gbs": round(abytes / (ms * 1e-3) / 1e9, 1),
                                             "distinct_copies": nb}
        del blocks, one
        torch.cuda.empty_cache()
    # 70B-shaped up-projection
    sh = synth.UP70B
    one = make_copy(lb, torch, sh, 7000)
    nc = copies_for(layer_bytes(one), args.copies_gb * 1e9)
    lays = [one] + [make_copy(lb, torch, sh, 7001 + i) for i in range(nc - 1)]
    for batch in (1, 16):
        x = torch.randn((batch, sh.n), device="cuda").half()
        y = torch.empty((batch, sh.m), dtype=torch.float16, device="cuda")
        ws = torch.zeros(lb.littlebit_linear_workspace_bytes(one, batch), dtype=torch.uint8, device="cuda")
        calls = [lambda l=l: lb.littlebit_linear_fwd(l, x, out=y, workspace=ws) for l in lays]
        ms = time_graph(torch, calls, max(8 * nc, 800), 2 * nc)
        abytes = algorithmic_bytes(sh.m, sh.n, sh.ranks, batch)
        out[f"up70b_b{batch}"] = {"us_per_call": round(ms * 1e3, 3), "tokens_per_s": round(batch * 1e3 / ms, 1),
                                  "algorithmic_bytes": abytes, "hbm_gbs": round(abytes / (ms * 1e-3) / 1e9, 1),
                                  "distinct_copies": nc}
    del lays, one
    torch.cuda.empty_cache()
    # prefill: 2048 tokens of the 7B up-projection (compute-bound; one copy)
    sh, M = synth.UP7B, synth.PREFILL_TOKENS
    lay = make_copy(lb, torch, sh, 8000)
    x = torch.randn((M, sh.n), device="cuda").half()
    y = torch.empty((M, sh.m), dtype=torch.float16, device="cuda")
    ws = torch.zeros(lb.littlebit_linear_workspace_bytes(lay, M), dtype=torch.uint8, device="cuda")
    ms = time_graph(torch, [lambda: lb.littlebit_linear_fwd(lay, x, out=y, workspace=ws)], 50, 5)
    flops = 2 * M * sum(r * (sh.m + sh.n) for r in sh.ranks)
    tflops = flops / (ms * 1e-3) / 1e12
    out["prefill_7b_up_2048"] = {"us_per_call": round(ms * 1e3, 2), "tokens_per_s": round(M * 1e3 / ms, 1),
                                 "flops": flops, "tflops": round(tflops, 1),
                                 "mfma_util": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                                 "peak_tflops": FP16_MFMA_PEAK_TFLOPS,
                                 "dense_fp16_library": dense_gemm_context(torch, M, sh.n, sum(sh.ranks), sh.m)}
    return out


def dense_gemm_context(torch, M, n, rsum, m):
    """Context for the prefill figure: the same two contractions as plain
    dense fp16 GEMMs through torch.matmul (the vendor GEMM library), with no
    sign expansion, in the faster of two operand layouts each.  Not part of
    the layer."""
    res = {}
    for name, (a_rows, k, b_cols) in (("gemm1", (M, n, rsum)), ("gemm2", (M, rsum, m))):
        a = torch.randn((a_rows, k), device="cuda").half()
        b_kn = torch.randn((k, b_cols), device="cuda").half()
        b_nk = torch.randn((b_cols, k), device="cuda").half()
        c = torch.empty((a_rows, b_cols), device="cuda", dtype=torch.float16)
        best = min(time_eager(torch, lambda: torch.matmul(a, b_kn, out=c), 30, 5),
                   time_eager(torch, lambda: torch.matmul(a, b_nk.t(), out=c), 30, 5))
        res[name + "_us"] = round(best * 1e3, 2)
        del a, b_kn, b_nk, c
    total = res["gemm1_us"] + res["gemm2_us"]
    flops = 2 * M * rsum * (n + m)
    res["total_us"] = round(total, 2)
    res["mfma_util"] = round(flops / (total * 1e-6) / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4)
    return res


def make_copy(lb, torch, shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    branches = []
    for r in shape.ranks:
        U = torch.randn((shape.m, r), device="cuda", generator=g)
        V = torch.randn((shape.n, r), device="cuda", generator=g)
        h = (torch.rand(shape.m, device="cuda", generator=g) + 0.5).half()
        l = (torch.rand(r, device="cuda", generator=g) + 0.5).half()
        gg = (torch.rand(shape.n, device="cuda", generator=g) + 0.5).half()
        branches.append(lb.LittleBitBranch(v_bits=lb.littlebit_pack(V, True),
                                           u_bits=lb.littlebit_pack(U, False),
                                           h=h, l=l, g=gg, r=r))
        del U, V
    return lb.LittleBitLayer(m=shape.m, n=shape.n, branches=branches)


PMC_SUMMARY = os.path.join(ROOT, "profiles", "lb_decode_7b_up_b1_pmc.md")
KERNEL_SOURCES = [os.path.join(ROOT, "binary_rank_gemv_amd", "csrc", f) for f in ("decode.hip", "lb_common.h")]


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    the decode kernel's sources have changed since the counters were taken."""
    import hashlib
    import re
    try:
        text = open(PMC_SUMMARY).read()
        h = hashlib.sha256(b"".join(open(f, "rb").read() for f in KERNEL_SOURCES)).hexdigest()
    except OSError:
        return None
    mt = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    mh = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    if not (mt and mh) or mh.group(1) != h:
        return None
    return int(mt.group(1))


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            return max(d["num_threads"] for d in info)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(shape, branches, x, seconds, y_gpu):
    """Time the float64 oracle on the host: whole batch-1 calls of its factored
    form, repeated for about `seconds`, plus a sample of output rows of its
    dense definition (rows of W built per call) for about a third of that.
    The oracle's result is also compared with the GPU's on the same input."""
    import oracle
    calls, t0 = 0, time.perf_counter()
    while calls < 3 or time.perf_counter() - t0 < seconds:
        yr = oracle.factored_forward(x, branches)
        calls += 1
    dt = time.perf_counter() - t0
    agreement = {"rel_l2": float(np.linalg.norm(y_gpu - yr) / np.linalg.norm(yr)),
                 "max_err_over_rms": float(np.max(np.abs(y_gpu - yr)) / np.sqrt(np.mean(yr ** 2)))}
    rows, t1 = 0, time.perf_counter()
    while rows < shape.m and (rows == 0 or time.perf_counter() - t1 < seconds / 3):
        blk = np.arange(rows, min(rows + 344, shape.m))
        oracle.rows_forward(x, branches, blk)
        rows += len(blk)
    dtd = time.perf_counter() - t1
    return {"value": round(x.shape[0] * calls / dt, 3), "unit": "tokens/s", "cores": int(_blas_threads()),
            "kind": "oracle",
            "sample": f"{calls} whole batch-1 calls of the float64 factored oracle in {dt:.1f} s",
            "dense_definition": {"value": round(x.shape[0] * (rows / shape.m) / dtd, 4), "unit": "tokens/s",
                                 "sample": f"{rows} of {shape.m} output rows of the dense float64 definition "
                                           f"in {dtd:.1f} s, scaled by {shape.m}/{rows}"},
            "gpu_agreement": agreement}


def bpw_sweep(lb, torch, synth, args):
    """Decode time of the 70B-shaped up-projection (8192 -> 28672, two
    branches) at 1.0, 0.8, 0.55, 0.3 and 0.1 bits per weight, batch 1 and 16,
    beside torch's fp16 dense product y = x W^T on the same shape (context)."""
    rows = []
    for bpw in sorted(synth.UP70B_BPW_SWEEP, reverse=True):
        sh = synth.up70b_at_bpw(bpw)
        one = make_copy(lb, torch, sh, 9000)
        nc = copies_for(layer_bytes(one), args.copies_gb * 1e9)
        lays = [one] + [make_copy(lb, torch, sh, 9001 + i) for i in range(nc - 1)]
        row = {"bpw": bpw, "rank": sh.ranks[0], "weight_bytes": layer_bytes(one), "distinct_copies": nc}
        for batch in (1, 16):
            x = torch.randn((batch, sh.n), device="cuda").half()
            y = torch.empty((batch, sh.m), dtype=torch.float16, device="cuda")
            ws = torch.zeros(lb.littlebit_linear_workspace_bytes(one, batch), dtype=torch.uint8, device="cuda")
            calls = [lambda l=l: lb.littlebit_linear_fwd(l, x, out=y, workspace=ws) for l in lays]
            ms = time_graph(torch, calls, max(8 * nc, 400), 2 * nc)
            abytes = algorithmic_bytes(sh.m, sh.n, sh.ranks, batch)
            row[f"b{batch}"] = {"us_per_call": round(ms * 1e3, 3), "tokens_per_s": round(batch * 1e3 / ms, 1),
                                "hbm_gbs": round(abytes / (ms * 1e-3) / 1e9, 1)}
        rows.append(row)
        del lays, one
        torch.cuda.empty_cache()
    # fp16 dense baseline: W^T stored [n, m] (no transposed view), copies > 1 GB
    m, n = synth.UP70B.m, synth.UP70B.n
    nw = max(2, int(np.ceil(args.copies_gb * 1e9 / (2 * m * n))))
    wts = [torch.randn((n, m), device="cuda", dtype=torch.float16) for _ in range(nw)]
    dense = {"distinct_copies": nw, "weight_bytes": 2 * m * n}
    for batch in (1, 16):
        x = torch.randn((batch, n), device="cuda").half()
        y = torch.empty((batch, m), dtype=torch.float16, device="cuda")
        calls = [lambda w=w: torch.matmul(x, w, out=y) for w in wts]
        ms = time_graph(torch, calls, max(8 * nw, 200), 2 * nw)
        dense[f"b{batch}"] = {"us_per_call": round(ms * 1e3, 3), "hbm_gbs": round((2 * m * n) / (ms * 1e-3) / 1e9, 1)}
    for row in rows:
        for batch in (1, 16):
            row[f"b{batch}"]["speedup_vs_fp16_dense"] = round(dense[f"b{batch}"]["us_per_call"] /
                                                              row[f"b{batch}"]["us_per_call"], 2)
    del wts
    torch.cuda.empty_cache()
    return {"bpw_sweep": rows, "fp16_dense": dense,
            "shape": {"m": m, "n": n, "branches": 2}, "data": "synthetic"}


def init_bench(lb, torch, synth, args):
    """Dual-SVID initialization (littlebit_dual_svid_init, the step before
    the layer) of a synthetic dense weight of the 7B up-projection's shape
    (11008 x 4096, decaying spectrum), two branches of rank 1472: seconds on
    the GPU and the relative reconstruction error; the float64 oracle is
    timed on a quarter-size sample (2752 x 1024, rank 368) as context."""
    import time
    sh = synth.UP7B
    r = sh.ranks[0]
    W = torch.from_numpy(synth.make_dense_weight(sh.m, sh.n, seed=7)).cuda()
    lb.littlebit_dual_svid_init(torch.from_numpy(synth.make_dense_weight(256, 128, seed=1)).cuda(), 8)  # library warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    brs = lb.littlebit_dual_svid_init(W, r, nbranches=2)
    torch.cuda.synchronize()
    gpu_s = time.perf_counter() - t0
    what = torch.zeros_like(W)
    for b in brs:
        su = torch.where(b["U"] < 0, -1.0, 1.0) * b["h"].float()[:, None] * b["l"].float()[None, :]
        sv = torch.where(b["V"] < 0, -1.0, 1.0) * b["g"].float()[:, None]
        what += su @ sv.T
        err = float(torch.linalg.norm(W - what) / torch.linalg.norm(W))
        b["error_after"] = err
    out = {"init": {"method": "dual-svid", "shape": {"m": sh.m, "n": sh.n, "rank": r, "branches": 2},
                    "gpu_seconds": round(gpu_s, 3),
                    "rel_error_branch1": round(brs[0]["error_after"], 5),
                    "rel_error_branches12": round(brs[1]["error_after"], 5), "data": "synthetic"}}
    # with a Joint-ITQ rotation of the latent factors (10 iterations per branch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    brs = lb.littlebit_dual_svid_init(W, r, nbranches=2, itq_iters=10)
    torch.cuda.synchronize()
    itq_s = time.perf_counter() - t0
    what = torch.zeros_like(W)
    for b in brs:
        su = torch.where(b["U"] < 0, -1.0, 1.0) * b["h"].float()[:, None] * b["l"].float()[None, :]
        sv = torch.where(b["V"] < 0, -1.0, 1.0) * b["g"].float()[:, None]
        what += su @ sv.T
    out["init"]["with_itq10"] = {"gpu_seconds": round(itq_s, 3),
                                 "rel_error_branches12": round(float(torch.linalg.norm(W - what) /
                                                                     torch.linalg.norm(W)), 5)}
    if args.cpu_seconds > 0:
        import oracle
        Wq = synth.make_dense_weight(sh.m // 4, sh.n // 4, seed=7).astype(np.float64)
        t0 = time.perf_counter()
        oracle.dual_svid_init(Wq, r // 4, nbranches=2)
        out["init"]["cpu_baseline"] = {"kind": "oracle", "seconds": round(time.perf_counter() - t0, 3),
                                       "cores": _blas_threads(),
                                       "sample": f"quarter-size weight {sh.m // 4} x {sh.n // 4}, rank {r // 4}"}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3840)
    ap.add_argument("--warmup", type=int, default=384)
    ap.add_argument("--copies-gb", type=float, default=1.0, help="total size of distinct layer copies")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="host time for the oracle baseline (0: skip)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 13B-block, 70B and prefill measurements")
    ap.add_argument("--bpw-sweep", action="store_true",
                    help="only the bits-per-weight sweep of the 70B up-projection against fp16 dense")
    ap.add_argument("--init", action="store_true",
                    help="only the Dual-SVID initialization of a 7B-shaped dense weight")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="no timing: one call per layer copy plus a 256 MiB device copy, for hardware counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is measured per GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from binary_rank_gemv_amd import littlebit as lb
    from binary_rank_gemv_amd import synth

    if args.bpw_sweep:
        torch.cuda.set_device(0)
        print(json.dumps(bpw_sweep(lb, torch, synth, args)))
        return
    if args.init:
        torch.cuda.set_device(0)
        print(json.dumps(init_bench(lb, torch, synth, args)))
        return

    shape, batch = synth.UP7B, 1
    branches, x_np = synth.make_layer(shape, batch=batch, seed=0)
    torch.cuda.set_device(0)
    x = torch.from_numpy(x_np).cuda()
    y = torch.empty((batch, shape.m), dtype=torch.float16, device="cuda")

    first = lb.LittleBitLayer.from_latents(branches)
    per_copy = sum(b.v_bits.numel() + b.u_bits.numel() + 2 * (b.h.numel() + b.l.numel() + b.g.numel())
                   for b in first.branches)
    ncopies = max(1, int(np.ceil(args.copies_gb * 1e9 / per_copy)))
    copies = [first] + [make_copy(lb, torch, shape, 1000 + i) for i in range(ncopies - 1)]
    need = lb.littlebit_linear_workspace_bytes(first, batch)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")

    if args.pmc_pass:
        # counter pass: every copy once (cold in the caches), then a plain
        # device copy of known size that calibrates the byte counters
        for c in copies:
            lb.littlebit_linear_fwd(c, x, out=y, workspace=ws)
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": True, "decode_calls": len(copies), "copy_bytes": src.numel()}))
        return

    # the measured configuration's output (first copy), compared with the
    # oracle in the cpu_baseline leg
    lb.littlebit_linear_fwd(first, x, out=y, workspace=ws)
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy().astype(np.float64)

    def time_path(path):
        """Milliseconds for `steps` calls cycling over the copies (HIP graph)."""
        calls = [lambda c=c: lb.littlebit_linear_fwd(c, x, out=y, workspace=ws, path=path) for c in copies]
        return time_graph(torch, calls, args.steps, args.warmup) * args.steps

    ms_two = time_path(lb.LB_DECODE_TWO_LAUNCHES)
    ms = time_path(lb.LB_PATH_AUTO)
    ms_per_step = ms / args.steps

    abytes = algorithmic_bytes(shape.m, shape.n, shape.ranks, batch)
    achieved = abytes / (ms_per_step * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "kernel": "lb_decode_kernel<2, true, false, 1> (one launch per call: V pass, tagged z exchange, U pass)",
                "algorithmic_bytes_per_call": abytes,
                "avg_call_us": round(ms_per_step * 1e3, 3),
                "two_launch_variant_us": round(ms_two / args.steps * 1e3, 3)}

    extra = None if args.no_extra else extra_measurements(lb, torch, synth, args)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(shape, branches, x_np, args.cpu_seconds, yg)

    out = {
        "metric": "decode tokens/s per layer",
        "value": round(batch * args.steps / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 operands, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "Llama2-7B-shaped MLP up-projection 4096->11008, 2 branches r=1472 "
                               "(~1.0 BPW), batch-1 decode",
                   "m": shape.m, "n": shape.n, "ranks": list(shape.ranks), "batch": batch,
                   "distinct_layer_copies": ncopies, "copies_bytes": ncopies * per_copy},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
