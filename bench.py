#!/usr/bin/env python3
"""Benchmark of the LittleBit layer on one MI355X.

Headline workload: the Llama2-70B-shaped MLP up-projection, 8192 -> 28672,
two branches of rank 1728 (about 0.55 bit per weight), fp16 scales
~U[0.5, 1.5], one fp16 token ~N(0, 1) per call (batch-1 decode GEMV) -- the
layer shape of the trueseeker.com case's A100 kernel benchmark ("The trace /
claim to source").  It is the largest configuration; the 7B up-projection,
the 70B layer at 16 tokens, the 13B decoder block at 0.55 and 0.1 bits per
weight and the 2048-token prefill of the 7B layer are measured the same way
under "extra".  Inputs are synthetic and seeded (binary_rank_gemv_amd.synth
for the first copy of the headline layer, torch's seeded GPU generator for
the other copies).

One step = one littlebit_linear_fwd call (every step of the layer for one
token).  To measure HBM rather than the 256 MB last-level cache, the calls
cycle through distinct copies of the layer totalling >= 1 GB, in one rotation
that runs on from the warm-up into the timed region: every timed call reads
a copy that no call has touched for at least 1 GB of other weights (or ever
since it was written).  The calls are captured in HIP graphs and replayed;
HIP events on the replay stream bracket exactly --steps calls.

Prints one JSON line, including a roofline object per configuration (HBM for
decode, matrix cores for prefill; `traffic` from the committed rocprofv3
counter summaries while the kernel sources match them) and a cpu_baseline
object for the float64 CPU oracle timed on a bounded sample of the headline
workload.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix-core peak
CSRC = os.path.join(ROOT, "binary_rank_gemv_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# Decode configurations: (kind, shape or block setting, tokens per call).
DECODE_CONFIGS = {
    "up70b_b1": ("linear", "UP70B", 1),
    "up70b_b16": ("linear", "UP70B", 16),
    "up7b_b1": ("linear", "UP7B", 1),
    "block13b_0.55_b1": ("block", "0.55", 1),
    "block13b_0.1_b1": ("block", "0.1", 1),
}
HEADLINE = "up70b_b1"
WORKLOAD_NAMES = {
    "up70b_b1": "Llama2-70B-shaped MLP up-projection 8192->28672, 2 branches r=1728 (~0.55 BPW), batch-1 decode",
    "up70b_b16": "Llama2-70B-shaped MLP up-projection 8192->28672, 2 branches r=1728, 16-token decode",
    "up7b_b1": "Llama2-7B-shaped MLP up-projection 4096->11008, 2 branches r=1472 (~1.0 BPW), batch-1 decode",
    "block13b_0.55_b1": "Llama2-13B-shaped decoder block (q,k,v,o,gate,up,down) at 0.55 BPW, batch-1 decode",
    "block13b_0.1_b1": "Llama2-13B-shaped decoder block (q,k,v,o,gate,up,down) at 0.1 BPW, batch-1 decode",
    "prefill_7b_up_2048": "2048-token prefill of the Llama2-7B-shaped up-projection 4096->11008, r=1472",
}


def algorithmic_bytes(m, n, ranks, batch):
    """Unpadded sign bits + fp16 scales + fp16 x + fp16 y for one call."""
    bits = sum(r * (m + n) for r in ranks)
    scales = sum(m + n + r for r in ranks) * 2
    return bits // 8 + scales + 2 * batch * n + 2 * batch * m


def rotation(n, start, count):
    """Copy indices of `count` calls starting at `start` in a rotation of n."""
    return [(start + i) % n for i in range(count)]


def graph_plan(n, start, count):
    """How `count` calls from `start` are replayed: `reps` replays of the
    whole cycle starting at `start`, then one replay of its first `rem`
    calls.  The cycle ends just before `start`, so repeats continue the
    rotation; the concatenation equals rotation(n, start, count)."""
    return count // n, count % n


def time_graph(torch, calls, steps, warmup):
    """Milliseconds per call over exactly `steps` calls that continue the
    rotation of `calls` from where `warmup` calls (from index 0) ended.  Each
    call's copy was last touched len(calls) calls earlier, or never."""
    n = len(calls)
    side = torch.cuda.Stream()

    def capture(idx):
        gr = torch.cuda.CUDAGraph()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(gr, stream=side):
                for i in idx:
                    calls[i]()
        torch.cuda.current_stream().wait_stream(side)
        return gr

    # one eager call (of the copy the rotation reaches last) loads the
    # kernels and the library's per-device state; capturing records
    # launches without running them
    calls[-1]()
    torch.cuda.synchronize()
    graphs = {}

    def replay(start, count):
        reps, rem = graph_plan(n, start, count)
        if reps:
            key = (start, n)
            if key not in graphs:
                graphs[key] = capture(rotation(n, start, n))
            for _ in range(reps):
                graphs[key].replay()
        if rem:
            key = (start, rem)
            if key not in graphs:
                graphs[key] = capture(rotation(n, start, rem))
            graphs[key].replay()

    # capture both phases before running either, so that capturing neither
    # touches the weights nor separates the warm-up from the timed region
    t0 = warmup % n
    for start, count in ((0, warmup), (t0, steps)):
        reps, rem = graph_plan(n, start, count)
        if reps and (start, n) not in graphs:
            graphs[(start, n)] = capture(rotation(n, start, n))
        if rem and (start, rem) not in graphs:
            graphs[(start, rem)] = capture(rotation(n, start, rem))
    torch.cuda.synchronize()
    replay(0, warmup)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    replay(t0, steps)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


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


def copies_for(bytes_per_copy, total_bytes):
    return max(2, int(np.ceil(total_bytes / bytes_per_copy)))


def layer_bytes(layer):
    return sum(b.v_bits.numel() + b.u_bits.numel() + 2 * (b.h.numel() + b.l.numel() + b.g.numel())
               for b in layer.branches)


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


# ------------------------------------------------------- counter summaries

def decode_sources():
    """The sources whose code runs in (or launches) the decode kernels."""
    files = sorted(glob.glob(os.path.join(CSRC, "decode*.hip"))) + [
        os.path.join(CSRC, "lb_common.h"), os.path.join(CSRC, "lb_sync.h"), os.path.join(CSRC, "littlebit_host.hip")]
    return files


def prefill_sources():
    return [os.path.join(CSRC, "prefill.hip"), os.path.join(CSRC, "lb_common.h"),
            os.path.join(CSRC, "littlebit_host.hip")]


def sources_hash(files):
    return hashlib.sha256(b"".join(open(f, "rb").read() for f in files)).hexdigest()


def pmc_summary_path(config):
    name = f"lb_{config}" if config.startswith("prefill") else f"lb_decode_{config}"
    return os.path.join(PROFILES, f"{name}_pmc.md")


def measured_traffic(config):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) from the
    committed counter summary of `config`, or None when there is none or the
    kernel sources have changed since the counters were taken."""
    files = prefill_sources() if config.startswith("prefill") else decode_sources()
    try:
        text = open(pmc_summary_path(config)).read()
        h = sources_hash(files)
    except OSError:
        return None
    mt = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    mh = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    if not (mt and mh) or mh.group(1) != h:
        return None
    return int(mt.group(1))


# ------------------------------------------------------------ workloads

class DecodeWorkload:
    """Distinct copies of one decode configuration and its call list."""

    def __init__(self, lb, torch, synth, config, copies_gb, first_branches=None, x_np=None):
        kind, what, batch = DECODE_CONFIGS[config]
        self.config, self.kind, self.batch = config, kind, batch
        if kind == "linear":
            shape = getattr(synth, what)
            self.shapes = [shape]
            first = (lb.LittleBitLayer.from_latents(first_branches) if first_branches is not None
                     else make_copy(lb, torch, shape, 7000))
            per = layer_bytes(first)
            nc = copies_for(per, copies_gb * 1e9)
            self.copies = [[first]] + [[make_copy(lb, torch, shape, 7001 + i)] for i in range(nc - 1)]
            x = (torch.from_numpy(x_np).cuda() if x_np is not None
                 else torch.randn((batch, shape.n), device="cuda").half())
            self.xs = [x]
            self.ys = [torch.empty((batch, shape.m), dtype=torch.float16, device="cuda")]
            self.ws = torch.zeros(lb.littlebit_linear_workspace_bytes(first, batch), dtype=torch.uint8,
                                  device="cuda")
            self.calls = [lambda c=c: lb.littlebit_linear_fwd(c[0], self.xs[0], out=self.ys[0], workspace=self.ws)
                          for c in self.copies]
        else:
            self.shapes = synth.block13b_shapes(what)
            one = [make_copy(lb, torch, sh, 5000 + i) for i, sh in enumerate(self.shapes)]
            per = sum(layer_bytes(l) for l in one)
            nc = copies_for(per, copies_gb * 1e9)
            self.copies = [one] + [[make_copy(lb, torch, sh, 6000 + 7 * j + i) for i, sh in enumerate(self.shapes)]
                                   for j in range(nc - 1)]
            self.xs = [torch.randn((batch, n), device="cuda").half() for n in (5120, 5120, 5120, 13824)]
            self.ys = [torch.empty((batch, sh.m), dtype=torch.float16, device="cuda") for sh in self.shapes]
            self.ws = torch.zeros(lb.littlebit_block_workspace_bytes(one, batch), dtype=torch.uint8, device="cuda")
            self.calls = [lambda c=c: lb.littlebit_block_fwd(c, *self.xs, outs=self.ys, workspace=self.ws)
                          for c in self.copies]
        self.per_copy = per
        self.algorithmic = sum(algorithmic_bytes(sh.m, sh.n, sh.ranks, batch) for sh in self.shapes)

    def measure(self, torch, steps, warmup):
        ms = time_graph(torch, self.calls, steps, warmup)
        achieved = self.algorithmic / (ms * 1e-3) / 1e9
        n = len(self.copies)
        return {
            "workload": WORKLOAD_NAMES[self.config],
            "us_per_call": round(ms * 1e3, 3),
            "tokens_per_s": round(self.batch * 1e3 / ms, 1),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(self.config),
                         "algorithmic_bytes_per_call": self.algorithmic},
            "rotation": {"distinct_copies": n, "copy_bytes": self.per_copy,
                         "reuse_distance_bytes": n * self.per_copy,
                         "timed_calls": steps, "timed_distinct_bytes": min(steps, n) * self.per_copy},
        }


def measure_prefill(lb, torch, synth):
    """2048 tokens of the 7B up-projection (compute-bound; one copy)."""
    sh, M = synth.UP7B, synth.PREFILL_TOKENS
    lay = make_copy(lb, torch, sh, 8000)
    x = torch.randn((M, sh.n), device="cuda").half()
    y = torch.empty((M, sh.m), dtype=torch.float16, device="cuda")
    ws = torch.zeros(lb.littlebit_linear_workspace_bytes(lay, M), dtype=torch.uint8, device="cuda")
    ms = time_graph(torch, [lambda: lb.littlebit_linear_fwd(lay, x, out=y, workspace=ws)], 50, 5)
    flops = 2 * M * sum(r * (sh.m + sh.n) for r in sh.ranks)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": WORKLOAD_NAMES["prefill_7b_up_2048"],
            "us_per_call": round(ms * 1e3, 2), "tokens_per_s": round(M * 1e3 / ms, 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_7b_up_2048"), "flops_per_call": flops},
            "dense_fp16_library": dense_gemm_context(torch, M, sh.n, sum(sh.ranks), sh.m)}


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


# ------------------------------------------------------------ CPU oracle

def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            return max(d["num_threads"] for d in info)
    except Exception:
        pass
    return None


def cpu_baseline(shape, branches, x, seconds, y_gpu):
    """Time the float64 oracle on the host: whole batch-1 calls of its factored
    form for about `seconds` with the BLAS library's own thread count, the
    same limited to one thread for about a third of that, and a sample of
    output rows of its dense definition (rows of W built per call).  The
    oracle's result is also compared with the GPU's on the same input."""
    import oracle
    from threadpoolctl import threadpool_limits

    def timed(fn, budget):
        calls, t0 = 0, time.perf_counter()
        out = None
        while calls < 1 or time.perf_counter() - t0 < budget:
            out = fn()
            calls += 1
        return calls, time.perf_counter() - t0, out

    calls, dt, yr = timed(lambda: oracle.factored_forward(x, branches), seconds)
    agreement = {"rel_l2": float(np.linalg.norm(y_gpu - yr) / np.linalg.norm(yr)),
                 "max_err_over_rms": float(np.max(np.abs(y_gpu - yr)) / np.sqrt(np.mean(yr ** 2)))}
    with threadpool_limits(limits=1):
        calls1, dt1, _ = timed(lambda: oracle.factored_forward(x, branches), seconds / 3)
    rows, t1 = 0, time.perf_counter()
    while rows < shape.m and (rows == 0 or time.perf_counter() - t1 < seconds / 3):
        blk = np.arange(rows, min(rows + 256, shape.m))
        oracle.rows_forward(x, branches, blk)
        rows += len(blk)
    dtd = time.perf_counter() - t1
    threads = _blas_threads()
    return {"value": round(x.shape[0] * calls / dt, 4), "unit": "tokens/s",
            "cores": threads if threads else len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{calls} whole batch-1 calls of the float64 factored oracle in {dt:.1f} s",
            "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": threads,
            "one_thread": {"value": round(x.shape[0] * calls1 / dt1, 4), "unit": "tokens/s", "cores": 1,
                           "sample": f"{calls1} whole calls with the BLAS library limited to one thread "
                                     f"in {dt1:.1f} s"},
            "dense_definition": {"value": round(x.shape[0] * (rows / shape.m) / dtd, 5), "unit": "tokens/s",
                                 "sample": f"{rows} of {shape.m} output rows of the dense float64 definition "
                                           f"in {dtd:.1f} s, scaled by {shape.m}/{rows}"},
            "gpu_agreement": agreement,
            "note": "the oracle is a correctness reference (plain NumPy float64), not a tuned CPU kernel"}


# ----------------------------------------------------------- other modes

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
            ms = time_graph(torch, calls, max(4 * nc, 200), nc)
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
    """Dual-SVID initialization (littlebit_dual_svid_init from the offline
    library, the step before the layer) of a synthetic dense weight of the
    7B up-projection's shape (11008 x 4096, decaying spectrum), two branches
    of rank 1472: seconds on the GPU and the relative reconstruction error;
    the float64 oracle is timed on a quarter-size sample (2752 x 1024, rank
    368) as context."""
    sh = synth.UP7B
    r = sh.ranks[0]
    W = torch.from_numpy(synth.make_dense_weight(sh.m, sh.n, seed=7)).cuda()
    lb.littlebit_dual_svid_init(torch.from_numpy(synth.make_dense_weight(256, 128, seed=1)).cuda(), 8)  # warm-up
    torch.cuda.synchronize()

    def run(itq):
        t0 = time.perf_counter()
        brs = lb.littlebit_dual_svid_init(W, r, nbranches=2, itq_iters=itq)
        torch.cuda.synchronize()
        secs = time.perf_counter() - t0
        what = torch.zeros_like(W)
        errs = []
        for b in brs:
            su = torch.where(b["U"] < 0, -1.0, 1.0) * b["h"].float()[:, None] * b["l"].float()[None, :]
            sv = torch.where(b["V"] < 0, -1.0, 1.0) * b["g"].float()[:, None]
            what += su @ sv.T
            errs.append(float(torch.linalg.norm(W - what) / torch.linalg.norm(W)))
        return secs, errs

    secs, errs = run(0)
    out = {"init": {"method": "dual-svid", "shape": {"m": sh.m, "n": sh.n, "rank": r, "branches": 2},
                    "gpu_seconds": round(secs, 3), "rel_error_branch1": round(errs[0], 5),
                    "rel_error_branches12": round(errs[1], 5), "data": "synthetic"}}
    secs, errs = run(10)
    out["init"]["with_itq10"] = {"gpu_seconds": round(secs, 3), "rel_error_branches12": round(errs[1], 5)}
    if args.cpu_seconds > 0:
        import oracle
        Wq = synth.make_dense_weight(sh.m // 4, sh.n // 4, seed=7).astype(np.float64)
        t0 = time.perf_counter()
        oracle.dual_svid_init(Wq, r // 4, nbranches=2)
        out["init"]["cpu_baseline"] = {"kind": "oracle", "seconds": round(time.perf_counter() - t0, 3),
                                       "cores": _blas_threads() or len(os.sched_getaffinity(0)),
                                       "sample": f"quarter-size weight {sh.m // 4} x {sh.n // 4}, rank {r // 4}"}
    return out


def pmc_pass(lb, torch, synth, config, copies_gb):
    """No timing: one call per distinct copy of `config` (cold caches), then a
    plain 256 MiB device copy that calibrates the byte counters."""
    if config == "prefill_7b_up_2048":
        sh, M = synth.UP7B, synth.PREFILL_TOKENS
        lay = make_copy(lb, torch, sh, 8000)
        x = torch.randn((M, sh.n), device="cuda").half()
        y = torch.empty((M, sh.m), dtype=torch.float16, device="cuda")
        ws = torch.zeros(lb.littlebit_linear_workspace_bytes(lay, M), dtype=torch.uint8, device="cuda")
        for _ in range(5):
            lb.littlebit_linear_fwd(lay, x, out=y, workspace=ws)
        ncalls = 5
    else:
        w = DecodeWorkload(lb, torch, synth, config, copies_gb)
        for c in w.calls:
            c()
        ncalls = len(w.calls)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    return {"pmc_pass": config, "calls": ncalls, "copy_bytes": src.numel()}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--copies-gb", type=float, default=1.0, help="total size of distinct layer copies")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="host time for the oracle baseline (0: skip)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other configurations (7B, 70B at 16 tokens, 13B block, prefill)")
    ap.add_argument("--only", choices=sorted(DECODE_CONFIGS) + ["prefill_7b_up_2048"],
                    help="time one configuration only")
    ap.add_argument("--bpw-sweep", action="store_true",
                    help="only the bits-per-weight sweep of the 70B up-projection against fp16 dense")
    ap.add_argument("--init", action="store_true",
                    help="only the Dual-SVID initialization of a 7B-shaped dense weight")
    ap.add_argument("--pmc-pass", choices=sorted(DECODE_CONFIGS) + ["prefill_7b_up_2048"],
                    help="no timing: one call per layer copy of a configuration plus a 256 MiB device copy, "
                         "for hardware counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is measured per GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from binary_rank_gemv_amd import littlebit as lb
    from binary_rank_gemv_amd import synth

    torch.cuda.set_device(0)
    if args.bpw_sweep:
        print(json.dumps(bpw_sweep(lb, torch, synth, args)))
        return
    if args.init:
        print(json.dumps(init_bench(lb, torch, synth, args)))
        return
    if args.pmc_pass:
        print(json.dumps(pmc_pass(lb, torch, synth, args.pmc_pass, args.copies_gb)))
        return
    if args.only == "prefill_7b_up_2048":
        print(json.dumps({args.only: measure_prefill(lb, torch, synth)}))
        return
    if args.only:
        w = DecodeWorkload(lb, torch, synth, args.only, args.copies_gb)
        print(json.dumps({args.only: w.measure(torch, args.steps, args.warmup)}))
        return

    # headline: the 70B up-projection at batch 1; its first copy is the
    # seeded synth layer, whose output is compared with the oracle
    shape, batch = synth.UP70B, 1
    branches, x_np = synth.make_layer(shape, batch=batch, seed=0)
    head = DecodeWorkload(lb, torch, synth, HEADLINE, args.copies_gb, first_branches=branches, x_np=x_np)
    head.calls[0]()
    torch.cuda.synchronize()
    yg = head.ys[0].float().cpu().numpy().astype(np.float64)
    res = head.measure(torch, args.steps, args.warmup)
    print(f"[bench] {HEADLINE}: {res['us_per_call']} us per call", file=sys.stderr, flush=True)
    ms_per_step = res["us_per_call"] * 1e-3
    roofline = dict(res["roofline"])
    roofline["kernel"] = ("lb_decode1_kernel<2, true, 1> (one launch per call: V pass, z exchange, U pass, "
                          "on the sparse matrix instruction)")
    roofline["avg_call_us"] = res["us_per_call"]
    two = time_graph(torch, [lambda c=c: lb.littlebit_linear_fwd(c[0], head.xs[0], out=head.ys[0],
                                                                  workspace=head.ws,
                                                                  path=lb.LB_DECODE_TWO_LAUNCHES)
                             for c in head.copies], max(len(head.copies), 100), len(head.copies))
    roofline["two_launch_variant_us"] = round(two * 1e3, 3)
    err = lb.littlebit_workspace_error(head.ws)
    torch.cuda.synchronize()
    poll_ok = int(err.item()) == 0
    del head
    torch.cuda.empty_cache()

    extra = None
    if not args.no_extra:
        extra = {}
        for cfg in DECODE_CONFIGS:
            if cfg == HEADLINE:
                continue
            w = DecodeWorkload(lb, torch, synth, cfg, args.copies_gb)
            nc = len(w.copies)
            extra[cfg] = w.measure(torch, max(4 * nc, 400), nc)
            del w
            torch.cuda.empty_cache()
            print(f"[bench] {cfg}: {extra[cfg]['us_per_call']} us per call", file=sys.stderr, flush=True)
        extra["prefill_7b_up_2048"] = measure_prefill(lb, torch, synth)
        print(f"[bench] prefill: {extra['prefill_7b_up_2048']['us_per_call']} us per call", file=sys.stderr,
              flush=True)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(shape, branches, x_np, args.cpu_seconds, yg)

    out = {
        "metric": "decode tokens/s per layer",
        "value": round(batch * 1e3 / ms_per_step, 1),
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
        "config": {"workload": WORKLOAD_NAMES[HEADLINE], "m": shape.m, "n": shape.n,
                   "ranks": list(shape.ranks), "batch": batch, **res["rotation"], "z_polls_ok": poll_ok},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
