"""Phase timeline of the one-token decode kernel, from the instrumented
library (``python -m binary_rank_gemv_amd.build --phase-stamps``).

    python -m binary_rank_gemv_amd.phase_timeline up70b_b1 up7b_b1 block13b_0.55_b1

For each configuration (bench.py's decode configurations at batch 1): one
call per layer copy to warm nothing but the code path, then 24 single calls,
each on a different copy; per call the percentiles over workgroups of each
phase point, in microseconds from the first workgroup's start, and the
median of those over the calls.  The points are the ones decode1.hip
records under LB_PHASE_STAMPS.
"""

import os
import sys

import numpy as np

POINTS = [(0, "start"), (1, "arguments + first u staged"), (7, "multi-layer tile staged"),
          (8, "first V products start"), (2, "first V products done"), (3, "first z round issued"),
          (4, "first z copied"), (5, "first U group products done"), (6, "end")]


def main(configs):
    from binary_rank_gemv_amd import build
    os.environ["LITTLEBIT_LIBRARY"] = build.STAMPED_LIB
    import ctypes
    import torch
    sys.path.insert(0, build.ROOT)
    import bench
    from binary_rank_gemv_amd import littlebit as lb, synth

    lib = ctypes.CDLL(build.STAMPED_LIB)
    torch.cuda.set_device(0)
    nwg = 1024
    stamps = torch.zeros(nwg * 16, dtype=torch.int64, device="cuda")
    if lib.littlebit_phase_stamps_set(ctypes.c_void_p(stamps.data_ptr())) != 0:
        raise RuntimeError("littlebit_phase_stamps_set failed")
    for cfg in configs:
        w = bench.DecodeWorkload(lb, torch, synth, cfg, 1.0)
        for c in w.calls:
            c()
        torch.cuda.synchronize()
        rows = []
        for i in range(24):
            stamps.zero_()
            w.calls[(7 * i) % len(w.calls)]()
            torch.cuda.synchronize()
            s = stamps.view(nwg, 16)[:, :9].cpu().numpy().astype(np.float64)
            used = s[:, 0] > 0
            s = s[used]
            t0 = s[:, 0].min()
            rows.append(np.where(s > 0, (s - t0) * 0.01, np.nan))  # 100 MHz ticks -> us
        a = np.stack(rows)
        print(f"== {cfg}: {a.shape[1]} workgroups; us from the first workgroup's start "
              f"(median over 24 calls of the per-call percentile over workgroups)")
        print(f"  {'point':30s} {'n':>4s} {'min':>7s} {'p10':>7s} {'p50':>7s} {'p90':>7s} {'max':>7s}")
        for j, name in POINTS:
            col = a[:, :, j]
            n = int(np.sum(~np.isnan(col[0])))
            if n == 0:
                continue
            v = [np.nanmedian(np.nanpercentile(col, q, axis=1)) for q in (0, 10, 50, 90, 100)]
            print(f"  {name:30s} {n:4d} " + " ".join(f"{x:7.2f}" for x in v))
        del w
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main(sys.argv[1:] or ["up70b_b1", "up7b_b1", "block13b_0.55_b1"])
