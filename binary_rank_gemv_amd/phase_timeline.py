"""Phase timeline of the decode kernels, from the instrumented library
(``python -m binary_rank_gemv_amd.build --phase-stamps``).

    python -m binary_rank_gemv_amd.phase_timeline up70b_b1 up7b_b1 block13b_0.55_b1 up70b_b16

For each configuration (bench.py's decode configurations): one call per
layer copy to warm nothing but the code path, then 24 single calls, each on
a different copy; per call the percentiles over workgroups of each phase
point, in microseconds from the first workgroup's start, and the median of
those over the calls.  The points are the ones decode1.hip (one token) and
decode.hip (several tokens) record under LB_PHASE_STAMPS.
"""

import os
import sys

import numpy as np

POINTS = [(0, "start"), (1, "arguments + first u staged"), (7, "multi-layer tile staged"),
          (13, "first unit's words landed"), (14, "next unit's words issued"),
          (8, "first V products start"), (2, "first V products done"), (15, "first unit's sums met"), (3, "first z round issued"),
          (9, "last V unit's z stored"), (4, "first z copied"), (10, "last z copy done"),
          (5, "first U group products done"), (6, "end")]
COUNTS = (11, 12)  # u stagings, z copies of a workgroup
MPOINTS = [(0, "start"), (10, "V pair slot 0 done"), (13, "V pair slot 3 done"), (14, "V pair slot 7 done"),
           (1, "phase-B loads issued"), (3, "V products done"), (2, "first V tile done"), (9, "last V tile done"), (4, "z copy done"),
           (5, "first U group done"), (8, "last U group begun"), (7, "last U group products issued"),
           (6, "end")]


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
    if lib.littlebit_phase_stamps_multi_set(ctypes.c_void_p(stamps.data_ptr())) != 0:
        raise RuntimeError("littlebit_phase_stamps_multi_set failed")
    for cfg in configs:
        w = bench.DecodeWorkload(lb, torch, synth, cfg, 1.0)
        multi = w.batch > 1
        points = MPOINTS if multi else POINTS
        for c in w.calls:
            c()
        torch.cuda.synchronize()
        rows, wrows = [], []
        for i in range(24):
            stamps.zero_()
            w.calls[(7 * i) % len(w.calls)]()
            torch.cuda.synchronize()
            s = stamps.view(nwg, 16)[:256, :16].cpu().numpy().astype(np.float64)  # one row per workgroup
            used = s[:, 0] > 0
            s = s[used]
            t0 = s[:, 0].min()
            t = np.where(s > 0, (s - t0) * 0.01, np.nan)  # 100 MHz ticks -> us
            t[:, COUNTS] = s[:, COUNTS]
            rows.append(t)
            # per-wave points (spare rows of the buffer): spread over waves
            wv = stamps.view(nwg, 16)[256:768, :8].cpu().numpy().astype(np.float64).reshape(2, 256, 8)
            wv = np.where(wv > 0, (wv - t0) * 0.01, np.nan)
            wrows.append(wv[:, used])
        a = np.stack(rows)
        print(f"== {cfg}: {a.shape[1]} workgroups; us from the first workgroup's start "
              f"(median over 24 calls of the per-call percentile over workgroups)")
        print(f"  {'point':30s} {'n':>4s} {'min':>7s} {'p10':>7s} {'p50':>7s} {'p90':>7s} {'max':>7s}")
        for j, name in points:
            col = a[:, :, j]
            n = int(np.sum(~np.isnan(col[0])))
            if n == 0:
                continue
            v = [np.nanmedian(np.nanpercentile(col, q, axis=1)) for q in (0, 10, 50, 90, 100)]
            print(f"  {name:30s} {n:4d} " + " ".join(f"{x:7.2f}" for x in v))
        wa = np.stack(wrows)  # call, region, workgroup, wave
        wnames = (((0, "z copy done"),) if multi else
                  ((0, "first V products done"), (1, "first U group products done")))
        for R, name in wnames:
            x = wa[:, R]
            if np.all(np.isnan(x)):
                continue
            spread = np.nanmax(x, axis=2) - np.nanmin(x, axis=2)
            print(f"  per wave, {name}: median over calls of the median workgroup's earliest / latest wave "
                  f"{np.nanmedian(np.nanmedian(np.nanmin(x, axis=2), axis=1)):.2f} / "
                  f"{np.nanmedian(np.nanmedian(np.nanmax(x, axis=2), axis=1)):.2f} us; "
                  f"median spread {np.nanmedian(spread):.2f} us; by wave: "
                  + " ".join(f"{np.nanmedian(x[:, :, k]):.2f}" for k in range(8)))
        # workgroups grouped by their counts of u stagings and z copies:
        # how many, and the median over calls of their median end
        keys = [] if multi else sorted({(int(a[0, i, 11]), int(a[0, i, 12])) for i in range(a.shape[1])})
        if keys:
            print("  by (u stagings, z copies): workgroups, median last z stored / last z copy done / end")
        for key in keys:
            sel = (a[0, :, 11] == key[0]) & (a[0, :, 12] == key[1])
            med = [np.nanmedian(np.nanmedian(a[:, sel, j], axis=1)) for j in (9, 10, 6)]
            print(f"    {str(key):10s} {int(sel.sum()):4d}   " + " ".join(f"{x:7.2f}" for x in med))
        del w
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main(sys.argv[1:] or ["up70b_b1", "up7b_b1", "block13b_0.55_b1"])
