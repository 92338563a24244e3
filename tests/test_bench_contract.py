"""Host-side checks of bench.py: the one-GPU rule and the committed counter
summary it reads (no GPU needed)."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_traffic_summary_matches_the_decode_sources():
    """The counter summary under profiles/ carries the hash of the decode
    kernel sources it was taken from; bench.py reports its traffic only while
    the sources still hash to it, so a stale summary yields null, never a
    number for other code."""
    b = _bench()
    t = b.measured_traffic()
    text = open(os.path.join(ROOT, "profiles", "lb_decode_7b_up_b1_pmc.md")).read()
    import hashlib
    import re
    h = hashlib.sha256(b"".join(open(f, "rb").read() for f in b.KERNEL_SOURCES)).hexdigest()
    stored = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text).group(1)
    if stored == h:
        assert t == int(re.search(r"traffic_bytes_per_launch:\s*(\d+)", text).group(1))
    else:
        assert t is None


def test_algorithmic_bytes_of_the_7b_layer():
    """Sign bits of both factors of both branches, fp16 scales, x and y: the
    per-call figure the roofline divides by the kernel time."""
    b = _bench()
    m, n, r = 11008, 4096, 1472
    bits = 2 * r * (m + n) // 8
    scales = 2 * 2 * (m + n + r)
    assert b.algorithmic_bytes(m, n, (r, r), 1) == bits + scales + 2 * n + 2 * m == 5654784
