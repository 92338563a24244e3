"""Host-side checks of bench.py: the one-GPU rule, the rotation of layer
copies around the timed region, and the committed counter summaries it reads
(no GPU needed)."""

import importlib.util
import os
import re
import subprocess
import sys
import types

import pytest

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


class _FakeCuda:
    """Just enough of torch.cuda for time_graph: graphs record the calls made
    while capturing and make them again on replay; everything else logs."""

    def __init__(self, log):
        self.log = log
        self.capturing = None
        fake = self

        class Stream:
            def wait_stream(self, other):
                pass

        class CUDAGraph:
            def __init__(self):
                self.calls = []

            def replay(self):
                for c in self.calls:
                    c()

        class _Ctx:
            def __init__(self, gr=None):
                self.gr = gr

            def __enter__(self):
                if self.gr is not None:
                    fake.capturing = self.gr

            def __exit__(self, *a):
                if self.gr is not None:
                    fake.capturing = None

        class Event:
            def __init__(self, enable_timing=False):
                self.t = 0

            def record(self):
                self.t = len(fake.log)
                fake.log.append("event")

            def elapsed_time(self, other):
                return 1.0

        self.Stream = Stream
        self.CUDAGraph = CUDAGraph
        self.Event = Event
        self.stream = lambda s: _Ctx()
        self.graph = lambda gr, stream=None: _Ctx(gr)
        self.current_stream = lambda: Stream()
        self.synchronize = lambda: None

    def call(self, i):
        def f():
            if self.capturing is not None:
                self.capturing.calls.append(f)
            else:
                self.log.append(i)
        return f


@pytest.mark.parametrize("n,steps,warmup", [(63, 20, 5), (63, 2000, 200), (178, 20, 5), (5, 17, 3),
                                            (7, 7, 0), (4, 9, 8)])
def test_every_timed_call_reads_a_cold_copy(n, steps, warmup):
    """time_graph replays exactly `steps` calls between its events, and each
    of them uses a copy that no call has touched during the previous n - 1
    calls: the rotation runs on from the warm-up (and the one eager call)
    into the timed region, so with n * copy_bytes >= 1 GB no timed call's
    weights can still sit in the 256 MB last-level cache."""
    b = _bench()
    log = []
    cuda = _FakeCuda(log)
    torch = types.SimpleNamespace(cuda=cuda)
    b.time_graph(torch, [cuda.call(i) for i in range(n)], steps, warmup)
    first, second = [i for i, e in enumerate(log) if e == "event"]
    timed = log[first + 1:second]
    assert len(timed) == steps
    assert timed == b.rotation(n, warmup % n, steps)
    for pos in range(first + 1, second):
        prev = [j for j in range(pos) if log[j] == log[pos]]
        assert not prev or pos - prev[-1] - sum(1 for j in range(prev[-1], pos) if log[j] == "event") >= n


def test_traffic_summaries_match_their_kernel_sources():
    """Each counter summary under profiles/ carries the hash of the kernel
    sources it was taken from; bench.py reports its traffic only while the
    sources still hash to it, so a stale summary yields null, never a number
    for other code."""
    b = _bench()
    for cfg in list(b.DECODE_CONFIGS) + ["prefill_7b_up_2048"]:
        path = b.pmc_summary_path(cfg)
        t = b.measured_traffic(cfg)
        if not os.path.exists(path):
            assert t is None
            continue
        text = open(path).read()
        files = b.prefill_sources() if cfg.startswith("prefill") else b.decode_sources()
        stored = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text).group(1)
        if stored == b.sources_hash(files):
            assert t == int(re.search(r"traffic_bytes_per_launch:\s*(\d+)", text).group(1))
        else:
            assert t is None


def test_algorithmic_bytes_of_the_7b_and_70b_layers():
    """Sign bits of both factors of both branches, fp16 scales, x and y: the
    per-call figure the roofline divides by the kernel time."""
    b = _bench()
    m, n, r = 11008, 4096, 1472
    bits = 2 * r * (m + n) // 8
    scales = 2 * 2 * (m + n + r)
    assert b.algorithmic_bytes(m, n, (r, r), 1) == bits + scales + 2 * n + 2 * m == 5654784
    assert b.algorithmic_bytes(28672, 8192, (1728, 1728), 1) == 16153344
    assert b.algorithmic_bytes(28672, 8192, (1728, 1728), 16) == 17259264


def test_headline_is_the_largest_single_gpu_configuration():
    b = _bench()
    assert b.HEADLINE == "up70b_b1"
    assert "8192->28672" in b.WORKLOAD_NAMES[b.HEADLINE]
