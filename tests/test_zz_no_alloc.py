"""GPU check of littlebit_linear_fwd_noalloc (the entry point that uses the
library's per-device scratch instead of a caller's workspace) against
littlebit_linear_fwd, through the C ABI: two calls in a row, the second with
a smaller input, for decode and for prefill (which runs in scratch-sized
token chunks).  Bar: the parity bar of the other tests (relative L2 error
<= 2e-3, max |err| <= 1e-2 * RMS) against the workspace entry point's
output, which runs the same kernels; decode is also expected bit-equal."""

import numpy as np
import pytest
import torch

import oracle
from binary_rank_gemv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    from binary_rank_gemv_amd import littlebit
    return littlebit


def _np(a):
    return a.float().cpu().numpy().astype(np.float64) if torch.is_tensor(a) else np.asarray(a, np.float64)


def _close(a, b, what):
    a64, b64 = _np(a), _np(b)
    assert np.isfinite(a64).all(), what
    rel = np.linalg.norm(a64 - b64) / np.linalg.norm(b64)
    mx = np.max(np.abs(a64 - b64)) / np.sqrt(np.mean(b64 ** 2))
    print(f"[noalloc] {what}: rel_l2={rel:.3e} max/rms={mx:.3e} equal={np.array_equal(a64, b64)}", flush=True)
    assert rel <= 2e-3 and mx <= 1e-2, what


def _run(lb, shape, batch, seed, path):
    br, x = synth.make_layer(shape, batch=batch, seed=seed)
    layer = lb.LittleBitLayer.from_latents(br)
    xt = torch.from_numpy(x).cuda()
    y_ws = lb.littlebit_linear_fwd(layer, xt, path=path).clone()
    y_na = lb.littlebit_linear_fwd_noalloc(layer, xt, path=path).clone()
    torch.cuda.synchronize()
    return br, x, y_ws, y_na


def test_noalloc_decode_two_calls_second_smaller(lb):
    print("[case] noalloc decode: 7B up batch 4, then tiny batch 1", flush=True)
    for shape, batch, seed in ((synth.UP7B, 4, 3), (synth.TINY, 1, 4)):
        br, x, y_ws, y_na = _run(lb, shape, batch, seed, lb.LB_PATH_AUTO)
        _close(y_na, y_ws, f"decode {shape.name} b={batch}")
        assert torch.equal(y_na, y_ws)
    ref = oracle.linear_forward(x, br)
    _close(y_na, ref, "decode tiny vs oracle")


def test_noalloc_prefill_two_calls_second_smaller(lb):
    print("[case] noalloc prefill: 7B up 2048 tokens, then 300 tokens of a ragged layer", flush=True)
    for shape, batch, seed in ((synth.UP7B, synth.PREFILL_TOKENS, 5),
                               (synth.LayerShape("ragged", 520, 4104, (264, 200)), 300, 6)):
        br, x, y_ws, y_na = _run(lb, shape, batch, seed, lb.LB_PATH_PREFILL)
        _close(y_na, y_ws, f"prefill {shape.name} {batch} tokens")
    rows = np.arange(0, 520, 37)
    _close(y_na[:, rows], oracle.rows_forward(x, br, rows), "prefill ragged vs oracle rows")
