"""GPU parity of the decode path in the cases that plain random inputs miss:
call sequences that mix the decode variants on one fresh workspace, negative
and subnormal scales, outputs and intermediates near the fp16 limit, and the
poll error word (littlebit_workspace_error) after every case.

Bar (per output array): relative L2 error <= 2e-3 and max |err| <= 1e-2 * RMS
of the oracle's output.  Inputs come from binary_rank_gemv_amd.synth (seeded)
and are then rescaled as each case says; the oracle always sees the exact
fp16 values the GPU sees.
"""

import numpy as np
import pytest
import torch

import oracle
from binary_rank_gemv_amd import synth

pytestmark = pytest.mark.gpu

REL_L2 = 2e-3
MAX_REL_RMS = 1e-2


@pytest.fixture(scope="module")
def lb():
    from binary_rank_gemv_amd import littlebit
    return littlebit


def _assert_parity(y_gpu, y_ref, what=""):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = y - y_ref
    rms = np.sqrt(np.mean(y_ref ** 2))
    rel = np.linalg.norm(err) / np.linalg.norm(y_ref)
    mx = np.max(np.abs(err)) / rms
    print(f"[parity] {what}: rel_l2={rel:.3e} max/rms={mx:.3e} max|y|={np.max(np.abs(y_ref)):.4g}", flush=True)
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e}"
    assert mx <= MAX_REL_RMS, f"{what}: max err {mx:.3e} x RMS"
    assert np.max(np.abs(y_ref)) < 65504, f"{what}: oracle output exceeds fp16 range"


def _no_poll_error(lb, ws, what):
    err = lb.littlebit_workspace_error(ws)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, f"{what}: a z poll gave up"


def _fresh_ws(nbytes):
    return torch.zeros(nbytes, dtype=torch.uint8, device="cuda")


# ------------------------------------------------ mixed call sequences

@pytest.mark.parametrize("shape,batch", [
    (synth.LayerShape("mix", 700, 900, (96, 96)), 1),
    (synth.LayerShape("mix16", 520, 640, (64, 48)), 16),
    (synth.UP7B, 1),
])
def test_two_launch_then_single_launch_on_fresh_workspace(lb, shape, batch):
    """A two-launch call with x1 and then a default (single-launch) call with
    x2 on one freshly zeroed workspace: the second call returns layer(x2),
    never a mix with x1's rank-space intermediate."""
    print(f"[case] mixed sequence {shape.name} batch={batch}", flush=True)
    br, x1 = synth.make_layer(shape, batch=batch, seed=21)
    x2 = synth.make_tokens(batch, shape.n, np.random.default_rng(22))
    layer = lb.LittleBitLayer.from_latents(br)
    ws = _fresh_ws(lb.littlebit_linear_workspace_bytes(layer, batch))
    y1 = lb.littlebit_linear_fwd(layer, torch.from_numpy(x1).cuda(), path=lb.LB_DECODE_TWO_LAUNCHES,
                                 workspace=ws).clone()
    y2 = lb.littlebit_linear_fwd(layer, torch.from_numpy(x2).cuda(), workspace=ws).clone()
    y3 = lb.littlebit_linear_fwd(layer, torch.from_numpy(x1).cuda(), workspace=ws).clone()
    torch.cuda.synchronize()
    _assert_parity(y1, oracle.factored_forward(x1, br), f"{shape.name} two-launch x1")
    _assert_parity(y2, oracle.factored_forward(x2, br), f"{shape.name} single launch x2 after two-launch x1")
    _assert_parity(y3, oracle.factored_forward(x1, br), f"{shape.name} single launch x1 again")
    assert torch.equal(y1, y3)
    _no_poll_error(lb, ws, shape.name)


def test_two_launch_then_block_on_fresh_workspace(lb):
    """The same sequence across entry points: a two-launch call of the q
    projection on the block's fresh workspace (its z lands where the block's
    q projection keeps z), then a block call with other inputs."""
    print("[case] mixed sequence: linear two-launch then block", flush=True)
    shapes, layers, xs = synth.make_block13b("0.1", batch=1, seed=31)
    _, _, xs2 = synth.make_block13b("0.1", batch=1, seed=32)
    dev = [lb.LittleBitLayer.from_latents(br) for br in layers]
    ws = _fresh_ws(lb.littlebit_block_workspace_bytes(dev, 1))
    lb.littlebit_linear_fwd(dev[0], torch.from_numpy(xs[0]).cuda(), path=lb.LB_DECODE_TWO_LAUNCHES, workspace=ws)
    ys = lb.littlebit_block_fwd(dev, *[torch.from_numpy(a).cuda() for a in xs2], workspace=ws)
    torch.cuda.synchronize()
    for i, (shape, br) in enumerate(zip(shapes, layers)):
        _assert_parity(ys[i], oracle.factored_forward(synth.block_inputs_for(i, xs2), br),
                       f"block after two-launch q: {shape.name}")
    _no_poll_error(lb, ws, "block after two-launch")


# ----------------------------------------------------- scales and range

def _rescaled(shape, batch, seed, h=None, l=None, g=None, x=None):
    """synth draws, then each scale array (and x) replaced by f(array, rng)
    rounded to fp16."""
    br, xs = synth.make_layer(shape, batch=batch, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    for b in br:
        for key, f in (("h", h), ("l", l), ("g", g)):
            if f is not None:
                b[key] = np.asarray(f(b[key].astype(np.float64), rng)).astype(np.float16)
    if x is not None:
        xs = np.asarray(x(xs.astype(np.float64), rng)).astype(np.float16)
    return br, xs


def _neg(a, rng):
    return a * rng.choice([-1.0, 1.0], a.shape)


@pytest.mark.parametrize("shape,batch", [
    (synth.LayerShape("neg", 300, 520, (40, 56)), 1),
    (synth.LayerShape("neg", 300, 520, (40, 56)), 5),
    (synth.LayerShape("neg16", 1000, 1000, (130, 70)), 16),
    (synth.UP7B, 1),
])
def test_decode_negative_scales(lb, shape, batch):
    """Half of every h, l and g negative (the decode twin of the prefill
    Hadamard case with negative scales)."""
    print(f"[case] negative scales {shape.name} batch={batch}", flush=True)
    br, x = _rescaled(shape, batch, 41, h=_neg, l=_neg, g=_neg)
    layer = lb.LittleBitLayer.from_latents(br)
    xt = torch.from_numpy(x).cuda()
    ws = _fresh_ws(lb.littlebit_linear_workspace_bytes(layer, batch))
    y = lb.littlebit_linear_fwd(layer, xt, workspace=ws)
    y2 = lb.littlebit_linear_fwd(layer, xt, path=lb.LB_DECODE_TWO_LAUNCHES, workspace=ws)
    _assert_parity(y, oracle.factored_forward(x, br), f"negative scales {shape.name} b={batch}")
    assert torch.equal(y, y2)
    _no_poll_error(lb, ws, "negative scales")


def test_decode_hadamard_negative_scales(lb):
    """sign(U) = sign(V) = Sylvester H, l = 2^-k, h and g of both signs: the
    layer is diag(sum_b h_b g_b), exactly."""
    print("[case] decode hadamard negative scales", flush=True)
    import scipy.linalg
    k = 7
    nn = 2 ** k
    H = scipy.linalg.hadamard(nn).astype(np.float32)
    rng = np.random.default_rng(29)
    br = [{"U": H * rng.uniform(0.1, 2, (nn, nn)).astype(np.float32),
           "V": H * rng.uniform(0.1, 2, (nn, nn)).astype(np.float32),
           "h": (rng.uniform(0.5, 1.5, nn) * rng.choice([-1, 1], nn)).astype(np.float16),
           "l": np.full(nn, 2.0 ** -k, dtype=np.float16),
           "g": (rng.uniform(0.5, 1.5, nn) * rng.choice([-1, 1], nn)).astype(np.float16)} for _ in range(2)]
    x = rng.standard_normal((4, nn)).astype(np.float16)
    y = lb.littlebit_linear_fwd(lb.LittleBitLayer.from_latents(br), torch.from_numpy(x).cuda())
    want = sum(b["h"].astype(np.float64) * b["g"].astype(np.float64) for b in br) * x.astype(np.float64)
    _assert_parity(y, want, "decode hadamard negative scales")


@pytest.mark.parametrize("batch", [1, 16])
def test_decode_outputs_near_fp16_max(lb, batch):
    """Row scales chosen so that max |y| is about 60000 (fp16 max 65504)."""
    print(f"[case] outputs near fp16 max batch={batch}", flush=True)
    shape = synth.LayerShape("range", 640, 768, (96, 64))
    br, x = synth.make_layer(shape, batch=batch, seed=51)
    peak = np.max(np.abs(oracle.factored_forward(x, br)))
    c = 60000.0 / peak / 1.02
    for b in br:
        b["h"] = (b["h"].astype(np.float64) * c).astype(np.float16)
    want = oracle.factored_forward(x, br)
    assert 45000 < np.max(np.abs(want)) < 65504
    y = lb.littlebit_linear_fwd(lb.LittleBitLayer.from_latents(br), torch.from_numpy(x).cuda())
    _assert_parity(y, want, f"outputs near fp16 max b={batch}")


@pytest.mark.parametrize("batch", [1, 16])
def test_decode_latent_near_fp16_max(lb, batch):
    """Latent scales chosen so that max |l * t| is about 30000 (z is held in
    fp16), row scales small enough that y stays in range."""
    print(f"[case] latent near fp16 max batch={batch}", flush=True)
    shape = synth.LayerShape("zrange", 512, 1024, (64, 64))
    br, x = synth.make_layer(shape, batch=batch, seed=53)
    xd = x.astype(np.float64)
    tmax = max(np.max(np.abs((xd * b["g"].astype(np.float64)) @ np.where(b["V"] < 0, -1.0, 1.0))) for b in br)
    c = 30000.0 / tmax / 1.5  # l is at most 1.5
    for b in br:
        b["l"] = (b["l"].astype(np.float64) * c).astype(np.float16)
        b["h"] = (b["h"].astype(np.float64) * 1e-3).astype(np.float16)
    zmax = max(np.max(np.abs(((xd * b["g"].astype(np.float64)) @ np.where(b["V"] < 0, -1.0, 1.0))
                             * b["l"].astype(np.float64))) for b in br)
    assert 15000 < zmax < 65504
    want = oracle.factored_forward(x, br)
    y = lb.littlebit_linear_fwd(lb.LittleBitLayer.from_latents(br), torch.from_numpy(x).cuda())
    _assert_parity(y, want, f"latent near fp16 max b={batch}")


@pytest.mark.parametrize("batch", [1, 5])
def test_decode_subnormal_scales(lb, batch):
    """Column and latent scales in the fp16 subnormal range (below 2^-14),
    activations and row scales large enough that u, z and y stay normal."""
    print(f"[case] subnormal scales batch={batch}", flush=True)
    shape = synth.LayerShape("subnormal", 384, 512, (48, 32))
    br, x = _rescaled(shape, batch, 61,
                      g=lambda a, rng: rng.uniform(2e-5, 5.5e-5, a.shape),
                      l=lambda a, rng: rng.uniform(2e-5, 5.5e-5, a.shape),
                      h=lambda a, rng: a * 64.0,
                      x=lambda a, rng: a * 4096.0)
    assert all((b["g"].astype(np.float64) < 2.0 ** -14).all() for b in br)
    want = oracle.factored_forward(x, br)
    y = lb.littlebit_linear_fwd(lb.LittleBitLayer.from_latents(br), torch.from_numpy(x).cuda())
    _assert_parity(y, want, f"subnormal g and l b={batch}")
