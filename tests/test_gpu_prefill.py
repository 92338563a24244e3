"""GPU parity of the prefill path (two matrix-core GEMMs) against the CPU oracle.

Same bar as the decode tests: relative L2 error <= 2e-3 and max |err| <=
1e-2 * RMS of the oracle's output, per output array.  Cases cover token
counts that leave partial 128-token blocks, ragged m / n / r (partial row
tiles, odd last 64-input units), n not a multiple of 8 and unaligned rows
(the element-wise staging path), one branch, branch masks, the Hadamard
special case, more than 8192 tokens (chunked calls), the 13B block, and the
2048-token prefill of the Llama2-7B-shaped up-projection.
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
    y = y_gpu.float().cpu().numpy().astype(np.float64) if torch.is_tensor(y_gpu) else y_gpu
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = y - y_ref
    rms = np.sqrt(np.mean(y_ref ** 2))
    rel = np.linalg.norm(err) / np.linalg.norm(y_ref)
    mx = np.max(np.abs(err)) / rms
    print(f"[parity] {what}: rel_l2={rel:.3e} max/rms={mx:.3e}", flush=True)
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e}"
    assert mx <= MAX_REL_RMS, f"{what}: max err {mx:.3e} x RMS"
    assert np.max(np.abs(y_ref)) < 65504, f"{what}: oracle output exceeds fp16 range"


def _layer(lb, branches):
    return lb.LittleBitLayer.from_latents(branches)


@pytest.mark.parametrize("batch", [1, 5, 17, 64, 130])
def test_prefill_tiny(lb, batch):
    print(f"[case] prefill tiny batch={batch}", flush=True)
    br, x = synth.make_layer(synth.TINY, batch=batch, seed=1)
    layer = _layer(lb, br)
    xt = torch.from_numpy(x).cuda()
    y = lb.littlebit_linear_fwd(layer, xt, path=lb.LB_PATH_PREFILL)
    _assert_parity(y, oracle.linear_forward(x, br), f"prefill tiny b={batch}")
    if batch > 16:   # the automatic choice takes the same path
        ya = lb.littlebit_linear_fwd(layer, xt)
        assert torch.equal(ya, y)


@pytest.mark.parametrize("m,n,ranks,batch", [
    (100, 200, (40, 24), 37),      # partial row tiles, odd last units, partial token block
    (24, 72, (8,), 130),           # one branch, rank 8
    (1000, 1000, (130, 70), 257),  # several row blocks, tails of 2 and 1 units
    (16, 8, (1, 1), 20),           # rank 1, n smaller than a step
    (520, 4104, (264, 264), 200),  # n not a multiple of 64
    (300, 100, (48, 72), 50),      # n % 8 != 0: element-wise staging
])
def test_prefill_ragged(lb, m, n, ranks, batch):
    print(f"[case] prefill ragged m={m} n={n} r={ranks} batch={batch}", flush=True)
    shape = synth.LayerShape("ragged", m, n, ranks)
    br, x = synth.make_layer(shape, batch=batch, seed=m + n + batch)
    y = lb.littlebit_linear_fwd(_layer(lb, br), torch.from_numpy(x).cuda(), path=lb.LB_PATH_PREFILL)
    _assert_parity(y, oracle.linear_forward(x, br), f"prefill ragged {m}x{n} r={ranks} b={batch}")


def test_prefill_strided_unaligned_rows(lb):
    print("[case] prefill strided", flush=True)
    br, x = synth.make_layer(synth.LayerShape("strided", 256, 320, (32, 48)), batch=40, seed=6)
    layer = _layer(lb, br)
    xbig = torch.zeros((40, 403), dtype=torch.float16, device="cuda")   # odd row stride
    xbig[:, 1:321] = torch.from_numpy(x).cuda()                          # 2-byte aligned start
    ybig = torch.full((40, 261), 7.0, dtype=torch.float16, device="cuda")
    lb.littlebit_linear_fwd(layer, xbig[:, 1:321], out=ybig[:, 3:259], path=lb.LB_PATH_PREFILL)
    _assert_parity(ybig[:, 3:259], oracle.linear_forward(x, br), "prefill strided")
    assert (ybig[:, :3] == 7.0).all() and (ybig[:, 259:] == 7.0).all()


@pytest.mark.parametrize("col0,width", [(8, 528), (3, 517)])
def test_prefill_output_views(lb, col0, width):
    """The main prefill kernels writing into a view of a wider output: a
    16-byte aligned start and row pitch (rows stored through LDS as whole
    16-byte pieces), and an odd start and pitch (direct stores).  Every value
    matches the oracle and nothing outside the view is written."""
    print(f"[case] prefill output view col0={col0} width={width}", flush=True)
    m, n, batch = 512, 256, 200
    br, x = synth.make_layer(synth.LayerShape("view", m, n, (64, 96)), batch=batch, seed=col0 + width)
    ybig = torch.full((batch, width), 7.0, dtype=torch.float16, device="cuda")
    lb.littlebit_linear_fwd(_layer(lb, br), torch.from_numpy(x).cuda(), out=ybig[:, col0:col0 + m],
                            path=lb.LB_PATH_PREFILL)
    _assert_parity(ybig[:, col0:col0 + m], oracle.linear_forward(x, br), f"prefill view col0={col0}")
    assert (ybig[:, :col0] == 7.0).all() and (ybig[:, col0 + m:] == 7.0).all()


def test_prefill_branch_masks(lb):
    print("[case] prefill branch masks", flush=True)
    br, x = synth.make_layer(synth.LayerShape("mask", 300, 512, (48, 72)), batch=33, seed=3)
    layer = _layer(lb, br)
    xt = torch.from_numpy(x).cuda()
    y1 = lb.littlebit_linear_fwd(layer, xt, branch_mask=1)
    y2 = lb.littlebit_linear_fwd(layer, xt, branch_mask=2)
    y3 = lb.littlebit_linear_fwd(layer, xt, branch_mask=3)
    _assert_parity(y1, oracle.linear_forward(x, br[:1]), "prefill primary only")
    _assert_parity(y2, oracle.linear_forward(x, br[1:]), "prefill residual only")
    _assert_parity(y3, oracle.linear_forward(x, br), "prefill both")


def test_prefill_hadamard_and_negative_scales(lb):
    """sign(U) = sign(V) = Sylvester H, l = 2^-k: the layer is diag(sum_b h_b g_b).
    Half of h and g are negative, which exercises the sign-folded row scale."""
    print("[case] prefill hadamard", flush=True)
    import scipy.linalg
    k = 7
    nn = 2 ** k
    H = scipy.linalg.hadamard(nn).astype(np.float32)
    rng = np.random.default_rng(19)
    br = [{"U": H * rng.uniform(0.1, 2, (nn, nn)).astype(np.float32),
           "V": H * rng.uniform(0.1, 2, (nn, nn)).astype(np.float32),
           "h": (rng.uniform(0.5, 1.5, nn) * rng.choice([-1, 1], nn)).astype(np.float16),
           "l": np.full(nn, 2.0 ** -k, dtype=np.float16),
           "g": (rng.uniform(0.5, 1.5, nn) * rng.choice([-1, 1], nn)).astype(np.float16)} for _ in range(2)]
    x = rng.standard_normal((70, nn)).astype(np.float16)
    y = lb.littlebit_linear_fwd(_layer(lb, br), torch.from_numpy(x).cuda(), path=lb.LB_PATH_PREFILL)
    want = sum(b["h"].astype(np.float64) * b["g"].astype(np.float64) for b in br) * x.astype(np.float64)
    _assert_parity(y, want, "prefill hadamard")


def test_prefill_matches_decode(lb):
    """The two paths on the same 16 tokens: both within the bar of the oracle."""
    print("[case] prefill vs decode", flush=True)
    br, x = synth.make_layer(synth.LayerShape("both", 640, 768, (96, 64)), batch=16, seed=8)
    layer = _layer(lb, br)
    xt = torch.from_numpy(x).cuda()
    yd = lb.littlebit_linear_fwd(layer, xt, path=lb.LB_PATH_DECODE)
    yp = lb.littlebit_linear_fwd(layer, xt, path=lb.LB_PATH_PREFILL)
    ref = oracle.linear_forward(x, br)
    _assert_parity(yd, ref, "decode 16")
    _assert_parity(yp, ref, "prefill 16")
    _assert_parity(yp, yd.float().cpu().numpy().astype(np.float64), "prefill vs decode")


@pytest.mark.parametrize("m,ranks,batch", [
    (256, (1728, 1728), 2048),  # GEMM 1 in 256-row blocks (224 workgroups), GEMM 2 in 192-row blocks
    (4000, (200, 1000), 300),   # both GEMMs in 192-row blocks, ragged last block and token block
    (11008, (32, 32), 2048),    # GEMM 2 split: 512 row tiles in 256-row blocks, 176 in 192-row blocks
])
def test_prefill_block_geometries(lb, m, ranks, batch):
    """Both row-block heights of the main prefill kernels (the library picks
    the one that fills the compute units in fewer rounds of rows)."""
    print(f"[case] prefill geometry m={m} r={ranks} batch={batch}", flush=True)
    n = 128 if m > 10000 else 256
    br, x = synth.make_layer(synth.LayerShape("geometry", m, n, ranks), batch=batch, seed=m + batch)
    y = lb.littlebit_linear_fwd(_layer(lb, br), torch.from_numpy(x).cuda(), path=lb.LB_PATH_PREFILL)
    _assert_parity(y, oracle.factored_forward(x, br), f"prefill geometry m={m} r={ranks} b={batch}")


def test_prefill_chunked_beyond_8192_tokens(lb):
    print("[case] prefill 8200 tokens", flush=True)
    br, x = synth.make_layer(synth.LayerShape("long", 96, 128, (16, 16)), batch=8200, seed=4)
    y = lb.littlebit_linear_fwd(_layer(lb, br), torch.from_numpy(x).cuda())
    _assert_parity(y, oracle.factored_forward(x, br), "prefill 8200 tokens")


def test_prefill_llama2_7b_up_2048_tokens(lb):
    print("[case] prefill 7b up 2048 tokens", flush=True)
    br, x = synth.make_layer(synth.UP7B, batch=synth.PREFILL_TOKENS, seed=0)
    y = lb.littlebit_linear_fwd(_layer(lb, br), torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy().astype(np.float64)
    _assert_parity(yg, oracle.factored_forward(x, br), "prefill 7B up 2048 (all outputs, factored oracle)")
    rng = np.random.default_rng(0)
    rows = rng.choice(synth.UP7B.m, 32, replace=False)
    toks = rng.choice(synth.PREFILL_TOKENS, 64, replace=False)
    _assert_parity(yg[np.ix_(toks, rows)], oracle.rows_forward(x[toks], br, rows),
                   "prefill 7B up 2048 (sampled outputs, dense oracle)")


def test_prefill_llama2_13b_block(lb):
    print("[case] prefill 13b block 0.1, 48 tokens", flush=True)
    shapes, layers, xs = synth.make_block13b("0.1", batch=48, seed=2)
    dev_layers = [_layer(lb, br) for br in layers]
    ys = lb.littlebit_block_fwd(dev_layers, *[torch.from_numpy(a).cuda() for a in xs])
    torch.cuda.synchronize()
    for i, (shape, br) in enumerate(zip(shapes, layers)):
        _assert_parity(ys[i], oracle.factored_forward(synth.block_inputs_for(i, xs), br),
                       f"prefill 13B 0.1 {shape.name}")
