"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar (per output array): relative L2 error <= 2e-3 and max |err| <= 1e-2 * RMS
of the oracle's output; packed sign bits are bit-exact against the oracle's
own packer.  Inputs come from binary_rank_gemv_amd.synth (seeded).  Full-size
configs compare every output against the oracle's factored float64
evaluator and a sample of outputs against the dense definition row by row.
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


# --------------------------------------------------------------------- packing

@pytest.mark.parametrize("R,K,transpose", [(16, 64, False), (20, 600, False), (600, 20, True),
                                           (1472, 4096, True), (11008, 1472, False),
                                           (168, 13824, False), (33, 130, True)])
def test_pack_bit_exact(lb, R, K, transpose):
    print(f"[case] pack R={R} K={K} transpose={transpose}", flush=True)
    rng = np.random.default_rng(R * 7 + K)
    shape = (K, R) if transpose else (R, K)
    lat = rng.standard_normal(shape).astype(np.float32)
    lat.flat[::97] = 0.0
    lat.flat[1::89] = -0.0
    got = lb.littlebit_pack(torch.from_numpy(lat).cuda(), transpose=transpose).cpu().numpy()
    want = oracle.pack_factor(oracle.sign_bits(lat, transpose=transpose))
    np.testing.assert_array_equal(got, want)


def test_pack_f16_and_strided(lb):
    print("[case] pack f16 strided", flush=True)
    rng = np.random.default_rng(11)
    lat = rng.standard_normal((100, 300)).astype(np.float16)
    lat[0, :5] = np.array([-0.0, 0.0, -6e-8, 6e-8, -65504], dtype=np.float16)
    full = torch.from_numpy(lat).cuda()
    view = full[:, 10:250]
    got = lb.littlebit_pack(view, transpose=False).cpu().numpy()
    want = oracle.pack_factor(oracle.sign_bits(lat[:, 10:250]))
    np.testing.assert_array_equal(got, want)
    got_t = lb.littlebit_pack(view, transpose=True).cpu().numpy()
    np.testing.assert_array_equal(got_t, oracle.pack_factor(oracle.sign_bits(lat[:, 10:250], transpose=True)))


# --------------------------------------------------------------- small layers

@pytest.mark.parametrize("two_launches", [False, True])
@pytest.mark.parametrize("batch", [1, 2, 5, 16])
def test_tiny_config_full_oracle(lb, batch, two_launches):
    print(f"[case] tiny batch={batch} two_launches={two_launches}", flush=True)
    br, x = synth.make_layer(synth.TINY, batch=batch, seed=0)
    layer = _layer(lb, br)
    path = lb.LB_DECODE_TWO_LAUNCHES if two_launches else lb.LB_PATH_AUTO
    y = lb.littlebit_linear_fwd(layer, torch.from_numpy(x).cuda(), path=path)
    _assert_parity(y, oracle.linear_forward(x, br), f"tiny b={batch} two={two_launches}")


@pytest.mark.parametrize("m,n,ranks,batch", [
    (100, 200, (40, 24), 3),      # ragged m, n, r: partial tiles, odd tail units
    (24, 72, (8,), 1),            # one branch, rank 8
    (1000, 1000, (130, 70), 7),   # several tiles, tails of 2 and 1 units
    (16, 8, (1, 1), 2),           # rank 1, n smaller than a step
    (520, 4104, (264, 264), 16),  # n not a multiple of 64, full batch
    # single launch with phase B's sign bytes copied to LDS during phase A:
    (81920, 64, (64, 64), 1),      # 20 tiles per workgroup: 16 copied, 4 read from memory
    (40960, 256, (1728, 1728), 1),  # 10 tiles of 6912 bytes: 9 fit the copy, 1 from memory
    (20000, 512, (1600,), 2),      # one branch, 5 tiles per workgroup
    (40000, 128, (96, 96), 5),     # batch 5: 9 tiles copied per workgroup, the rest from memory
    (600, 300, (3000, 3000), 13),  # z of 13 tokens exceeds the LDS: launches of 9 and 4 tokens
    # one token, more V tiles than workgroups (two tiles per unit): odd tile
    # counts (the last unit's second tile is its first) and partial tiles
    (700, 520, (2600, 2072), 1),   # 163 + 130 tiles
    (300, 200, (4088, 1000), 1),   # 256 + 63 tiles, rank near its limit
    # phase A's staging of g*x: n % 8 != 0 (element-wise loads), and n > 8192
    # (a second batch of sign words, a chunk cut at the batch's end)
    (90, 130, (24, 40), 3),
    (64, 1001, (32,), 1),
    (256, 9000, (48, 48), 4),
    (200, 9001, (40, 24), 16),
])
def test_ragged_shapes(lb, m, n, ranks, batch):
    print(f"[case] ragged m={m} n={n} r={ranks} batch={batch}", flush=True)
    shape = synth.LayerShape("ragged", m, n, ranks)
    br, x = synth.make_layer(shape, batch=batch, seed=m + n)
    layer = _layer(lb, br)
    xt = torch.from_numpy(x).cuda()
    y = lb.littlebit_linear_fwd(layer, xt)
    _assert_parity(y, oracle.linear_forward(x, br), f"ragged {m}x{n} r={ranks} b={batch}")
    # the single launch and the two-launch path sum in the same order
    assert torch.equal(y, lb.littlebit_linear_fwd(layer, xt, path=lb.LB_DECODE_TWO_LAUNCHES))


@pytest.mark.parametrize("batch", [1, 5, 16])
def test_unaligned_activations(lb, batch):
    """x as a view whose rows start 2 bytes past a 16-byte boundary and whose
    row stride is odd: phase A stages g*x with element-wise loads."""
    print(f"[case] unaligned x batch={batch}", flush=True)
    shape = synth.LayerShape("unaligned", 300, 520, (40, 56))
    br, x = synth.make_layer(shape, batch=batch, seed=11)
    layer = _layer(lb, br)
    big = torch.zeros((batch, 521), dtype=torch.float16, device="cuda")
    big[:, 1:] = torch.from_numpy(x).cuda()
    xv = big[:, 1:]
    assert xv.data_ptr() % 16 == 2 and xv.stride(0) == 521
    y = lb.littlebit_linear_fwd(layer, xv)
    _assert_parity(y, oracle.linear_forward(x, br), f"unaligned x b={batch}")
    assert torch.equal(y, lb.littlebit_linear_fwd(layer, torch.from_numpy(x).cuda()))


def test_branch_masks_and_additivity(lb):
    print("[case] branch masks", flush=True)
    br, x = synth.make_layer(synth.LayerShape("mask", 300, 500, (48, 72)), batch=4, seed=3)
    layer = _layer(lb, br)
    xt = torch.from_numpy(x).cuda()
    y1 = lb.littlebit_linear_fwd(layer, xt, branch_mask=1)
    y2 = lb.littlebit_linear_fwd(layer, xt, branch_mask=2)
    y3 = lb.littlebit_linear_fwd(layer, xt, branch_mask=3)
    _assert_parity(y1, oracle.linear_forward(x, br[:1]), "primary only")
    _assert_parity(y2, oracle.linear_forward(x, br[1:]), "residual only")
    _assert_parity(y3, oracle.linear_forward(x, br), "both")
    _assert_parity(y1.float() + y2.float(), oracle.linear_forward(x, br), "sum of single branches")


def test_hadamard_special_case_on_gpu(lb):
    """sign(U) = sign(V) = Sylvester H, l = 2^-k: the layer is diag(sum_b h_b g_b)."""
    print("[case] hadamard", flush=True)
    import scipy.linalg
    k = 6
    nn = 2 ** k
    H = scipy.linalg.hadamard(nn).astype(np.float32)
    rng = np.random.default_rng(9)
    br = [{"U": H * rng.uniform(0.1, 2, (nn, nn)).astype(np.float32),
           "V": H * rng.uniform(0.1, 2, (nn, nn)).astype(np.float32),
           "h": rng.uniform(0.5, 1.5, nn).astype(np.float16),
           "l": np.full(nn, 2.0 ** -k, dtype=np.float16),
           "g": rng.uniform(0.5, 1.5, nn).astype(np.float16)} for _ in range(2)]
    x = rng.standard_normal((3, nn)).astype(np.float16)
    y = lb.littlebit_linear_fwd(_layer(lb, br), torch.from_numpy(x).cuda())
    want = sum(b["h"].astype(np.float64) * b["g"].astype(np.float64) for b in br) * x.astype(np.float64)
    _assert_parity(y, want, "hadamard")


def test_determinism_and_poisoned_buffers(lb):
    print("[case] determinism", flush=True)
    br, x = synth.make_layer(synth.LayerShape("det", 700, 900, (96, 96)), batch=3, seed=5)
    layer = _layer(lb, br)
    xt = torch.from_numpy(x).cuda()
    need = lb.littlebit_linear_workspace_bytes(layer, 3)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")   # garbage data region
    ws[:4096] = 0                                                       # zeroed sync header
    out = torch.full((3, 700), float("nan"), dtype=torch.float16, device="cuda")
    y_a = lb.littlebit_linear_fwd(layer, xt, out=out, workspace=ws).clone()
    y_b = lb.littlebit_linear_fwd(layer, xt).clone()
    y_c = lb.littlebit_linear_fwd(layer, xt, path=lb.LB_DECODE_TWO_LAUNCHES).clone()
    for _ in range(5):
        lb.littlebit_linear_fwd(layer, xt, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_b) and torch.equal(y_a, y_c) and torch.equal(out, y_a)
    _assert_parity(y_a, oracle.linear_forward(x, br), "poisoned")
    # header: one 64-bit call counter per workgroup of the single launch
    # (bytes 8*w, at most 256 workgroups), error word at byte 2048.  Six
    # single-launch calls ran on this workspace.
    hdr = ws[:4096].cpu()
    counters = hdr[:2048].view(torch.int64).tolist()
    grid = min(torch.cuda.get_device_properties(0).multi_processor_count, 256)
    assert int(hdr[2048:2052].view(torch.int32)) == 0, "z poll spin limit hit"
    assert counters[:grid] == [6] * grid and not any(counters[grid:]), counters


@pytest.mark.parametrize("setting", ["0.55", "0.1"])
def test_block_repeated_calls_one_workspace(lb, setting):
    """Consecutive block calls on one workspace: each equals the first bit for
    bit, no z poll gave up, and every workgroup's call counter advanced once
    per call (a tag taken before the counter is read would fail from the
    second call on)."""
    print(f"[case] 13b block {setting} repeated calls", flush=True)
    shapes, layers, xs = synth.make_block13b(setting, batch=1, seed=3)
    dev_layers = [_layer(lb, br) for br in layers]
    xt = [torch.from_numpy(a).cuda() for a in xs]
    ws = torch.zeros((lb.littlebit_block_workspace_bytes(dev_layers, 1),), dtype=torch.uint8, device="cuda")
    first = [y.clone() for y in lb.littlebit_block_fwd(dev_layers, *xt, workspace=ws)]
    for _ in range(3):
        ys = lb.littlebit_block_fwd(dev_layers, *xt, workspace=ws)
        for a, b in zip(first, ys):
            assert torch.equal(a, b)
    torch.cuda.synchronize()
    hdr = ws[:4096].cpu()
    assert int(hdr[2048:2052].view(torch.int32)) == 0, "z poll spin limit hit"
    counters = hdr[:2048].view(torch.int64).tolist()
    grid = min(torch.cuda.get_device_properties(0).multi_processor_count, 256)
    assert counters[:grid] == [4] * grid and not any(counters[grid:]), counters
    for i in (0, 6):
        xi = synth.block_inputs_for(i, xs)
        _assert_parity(first[i], oracle.factored_forward(xi, layers[i]), f"13B {setting} {shapes[i].name} repeated")


def test_strided_rows(lb):
    print("[case] strided x/y", flush=True)
    br, x = synth.make_layer(synth.LayerShape("strided", 256, 320, (32, 32)), batch=4, seed=6)
    layer = _layer(lb, br)
    xbig = torch.zeros((4, 400), dtype=torch.float16, device="cuda")
    xbig[:, :320] = torch.from_numpy(x).cuda()
    ybig = torch.full((4, 264), 7.0, dtype=torch.float16, device="cuda")
    lb.littlebit_linear_fwd(layer, xbig[:, :320], out=ybig[:, :256])
    _assert_parity(ybig[:, :256], oracle.linear_forward(x, br), "strided")
    assert (ybig[:, 256:] == 7.0).all()


# ------------------------------------------------------------ full-size configs

def _full_size_check(lb, br, x, what, nrows=64, path=None):
    layer = _layer(lb, br)
    xt = torch.from_numpy(x).cuda()
    y = (lb.littlebit_linear_fwd(layer, xt) if path is None
         else lb.littlebit_linear_fwd(layer, xt, path=path))
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy().astype(np.float64)
    _assert_parity(yg, oracle.factored_forward(x, br), what + " (all outputs, factored oracle)")
    rows = np.random.default_rng(0).choice(br[0]["U"].shape[0], nrows, replace=False)
    _assert_parity(yg[:, rows], oracle.rows_forward(x, br, rows), what + " (sampled rows, dense oracle)")
    return layer, xt, y


@pytest.mark.parametrize("two_launches", [False, True])
def test_llama2_7b_up_batch1(lb, two_launches):
    print(f"[case] 7b up batch 1 two_launches={two_launches}", flush=True)
    br, x = synth.make_layer(synth.UP7B, batch=1, seed=0)
    _full_size_check(lb, br, x, f"7B up b=1 two={two_launches}",
                     path=lb.LB_DECODE_TWO_LAUNCHES if two_launches else None)


@pytest.mark.parametrize("batch", [1, 16])
def test_llama2_70b_up(lb, batch):
    print(f"[case] 70b up batch {batch}", flush=True)
    br, x = synth.make_layer(synth.UP70B, batch=batch, seed=0)
    _full_size_check(lb, br, x, f"70B up b={batch}")


@pytest.mark.parametrize("bpw,batch", [(1.0, 1), (0.8, 1), (0.3, 1), (0.1, 1), (0.1, 16), (1.0, 16)])
def test_70b_bpw_sweep_ranks(lb, bpw, batch):
    """The ranks of the bits-per-weight sweep (0.55 is the 70B case above)."""
    print(f"[case] 70b up {bpw} bpw batch {batch}", flush=True)
    br, x = synth.make_layer(synth.up70b_at_bpw(bpw), batch=batch, seed=1)
    _full_size_check(lb, br, x, f"70B up {bpw} BPW b={batch}")


@pytest.mark.parametrize("setting,batch", [("0.1", 16), ("0.55", 4)])
def test_llama2_13b_block_several_tokens(lb, setting, batch):
    """The multi-layer launch at several tokens (the multi-token kernels):
    every projection against the oracle, and equal to the single-launch
    per-layer call's sums order (two-launch path) bit for bit."""
    print(f"[case] 13b block {setting} batch {batch}", flush=True)
    shapes, layers, xs = synth.make_block13b(setting, batch=batch, seed=4)
    dev_layers = [_layer(lb, br) for br in layers]
    xt = [torch.from_numpy(a).cuda() for a in xs]
    ys = lb.littlebit_block_fwd(dev_layers, *xt)
    torch.cuda.synchronize()
    for i, (shape, br) in enumerate(zip(shapes, layers)):
        xi = synth.block_inputs_for(i, xs)
        _assert_parity(ys[i], oracle.factored_forward(xi, br), f"13B {setting} b={batch} {shape.name}")
        y2 = lb.littlebit_linear_fwd(dev_layers[i], torch.from_numpy(xi).cuda(), path=lb.LB_DECODE_TWO_LAUNCHES)
        assert torch.equal(ys[i], y2), f"13B {setting} b={batch} {shape.name}: block and two-launch differ"


@pytest.mark.parametrize("ranks", [
    # gate/up with 12 pairs per branch (3 per wave in phase B), the others 6-8
    {"attn": (688, 112), "mlp": (1472, 168), "down": (1008, 1008)},
    # one-branch layers among the two-branch ones
    {"attn": (688,), "mlp": (1008, 168), "down": (256,)},
])
def test_block_one_token_mixed_ranks(lb, ranks):
    """A seven-projection call at one token on smaller dimensions with mixed
    ranks and branch counts: every projection against the oracle, and equal
    bit for bit to the same projection's two-launch call."""
    print(f"[case] block one token ranks {ranks}", flush=True)
    d, f = 1024, 2816
    shapes = [synth.LayerShape(nm, mm, nn, ranks[key]) for nm, mm, nn, key in (
        ("q", d, d, "attn"), ("k", d, d, "attn"), ("v", d, d, "attn"), ("o", d, d, "attn"),
        ("gate", f, d, "mlp"), ("up", f, d, "mlp"), ("down", d, f, "down"))]
    rng = np.random.default_rng(11)
    layers = [synth.make_branches(sh, rng) for sh in shapes]
    xs = (synth.make_tokens(1, d, rng), synth.make_tokens(1, d, rng), synth.make_tokens(1, d, rng),
          synth.make_tokens(1, f, rng))
    dev_layers = [_layer(lb, br) for br in layers]
    xt = [torch.from_numpy(a).cuda() for a in xs]
    ws = torch.zeros((lb.littlebit_block_workspace_bytes(dev_layers, 1),), dtype=torch.uint8, device="cuda")
    ys = lb.littlebit_block_fwd(dev_layers, *xt, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[2048:2052].cpu().view(torch.int32)) == 0, "z poll spin limit hit"
    for i, (shape, br) in enumerate(zip(shapes, layers)):
        xi = synth.block_inputs_for(i, xs)
        _assert_parity(ys[i], oracle.factored_forward(xi, br), f"block {shape.name} {ranks}")
        y2 = lb.littlebit_linear_fwd(dev_layers[i], torch.from_numpy(xi).cuda(), path=lb.LB_DECODE_TWO_LAUNCHES)
        assert torch.equal(ys[i], y2), f"block {shape.name} {ranks}: block and two-launch differ"


@pytest.mark.parametrize("setting", ["0.55", "0.1"])
def test_llama2_13b_block(lb, setting):
    print(f"[case] 13b block {setting}", flush=True)
    shapes, layers, xs = synth.make_block13b(setting, batch=1, seed=0)
    dev_layers = [_layer(lb, br) for br in layers]
    xt = [torch.from_numpy(a).cuda() for a in xs]
    ys = lb.littlebit_block_fwd(dev_layers, *xt)
    torch.cuda.synchronize()
    for i, (shape, br) in enumerate(zip(shapes, layers)):
        xi = synth.block_inputs_for(i, xs)
        _assert_parity(ys[i], oracle.factored_forward(xi, br), f"13B {setting} {shape.name}")
        # the block call agrees with the single-layer call on the same projection
        if i in (0, 6):
            y1 = lb.littlebit_linear_fwd(dev_layers[i], torch.from_numpy(xi).cuda())
            _assert_parity(y1, oracle.factored_forward(xi, br), f"13B {setting} {shape.name} single")
