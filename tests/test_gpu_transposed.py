"""The transposed product dx = W^T dy (the backward-input of quantization-aware
training) through the same kernels: the packed factors are transposed on the
GPU (bit-exact against the oracle's packer of the transposed signs) and the
layer of W^T runs through littlebit_linear_fwd (parity against the oracle's
transposed_forward, the dense W^T in float64)."""

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


def _assert_parity(y_gpu, y_ref, what):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = y - y_ref
    rms = np.sqrt(np.mean(y_ref ** 2))
    rel = np.linalg.norm(err) / np.linalg.norm(y_ref)
    mx = np.max(np.abs(err)) / rms
    print(f"[parity] {what}: rel_l2={rel:.3e} max/rms={mx:.3e}", flush=True)
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e}"
    assert mx <= MAX_REL_RMS, f"{what}: max err {mx:.3e} x RMS"


@pytest.mark.parametrize("R,K", [(16, 64), (20, 600), (33, 130), (1472, 4096), (600, 20), (7, 1), (168, 13824)])
def test_transpose_packed_bit_exact(lb, R, K):
    """transpose(pack(S)) == pack(S^T), pad bits zero, odd units and ragged tiles."""
    print(f"[case] transpose R={R} K={K}", flush=True)
    rng = np.random.default_rng(R + 31 * K)
    lat = rng.standard_normal((R, K)).astype(np.float32)
    lat.flat[::53] = 0.0
    bits = lb.littlebit_pack(torch.from_numpy(lat).cuda(), transpose=False)
    got = lb.littlebit_transpose_packed(bits, R, K).cpu().numpy()
    want = oracle.pack_factor(oracle.sign_bits(lat, transpose=True))
    np.testing.assert_array_equal(got, want)
    # transposing twice gives the original packing back
    back = lb.littlebit_transpose_packed(lb.littlebit_transpose_packed(bits, R, K), K, R)
    assert torch.equal(back, bits)


@pytest.mark.parametrize("m,n,ranks,batch", [
    (512, 512, (32, 32), 1),       # the tiny configuration, decode
    (300, 1000, (130, 70), 5),     # ragged m, n, r; decode
    (1000, 200, (64,), 16),        # one branch, full decode batch
    (700, 900, (96, 96), 100),     # prefill
    (11008, 4096, (1472, 1472), 1),  # the 7B up-projection's transpose, batch 1
])
def test_transposed_product(lb, m, n, ranks, batch):
    print(f"[case] transposed m={m} n={n} r={ranks} batch={batch}", flush=True)
    shape = synth.LayerShape("transposed", m, n, ranks)
    br, _ = synth.make_layer(shape, batch=1, seed=m + n + batch)
    dy = synth.make_tokens(batch, m, np.random.default_rng(batch))
    layer = lb.LittleBitLayer.from_latents(br)
    lt = layer.transposed()
    assert (lt.m, lt.n) == (n, m)
    dx = lb.littlebit_linear_fwd(lt, torch.from_numpy(dy).cuda())
    _assert_parity(dx, oracle.transposed_forward(dy, br), f"W^T dy {m}x{n} r={ranks} b={batch}")
