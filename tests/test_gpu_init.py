"""GPU parity of the Dual-SVID initialization (littlebit_dual_svid_init,
through the C ABI), with and without the Joint-ITQ rotation, against the
float64 oracle (oracle.dual_svid_init).

Bar (a reading: the method reaches the oracle's result up to floating-point
rounding, and the singular vectors are oriented by the same rule on both
sides):
* signs of the latent factors: equal everywhere except entries whose float64
  oracle value is below 1e-9 of the largest entry of its column (none in these
  cases);
* latent values (fp32 on the GPU): relative error <= 1e-4 of the column norm;
* fp16 scales h, l, g: within 1 unit in the last place;
* reconstruction error ||W - W_1 - W_2|| / ||W||: equal to the oracle's within
  1e-5 (absolute);
* the layer built from the GPU branches computes the oracle's forward of the
  same branches within the layer's own bar.
"""

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


def _ulp_close(a16, b16):
    a = a16.astype(np.float16).view(np.uint16).astype(np.int32)
    b = b16.astype(np.float16).view(np.uint16).astype(np.int32)
    return np.max(np.abs(a - b)) <= 1


@pytest.mark.parametrize("m,n,r,seed,itq", [(300, 200, 16, 0, 0), (150, 260, 24, 1, 0), (1024, 768, 96, 2, 0),
                                            (2048, 1536, 192, 3, 0), (300, 200, 16, 0, 10), (150, 260, 24, 1, 5),
                                            (1024, 768, 96, 2, 8)])
def test_dual_svid_matches_the_oracle(lb, m, n, r, seed, itq):
    print(f"[case] dual-svid m={m} n={n} r={r} itq={itq}", flush=True)
    W = synth.make_dense_weight(m, n, seed=seed)
    ref = oracle.dual_svid_init(W.astype(np.float64), r, nbranches=2, itq_iters=itq)
    got = lb.littlebit_dual_svid_init(torch.from_numpy(W).cuda(), r, nbranches=2, itq_iters=itq)
    torch.cuda.synchronize()
    gb = [{k: v.cpu().numpy() for k, v in b.items()} for b in got]
    for b, (g, o) in enumerate(zip(gb, ref)):
        for key in ("U", "V"):
            lat, want = g[key].astype(np.float64), o[key]
            colmax = np.max(np.abs(want), axis=0)
            decided = np.abs(want) > 1e-9 * colmax
            assert np.array_equal(lat[decided] < 0, want[decided] < 0), f"branch {b} {key} signs"
            err = np.linalg.norm(lat - want, axis=0) / np.linalg.norm(want, axis=0)
            assert err.max() <= 1e-4, f"branch {b} {key} latent rel err {err.max():.2e}"
        for key in ("h", "l", "g"):
            assert _ulp_close(g[key], o[key]), f"branch {b} {key}"
    e_ref = oracle.reconstruction_error(W, ref)
    got_np = [{"U": b["U"], "V": b["V"], "h": b["h"], "l": b["l"], "g": b["g"]} for b in gb]
    e_got = oracle.reconstruction_error(W, got_np)
    print(f"[parity] dual-svid {m}x{n} r={r} itq={itq}: error gpu {e_got:.6f} oracle {e_ref:.6f}", flush=True)
    assert abs(e_got - e_ref) <= 1e-5
    assert e_got < oracle.reconstruction_error(W, got_np[:1])


def test_dual_svid_branches_run_as_a_layer(lb):
    """End to end: W -> initialization on the GPU -> packed layer -> decode,
    against the oracle's forward of the same branches."""
    print("[case] dual-svid layer", flush=True)
    W = synth.make_dense_weight(512, 384, seed=4)
    got = lb.littlebit_dual_svid_init(torch.from_numpy(W).cuda(), 32)
    layer = lb.LittleBitLayer.from_latents(got)
    x = np.random.default_rng(5).standard_normal((3, 384)).astype(np.float16)
    y = lb.littlebit_linear_fwd(layer, torch.from_numpy(x).cuda()).float().cpu().numpy().astype(np.float64)
    brs = [{k: v.cpu().numpy() for k, v in b.items()} for b in got]
    want = oracle.linear_forward(x, brs)
    rel = np.linalg.norm(y - want) / np.linalg.norm(want)
    assert rel <= 2e-3, rel


def test_dual_svid_rank1_sign_magnitude_weight(lb):
    """The oracle's exact case on the GPU: W = (h * s)(g * t)^T, one branch
    of rank 1, reconstructs W within the fp16 rounding of the scales."""
    print("[case] dual-svid rank-1", flush=True)
    rng = np.random.default_rng(6)
    h, g = rng.uniform(0.5, 2.0, 64), rng.uniform(0.5, 2.0, 48)
    s_, t_ = np.where(rng.random(64) < 0.5, -1.0, 1.0), np.where(rng.random(48) < 0.5, -1.0, 1.0)
    W = np.outer(h * s_, g * t_).astype(np.float32)
    got = lb.littlebit_dual_svid_init(torch.from_numpy(W).cuda(), 1, nbranches=1)
    b = {k: v.cpu().numpy() for k, v in got[0].items()}
    assert oracle.reconstruction_error(W, [b]) < 2e-3
