"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand derivation stored in
tests/golden, exact rational arithmetic, a textbook special case (Sylvester
Hadamard matrices, via scipy), a closed form, an invariant of the definition,
or numbers printed on the pages.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
from binary_rank_gemv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _branches_from_json(d):
    out = []
    for b in d["branches"]:
        out.append({k: np.asarray(b[k], dtype=np.float64) if k in ("U", "V")
                    else np.asarray(b[k], dtype=np.float16) for k in b})
    return out


def _random_layer(rng, m, n, ranks):
    out = []
    for r in ranks:
        out.append({
            "U": rng.standard_normal((m, r)).astype(np.float32),
            "V": rng.standard_normal((n, r)).astype(np.float32),
            "h": rng.uniform(0.5, 1.5, m).astype(np.float16),
            "l": rng.uniform(0.5, 1.5, r).astype(np.float16),
            "g": rng.uniform(0.5, 1.5, n).astype(np.float16),
        })
    return out


# ---------------------------------------------------------------- hand example

def test_hand_example_all_evaluators():
    d = _load("hand_example_two_branch.json")
    br = _branches_from_json(d)
    x = np.asarray(d["x"], dtype=np.float16)
    want = np.asarray(d["y"])
    np.testing.assert_array_equal(oracle.linear_forward(x, br), want)
    np.testing.assert_array_equal(oracle.factored_forward(x, br), want)
    exact = oracle.exact_forward(x, br)
    assert exact == [[Fraction(10), Fraction(-19)]]
    np.testing.assert_array_equal(oracle.rows_forward(x, br, [1, 0]), want[:, ::-1])


def test_sign_reading_zero_and_negative_zero():
    v = np.array([-1.0, -0.0, 0.0, 1e-30, -1e-30, np.nan], dtype=np.float64)
    np.testing.assert_array_equal(oracle.sign_matrix(v), [-1, 1, 1, 1, -1, 1])
    v16 = np.array([-0.0, 0.0, -6e-8, 6e-8], dtype=np.float16)   # fp16 subnormals
    np.testing.assert_array_equal(oracle.sign_matrix(v16), [1, 1, -1, 1])


# ------------------------------------------------------------ exact arithmetic

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_float64_matches_exact_rational(seed):
    rng = np.random.default_rng(100 + seed)
    m, n = 11, 13
    br = _random_layer(rng, m, n, (5, 3))
    x = rng.standard_normal((2, n)).astype(np.float16)
    exact = oracle.exact_forward(x, br)
    ex = np.array([[float(v) for v in row] for row in exact])
    scale = np.max(np.abs(ex))
    for y in (oracle.linear_forward(x, br), oracle.factored_forward(x, br)):
        assert np.max(np.abs(y - ex)) <= 1e-13 * scale


# -------------------------------------------------------------- special cases

@pytest.mark.parametrize("k", [1, 3, 5])
def test_hadamard_factors_reduce_to_elementwise_scaling(k):
    """sign(U) = sign(V) = H (Sylvester), l = 2^-k  =>  H diag(l) H^T = I,
    so each branch is diag(h*g) and y = sum_b h_b*g_b*x."""
    n = 2 ** k
    H = scipy.linalg.hadamard(n).astype(np.float64)
    rng = np.random.default_rng(k)
    br = []
    for _ in range(2):
        br.append({"U": H * rng.uniform(0.1, 2.0, (n, n)),
                   "V": H * rng.uniform(0.1, 2.0, (n, n)),
                   "h": rng.uniform(0.5, 1.5, n).astype(np.float16),
                   "l": np.full(n, 2.0 ** -k, dtype=np.float16),
                   "g": rng.uniform(0.5, 1.5, n).astype(np.float16)})
    x = rng.standard_normal((3, n)).astype(np.float16)
    want = sum(b["h"].astype(np.float64) * b["g"].astype(np.float64) for b in br) * x.astype(np.float64)
    np.testing.assert_allclose(oracle.linear_forward(x, br), want, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(oracle.factored_forward(x, br), want, rtol=1e-14, atol=1e-12)


def test_all_positive_signs_closed_form():
    """All signs +1: W_b = h_b (sum_j l_bj) g_b^T, so
    y_i = sum_b h_bi (sum_j l_bj) (sum_k g_bk x_k)."""
    rng = np.random.default_rng(7)
    m, n = 9, 6
    br = _random_layer(rng, m, n, (4, 2))
    for b in br:
        b["U"] = np.abs(b["U"])
        b["V"] = np.abs(b["V"])
    x = rng.standard_normal((2, n)).astype(np.float16)
    x64 = x.astype(np.float64)
    want = np.zeros((2, m))
    for b in br:
        h, l, g = (b[k].astype(np.float64) for k in ("h", "l", "g"))
        want += np.outer(x64 @ g, h) * l.sum()
    np.testing.assert_allclose(oracle.linear_forward(x, br), want, rtol=1e-13)


# ----------------------------------------------------------------- invariants

def test_dense_and_factored_agree_tiny_config():
    br, x = synth.make_layer(synth.TINY, batch=3, seed=0)
    yd = oracle.linear_forward(x, br)
    yf = oracle.factored_forward(x, br)
    assert np.max(np.abs(yd - yf)) <= 1e-12 * np.max(np.abs(yd))


def test_gauge_flip_of_latent_column_leaves_output_unchanged():
    rng = np.random.default_rng(3)
    br = _random_layer(rng, 20, 24, (6, 6))
    x = rng.standard_normal((2, 24)).astype(np.float16)
    y0 = oracle.linear_forward(x, br)
    flipped = [dict(b) for b in br]
    for j in (0, 4):
        flipped[0]["U"] = flipped[0]["U"].copy(); flipped[0]["U"][:, j] *= -1
        flipped[0]["V"] = flipped[0]["V"].copy(); flipped[0]["V"][:, j] *= -1
    assert not np.array_equal(oracle.sign_matrix(br[0]["U"]), oracle.sign_matrix(flipped[0]["U"]))
    np.testing.assert_allclose(oracle.linear_forward(x, flipped), y0, rtol=1e-13, atol=1e-12)


def test_latent_permutation_leaves_output_unchanged():
    rng = np.random.default_rng(4)
    br = _random_layer(rng, 17, 15, (7,))
    x = rng.standard_normal((2, 15)).astype(np.float16)
    perm = rng.permutation(7)
    pb = [{"U": br[0]["U"][:, perm], "V": br[0]["V"][:, perm], "l": br[0]["l"][perm],
           "h": br[0]["h"], "g": br[0]["g"]}]
    np.testing.assert_allclose(oracle.linear_forward(x, pb), oracle.linear_forward(x, br),
                               rtol=1e-13, atol=1e-12)


def test_branch_additivity_and_linearity():
    rng = np.random.default_rng(5)
    br = _random_layer(rng, 14, 10, (3, 5))
    x1 = rng.standard_normal((2, 10)).astype(np.float16)
    x2 = rng.standard_normal((2, 10)).astype(np.float16)
    y = oracle.linear_forward(x1, br)
    np.testing.assert_allclose(y, oracle.linear_forward(x1, br[:1]) + oracle.linear_forward(x1, br[1:]),
                               rtol=1e-13, atol=1e-12)
    xs = (x1.astype(np.float64) + x2.astype(np.float64))
    np.testing.assert_allclose(oracle.linear_forward(xs, br),
                               y + oracle.linear_forward(x2, br), rtol=1e-12, atol=1e-11)


def test_rows_forward_matches_full():
    br, x = synth.make_layer(synth.TINY, batch=2, seed=1)
    rows = [0, 5, 511, 100]
    np.testing.assert_allclose(oracle.rows_forward(x, br, rows),
                               oracle.linear_forward(x, br)[:, rows], rtol=1e-12, atol=1e-9)


def test_transposed_is_adjoint_of_forward():
    rng = np.random.default_rng(6)
    br = _random_layer(rng, 12, 9, (4, 3))
    x = rng.standard_normal((1, 9))
    d = rng.standard_normal((1, 12))
    lhs = (oracle.linear_forward(x, br) @ d.T).item()
    rhs = (x @ oracle.transposed_forward(d, br).T).item()
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    np.testing.assert_allclose(oracle.transposed_forward(d, br), d @ oracle.dense_weight(br),
                               rtol=1e-14)


# --------------------------------------------------------- bits per weight

def test_bits_per_weight_counts_the_arrays_of_a_layer():
    for shape in (synth.TINY, synth.LayerShape("odd", 40, 72, (9, 9))):
        br, _ = synth.make_layer(shape, batch=1, seed=0)
        bits = sum(b["U"].size + b["V"].size + 16 * (b["h"].size + b["l"].size + b["g"].size)
                   for b in br)
        assert bits / (shape.m * shape.n) == pytest.approx(
            oracle.bits_per_weight(shape.m, shape.n, shape.ranks[0], len(shape.ranks)), rel=1e-15)


@pytest.mark.parametrize("m,n,r,stated", [
    (512, 512, 32, 0.38), (11008, 4096, 1472, 1.0), (5120, 5120, 688, 0.55),
    (5120, 5120, 112, 0.1), (13824, 5120, 1008, 0.55), (5120, 13824, 168, 0.1),
    (28672, 8192, 1728, 0.55)])
def test_config_ranks_give_the_stated_bits_per_weight(m, n, r, stated):
    assert oracle.bits_per_weight(m, n, r) == pytest.approx(stated, rel=0.02)
    assert abs(oracle.rank_for_bpw(m, n, oracle.bits_per_weight(m, n, r)) - r) < 1e-9


@pytest.mark.parametrize("bpw", sorted(synth.UP70B_BPW_SWEEP))
def test_bpw_sweep_ranks_are_the_nearest_multiples_of_16(bpw):
    """Each sweep rank is the multiple of 16 nearest the closed-form rank, and
    its stored bits per weight are within 1.2% of the target."""
    r = synth.UP70B_BPW_SWEEP[bpw]
    assert r % 16 == 0
    exact = oracle.rank_for_bpw(28672, 8192, bpw)
    assert abs(r - exact) <= 8
    assert oracle.bits_per_weight(28672, 8192, r) == pytest.approx(bpw, rel=0.012)


def test_model_footprints_match_the_pages():
    d = _load("model_sizes.json")
    tol = d["tolerance"]
    for mdl in d["models"]:
        dims = (mdl["hidden"], mdl["intermediate"], mdl["layers"], mdl["vocab"])
        for key, gb in mdl["sizes_gb"].items():
            got = oracle.model_footprint_bytes(*dims, bpw=None if key == "fp16" else float(key)) / 1e9
            rel = tol["fp16"] if key == "fp16" else tol["quantised"]
            assert got == pytest.approx(gb, rel=rel), (mdl["name"], key, got, gb)


# -------------------------------------------------------------------- packing

def test_pack_worked_examples():
    d = _load("pack_worked_examples.json")
    for case in d["cases"]:
        neg = np.zeros((case["R"], case["K"]), dtype=bool)
        for a, k in case["negative"]:
            neg[a, k] = True
        p = oracle.pack_factor(neg)
        assert p.size == case["total_bytes"] == oracle.packed_factor_bytes(case["R"], case["K"])
        want = np.zeros(p.size, dtype=np.uint8)
        for off, val in case["nonzero_bytes"].items():
            want[int(off)] = val
        np.testing.assert_array_equal(p, want)


@pytest.mark.parametrize("R,K", [(16, 64), (20, 600), (33, 1472), (7, 40), (48, 4096)])
def test_pack_roundtrip_and_popcount(R, K):
    rng = np.random.default_rng(R * 1000 + K)
    neg = rng.random((R, K)) < 0.5
    p = oracle.pack_factor(neg)
    np.testing.assert_array_equal(oracle.unpack_factor(p, R, K), neg)
    assert int(np.unpackbits(p).sum()) == int(neg.sum())


def test_pack_all_negative_and_all_positive():
    for R, K in ((16, 64), (20, 600)):
        p1 = oracle.pack_factor(np.ones((R, K), dtype=bool))
        assert int(np.unpackbits(p1).sum()) == R * K        # pad bits stay 0
        p0 = oracle.pack_factor(np.zeros((R, K), dtype=bool))
        assert not p0.any()
    # a full 16 x 64 tile of -1 is all ones
    assert (oracle.pack_factor(np.ones((16, 64), dtype=bool)) == 0xFF).all()


def test_sign_bits_transpose():
    v = np.array([[1.0, -2.0, 0.0], [-0.0, -1.0, 3.0]], dtype=np.float32)
    np.testing.assert_array_equal(oracle.sign_bits(v), [[False, True, False], [False, True, False]])
    np.testing.assert_array_equal(oracle.sign_bits(v, transpose=True),
                                  [[False, False], [True, True], [False, False]])


# ------------------------------------------------ planted mistakes are caught

def _hand_case():
    d = _load("hand_example_two_branch.json")
    return _branches_from_json(d), np.asarray(d["x"], dtype=np.float16), np.asarray(d["y"])


@pytest.mark.parametrize("mistake", ["drop_g", "drop_l", "l_index_reversed", "negated_u",
                                     "sign_zero_negative", "drop_residual"])
def test_pins_catch_planted_oracle_mistakes(mistake, monkeypatch):
    """Each plausible slip in the definition changes the hand example's y."""
    import oracle.littlebit_oracle as lo

    def bad_bw(br):
        su, sv = lo.sign_matrix(br["U"]), lo.sign_matrix(br["V"])
        h, l, g = (np.asarray(br[k], dtype=np.float64) for k in ("h", "l", "g"))
        if mistake == "drop_g":
            return h[:, None] * ((su * l) @ sv.T)
        if mistake == "drop_l":
            return h[:, None] * (su @ sv.T) * g[None, :]
        if mistake == "l_index_reversed":
            return h[:, None] * ((su * l[::-1]) @ sv.T) * g[None, :]
        assert mistake == "negated_u"
        return h[:, None] * ((-su * l) @ sv.T) * g[None, :]

    br, x, want = _hand_case()
    if mistake == "sign_zero_negative":
        monkeypatch.setattr(lo, "sign_matrix",
                            lambda a: np.where(np.signbit(np.asarray(a, dtype=np.float64)), -1.0, 1.0))
    elif mistake == "drop_residual":
        br = br[:1]
    else:
        monkeypatch.setattr(lo, "branch_weight", bad_bw)
    y = lo.linear_forward(x, br)
    assert not np.array_equal(y, want), mistake


# ------------------------------------------------------ Dual-SVID initialization

def _orthonormal(rng, rows, cols):
    q, _ = np.linalg.qr(rng.standard_normal((rows, cols)))
    return q


def test_truncated_svd_factors_meet_the_eckart_young_closed_form():
    """A weight built as P diag(s) Q^T with known orthonormal P, Q and
    decreasing s: U'V'^T equals P_r diag(s_r) Q_r^T and the squared error
    is the sum of the discarded s_i^2."""
    rng = np.random.default_rng(11)
    m, n, k, r = 40, 30, 30, 7
    P, Q = _orthonormal(rng, m, k), _orthonormal(rng, n, k)
    s = np.sort(rng.uniform(0.5, 4.0, k))[::-1] + np.arange(k)[::-1] * 0.1
    W = (P * s) @ Q.T
    U, V = oracle.truncated_svd_factors(W, r)
    np.testing.assert_allclose(U @ V.T, (P[:, :r] * s[:r]) @ Q[:, :r].T, atol=1e-10)
    assert abs(np.linalg.norm(W - U @ V.T) ** 2 - np.sum(s[r:] ** 2)) < 1e-9
    # singular values split evenly: column norms of U' and V' are both sqrt(s)
    np.testing.assert_allclose(np.linalg.norm(U, axis=0), np.sqrt(s[:r]), rtol=1e-10)
    np.testing.assert_allclose(np.linalg.norm(V, axis=0), np.sqrt(s[:r]), rtol=1e-10)
    for j in range(r):  # orientation rule
        assert V[np.argmax(np.abs(V[:, j])), j] > 0


def test_svid_recovers_a_sign_times_rank1_magnitude_matrix():
    rng = np.random.default_rng(12)
    p, q = rng.uniform(0.2, 3.0, 25), rng.uniform(0.2, 3.0, 9)
    S = np.where(rng.random((25, 9)) < 0.5, -1.0, 1.0)
    signs, a, b = oracle.svid(S * np.outer(p, q))
    np.testing.assert_array_equal(signs, S)
    assert (a > 0).all() and (b > 0).all()
    np.testing.assert_allclose(np.outer(a, b), np.outer(p, q), rtol=1e-12)


def test_dual_svid_rank1_sign_magnitude_weight_is_exact():
    """W = (h * s)(g * t)^T with sign vectors s, t: one branch of rank 1
    reproduces W exactly before the fp16 rounding of its scales."""
    rng = np.random.default_rng(13)
    h, g = rng.uniform(0.5, 2.0, 12), rng.uniform(0.5, 2.0, 8)
    s_, t_ = np.where(rng.random(12) < 0.5, -1.0, 1.0), np.where(rng.random(8) < 0.5, -1.0, 1.0)
    W = np.outer(h * s_, g * t_)
    br = oracle.dual_svid_branch(W, 1)
    what = (br["h64"][:, None] * oracle.sign_matrix(br["U"]) * br["l64"]) @ (oracle.sign_matrix(br["V"]) * br["g64"][:, None]).T
    np.testing.assert_allclose(what, W, rtol=1e-10, atol=1e-12)
    # the deployed (fp16-scaled) branch is within fp16 rounding of W
    assert oracle.reconstruction_error(W, [br]) < 2e-3


def test_dual_svid_is_positively_homogeneous():
    rng = np.random.default_rng(14)
    W = rng.standard_normal((20, 16))
    b1, b2 = oracle.dual_svid_branch(W, 4), oracle.dual_svid_branch(3.0 * W, 4)
    rec = lambda b: (b["h64"][:, None] * oracle.sign_matrix(b["U"]) * b["l64"]) @ (oracle.sign_matrix(b["V"]) * b["g64"][:, None]).T
    np.testing.assert_allclose(rec(b2), 3.0 * rec(b1), rtol=1e-9, atol=1e-12)
    np.testing.assert_array_equal(oracle.sign_matrix(b1["U"]), oracle.sign_matrix(b2["U"]))


def test_dual_svid_residual_branch_lowers_the_error():
    from binary_rank_gemv_amd import synth
    W = synth.make_dense_weight(96, 64, seed=3).astype(np.float64)
    brs = oracle.dual_svid_init(W, 16, nbranches=2)
    e1, e2 = oracle.reconstruction_error(W, brs[:1]), oracle.reconstruction_error(W, brs)
    assert e2 < e1 < 1.0
    # branch 2 was fitted to W minus the deployed branch 1
    R = W - oracle.branch_weight(brs[0])
    ref = oracle.dual_svid_branch(R, 16)
    np.testing.assert_array_equal(ref["h"], brs[1]["h"])


def test_dual_svid_block_diagonal_weight_splits_into_the_two_branches():
    """W = blockdiag(B1, B2), each block a rank-1 sign-magnitude matrix, with
    ||B1|| > ||B2||, rank 1 per branch: the first branch is the best rank-1
    approximation of W, i.e. B1 (zero outside its block), and the second is
    fitted to what is left, i.e. B2.  Each is exact up to the fp16 rounding of
    its scales.  A second branch fitted to W rather than to the residual
    would reproduce B1 again; one fitted with the wrong sign, -B2."""
    rng = np.random.default_rng(3)
    m1, n1, m2, n2 = 24, 20, 16, 12

    def block(m, n, scale):
        s, t = rng.choice([-1.0, 1.0], m), rng.choice([-1.0, 1.0], n)
        return scale * np.outer(rng.uniform(0.5, 1.5, m) * s, rng.uniform(0.5, 1.5, n) * t)

    B1, B2 = block(m1, n1, 3.0), block(m2, n2, 1.0)
    W = np.zeros((m1 + m2, n1 + n2))
    W[:m1, :n1], W[m1:, n1:] = B1, B2
    brs = oracle.dual_svid_init(W, 1, nbranches=2)
    W1, W2 = oracle.branch_weight(brs[0]), oracle.branch_weight(brs[1])
    E1, E2 = np.zeros_like(W), np.zeros_like(W)
    E1[:m1, :n1], E2[m1:, n1:] = B1, B2
    assert np.linalg.norm(W1 - E1) / np.linalg.norm(B1) < 2e-3
    assert np.linalg.norm(W2 - E2) / np.linalg.norm(B2) < 2e-3
    assert np.abs(W1[m1:, :]).max() == 0 and np.abs(W1[:, n1:]).max() == 0
    assert np.abs(W2[:m1, :]).max() == 0 and np.abs(W2[:, :n1]).max() == 0


# ---------------------------------------------------- Joint-ITQ latent rotation

def test_itq_rotation_is_orthogonal_keeps_the_product_and_never_lowers_the_objective():
    rng = np.random.default_rng(21)
    U, V = rng.standard_normal((40, 8)) * np.linspace(2, 0.5, 8), rng.standard_normal((30, 8))
    prev = oracle.itq_objective(U, V, np.eye(8))
    for it in (1, 2, 3, 5, 8, 13):
        R = oracle.itq_rotation(U, V, it)
        np.testing.assert_allclose(R.T @ R, np.eye(8), atol=1e-12)
        np.testing.assert_allclose((U @ R) @ (V @ R).T, U @ V.T, atol=1e-10)
        obj = oracle.itq_objective(U, V, R)
        assert obj >= prev - 1e-9
        prev = obj


def test_itq_recovers_a_rotated_sign_matrix_in_one_iteration():
    """Z = H Q^T, H a 32 x 8 sign matrix with orthogonal columns (columns
    1..8 of a Sylvester-Hadamard matrix, rows split over U and V) and Q a
    small rotation: sign(Z) = H, the Procrustes step gives R = Q and Z R = H."""
    from scipy.linalg import expm, hadamard
    rng = np.random.default_rng(22)
    H = hadamard(32).astype(np.float64)[:, 1:9]
    A = rng.standard_normal((8, 8)) * 0.02
    Q = expm(A - A.T)
    Z = H @ Q.T
    assert np.array_equal(np.where(Z < 0, -1.0, 1.0), H)
    R = oracle.itq_rotation(Z[:20], Z[20:], 1)
    np.testing.assert_allclose(R, Q, atol=1e-12)
    np.testing.assert_allclose(Z @ R, H, atol=1e-12)
    assert abs(oracle.itq_objective(Z[:20], Z[20:], R) - np.abs(H).sum()) < 1e-9


def test_dual_svid_with_itq_keeps_the_latent_product():
    from binary_rank_gemv_amd import synth
    W = synth.make_dense_weight(80, 60, seed=5).astype(np.float64)
    plain, rot = oracle.dual_svid_branch(W, 12), oracle.dual_svid_branch(W, 12, itq_iters=10)
    np.testing.assert_allclose(rot["U"] @ rot["V"].T, plain["U"] @ plain["V"].T, atol=1e-10)
