"""Float64 oracle of the Dual-SVID initialization and residual fit.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

The explainx.ai explainer, "How it works" item 3, describes the initialization
in three steps, which this module takes in order:

1. a truncated SVD of the real weights W (m x n) to rank r;
2. the signs and magnitudes of the resulting latent factors are mapped into
   the learnable parameters (signs -> sign(U), sign(V); magnitudes -> the
   scales h, l, g);
3. a second branch is fitted to the residual, the part of W that the first
   branch does not capture.

The page names the decomposition "Sign-Value-Independent": a matrix is split
into its sign pattern and a magnitude part that does not depend on the signs.
Readings where the page is silent (each also listed in the design notes):

* Latent factors of the truncated SVD W ~ P S Q^T: U' = P S^(1/2),
  V' = Q S^(1/2) (the singular values split evenly, so U' V'^T is the best
  rank-r approximation).  Singular vectors are defined up to a joint sign
  per component: the column of V' is oriented so that its entry of largest
  magnitude (the first such index) is positive, and U' follows.
* Magnitudes to scales: |U'| (m x r) is approximated by the rank-1 outer
  product a b^T of its leading singular triplet (sigma, p, q), with
  a = sqrt(sigma) p and b = sqrt(sigma) q, both non-negative (the leading
  singular vectors of a non-negative matrix).  Then h = a_U, g = a_V and
  l = b_U * b_V elementwise, so that diag(h) sign(U') diag(l) sign(V')^T
  diag(g) has entries h_i g_k sum_j l_j s^U_ij s^V_kj: the rank-1 magnitude
  model of both factors applied to the sign pattern.
* Scales are stored as fp16 (round to nearest even), as the deployed layer
  uses them; the residual for branch 2 is W minus the deployed (fp16-scaled)
  branch 1: branch 2 is fitted to the error the deployed first branch leaves.
* Both branches use the same rank r.

Parity status (tests/test_oracle.py):

* ``truncated_svd_factors``: pinned by the Eckart-Young closed form
  ||W - U'V'^T||_F^2 = sum of the discarded squared singular values, and by
  the orientation rule.
* ``svid``: pinned by exact recovery of a matrix diag(p) S diag(q) with S a
  sign matrix and p, q > 0, and by the positivity of the magnitude vectors.
* ``itq_rotation``: pinned by orthogonality of R, invariance of the product
  U R (V R)^T = U V^T, the monotone objective (no iteration lowers
  sum |[U; V] R|), and exact recovery in one iteration when the stacked
  factors are a sign matrix H with orthogonal columns times a small rotation
  Q^T (sign(H Q^T) = H, so the Procrustes step returns R = Q and Z R = H).
* ``dual_svid_init``: pinned by exact reconstruction of a rank-1
  sign-magnitude weight (h * s)(g * t)^T with r = 1 (before fp16 rounding),
  by positive homogeneity (scaling W scales the unrounded reconstruction),
  by the residual branch lowering the error on synthetic weights with a
  decaying spectrum, and by a block-diagonal weight of two rank-1
  sign-magnitude blocks, which rank-1 branches split exactly (up to the fp16
  rounding of the scales): branch 1 reproduces the larger block and branch 2
  the smaller one, each zero outside its block.
"""

from __future__ import annotations

import numpy as np

from .littlebit_oracle import branch_weight


def truncated_svd_factors(W: np.ndarray, r: int):
    """Latent factors U' (m x r) and V' (n x r) of the rank-r truncated SVD,
    U' V'^T = P_r S_r Q_r^T, singular values split evenly; each column of V'
    oriented so its largest-magnitude entry (first index on ties) is positive.

    explainx.ai explainer, "How it works" item 3 (truncated SVD of the real
    weights).
    """
    W = np.asarray(W, dtype=np.float64)
    P, S, Qt = np.linalg.svd(W, full_matrices=False)
    r = min(r, S.size)
    root = np.sqrt(S[:r])
    U = P[:, :r] * root
    V = Qt[:r, :].T * root
    for j in range(r):
        k = int(np.argmax(np.abs(V[:, j])))
        if V[k, j] < 0:
            U[:, j] = -U[:, j]
            V[:, j] = -V[:, j]
    return U, V


def svid(M: np.ndarray):
    """Sign-value-independent split of M: (sign(M) as +-1, a, b) with a b^T
    the rank-1 approximation of |M| from its leading singular triplet,
    a = sqrt(sigma) p, b = sqrt(sigma) q, non-negative.

    explainx.ai explainer, "How it works" item 3 (signs and magnitudes mapped
    into the parameters).  Sign of 0 is +1, as for the layer itself.
    """
    M = np.asarray(M, dtype=np.float64)
    signs = np.where(M < 0, -1.0, 1.0)
    P, S, Qt = np.linalg.svd(np.abs(M), full_matrices=False)
    p, q = P[:, 0], Qt[0, :]
    if p.sum() < 0:  # leading vectors of a non-negative matrix: take the non-negative orientation
        p, q = -p, -q
    root = np.sqrt(S[0])
    return signs, np.abs(p) * root, np.abs(q) * root


def itq_rotation(U: np.ndarray, V: np.ndarray, iters: int) -> np.ndarray:
    """Orthogonal R (r x r) of Joint-ITQ for the latent factors U (m x r) and
    V (n x r): from R = I, each iteration takes B = sign([U; V] R) (-1 iff
    < 0) and then the R that best maps [U; V] onto B, R = P Q^T from the SVD
    P S Q^T of [U; V]^T B (orthogonal Procrustes).

    explainx.ai explainer, the LittleBit-2 paragraph: Internal Latent Rotation
    with Joint Iterative Quantization aligns the SVD-derived latent factors
    with the binary hypercube before training.  Reading: one rotation shared
    by both factors, so U R (V R)^T = U V^T and the product is unchanged;
    "joint" = both factors stacked in one objective; start R = I, a fixed
    iteration count.
    """
    Z = np.vstack([np.asarray(U, np.float64), np.asarray(V, np.float64)])
    R = np.eye(Z.shape[1])
    for _ in range(iters):
        B = np.where(Z @ R < 0, -1.0, 1.0)
        P, _, Qt = np.linalg.svd(Z.T @ B)
        R = P @ Qt
    return R


def itq_objective(U: np.ndarray, V: np.ndarray, R: np.ndarray) -> float:
    """sum |[U; V] R|, the alignment with the hypercube that each ITQ step
    cannot lower (it equals max over sign matrices B of tr(B^T [U; V] R))."""
    return float(np.abs(np.vstack([U, V]) @ R).sum())


def dual_svid_branch(R: np.ndarray, r: int, itq_iters: int = 0) -> dict:
    """One branch from the matrix it approximates: truncated SVD, an optional
    Joint-ITQ rotation of the latent factors, then the sign-value split of
    both latent factors; scales rounded to fp16.

    explainx.ai explainer, "How it works" items 2 and 3, and the LittleBit-2
    paragraph (the rotation).
    """
    U, V = truncated_svd_factors(R, r)
    if itq_iters > 0:
        Q = itq_rotation(U, V, itq_iters)
        U, V = U @ Q, V @ Q
    _, hU, lU = svid(U)
    _, gV, lV = svid(V)
    return {"U": U, "V": V, "h": hU.astype(np.float16), "l": (lU * lV).astype(np.float16),
            "g": gV.astype(np.float16), "h64": hU, "l64": lU * lV, "g64": gV}


def dual_svid_init(W: np.ndarray, r: int, nbranches: int = 2, itq_iters: int = 0) -> list:
    """Branches of the Dual-SVID initialization of W: branch 1 from W, each
    later branch from the residual W minus the deployed earlier branches.

    explainx.ai explainer, "How it works" item 3 (the second branch takes
    over the part of the weight that the first leaves).
    """
    W = np.asarray(W, dtype=np.float64)
    out = []
    R = W.copy()
    for _ in range(nbranches):
        br = dual_svid_branch(R, r, itq_iters)
        out.append(br)
        R = R - branch_weight(br)
    return out


def reconstruction_error(W: np.ndarray, branches) -> float:
    """Relative Frobenius error ||W - sum_b W_b|| / ||W|| of a set of branches
    (their deployed fp16 scales)."""
    W = np.asarray(W, dtype=np.float64)
    What = sum(branch_weight(b) for b in branches)
    return float(np.linalg.norm(W - What) / np.linalg.norm(W))
