"""Float64 / exact-rational oracle of the LittleBit factored binary linear layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What the layer computes
-----------------------
The explainx.ai explainer, "How it works" item 1, approximates a weight matrix
W by the product of two thin matrices U and V and keeps, for inference, only
the signs (+1 or -1) of their entries.  Item 2 ("Multi-scale compensation")
adds learned FP16 scale vectors on three axes: rows, columns and the latent
dimension.  Item 3 adds a second, residual branch for the part of the weight
the first one leaves.  With W of shape out x in = m x n, U of shape m x r and V of shape
n x r, the only placement of one scale per named axis is

    W_b = diag(h_b) . sign(U_b) . diag(l_b) . sign(V_b)^T . diag(g_b)

with h_b on the m output rows, g_b on the n input columns and l_b on the r
latent indices, and the branches add: W = W_1 + W_2.  A token x (length n) maps
to y = W x.  This is the plain definition the oracle evaluates.

Readings where the pages are silent (each also listed in the design notes):

* sign(0): the pages only say "+1 or -1".  The oracle maps a latent value v to
  -1 exactly when ``v < 0``; +0.0, -0.0 and NaN all give +1.
* Activations are not quantised: the pages count bits per *weight* only
  (explainx.ai explainer, "What LittleBit is").  x, h, l, g are the exact
  fp16 values, upcast to float64 without rounding.
* The oracle itself never rounds to fp16: it defines the exact result, and a
  GPU path that stores intermediates in fp16 is compared within a tolerance.

Parity status (what pins each function; tests/test_oracle.py):

* ``linear_forward`` / ``dense_weight`` / ``branch_weight``: pinned by the
  exact-rational evaluator on tiny inputs, the hand-derived 2x2 example in
  tests/golden, the Sylvester-Hadamard special case (reduces to an
  elementwise product), the all-positive closed form, and the gauge,
  permutation, additivity and linearity invariants.
* ``factored_forward`` and ``rows_forward``: pinned by agreement with the
  dense definition (and therefore with the pins above).
* ``exact_forward``: pinned by the hand example and the Hadamard case.
* ``transposed_forward``: pinned by the adjoint identity <W x, d> = <x, W^T d>
  against ``linear_forward`` and by an explicit transpose of ``dense_weight``.
* ``bits_per_weight`` / ``model_footprint_bytes``: pinned by counting the
  entries of a concrete layer's arrays, and by the model sizes the trueseeker
  fact-check prints (Llama2-7B 13.49 GB fp16, 0.79 GB at 0.3 BPW, 0.63 GB at
  0.1 BPW; Llama2-13B 26.06 GB fp16, 0.84 GB at 0.1 BPW) to within 5 %.
* ``rank_for_bpw``: pinned by inversion of ``bits_per_weight``.
"""

from __future__ import annotations

from fractions import Fraction
from typing import Iterable, Sequence

import numpy as np

# A branch is a mapping with keys "U" (m x r latent), "V" (n x r latent),
# "h" (m,), "l" (r,), "g" (n,).  Latents may be any float dtype; scales are
# normally float16 and are upcast exactly.


def sign_matrix(latent: np.ndarray) -> np.ndarray:
    """Signs of a latent factor as float64 +-1.

    explainx.ai explainer, "How it works" item 1: only the signs of U and V
    are used at inference time.  Reading for the silent case: -1 iff v < 0.
    """
    a = np.asarray(latent)
    return np.where(a < 0, -1.0, 1.0).astype(np.float64)


def _f64(v) -> np.ndarray:
    return np.asarray(v).astype(np.float64)


def branch_weight(br) -> np.ndarray:
    """Dense m x n weight of one branch: diag(h) sign(U) diag(l) sign(V)^T diag(g).

    explainx.ai explainer, "How it works" items 1 (thin binary factors) and 2
    (scales on rows, latent dimension and columns).
    """
    su = sign_matrix(br["U"])          # m x r
    sv = sign_matrix(br["V"])          # n x r
    h, l, g = _f64(br["h"]), _f64(br["l"]), _f64(br["g"])
    inner = (su * l[None, :]) @ sv.T   # m x n : sign(U) diag(l) sign(V)^T
    return h[:, None] * inner * g[None, :]


def dense_weight(branches: Sequence) -> np.ndarray:
    """Sum of the branch weights (explainx.ai explainer, "How it works" item 3:
    the residual branch covers what the primary branch leaves over, so the
    two approximations add)."""
    w = None
    for br in branches:
        wb = branch_weight(br)
        w = wb if w is None else w + wb
    return w


def linear_forward(x: np.ndarray, branches: Sequence) -> np.ndarray:
    """The layer's output y = W x for each token row of x (batch x n -> batch x m).

    This is the definition: build the dense W and multiply, in float64.
    """
    x64 = np.atleast_2d(_f64(x))
    return x64 @ dense_weight(branches).T


def factored_forward(x: np.ndarray, branches: Sequence) -> np.ndarray:
    """Same result as ``linear_forward`` evaluated without forming W.

    Per branch: scale the input by g, contract with sign(V) over the n inputs,
    scale by l, contract with sign(U) over the r latent indices, scale by h;
    then sum the branches.  Float64 throughout.
    """
    x64 = np.atleast_2d(_f64(x))
    y = np.zeros((x64.shape[0], np.asarray(branches[0]["U"]).shape[0]))
    for br in branches:
        u = x64 * _f64(br["g"])[None, :]                 # batch x n
        t = u @ sign_matrix(br["V"])                     # batch x r
        z = t * _f64(br["l"])[None, :]                   # batch x r
        s = z @ sign_matrix(br["U"]).T                   # batch x m
        y += s * _f64(br["h"])[None, :]
    return y


def rows_forward(x: np.ndarray, branches: Sequence, rows: Iterable[int]) -> np.ndarray:
    """Outputs y[:, i] for the listed rows i only, each from its own row of W.

    Row i of W_b is h_i * sign(U)[i, :] diag(l) sign(V)^T diag(g); the cost is
    O(r n) per row, so full-size layers can be sampled one output at a time.
    """
    rows = np.asarray(list(rows), dtype=np.int64)
    x64 = np.atleast_2d(_f64(x))
    out = np.zeros((x64.shape[0], rows.size))
    for br in branches:
        su = sign_matrix(np.asarray(br["U"])[rows, :])   # k x r
        sv = sign_matrix(br["V"])                        # n x r
        h, l, g = _f64(br["h"])[rows], _f64(br["l"]), _f64(br["g"])
        wrows = h[:, None] * ((su * l[None, :]) @ sv.T) * g[None, :]  # k x n
        out += x64 @ wrows.T
    return out


def transposed_forward(dy: np.ndarray, branches: Sequence) -> np.ndarray:
    """The adjoint product dx = W^T dy (batch x m -> batch x n).

    This is the input-gradient of the layer used by quantisation-aware
    training (explainx.ai explainer, "How it works", the paragraph after the
    figure: training sees the binarised forward pass).  Definition: dense W,
    transposed, multiplied in float64.
    """
    dy64 = np.atleast_2d(_f64(dy))
    return dy64 @ dense_weight(branches)


def exact_forward(x: Sequence[Sequence[float]], branches: Sequence) -> list:
    """Exact rational y for tiny layers (pure-Python loops over Fractions).

    Every fp16 value is a dyadic rational, so Fraction(float(v)) is exact and
    the sums below carry no rounding at all.  Same definition as
    ``linear_forward``: W_b[i][k] = h_i * sum_j sU[i][j] l_j sV[k][j] * g_k.
    """
    xs = [[Fraction(float(v)) for v in row] for row in np.atleast_2d(np.asarray(x))]
    m = np.asarray(branches[0]["U"]).shape[0]
    n = np.asarray(branches[0]["V"]).shape[0]
    w = [[Fraction(0)] * n for _ in range(m)]
    for br in branches:
        U, V = np.asarray(br["U"]), np.asarray(br["V"])
        r = U.shape[1]
        h = [Fraction(float(v)) for v in np.asarray(br["h"])]
        l = [Fraction(float(v)) for v in np.asarray(br["l"])]
        g = [Fraction(float(v)) for v in np.asarray(br["g"])]
        for i in range(m):
            for k in range(n):
                acc = Fraction(0)
                for j in range(r):
                    su = -1 if U[i, j] < 0 else 1
                    sv = -1 if V[k, j] < 0 else 1
                    acc += su * l[j] * sv
                w[i][k] += h[i] * acc * g[k]
    return [[sum((w[i][k] * xr[k] for k in range(n)), Fraction(0)) for i in range(m)]
            for xr in xs]


def bits_per_weight(m: int, n: int, r: int, nbranches: int = 2) -> float:
    """Stored bits per original weight of an m x n layer.

    Per branch the layer stores r(m + n) sign bits (explainx.ai explainer,
    "How it works" item 1: one bit per entry of the thin factors) and
    m + n + r FP16 scales (item 2), i.e. 16 bits each.  Divided by the m n
    weights it replaces.
    """
    return nbranches * (r * (m + n) + 16 * (m + n + r)) / (m * n)


def rank_for_bpw(m: int, n: int, bpw: float, nbranches: int = 2) -> float:
    """Real-valued rank r at which ``bits_per_weight`` equals ``bpw``.

    The explainx.ai explainer ("What the repository lets you do today") says
    the effective-bit flag sets the bits per weight; the pages give no rounding
    rule, so this returns the unrounded solution of the linear equation.
    """
    return (bpw * m * n / nbranches - 16 * (m + n)) / (m + n + 16)


def model_footprint_bytes(hidden: int, intermediate: int, layers: int, vocab: int,
                          bpw: float | None) -> float:
    """Stored bytes of a Llama-style model under the pages' accounting.

    trueseeker fact-check: quantisation applies to the Transformer blocks only;
    the embedding and the output head stay FP16, and BPW is counted over the
    block linears.  A block has q, k, v, o (hidden x hidden) and gate, up, down
    (hidden x intermediate).  ``bpw=None`` gives the all-FP16 size.  Norm
    vectors (2 per block + 1 final, hidden each) are counted in FP16.
    """
    block_linear = layers * (4 * hidden * hidden + 3 * hidden * intermediate)
    fp16_params = 2 * vocab * hidden + (2 * layers + 1) * hidden
    if bpw is None:
        return 2.0 * (block_linear + fp16_params)
    return block_linear * bpw / 8.0 + 2.0 * fp16_params
