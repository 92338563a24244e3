"""Seeded synthetic inputs for the LittleBit layer.

This module only draws random numbers and casts them; it contains none of the
layer's arithmetic, so both the HIP path's tests and the CPU oracle can take
their inputs from it.

Draw order (per layer, one ``numpy.random.default_rng(seed)`` stream): for
each branch in turn U (m x r, float32 N(0,1)), V (n x r, float32 N(0,1)),
h (m), l (r), g (n) (float64 U[0.5, 1.5] rounded to float16); then the token
batch x (batch x n, float32 N(0,1) rounded to float16).  Latents stay float32:
rounding them to float16 first would create +-0 ties that the sign rule then
has to break.

Workloads: the layer shapes of the pages' models (Llama2-7B up-projection,
Llama2-13B decoder block at 0.55 and 0.1 bits per weight, the Llama2-70B
8192 x 28672 MLP layer, a 2048-token prefill of the 7B up-projection) and a
tiny 512 x 512 layer.  No dataset or trained weight is involved.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np


@dataclass(frozen=True)
class LayerShape:
    name: str
    m: int            # outputs
    n: int            # inputs
    ranks: Tuple[int, ...]   # one rank per branch


# Shapes of the seven projections of a Llama2-13B decoder block, in the order
# q, k, v, o, gate, up, down, at the two rank settings used for 0.55 and 0.1
# bits per weight.
BLOCK13B_RANKS = {
    "0.55": {"attn": 688, "mlp": 1008},
    "0.1": {"attn": 112, "mlp": 168},
}
BLOCK13B_NAMES = ("q", "k", "v", "o", "gate", "up", "down")


def block13b_shapes(setting: str) -> List[LayerShape]:
    ra = BLOCK13B_RANKS[setting]["attn"]
    rm = BLOCK13B_RANKS[setting]["mlp"]
    d, f = 5120, 13824
    return [
        LayerShape("q", d, d, (ra, ra)),
        LayerShape("k", d, d, (ra, ra)),
        LayerShape("v", d, d, (ra, ra)),
        LayerShape("o", d, d, (ra, ra)),
        LayerShape("gate", f, d, (rm, rm)),
        LayerShape("up", f, d, (rm, rm)),
        LayerShape("down", d, f, (rm, rm)),
    ]


TINY = LayerShape("tiny_512x512_r32", 512, 512, (32, 32))
UP7B = LayerShape("llama2_7b_up_4096x11008_r1472", 11008, 4096, (1472, 1472))
UP70B = LayerShape("llama2_70b_up_8192x28672_r1728", 28672, 8192, (1728, 1728))
# The bits-per-weight sweep on the 70B-shaped up-projection: per target BPW,
# the rank (a multiple of 16) whose stored bits per weight come nearest to it
# with two branches (1.0 -> 0.9999, 0.8 -> 0.7989, 0.55 -> 0.5477, 0.3 ->
# 0.3015, 0.1 -> 0.1005; a CPU test recomputes these from the closed form).
UP70B_BPW_SWEEP = {1.0: 3168, 0.8: 2528, 0.55: 1728, 0.3: 944, 0.1: 304}


def up70b_at_bpw(bpw: float) -> LayerShape:
    r = UP70B_BPW_SWEEP[bpw]
    return LayerShape(f"llama2_70b_up_8192x28672_r{r}_{bpw}bpw", 28672, 8192, (r, r))
PREFILL_TOKENS = 2048


def make_branches(shape: LayerShape, rng: np.random.Generator) -> list:
    """Draw every branch of one layer from ``rng`` in the documented order."""
    out = []
    for r in shape.ranks:
        U = rng.standard_normal((shape.m, r), dtype=np.float32)
        V = rng.standard_normal((shape.n, r), dtype=np.float32)
        h = rng.uniform(0.5, 1.5, shape.m).astype(np.float16)
        l = rng.uniform(0.5, 1.5, r).astype(np.float16)
        g = rng.uniform(0.5, 1.5, shape.n).astype(np.float16)
        out.append({"U": U, "V": V, "h": h, "l": l, "g": g})
    return out


def make_tokens(batch: int, n: int, rng: np.random.Generator) -> np.ndarray:
    return rng.standard_normal((batch, n), dtype=np.float32).astype(np.float16)


def make_layer(shape: LayerShape, batch: int, seed: int = 0):
    """(branches, x) for one layer and one token batch."""
    rng = np.random.default_rng(seed)
    branches = make_branches(shape, rng)
    x = make_tokens(batch, shape.n, rng)
    return branches, x


def make_block13b(setting: str, batch: int, seed: int = 0):
    """Seven layers (q, k, v, o, gate, up, down) and the four input batches.

    Layers are drawn in order from one stream, then x_qkv (n=5120), x_o
    (5120), x_gu (5120) and x_down (13824).
    """
    rng = np.random.default_rng(seed)
    shapes = block13b_shapes(setting)
    layers = [make_branches(s, rng) for s in shapes]
    x_qkv = make_tokens(batch, 5120, rng)
    x_o = make_tokens(batch, 5120, rng)
    x_gu = make_tokens(batch, 5120, rng)
    x_down = make_tokens(batch, 13824, rng)
    return shapes, layers, (x_qkv, x_o, x_gu, x_down)


def make_dense_weight(m: int, n: int, seed: int = 0, decay: float = 0.75, noise: float = 0.05) -> np.ndarray:
    """A synthetic dense weight (m x n float32) with a decaying spectrum, the
    input of the initialization: Gaussian factors A (m x k) and B (n x k),
    k = min(m, n), with column i of A weighted by (i + 1)^-decay, times
    1/sqrt(k), plus independent Gaussian noise of standard deviation
    ``noise``.  Drawn from one ``default_rng(seed)`` stream: A, B, noise."""
    rng = np.random.default_rng(seed)
    k = min(m, n)
    A = rng.standard_normal((m, k), dtype=np.float32)
    B = rng.standard_normal((n, k), dtype=np.float32)
    w = (np.arange(1, k + 1, dtype=np.float32) ** np.float32(-decay)) / np.float32(np.sqrt(k))
    W = (A * w) @ B.T
    W += np.float32(noise) * rng.standard_normal((m, n), dtype=np.float32)
    return W


def block_inputs_for(index: int, xs: Sequence[np.ndarray]) -> np.ndarray:
    """Which of the four block inputs feeds projection ``index`` (0..6)."""
    x_qkv, x_o, x_gu, x_down = xs
    return (x_qkv, x_qkv, x_qkv, x_o, x_gu, x_gu, x_down)[index]
