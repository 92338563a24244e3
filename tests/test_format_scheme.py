"""The LB16 bit order supports an exact shift-and-mask sign unpack.

These CPU tests model, in plain Python, how a 64-lane matrix-core fragment is
formed from LB16 bytes (packed here by the oracle's packer): a lane loads one
aligned 32-bit word per pair of 16-bit units (an odd last unit comes with its
neighbour lane's unit) and rearranges its bytes with a byte permutation; then
operand dword q (q = 4*step + d, two fp16 values) is the word shifted left by
q, masked to bits 15 and 31, and OR-ed with the bits of 1.0 in both halves.
Every fragment entry must come out as exactly the sign, +1.0 or -1.0, at the
row and input index the fragment layout assigns to it.  Nothing here is the
GPU code; it checks that the format makes that scheme exact.
"""

import numpy as np
import pytest

import oracle


def _perm(mem, sel):
    """Byte permutation of one 32-bit word: selector byte 0..3 (or 4..7) picks
    that byte of the word, 0x0C gives 0x00."""
    out = 0
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        v = (mem >> (8 * (b & 3))) & 0xFF if b < 8 else 0
        assert b < 8 or b == 0x0C
        out |= v << (8 * i)
    return out


def _pair_reg(packed, T, L, p, R, K):
    """The register word a lane forms for pair p: one aligned 32-bit load
    (units 2p, 2p+1 at 256p + 4L; an odd last unit through the aligned word
    at 256p + 4*(L//2) that it shares with its neighbour) and a byte
    selection that puts the lane's units in place."""
    rp, kp = 16 * ((R + 15) // 16), 64 * ((K + 63) // 64)
    nu = kp // 64
    full = 2 * p + 1 < nu
    rel = 256 * p + (4 * L if full else 4 * (L // 2))
    off = T * 2 * kp + rel
    assert off + 4 <= len(packed) and rel + 4 <= 2 * kp   # stays inside the tile
    mem = int.from_bytes(bytes(packed[off:off + 4]), "little")
    sel = 0x01030002 if full else (0x030C020C if L & 1 else 0x010C000C)
    return _perm(mem, sel)


def _fp16_bits_to_float(bits16):
    return float(np.array([bits16], dtype=np.uint16).view(np.float16)[0])


def _fragment_values(packed, R, K):
    """A[a, k] as the lanes would build them (NaN where no lane writes)."""
    rp, kp = 16 * ((R + 15) // 16), 64 * ((K + 63) // 64)
    nt, nu = rp // 16, kp // 64
    A = np.full((nt * 16, kp), np.nan)
    for T in range(nt):
        for L in range(64):
            row, c = 16 * T + L % 16, L // 16
            for p in range((nu + 1) // 2):
                reg = _pair_reg(packed, T, L, p, R, K)
                for q in range(16):
                    step = 4 * p + q // 4
                    if 32 * step >= kp:
                        continue
                    dw = (((reg << q) & 0xFFFFFFFF) & 0x80008000) | 0x3C003C00
                    d = q % 4
                    for half, e in ((0, 2 * d), (1, 2 * d + 1)):
                        k = 32 * step + 8 * c + e
                        assert np.isnan(A[row, k]), "two lanes write one entry"
                        A[row, k] = _fp16_bits_to_float((dw >> (16 * half)) & 0xFFFF)
    return A


@pytest.mark.parametrize("R,K", [(16, 64), (16, 128), (16, 192), (20, 600), (40, 320), (32, 1472)])
def test_fragment_unpack_reproduces_signs(R, K):
    rng = np.random.default_rng(R + K)
    neg = rng.random((R, K)) < 0.5
    A = _fragment_values(oracle.pack_factor(neg), R, K)
    s = np.where(neg, -1.0, 1.0)
    np.testing.assert_array_equal(A[:R, :K], s)
    # padding (rows >= R, inputs >= K) unpacks to +1: the kernels pair it with
    # zero activations and never store padded rows
    assert not np.isnan(A).any()
    assert (A[R:, :] == 1.0).all() and (A[:, K:] == 1.0).all()
    # exact signed contraction
    u = rng.standard_normal(K)
    np.testing.assert_allclose(A[:R, :K] @ u, s @ u, rtol=1e-12, atol=1e-12)
