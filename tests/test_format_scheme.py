"""The LB16 bit order supports an exact shift-and-mask sign unpack.

These CPU tests model, in plain Python, how a 64-lane matrix-core fragment is
formed from LB16 bytes (packed here by the oracle's packer): a lane joins two
16-bit units into a 32-bit word with a byte permutation, then for q = 0..15
shifts the word left by 2*floor(q/2) and masks either bits 15/31 (q even,
giving fp16 +-1 after OR-ing in 1.0) or bits 14/30 (q odd, giving fp16 0 or
2).  Element k lands in the q-odd class exactly when (k & 2) != 0, so a
contraction with the q-odd operand entries negated, plus the sum of those
operand entries, equals the signed contraction.  Nothing here is the GPU
code; it checks that the format makes that scheme exact.
"""

import numpy as np
import pytest

import oracle


def _units(packed, R, K):
    """units[T, L, u] read back from the bytes with the placement rule."""
    rp, kp = 16 * ((R + 15) // 16), 64 * ((K + 63) // 64)
    nt, nu = rp // 16, kp // 64
    nf = nu // 8
    out = np.zeros((nt, 64, nu), dtype=np.uint32)
    for T in range(nt):
        for L in range(64):
            for u in range(nu):
                j, tu = u - 8 * nf, nu - 8 * nf
                if u < 8 * nf:
                    rel = 1024 * (u // 8) + 16 * L + 2 * (u % 8)
                elif j < 2 * (tu // 2):
                    rel = 1024 * nf + 256 * (j // 2) + 4 * L + 2 * (j % 2)
                else:
                    rel = 1024 * nf + 256 * (tu // 2) + 2 * L
                off = T * 2 * kp + rel
                out[T, L, u] = int(packed[off]) | (int(packed[off + 1]) << 8)
    return out


def _fp16_bits_to_float(bits16):
    return float(np.array([bits16], dtype=np.uint16).view(np.float16)[0])


def _fragment_values(units, R, K):
    """A[a, k] as the lanes would build them; cls[k] = True for the q-odd class."""
    nt, _, nu = units.shape
    kp = 64 * nu
    A = np.full((nt * 16, kp), np.nan)
    cls = np.zeros(kp, dtype=bool)
    for T in range(nt):
        for L in range(64):
            row, c = 16 * T + L % 16, L // 16
            for p in range((nu + 1) // 2):
                u0 = units[T, L, 2 * p]
                u1 = units[T, L, 2 * p + 1] if 2 * p + 1 < nu else 0
                mem = u0 | (u1 << 16)
                mb = [(mem >> (8 * i)) & 0xFF for i in range(4)]
                reg = mb[2] | (mb[0] << 8) | (mb[3] << 16) | (mb[1] << 24)
                for q in range(16):
                    step = 4 * p + q // 4
                    if 32 * step >= kp:
                        continue
                    ws = (reg << (2 * (q // 2))) & 0xFFFFFFFF
                    dw = ((ws & 0x80008000) | 0x3C003C00) if q % 2 == 0 else (ws & 0x40004000)
                    d = q % 4
                    for half, e in ((0, 2 * d), (1, 2 * d + 1)):
                        k = 32 * step + 8 * c + e
                        A[row, k] = _fp16_bits_to_float((dw >> (16 * half)) & 0xFFFF)
                        cls[k] = (q % 2 == 1)
    return A, cls


@pytest.mark.parametrize("R,K", [(16, 64), (16, 128), (20, 600), (32, 1472)])
def test_fragment_unpack_reproduces_signs(R, K):
    rng = np.random.default_rng(R + K)
    neg = rng.random((R, K)) < 0.5
    units = _units(oracle.pack_factor(neg), R, K)
    A, cls = _fragment_values(units, R, K)
    kk = np.arange(A.shape[1])
    np.testing.assert_array_equal(cls, (kk & 2) != 0)
    s = np.where(neg, -1.0, 1.0)
    for k in range(K):
        if cls[k]:
            np.testing.assert_array_equal(A[:R, k], np.where(neg[:, k], 2.0, 0.0))
        else:
            np.testing.assert_array_equal(A[:R, k], s[:, k])
    # exact signed contraction through the class rule
    u = rng.standard_normal(K)
    Bp = np.where(cls[:K], -u, u)
    got = A[:R, :K] @ Bp + u[cls[:K]].sum()
    np.testing.assert_allclose(got, s @ u, rtol=1e-12, atol=1e-12)
