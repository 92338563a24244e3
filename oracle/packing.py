"""Oracle implementation of the LB16 packed sign-bit format.

TEST INFRASTRUCTURE ONLY: never imported by the product path.  Written from
the format's text specification (repeated below); it shares no code or table
with the GPU packer.

Why bits at all: the explainx.ai explainer, "How it works" item 1, keeps only
the signs of the thin factors at inference time, and a matrix of signs needs
one bit per entry.  The bit order below is this project's own choice (the
pages give none).

LB16 format (one packed factor F with R rows and reduction length K)
--------------------------------------------------------------------
* F[a][k] is +1 or -1; it is stored as one bit, 1 meaning -1.  For a latent
  value v the bit is 1 exactly when v < 0.
* Rp = 16 * ceil(R / 16) rows and Kp = 64 * ceil(K / 64) columns are stored;
  padding elements (a >= R or k >= K) are stored as 0.
* Tile T holds rows 16T .. 16T+15 and occupies 2*Kp bytes starting at byte
  T * 2 * Kp.
* Inside a tile there are 64 lanes L = 0..63.  Lane L covers row
  a = 16T + (L mod 16) and column group c = floor(L / 16).
* K is cut into steps of 32 columns.  In step s lane L owns the 8 elements
  k = 32 s + 8 c + e, e = 0..7.
* A lane's elements form 16-bit units.  Unit u (0 <= u < NU = Kp / 64) holds
  steps 2u and 2u+1; element (step 2u + q, e), q in {0, 1}, is bit
  8 * (e mod 2) + 7 - (4 q + floor(e / 2)) of the unit.
* Units are stored little-endian.  Units 2p and 2p+1 of lane L form the
  aligned 32-bit word at tile byte 256 p + 4 L (unit 2p in the low half);
  when NU is odd the last unit sits alone at tile byte 256 floor(NU / 2) + 2 L.
"""

from __future__ import annotations

import numpy as np


def sign_bits(latent: np.ndarray, transpose: bool = False) -> np.ndarray:
    """Boolean matrix of the factor to pack: True where the latent value is < 0.

    ``transpose=True`` packs the transpose of ``latent`` (rows and columns
    swapped), as is done for sign(V)^T, whose reduction runs over the n inputs.
    """
    a = np.asarray(latent)
    neg = a < 0
    return np.ascontiguousarray(neg.T if transpose else neg)


def packed_factor_bytes(R: int, K: int) -> int:
    """Size in bytes of a packed R x K factor (padding included)."""
    rp = 16 * ((R + 15) // 16)
    kp = 64 * ((K + 63) // 64)
    return rp * kp // 8


def _unit_bit_position(q: int, e: int) -> int:
    # Bit of element (step 2u + q, e) inside its 16-bit unit.
    return 8 * (e % 2) + 7 - (4 * q + e // 2)


def _unit_byte_offsets(nu: int) -> np.ndarray:
    """offsets[L, u] = byte offset of lane L's unit u inside a tile."""
    out = np.zeros((64, nu), dtype=np.int64)
    for lane in range(64):
        for u in range(nu):
            if u < 2 * (nu // 2):
                out[lane, u] = 256 * (u // 2) + 4 * lane + 2 * (u % 2)
            else:
                out[lane, u] = 256 * (nu // 2) + 2 * lane
    return out


def pack_factor(neg: np.ndarray) -> np.ndarray:
    """Pack a boolean R x K matrix (True = -1) into LB16 bytes (uint8 array)."""
    neg = np.asarray(neg, dtype=bool)
    R, K = neg.shape
    rp, kp = 16 * ((R + 15) // 16), 64 * ((K + 63) // 64)
    full = np.zeros((rp, kp), dtype=bool)
    full[:R, :K] = neg
    ntiles, nu = rp // 16, kp // 64
    # column k = 64 u + 32 q + 8 c + e ; row a = 16 T + row16
    b = full.reshape(ntiles, 16, nu, 2, 4, 8).astype(np.uint32)   # [T,row16,u,q,c,e]
    units = np.zeros((ntiles, 16, nu, 4), dtype=np.uint32)          # [T,row16,u,c]
    for q in range(2):
        for e in range(8):
            units |= b[:, :, :, q, :, e] << np.uint32(_unit_bit_position(q, e))
    # lane L = 16 c + row16  ->  [T, L, u]
    lane_units = units.transpose(0, 3, 1, 2).reshape(ntiles, 64, nu)
    tile_bytes = 2 * kp
    out = np.zeros(ntiles * tile_bytes, dtype=np.uint8)
    offs = _unit_byte_offsets(nu)                                    # [L, u]
    base = (np.arange(ntiles, dtype=np.int64) * tile_bytes)[:, None, None]
    pos = base + offs[None, :, :]
    out[pos] = (lane_units & 0xFF).astype(np.uint8)
    out[pos + 1] = (lane_units >> 8).astype(np.uint8)
    return out


def unpack_factor(packed: np.ndarray, R: int, K: int) -> np.ndarray:
    """Inverse of ``pack_factor``: LB16 bytes -> boolean R x K (True = -1)."""
    packed = np.asarray(packed, dtype=np.uint8)
    rp, kp = 16 * ((R + 15) // 16), 64 * ((K + 63) // 64)
    ntiles, nu = rp // 16, kp // 64
    tile_bytes = 2 * kp
    if packed.size != ntiles * tile_bytes:
        raise ValueError("packed buffer has the wrong size for R x K")
    offs = _unit_byte_offsets(nu)
    base = (np.arange(ntiles, dtype=np.int64) * tile_bytes)[:, None, None]
    pos = base + offs[None, :, :]
    lane_units = packed[pos].astype(np.uint32) | (packed[pos + 1].astype(np.uint32) << 8)
    units = lane_units.reshape(ntiles, 4, 16, nu).transpose(0, 2, 3, 1)  # [T,row16,u,c]
    b = np.zeros((ntiles, 16, nu, 2, 4, 8), dtype=bool)
    for q in range(2):
        for e in range(8):
            b[:, :, :, q, :, e] = (units >> np.uint32(_unit_bit_position(q, e))) & 1
    full = b.reshape(rp, kp)
    return full[:R, :K].copy()
