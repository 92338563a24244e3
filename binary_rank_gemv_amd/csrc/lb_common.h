// Shared device helpers for the LittleBit gfx950 kernels: LB16 addressing and
// the shift-and-mask conversion of packed signs into matrix-core operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LB_WAVE 64
#define LB_MAX_LAYERS 7

// ---------------------------------------------------------------- LB16 layout
// A packed factor with R rows and reduction length K is a sequence of tiles of
// 16 rows; a tile holds 64 lanes x NU 16-bit units, NU = ceil(K/64).  Units
// 2p and 2p+1 of a lane form one aligned 32-bit word ("pair p"), except the
// last unit when NU is odd.

__host__ __device__ inline int lb16_units(int K) { return (K + 63) >> 6; }
__host__ __device__ inline long lb16_tile_bytes(int K) { return 128L * lb16_units(K); }

// Byte offset, inside a tile, of lane `lane`'s pair p (or of its odd last unit).
__device__ inline int lb16_pair_offset(int p, int lane, int nu) {
  const int nf = nu >> 3;
  if (2 * p < 8 * nf) return 1024 * (p >> 2) + 16 * lane + 4 * (p & 3);
  const int j = 2 * p - 8 * nf, tu = nu - 8 * nf;
  if (j + 1 < tu) return 1024 * nf + 256 * (j >> 1) + 4 * lane;
  return 1024 * nf + 256 * (tu >> 1) + 2 * lane;  // odd last unit (16 bits)
}

// Load lane `lane`'s pair p of a tile as a 32-bit word in memory order (the
// odd last unit is zero-extended).
__device__ inline uint32_t lb16_load_pair(const uint8_t* tile, int p, int lane, int nu) {
  const int off = lb16_pair_offset(p, lane, nu);
  if (2 * p + 1 < nu) return *reinterpret_cast<const uint32_t*>(tile + off);
  return (uint32_t)(*reinterpret_cast<const uint16_t*>(tile + off));
}

// Memory bytes [m0 m1 m2 m3] (units 2p, 2p+1) -> register word [m2 m0 m3 m1]:
// bit 15-q holds the low element and bit 31-q the high element of operand
// dword q = 4*step + d (step 0..3 of the pair, d = 0..3).
__device__ inline uint32_t lb16_reg_word(uint32_t mem) {
  return __builtin_amdgcn_perm(mem, mem, 0x01030002u);
}

// The four operand dwords (8 fp16 values) of step `st` (0..3) of a register
// word.  Even q: bits 15/31 after the shift are signs -> +-1.0 (0x3C00).
// Odd q: bits 14/30 -> 0.0 or 2.0; the matching activations are stored
// negated and their sum is added back, so  A.B' + sum = sum_k sign_k * act_k.
__device__ inline f16x8 lb16_step_operand(uint32_t reg, int st) {
  const uint32_t w0 = reg << (4 * st);
  const uint32_t w1 = reg << (4 * st + 2);
  u32x4 d;
  d[0] = (w0 & 0x80008000u) | 0x3C003C00u;
  d[1] = w0 & 0x40004000u;
  d[2] = (w1 & 0x80008000u) | 0x3C003C00u;
  d[3] = w1 & 0x40004000u;
  return __builtin_bit_cast(f16x8, d);
}

// Activation index k belongs to the "odd q" operand class iff (k & 2) != 0.
__host__ __device__ inline bool lb16_negated_class(int k) { return (k & 2) != 0; }

__device__ inline f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline float h2f(uint16_t v) { return (float)__builtin_bit_cast(f16, v); }
__device__ inline uint16_t f2h(float v) { return __builtin_bit_cast(uint16_t, (f16)v); }

// ------------------------------------------------------------ layer arguments
struct LbBranchArgs {
  const uint8_t* vbits;   // LB16 sign(V)^T : R = r, K = n
  const uint8_t* ubits;   // LB16 sign(U)   : R = m, K = r
  const uint16_t* h;
  const uint16_t* l;
  const uint16_t* g;
  int r;
  int zoff;               // offset of this branch's z inside a z row (halves)
  int csum_off;           // offset (floats) of this branch's tile sums
};

struct LbLayerArgs {
  LbBranchArgs br[2];
  int nb;                 // active branches (1 or 2)
  int m, n;
  const uint16_t* x; long ldx;
  uint16_t* y; long ldy;
  uint16_t* z;            // workspace: [batch][zs] fp16 (negated class stored negated)
  float* csum;            // workspace: per branch [ceil(r/16)][16] floats
  int zs;                 // z row stride (halves)
  int vt_begin[2];        // first global V-tile index of each branch
  int ut_begin;           // first global U-tile index
};

struct LbDecodeArgs {
  LbLayerArgs L[LB_MAX_LAYERS];
  int nlayers;
  int batch;
  int nvt;                // total V tiles
  int nut;                // total U tiles
};
