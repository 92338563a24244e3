// Shared device helpers for the LittleBit gfx950 kernels: LB16 addressing and
// the shift-and-mask conversion of packed signs into matrix-core operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LB_MAX_LAYERS 7
#define LB_MAX_GRID 256  // workgroups of the single-launch decode kernel
#define LB_DECODE_LDS_MAX (120 * 1024)  // dynamic LDS limit of a decode launch (bytes)
#define LB_DECODE1_LDS_MAX (64 * 1024)  // the same, one-token kernels (u of n <= 32768 in sparse order)

// ---------------------------------------------------------------- LB16 layout
// A packed factor with R rows and reduction length K is a sequence of tiles of
// 16 rows; a tile holds 64 lanes x NU 16-bit units, NU = ceil(K/64).  Units
// 2p and 2p+1 of lane L ("pair p") are the aligned 32-bit word at tile byte
// 256p + 4L; when NU is odd the last unit is alone at 256*(NU/2) + 2L.

__host__ __device__ inline int lb16_units(int K) { return (K + 63) >> 6; }
__host__ __device__ inline long lb16_tile_bytes(int K) { return 128L * lb16_units(K); }

// Lane `lane`'s pair p of a tile as one aligned 32-bit load: units 2p, 2p+1,
// or, for an odd last unit, the word holding the lane's unit and its
// neighbour's (lb16_pair_sel picks the right half).  p must be wave-uniform.
__device__ inline uint32_t lb16_load_pair(const uint8_t* tile, int p, int lane, int nu) {
  const int off = (2 * p + 1 < nu) ? 4 * lane : 4 * (lane >> 1);
  return *reinterpret_cast<const uint32_t*>(tile + 256 * p + off);
}

// Byte selector of lb16_reg_word for pair p.  Memory bytes [m0 m1 m2 m3] of a
// full pair give the register word [m2 m0 m3 m1] (byte 0 first); an odd last
// unit stands in for unit 2p with unit 2p+1 = 0: [0 m0 0 m1] for an even lane
// (its unit is bytes m0 m1), [0 m2 0 m3] for an odd lane.  Selector byte 0x0C
// yields 0x00.
__device__ inline uint32_t lb16_pair_sel(int p, int lane, int nu) {
  return (2 * p + 1 < nu) ? 0x01030002u : ((lane & 1) ? 0x030C020Cu : 0x010C000Cu);
}

// Register word of a pair: bit 15-q holds the low element and bit 31-q the
// high element of operand dword q = 4*step + d (step 0..3 of the pair, d = 0..3).
__device__ inline uint32_t lb16_reg_word(uint32_t mem, uint32_t sel) {
  return __builtin_amdgcn_perm(mem, mem, sel);
}

// Constants of the sign expansion, held in registers so that the compiler
// can use one and-or per value pair (a 3-operand instruction takes no
// literals on this architecture).
struct LbSignConsts {
  uint32_t sign_mask;  // 0x80008000 (scalar register)
  uint32_t one_pair;   // 0x3C003C00 = (1.0, 1.0) in fp16 (vector register)
};

__device__ inline LbSignConsts lb16_sign_consts() {
  LbSignConsts c;
  c.sign_mask = 0x80008000u;
  c.one_pair = 0x3C003C00u;
  __asm__ volatile("" : "+s"(c.sign_mask));
  __asm__ volatile("" : "+v"(c.one_pair));
  return c;
}

// The four operand dwords (8 fp16 values) of step `st` (0..3) of a pair's
// register word, every value exactly +-v, where `vpair` holds the fp16 bits
// of v >= 0 in both halves (v = 1.0: 0x3C003C00).  Dword q's two signs sit
// at bits 15-(4st+q) and 31-(4st+q): a left shift by 4st+q brings them to
// the fp16 sign positions.  Two instructions per value pair.  (A negative scale is applied by inverting
// every bit of the register word first: all values of a lane share one row.)
__device__ inline f16x8 lb16_step_operand_val(uint32_t reg, int st, uint32_t sign_mask, uint32_t vpair) {
  u32x4 d;
  d[0] = ((reg << (4 * st)) & sign_mask) | vpair;
  d[1] = ((reg << (4 * st + 1)) & sign_mask) | vpair;
  d[2] = ((reg << (4 * st + 2)) & sign_mask) | vpair;
  d[3] = ((reg << (4 * st + 3)) & sign_mask) | vpair;
  return __builtin_bit_cast(f16x8, d);
}

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
};

struct LbLayerArgs {
  LbBranchArgs br[2];
  int nb;                 // active branches (1 or 2)
  int m, n;
  const uint16_t* x; long ldx;
  uint16_t* y; long ldy;
  uint64_t* z;            // workspace: [batch][zs/2] tagged words (see decode.hip)
  int zs;                 // z row length (halves; a multiple of 64)
};

// Kernel arguments of the decode kernels.  The header (first 128 bytes) holds
// everything needed to map a global tile index to its layer without further
// memory traffic; tiles are numbered layer by layer (V tiles branch by branch).
struct LbDecodeArgs {
  int nlayers;
  int batch;
  int nvt;                          // total V tiles
  int nut;                          // total U tiles
  int ut_end[LB_MAX_LAYERS];        // cumulative U-tile count after layer i
  int vt_end[2 * LB_MAX_LAYERS];    // cumulative V-tile count after (layer i, branch b) = 2i+b
  int vq, vr;                       // V tiles of workgroup w: vq + (w < vr), contiguous
  int uq, ur;                       // U tiles likewise
  int vtpu;                         // one-token kernels: V tiles per unit of V work (1 or 2)
  int pad_[2];
  LbLayerArgs L[LB_MAX_LAYERS];
  // single launch of several layers: workgroup w takes V tiles
  // [vt_begin[w], vt_begin[w + 1]) and U tiles [ut_begin[w], ut_begin[w + 1]),
  // contiguous ranges balanced by their cost (one layer splits evenly with
  // vq/vr and uq/ur instead)
  int vt_begin[LB_MAX_GRID + 1];
  int ut_begin[LB_MAX_GRID + 1];
};

// Kernel arguments of the prefill (matrix-core GEMM) kernels for one layer
// and up to LB_PREFILL_MAX_TOKENS tokens.  z: [M][zs] fp16, branch b's
// latent values at zoff (halves), zero-padded to 64*ceil(r/64).
#define LB_PREFILL_MAX_TOKENS 8192
struct LbPrefillArgs {
  LbBranchArgs br[2];
  int nb;
  int m, n;
  int M;                  // tokens
  const uint16_t* x; long ldx;
  uint16_t* y; long ldy;
  uint16_t* z;
  int zs;                 // z row length (halves; a multiple of 64)
};
