// One-token decode of the LittleBit layer on gfx950's sparse matrix
// instruction (v_smfmac_f32_16x16x64_f16).
//
// Per branch (explainx.ai explainer, "How it works" items 1-3):
//   u = g*x (fp16), t = sign(V)^T u, z = l*t (fp16), s = sign(U) z, y = sum_b h_b*s_b.
//
// The signs never become operand values.  The sparse instruction's A operand
// is 16 rows x 64 positions in which every group of 4 positions holds 2
// values, each placed by a 2-bit index.  Here every row of A holds the
// activations of its lane group (a lane's 8 values) and the index carries
// the signs: B's column 0 holds -1 where bit 0 of the in-group position is
// set and column 1 where bit 1 is, +1 elsewhere (sign_columns).  With bit 0
// of each index the sign bit of one tile's row and bit 1 that of a second
// tile's, column 0 of the product is the first row's sum of +-a and column 1
// the second's, exactly: one instruction serves two 16-row tiles.  The raw
// LB16 words give the indices with two or three VALU operations per word;
// the activations are stored in the matching order ("sparse order", below),
// so no bit is moved.
//
// Structure (as in the multi-token kernels of decode.hip): phase A runs the V
// pass over pairs of 16-row tiles of sign(V)^T (the 8 waves of a workgroup split the
// reduction; the activation operands reach each 16-lane row by a DPP row
// broadcast) and stores z as tagged 64-bit words [call tag | two fp16];
// phase B polls the z range of each wave, then runs the U pass over groups
// of 16-row output tiles, two tiles per instruction, with the h epilogue.
// The first U block of each wave is copied straight into LDS during phase A.
// One launch of one 512-thread workgroup per compute unit (MODE 2), or two
// launches (MODE 0: phase A with tag 0, MODE 1: phase B without polling).  A
// tile's sums do not depend on the workgroup or launch that runs it, so every
// path returns the same bits.
#include <stddef.h>

#include "lb_common.h"
#include "lb_sync.h"

// Phase timestamps, in an instrumented build only (-DLB_PHASE_STAMPS; the
// regular library has none of this).  Every workgroup keeps the 100 MHz
// real-time counter at fixed points of a call in registers and writes them
// after its last phase to the device buffer given to
// littlebit_phase_stamps_set: slot 16 w + i for workgroup w and point i
// (0 start, 1 arguments and first u staged, 8 first V products start,
// 2 first V products done, 3 first z round issued, 4 first z copied,
// 5 first U group's products done, 6 end; 7 a multi-layer tile staged;
// 9 last V unit's z stored, 10 last z copy done, 13 first unit's words
// landed, 14 next unit's words issued, 15 first unit's partial sums met)
// and two counts (11 u stagings, 12 z copies).
#ifdef LB_PHASE_STAMPS
__device__ uint64_t* g_phase_stamps;
#define LB_STAMP_N 16
#define LB_STAMP_DECL uint64_t ts_[LB_STAMP_N] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#define LB_STAMP(i) (ts_[i] = __builtin_amdgcn_s_memrealtime())
#define LB_COUNT(i) (++ts_[i])
#define LB_STAMP_WRITE()                                                              \
  do {                                                                               \
    uint64_t* sp_ = g_phase_stamps;                                                  \
    if (threadIdx.x == 0 && sp_)                                                     \
      for (int i_ = 0; i_ < LB_STAMP_N; ++i_) sp_[16 * blockIdx.x + i_] = ts_[i_];   \
  } while (0)
// Per-wave points, lane 0 of every wave, in the buffer's spare rows:
// 16 (256 R + w) + wave for region R (0 first V products done, 1 first U
// group's products done) of workgroup w < 256.
#define LB_WSTAMP(R)                                                                 \
  do {                                                                               \
    uint64_t* sp_ = g_phase_stamps;                                                  \
    if ((threadIdx.x & 63) == 0 && sp_ && blockIdx.x < 256)                          \
      sp_[16 * (256 * (R + 1) + blockIdx.x) + (threadIdx.x >> 6)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
extern "C" int littlebit_phase_stamps_set(void* p) {
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_phase_stamps), &p, sizeof(p));
}
#else
#define LB_STAMP_DECL
#define LB_STAMP(i) ((void)0)
#define LB_COUNT(i) ((void)0)
#define LB_WSTAMP(R) ((void)0)
#define LB_STAMP_WRITE() ((void)0)
#endif

#define DK_WAVES 8
#define DK_THREADS (64 * DK_WAVES)
#define DK_VPW 8   // V-pass pairs per wave per batch of sign words
#define DK_UTG 8   // U tiles per group (one epilogue), at most; launches whose
                   // workgroups hold at most 4 U tiles use groups of 4
#define DK_UPW 4   // U-pass pairs per wave per block of sign words

namespace {

typedef f16 f16x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------ sparse order
// Reduction index k of a packed factor (k < 64 NU) is stored at
// sparse_pos(k): unit u = k / 64 holds steps 2u (q = 0) and 2u + 1 (q = 1);
// lane group G owns k = 64u + 32q + 8G + e, e = 0..7.  For unit u and group G
// the 16 halves at 64u + 16G are the A operands of two instructions, "even"
// (the signs at the even bits of the lane's 16-bit unit) then "odd".  Bit b
// of the unit is element (q, e) with 8(e%2) + 7 - (4q + e/2) = b (LB16);
// (unit & 0x5555) puts the bits 4d and 4d+2 in index nibble d, whose two
// values are the operand's slots 2d and 2d+1, and likewise for unit >> 1.
// Worked out: element (q, e) is slot 2 dword + half of operand `which` with
//   which = 1 - (e/2 % 2), dword = 2 (e % 2) + 1 - q, half = 1 - e/4.
__host__ __device__ inline int sparse_pos(int k) {
  const int u = k >> 6, q = (k >> 5) & 1, G = (k >> 3) & 3, e = k & 7;
  const int which = 1 - ((e >> 1) & 1), dword = 2 * (e & 1) + 1 - q, half = 1 - (e >> 2);
  return 64 * u + 16 * G + 8 * which + 2 * dword + half;
}

// Workgroup barrier that orders LDS only.  Global loads stay in flight across
// it (__syncthreads' fence would also wait for every outstanding global load,
// which would serialise the prefetches with each barrier).  The kernels share
// data between waves only through LDS.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier for LDS data written by ds instructions, without a
// memory fence: loads that write LDS straight from memory and are still in
// flight (the first U block's, read only in phase B) are not waited for.
// The asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier_nf() {
  compiler_memory_barrier();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
  __builtin_amdgcn_s_barrier();
  compiler_memory_barrier();
}

// B operand.  The in-group index t (0..3) of an A value selects the B row
// 4 g + t of its group g; here column 0 holds -1 where bit 0 of t is set and
// column 1 where bit 1 is set, +1 elsewhere, and columns 2..15 are zero.  So
// column 0 of the product sums the values signed by their index's bit 0 and
// column 1 by its bit 1: one instruction serves two rows of signs (lane
// element e of B sits at a position p with p % 4 = e % 4).  The instruction
// gathers B rows for any pair of indices of a group, equal ones included.
__device__ inline f16x16 sign_columns() {
  const int col = threadIdx.x & 15;
  uint32_t d0 = col == 0 ? 0xBC003C00u : (col == 1 ? 0x3C003C00u : 0u);  // t = 0, 1
  uint32_t d1 = col == 0 ? 0xBC003C00u : (col == 1 ? 0xBC00BC00u : 0u);  // t = 2, 3
  __asm__ volatile("" : "+v"(d0), "+v"(d1));
  typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
  u32x8 v = {d0, d1, d0, d1, d0, d1, d0, d1};
  return __builtin_bit_cast(f16x16, v);
}

__device__ __forceinline__ f32x4 smfmac(f16x8 a, f16x16 b, f32x4 c, int idx, int abid) {
  if (abid == 0) return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c, idx, 0, 0);
  return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c, idx, 0, 1);
}

// A lane's activation operands of one pair (sparse order): even and odd
// operands of the pair's two units (the second unit's only when it exists).
struct PairAct {
  f16x8 e0, o0, e1, o1;
};

__device__ __forceinline__ PairAct load_pair_act(const uint16_t* act, bool two_units) {
  const int G = (threadIdx.x & 63) >> 4;
  const uint16_t* a0 = act + 16 * G;
  PairAct a;
  a.e0 = *reinterpret_cast<const f16x8*>(a0);
  a.o0 = *reinterpret_cast<const f16x8*>(a0 + 8);
  a.e1 = two_units ? *reinterpret_cast<const f16x8*>(a0 + 64) : a.e0;
  a.o1 = two_units ? *reinterpret_cast<const f16x8*>(a0 + 72) : a.o0;
  return a;
}

// The products of one pair of units for two tiles at once: raw LB16 words
// wa, wb of the tiles (for an odd last unit, the lane's unit in bits 0..15
// and two_units false).  The sign bit of tile a's row becomes bit 0 and tile
// b's bit 1 of each index, so column 0 sums tile a's row and column 1 tile
// b's; four VALU operations make the indices of up to four instructions.
__device__ __forceinline__ void pair_products2(const PairAct& a, uint32_t wa, uint32_t wb, bool two_units,
                                               const f16x16& B, f32x4& acc0, f32x4& acc1) {
  const int ie = (int)((wa & 0x55555555u) | ((wb << 1) & 0xAAAAAAAAu));
  const int io = (int)(((wa >> 1) & 0x55555555u) | (wb & 0xAAAAAAAAu));
  acc0 = smfmac(a.e0, B, acc0, ie, 0);
  acc1 = smfmac(a.o0, B, acc1, io, 0);
  if (two_units) {
    acc0 = smfmac(a.e1, B, acc0, ie, 1);
    acc1 = smfmac(a.o1, B, acc1, io, 1);
  }
}

// Lane's raw word of pair p of a tile (units 2p, 2p + 1), or, for an odd last
// unit, the lane's own 16-bit unit in the low half.
// The address is selected first, so every call is one load that is not waited
// for here (two conditional loads would each be waited for in turn).
__device__ __forceinline__ uint32_t pair_word(const uint8_t* tile, int p, int nu) {
  const int lane = threadIdx.x & 63;
  const bool full = 2 * p + 1 < nu;
  return *reinterpret_cast<const uint32_t*>(tile + 256 * p + (full ? 4 * lane : 4 * (lane >> 1)));
}

// The word as pair_products takes it: an odd last unit's word holds this
// lane's unit and its neighbour's; the lane's own goes to bits 0..15.
__device__ __forceinline__ uint32_t pair_bits(uint32_t w, bool full) {
  const int lane = threadIdx.x & 63;
  return full ? w : ((lane & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// ------------------------------------------------------------- arguments
// The kernels read the header and layer records of the argument block from
// an LDS copy: one round of 16-byte loads at kernel start, overlapping the
// first sign-word loads, instead of scalar loads on the critical path.
// Fields that steer control flow or form addresses are read into scalar
// registers (readfirstlane: every lane of a wave holds the same value).
#define DK_ARGS_BYTES ((int)offsetof(LbDecodeArgs, vt_begin))  // header + layer records
static_assert(DK_ARGS_BYTES % 16 == 0, "16-byte copy of the argument block");

// Waits for every outstanding vector memory load of the wave.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }
// A pointer into device memory read from the LDS copy: made wave-uniform and
// marked as global, so that its loads are global (vector memory counter only)
// rather than flat ones, which the LDS waits would also have to drain.
template <class T>
__device__ __forceinline__ T* rflp(T* p) {
  typedef __attribute__((address_space(1))) T GT;
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)rfl((int)(uint32_t)u), hi = (uint32_t)rfl((int)(uint32_t)(u >> 32));
  return (T*)(GT*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// One layer's fields, wave-uniform; branch fields are selected with
// `b ? x1 : x0`, so no array is indexed at run time.
struct SL {
  const uint8_t *vb0, *vb1, *ub0, *ub1;
  const uint16_t *h0, *h1, *l0, *l1, *g0, *g1;
  const uint16_t* x;
  uint16_t* y;
  uint64_t* z;
  int r0, r1, zoff0, zoff1, nb, m, n;
  __device__ int r(int b) const { return b ? r1 : r0; }
  __device__ int zoff(int b) const { return b ? zoff1 : zoff0; }
  __device__ const uint8_t* vb(int b) const { return b ? vb1 : vb0; }
  __device__ const uint8_t* ub(int b) const { return b ? ub1 : ub0; }
  __device__ const uint16_t* l(int b) const { return b ? l1 : l0; }
  __device__ const uint16_t* g(int b) const { return b ? g1 : g0; }
};

// The record (in the LDS copy) is read in one batch of 16-byte reads and
// waited for once; field by field, each read would be waited for before its
// readfirstlane, a round trip per field.
__device__ __forceinline__ SL scalar_layer(const LbLayerArgs& rec) {
  static_assert(sizeof(LbLayerArgs) % 16 == 0 && (int)offsetof(LbDecodeArgs, L) % 16 == 0,
                "layer records are whole 16-byte chunks");
  constexpr int NQ = (int)(sizeof(LbLayerArgs) / 16);
  u32x4 q[NQ];
  const u32x4* src = reinterpret_cast<const u32x4*>(&rec);
#pragma unroll
  for (int i = 0; i < NQ; ++i) q[i] = src[i];
  LbLayerArgs L;
  __builtin_memcpy(&L, q, sizeof(L));
  SL s;
  s.vb0 = rflp(L.br[0].vbits);
  s.vb1 = rflp(L.br[1].vbits);
  s.ub0 = rflp(L.br[0].ubits);
  s.ub1 = rflp(L.br[1].ubits);
  s.h0 = rflp(L.br[0].h);
  s.h1 = rflp(L.br[1].h);
  s.l0 = rflp(L.br[0].l);
  s.l1 = rflp(L.br[1].l);
  s.g0 = rflp(L.br[0].g);
  s.g1 = rflp(L.br[1].g);
  s.x = rflp(L.x);
  s.y = rflp(L.y);
  s.z = rflp(L.z);
  s.r0 = rfl(L.br[0].r);
  s.r1 = rfl(L.br[1].r);
  s.zoff0 = rfl(L.br[0].zoff);
  s.zoff1 = rfl(L.br[1].zoff);
  s.nb = rfl(L.nb);
  s.m = rfl(L.m);
  s.n = rfl(L.n);
  return s;
}

// ------------------------------------------------------------- tile map
__host__ __device__ inline int nunits(int k) { return (k + 63) >> 6; }

// Layer and branch slot (2 layer + branch) of global V tile t, and the tile
// inside its branch.
template <bool SINGLE>
__device__ __forceinline__ int v_slot1(const LbDecodeArgs& A, int t, int& tile) {
  int k = 0;
  if (SINGLE) {
    k = t >= A.vt_end[0] ? 1 : 0;
  } else {
    const int nl = rfl(A.nlayers);
#pragma unroll
    for (int q = 0; q < 2 * LB_MAX_LAYERS - 1; ++q)
      if (q < 2 * nl - 1 && t >= A.vt_end[q]) k = q + 1;
  }
  k = rfl(k);
  tile = rfl(t - (k > 0 ? A.vt_end[k - 1] : 0));
  return k;
}

// Layer of global U tile t and the tile inside it.
template <bool SINGLE>
__device__ __forceinline__ int u_layer1(const LbDecodeArgs& A, int t, int& tile) {
  int li = 0;
  if (!SINGLE) {
    const int nl = rfl(A.nlayers);
#pragma unroll
    for (int i = 0; i < LB_MAX_LAYERS - 1; ++i)
      if (i < nl - 1 && t >= A.ut_end[i]) li = i + 1;
  }
  li = rfl(li);
  tile = rfl(t - (li > 0 ? A.ut_end[li - 1] : 0));
  return li;
}

__device__ __forceinline__ void share1(int q, int r, int i, int& beg, int& end) {
  beg = i * q + min(i, r);
  end = beg + q + (i < r ? 1 : 0);
}

// ------------------------------------------------------------- phase A
// u = fp16(g*x) of one branch of one layer, in sparse order, into LDS (all
// 64 nu values; zero beyond n).  Thread i builds natural groups of 8 inputs
// i, i + 512, ...; the 8 values of a group share unit, step and lane group
// and land as four 32-bit pairs.
__device__ __forceinline__ void stage_u(const uint16_t* x, const uint16_t* g, int n, uint16_t* up) {
  const int nu = nunits(n);
  const bool aligned16 = (((uintptr_t)x) & 15) == 0;  // g is 16-byte aligned by contract
  for (int grp = threadIdx.x; grp < 8 * nu; grp += DK_THREADS) {
    const int k = 8 * grp;
    // products as packed pairs: dword d holds elements 2d (low) and 2d + 1
    // (one fp16 rounding of the exact product, as fp32 then fp16 would give)
    u32x4 uw;
    if (aligned16 && k + 8 <= n) {
      const uint4 xr = *reinterpret_cast<const uint4*>(x + k);
      const uint4 gr = *reinterpret_cast<const uint4*>(g + k);
      uw = __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, xr) * __builtin_bit_cast(f16x8, gr));
    } else {
      // element by element from always-valid indices (no branch, so the 16
      // loads are in flight together), zero at and beyond n
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = min(k + e, n - 1);
        const f16 uv = __builtin_bit_cast(f16, x[kk]) * __builtin_bit_cast(f16, g[kk]);
        h[e] = (k + e < n) ? (uint32_t)__builtin_bit_cast(uint16_t, uv) : 0u;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) uw[d] = h[2 * d] | (h[2 * d + 1] << 16);
    }
    // elements (e + 4, e) share a 32-bit pair (low, high) for e = 0..3
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = (uw[(e + 4) >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      const uint32_t hi = (uw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      *reinterpret_cast<uint32_t*>(up + sparse_pos(k + e + 4)) = lo | (hi << 16);  // even position: low half
    }
  }
}

// Word (of a branch's z region) holding z value pair j (0..7) of V tile T in
// sparse order: tile T covers rows 64u + 16 tl + i (u = T / 4, tl = T % 4),
// i.e. step q = tl / 2, lane groups 2 (tl % 2) and 2 (tl % 2) + 1; pair j
// is group 2 (tl % 2) + j / 4, elements (e + 4, e) with e = j % 4, which
// share one word (low, high halves) and belong to rows i + 4 and i,
// i = 8 (j / 4) + e.
__device__ __forceinline__ int z_word(int T, int j) {
  const int u = T >> 2, tl = T & 3, q = tl >> 1;
  const int G = 2 * (tl & 1) + (j >> 2), e = j & 3;
  const int which = 1 - ((e >> 1) & 1), dword = 2 * (e & 1) + 1 - q;
  return 32 * u + 8 * G + 4 * which + dword;
}

// Stores the 16 z values of V tile T of branch b (zv in LDS) as 8 tagged
// words in sparse order; the branch's last tile also writes the tagged zero
// words of the padding tiles up to 64 nu rows.
__device__ __forceinline__ void store_z_tile(const SL& L, int b, int T, uint32_t tag, const uint16_t* zv) {
  const int tid = threadIdx.x;
  const int r = L.r(b), nu = nunits(r);
  uint64_t* zb = L.z + (L.zoff(b) >> 1);
  if (tid < 8) {
    const int i = 8 * (tid >> 2) + (tid & 3);
    const uint32_t v = (uint32_t)zv[i + 4] | ((uint32_t)zv[i] << 16);
    st64c(zb + z_word(T, tid), (uint64_t)tag | ((uint64_t)v << 32));
  }
  const int ntv = (r + 15) >> 4;
  if (T == ntv - 1) {
    for (int w = tid; w < 8 * (4 * nu - ntv); w += DK_THREADS) st64c(zb + z_word(ntv + (w >> 3), w & 7), (uint64_t)tag);
  }
}

// The V pass over a pair of tiles of one branch (T0, T1; T1 == T0 for an
// odd last tile): wave w sums its even share [pa, pb) of the tiles' unit
// pairs, the sign words of both tiles in batches of DK_VPW pairs per wave.
struct VTile {
  const uint8_t *tile0, *tile1;
  int nu, pa, pb;
};

__device__ __forceinline__ VTile v_tile_geom(const uint8_t* vbits, int n, int T0, int T1) {
  VTile v;
  v.nu = nunits(n);
  const int np = (v.nu + 1) >> 1, wave = wave_id();
  v.tile0 = vbits + (long)T0 * lb16_tile_bytes(n);
  v.tile1 = vbits + (long)T1 * lb16_tile_bytes(n);
  v.pa = (np * wave) >> 3;
  v.pb = (np * (wave + 1)) >> 3;
  return v;
}

// Unit u of V work (tpu = 1 or 2 16-rank tiles) of a branch with ntv tiles:
// tiles T0 and T1 (T1 == T0 for one tile).
__device__ __forceinline__ void v_pair_tiles(int u, int ntv, int tpu, int& T0, int& T1) {
  T0 = tpu * u;
  T1 = min(T0 + tpu - 1, ntv - 1);
}

struct VWords {
  uint32_t w0[DK_VPW], w1[DK_VPW];
};

// Sign words of batch [pc, pc + DK_VPW), in groups of four pairs; groups
// that start beyond the share are not loaded (their words are never used),
// and the last group's slots beyond pb repeat its last word.  TPU = 1: the
// unit is one tile (T1 == T0) and only its words are loaded.
template <int TPU>
__device__ __forceinline__ void v_load_words(const VTile& v, int pc, VWords& w) {
  const int plast = max(v.pb - 1, 0);
#pragma unroll
  for (int j = 0; j < DK_VPW / 4; ++j)
    if (j == 0 || pc + 4 * j < v.pb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w.w0[4 * j + i] = pair_word(v.tile0, min(pc + 4 * j + i, plast), v.nu);
      if (TPU == 2)
#pragma unroll
        for (int i = 0; i < 4; ++i) w.w1[4 * j + i] = pair_word(v.tile1, min(pc + 4 * j + i, plast), v.nu);
    }
}

// A unit's first two batches of sign words.  Both are loaded before the
// workgroup issues any later load (the first U block's copy above all):
// loads complete in issue order, so a second batch loaded at its use would
// wait for everything issued before it.
struct VWords2 {
  VWords b0, b1;
};

// The second batch's first group of four pairs is loaded even when the share
// has no second batch (v_load_words clamps it to the share's last pair, and
// its words are then never used): a load under a branch would make the
// compiler keep the words in memory.
template <int TPU>
__device__ __forceinline__ void v_load_first(const VTile& v, VWords2& w) {
  v_load_words<TPU>(v, v.pa, w.b0);
  v_load_words<TPU>(v, v.pa + DK_VPW, w.b1);
}

// V activations through a row broadcast.  Every lane of a 16-lane row (one
// lane group) needs the same 8 activations for an instruction; rather than
// each lane reading them (16 bytes per lane per instruction), lane r of each
// row reads operand r of a group of four pairs (pair r / 4, unit (r / 2) % 2
// of the pair, even or odd operand r % 2) and each instruction's operand is
// broadcast from its lane across the row (DPP row broadcast, one move per
// dword): a sixteenth of the LDS traffic, for four moves per instruction.
// Every lane of every row is written (all rows and banks enabled, the source
// lane always valid), so the moves take no prior value of the destination
// and need no instruction to set one.
template <int N>
__device__ __forceinline__ f16x8 bcast_operand(const u32x4& q) {
  u32x4 d;
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)q[i], 0x150 + N, 0xF, 0xF, false);
  return __builtin_bit_cast(f16x8, d);
}

// This lane's operand of the group of pairs [pc, pc + 4), clamped to the
// share and to the staged units.
__device__ __forceinline__ u32x4 load_act_group(const uint16_t* up, int pc, int plast, int nu) {
  const int lane = threadIdx.x & 63, r = lane & 15, G = lane >> 4;
  const int p = min(pc + (r >> 2), plast);
  const int unit = min(2 * p + ((r >> 1) & 1), nu - 1);
  return *reinterpret_cast<const u32x4*>(up + 64 * unit + 16 * G + 8 * (r & 1));
}

// Pair I (0..3) of a group: its four operands from the group's reads.
template <int I>
__device__ __forceinline__ PairAct bcast_pair(const u32x4& q) {
  PairAct a;
  a.e0 = bcast_operand<4 * I + 0>(q);
  a.o0 = bcast_operand<4 * I + 1>(q);
  a.e1 = bcast_operand<4 * I + 2>(q);
  a.o1 = bcast_operand<4 * I + 3>(q);
  return a;
}

template <int TPU, int J, int I>
__device__ __forceinline__ void v_pair(const VTile& v, int pc, const u32x4& q, const VWords& w, const f16x16& B,
                                       f32x4& acc0, f32x4& acc1) {
  const int p = pc + 4 * J + I;
  if (p < v.pb) {
    const bool two = 2 * p + 1 < v.nu;
    const uint32_t b0 = pair_bits(late(w.w0[4 * J + I]), two);
    pair_products2(bcast_pair<I>(q), b0, TPU == 2 ? pair_bits(late(w.w1[4 * J + I]), two) : b0, two, B, acc0, acc1);
  }
  __builtin_amdgcn_sched_barrier(0);  // one pair's operands live at a time
}

template <int TPU, int J>
__device__ __forceinline__ void v_group(const VTile& v, int pc, const u32x4& q, const VWords& w, const f16x16& B,
                                        f32x4& acc0, f32x4& acc1) {
  v_pair<TPU, J, 0>(v, pc, q, w, B, acc0, acc1);
  v_pair<TPU, J, 1>(v, pc, q, w, B, acc0, acc1);
  v_pair<TPU, J, 2>(v, pc, q, w, B, acc0, acc1);
  v_pair<TPU, J, 3>(v, pc, q, w, B, acc0, acc1);
}

// Returns this lane's partial sums (rows 4 (lane / 16) + q of column
// lane % 16: tile T0 in column 0, T1 in column 1); `w` holds the first two
// batches' words on entry.
template <int TPU>
__device__ __forceinline__ f32x4 v_tile_sums(const VTile& v, const uint16_t* up, const f16x16& B, const VWords2& w) {
  static_assert(DK_VPW == 8, "two activation groups per batch");
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int plast = max(v.pb - 1, 0);
  // The first two batches stand outside the loop.  Inside it, a batch's
  // words are loaded at the top and used at once, and the compiler's wait for
  // them is counted from there; had the first batches been iterations, their
  // words (loaded much earlier) would get that same wait, i.e. for all but
  // the last few loads issued since: the first U block's copy among them.
  // (Pairs beyond the share are skipped by v_pair.)
  v_group<TPU, 0>(v, v.pa, load_act_group(up, v.pa, plast, v.nu), w.b0, B, acc0, acc1);
  v_group<TPU, 1>(v, v.pa, load_act_group(up, v.pa + 4, plast, v.nu), w.b0, B, acc0, acc1);
  if (v.pa + DK_VPW < v.pb) {
    const int pc = v.pa + DK_VPW;
    v_group<TPU, 0>(v, pc, load_act_group(up, pc, plast, v.nu), w.b1, B, acc0, acc1);
    v_group<TPU, 1>(v, pc, load_act_group(up, pc + 4, plast, v.nu), w.b1, B, acc0, acc1);
  }
  for (int pc = v.pa + 2 * DK_VPW; pc < v.pb; pc += DK_VPW) {
    VWords wl;
    v_load_words<TPU>(v, pc, wl);
    v_group<TPU, 0>(v, pc, load_act_group(up, pc, plast, v.nu), wl, B, acc0, acc1);
    v_group<TPU, 1>(v, pc, load_act_group(up, pc + 4, plast, v.nu), wl, B, acc0, acc1);
  }
  return acc0 + acc1;
}

// ------------------------------------------------------------- phase B
// Copies units [u0, u1) of branch b's z (tagged words) into zl (sparse order,
// values only), polling until every word carries `tag` (unless !check).
// Chunk c (16 bytes: two words) of the range is load c / 64 of lane c % 64,
// in rounds of 64 NL chunks.  zc_begin issues the first round's loads and
// zc_finish completes the copy, so that other loads can be issued between
// the two while the first round is in flight.
template <int NL>
struct ZCopy {
  __amdgpu_buffer_rsrc_t rs;
  uint16_t* dst;
  int nchunks;
  uint32_t todo;  // loads of the current round still to land with the tag
  u32x4 q[NL];
};

template <int NL>
__device__ __forceinline__ uint32_t zc_round_bits(int nchunks, int c0) {
  uint32_t todo = 0;
#pragma unroll
  for (int i = 0; i < NL; ++i)
    if (c0 + 64 * i < nchunks) todo |= 1u << i;
  return todo;
}

template <int NL>
__device__ __forceinline__ void zc_issue(ZCopy<NL>& c, int c0) {
  const int lane = threadIdx.x & 63;
  compiler_memory_barrier();
#pragma unroll
  for (int i = 0; i < NL; ++i)
    if (c.todo & (1u << i)) c.q[i] = ld_tagged2(c.rs, 16 * (c0 + 64 * i + lane));  // beyond the range: zeros
}

template <int NL>
__device__ __forceinline__ void zc_begin(ZCopy<NL>& c, const SL& L, int b, int u0, int u1, uint16_t* zl) {
  c.nchunks = max(16 * (u1 - u0), 0);
  const uint8_t* base = reinterpret_cast<const uint8_t*>(L.z + (L.zoff(b) >> 1) + 32 * u0);
  c.rs = make_rsrc(base, 16 * c.nchunks);
  c.dst = zl + L.zoff(b) + 64 * u0;
  c.todo = zc_round_bits<NL>(c.nchunks, 0);
  zc_issue(c, 0);
}

template <int NL>
__device__ __forceinline__ void zc_finish(ZCopy<NL>& c, uint32_t tag, bool check, uint8_t* sync) {
  const int lane = threadIdx.x & 63;
  for (int c0 = 0; c0 < c.nchunks; c0 += 64 * NL) {
    if (c0 != 0) {
      c.todo = zc_round_bits<NL>(c.nchunks, c0);
      zc_issue(c, c0);
    }
    int spins = 0;
    while (check) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        if (c.todo & (1u << i)) {
          const bool in = c0 + 64 * i + lane < c.nchunks;
          const bool ok = !in || ((c.q[i][0] == tag) & (c.q[i][2] == tag));
          if (__all(ok)) c.todo &= ~(1u << i);
        }
      }
      if (c.todo == 0) break;
      if (++spins > LB_SPIN_LIMIT) {
        st32c(sync + LB_SYNC_ERR, 1u);
        break;
      }
      zc_issue(c, c0);  // the words not yet tagged, again
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int ch = c0 + 64 * i + lane;
      if (ch < c.nchunks) {
        uint2 d;
        d.x = c.q[i][1];
        d.y = c.q[i][3];
        *reinterpret_cast<uint2*>(c.dst + 4 * ch) = d;
      }
    }
  }
}

template <int NL>
__device__ __forceinline__ void copy_z(const SL& L, int b, int u0, int u1, uint32_t tag, bool check, uint8_t* sync,
                                       uint16_t* zl) {
  ZCopy<NL> c;
  zc_begin(c, L, b, u0, u1, zl);
  zc_finish(c, tag, check, sync);
}

// Wave's phase-B role for a layer: branch and pair range of that branch.
// With two branches, waves w and w + 4 (which share a SIMD) take quarters w
// and 3 - w, so that uneven quarters even out per SIMD.
__device__ __forceinline__ void u_role1(const SL& L, int wave, int& b, int& p0, int& p1) {
  if (L.nb == 2) {
    b = wave >> 2;
    const int np = (nunits(L.r(b)) + 1) >> 1, w = b ? 3 - (wave & 3) : (wave & 3);
    p0 = (np * w) >> 2;
    p1 = (np * (w + 1)) >> 2;
  } else {
    b = 0;
    const int np = (nunits(L.r0) + 1) >> 1;
    p0 = (np * wave) >> 3;
    p1 = (np * (wave + 1)) >> 3;
  }
}

// A block of U sign words: tiles [t0, t0 + nt) of one layer (nt <= UTG),
// this wave's pairs [pc, pc + DK_UPW) of its range (clamped loads keep the
// wait counts static).
template <int UTG>
struct UBlock {
  uint32_t w[UTG][DK_UPW];
};

// Row scales (fp16 bits) of this thread's epilogue entry of a group of tiles
// [t0, t0 + nt): tile (tid / 16) % UTG, row tid % 16, clamped to a valid
// row (threads beyond the group's entries never store).  Unconditional loads,
// so no wait is placed at a branch join.
struct HPair {
  uint32_t h0, h1;
};

template <int UTG>
__device__ __forceinline__ HPair load_group_h(const SL& L, int t0, int nt) {
  const int tid = threadIdx.x;
  const int row = min(16 * (t0 + min((tid >> 4) % UTG, nt - 1)) + (tid & 15), L.m - 1);
  const uint16_t* h1p = L.nb == 2 ? L.h1 : L.h0;
  HPair h;
  h.h0 = L.h0[row];
  h.h1 = h1p[row];
  return h;
}

// Words of tile k of a U block (pairs [pc, pc + DK_UPW) of the wave's range
// ending at p1, tiles clamped to the group).
__device__ __forceinline__ void load_utile(const SL& L, int b, int t0, int nt, int pc, int p1, int k,
                                           uint32_t (&w)[DK_UPW]) {
  const int r = L.r(b), nu = nunits(r);
  const uint8_t* tile = L.ub(b) + (long)(t0 + min(k, nt - 1)) * lb16_tile_bytes(r);
  const int plast = max(p1 - 1, 0);
#pragma unroll
  for (int i = 0; i < DK_UPW; ++i) w[i] = pair_word(tile, min(pc + i, plast), nu);
}

template <int UTG>
__device__ __forceinline__ void load_ublock(const SL& L, int b, int t0, int nt, int pc, int p1, UBlock<UTG>& U) {
#pragma unroll
  for (int k = 0; k < UTG; ++k) load_utile(L, b, t0, nt, pc, p1, k, U.w[k]);
}

// The same block straight into LDS (no registers held while it is in
// flight): tile k's pairs [pc, pc + PPT), contiguous in the LB16 layout, to
// dst + 64 PPT k with one 16-byte load per lane, 4 / PPT tiles per load
// (lanes 16 PPT j .. take tile k + j).  Word (k, i) of a lane is then
// dst[64 (PPT k + i) + lane] (lane / 2 for an odd last unit), as pair_word
// reads it from memory.  The copy costs in proportion to its bytes, so it
// takes CT tiles (a group's last tile repeated past nt; groups of 4 where no
// workgroup holds more, 7 of a group of 8 where none holds 8: the eighth
// slot is then never a tile of the group, and its column of the last tile
// pair is discarded) and PPT pairs of each (2 where no wave's range is
// longer, else 4).  Reads are bounded by the end of the factor.
template <int UTG, int PPT, int CT = UTG>
__device__ __forceinline__ void dma_ublock(const SL& L, int b, int t0, int nt, int pc, uint32_t* dst) {
  static_assert(PPT == 2 || PPT == 4, "2 or 4 pairs per tile");
  constexpr int TPL = 4 / PPT;  // tiles per load
  const int r = L.r(b), lane = threadIdx.x & 63;
  const long tb = lb16_tile_bytes(r);
  const int ntf = (L.m + 15) >> 4;
  static_assert(CT == UTG || (CT <= UTG && CT % TPL == 0), "whole loads");
#pragma unroll
  for (int k = 0; k < CT; k += TPL) {
    const int ta = t0 + min(k, nt - 1), tl = t0 + min(k + lane / (16 * PPT), nt - 1);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(L.ub(b) + (long)ta * tb, (int)((ntf - ta) * tb));
    const int off = (int)((tl - ta) * tb) + 256 * pc + 16 * (lane & (16 * PPT - 1));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 64 * PPT * k), 16, off,
                                             0, 0, 0);
  }
}

// A block's words from its LDS copy; pairs past PPT (past every wave's
// range) are zero.
template <int UTG, int PPT>
__device__ __forceinline__ void lds_ublock(const uint32_t* src, int pc, int nu, UBlock<UTG>& U) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < DK_UPW; ++i) {
    const int li = 2 * (pc + i) + 1 < nu ? lane : lane >> 1;
#pragma unroll
    for (int k = 0; k < UTG; ++k) U.w[k][i] = i < PPT ? src[64 * (PPT * k + i) + li] : 0u;
  }
}

// The h epilogue of a group: cross-wave sums in wave order, y = h0 s0 + h1 s1.
// acc[j] holds tiles 2j (column 0) and 2j + 1 (column 1).
template <int UTG>
__device__ __forceinline__ void u_epilogue(const SL& L, int t0, int nt, const f32x4 (&acc)[UTG / 2],
                                           float (*red)[DK_WAVES][16], uint32_t h0raw, uint32_t h1raw) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int col = lane & 15;
  if (col < 2) {
#pragma unroll
    for (int j = 0; j < UTG / 2; ++j)
      if (2 * j + col < nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[2 * j + col][wave][4 * (lane >> 4) + q] = acc[j][q];
  }
  lds_barrier();
  if (tid < 16 * nt) {
    const int k = tid >> 4, i = tid & 15;
    const int row = 16 * (t0 + k) + i;
    if (row < L.m) {
      float y;
      if (L.nb == 2) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int w = 0; w < DK_WAVES / 2; ++w) {
          s0 += red[k][w][i];
          s1 += red[k][w + DK_WAVES / 2][i];
        }
        y = fmaf(h2f((uint16_t)h0raw), s0, h2f((uint16_t)h1raw) * s1);
      } else {
        float s0 = 0.f;
#pragma unroll
        for (int w = 0; w < DK_WAVES; ++w) s0 += red[k][w][i];
        y = h2f((uint16_t)h0raw) * s0;
      }
      L.y[row] = f2h(y);
    }
  }
}

}  // namespace

// The kernels' explicit arguments in order, as laid out in the kernel
// argument segment (each at its natural alignment, as in a struct).  The
// leading 14 dwords are preloaded into scalar registers by the dispatch: a
// single-layer launch issues its first sign-word, activation and counter
// loads from them without waiting for an argument fetch.
struct Dk1Kernargs {
  const uint8_t *pre_vb0, *pre_vb1;
  const uint16_t *pre_x, *pre_g0, *pre_g1;
  uint8_t* sync;
  int pre_n;          // n | (V tiles of branch 0) << 16
  uint32_t pre_misc;  // vq | vr << 8 | (V tiles of branch 1) << 17 (V units of workgroup w: vq + (w < vr))
  LbDecodeArgs A;
};

// The argument block in the kernel argument segment (for the 16-byte copy
// and the per-workgroup tile-range tables).
__device__ __forceinline__ const LbDecodeArgs* dk1_kernarg_args() {
  return (const LbDecodeArgs*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(Dk1Kernargs, A));
}

// MODE 0: phase A only (z tagged 0); 1: phase B only (no polling); 2: both in
// one launch of one workgroup per compute unit.  SINGLE: one layer (tile
// ranges split evenly: V by pre_misc, U by uq/ur); else the cost-balanced
// ranges vt_begin / ut_begin of the argument block (two launches: vq/vr,
// uq/ur).  TPU: 16-rank tiles per unit of V work (1, or 2 on one
// instruction: the host takes 2 when there are more tiles than workgroups).
template <int MODE, bool SINGLE, int TPU, int UTG = DK_UTG, int PPT = DK_UPW, int CT = UTG>
__global__ __launch_bounds__(DK_THREADS) void lb_decode1_kernel(const uint8_t* pre_vb0, const uint8_t* pre_vb1,
                                                                const uint16_t* pre_x, const uint16_t* pre_g0,
                                                                const uint16_t* pre_g1, uint8_t* sync, int pre_n,
                                                                uint32_t pre_misc, LbDecodeArgs) {
  extern __shared__ __align__(16) uint16_t dyn[];  // u in sparse order (phase A), z (phase B)
  __shared__ __align__(16) uint8_t sA_bytes[DK_ARGS_BYTES];
  __shared__ float vred[DK_WAVES][32];
  __shared__ uint16_t zv[32];
  __shared__ float ured[2][DK_UTG][DK_WAVES][16];
  __shared__ __align__(16) uint32_t ublk[DK_WAVES][DK_UTG * DK_UPW * 64];  // each wave's first U block
  const LbDecodeArgs& A = *reinterpret_cast<const LbDecodeArgs*>(sA_bytes);

  const int wg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  LB_STAMP_DECL
  LB_STAMP(0);
  const f16x16 B = sign_columns();
  const LbDecodeArgs* KA = dk1_kernarg_args();

  // ---------------- start
  // Load order (loads complete in issue order): the first V unit's sign
  // words (single layer: from the preloaded arguments), the argument block's
  // copy, this workgroup's call counter, the staging loads of x and g.
  // V work comes in units of two 16-rank tiles of one branch (T0, T1).
  int vt0 = 0, vt1 = 0;
  int k = 0, T0 = 0, T1 = 0;
  VTile v;
  VWords2 w;
  const int n1 = pre_n & 0xFFFF;  // the single layer's n, and its branches' V tile counts
  const int ntv0 = (int)((uint32_t)pre_n >> 16), ntv1 = (int)(pre_misc >> 17);
  const int vsplit = (ntv0 + TPU - 1) / TPU;  // V units of branch 0
  if (SINGLE && MODE != 1) {
    share1((int)(pre_misc & 255u), (int)((pre_misc >> 8) & 255u), wg, vt0, vt1);
    if (vt0 < vt1) {
      k = vt0 >= vsplit ? 1 : 0;
      v_pair_tiles(vt0 - (k ? vsplit : 0), k ? ntv1 : ntv0, TPU, T0, T1);
      v = v_tile_geom(k ? pre_vb1 : pre_vb0, n1, T0, T1);
      v_load_first<TPU>(v, w);
    }
  }
  u32x4 acopy = {0u, 0u, 0u, 0u};
  if (tid < DK_ARGS_BYTES / 16) acopy = reinterpret_cast<const u32x4*>(KA)[tid];
  uint32_t ctr = 0;  // call counter; the tag (0 in the two-launch path, which no poll accepts) is taken at first use
  if (MODE == 2) ctr = ld32c(sync + LB_SYNC_CTR + 8 * wg);
  int ut0 = 0, ut1 = 0;
  if (!SINGLE && MODE == 2) {
    vt0 = KA->vt_begin[wg];
    vt1 = KA->vt_begin[wg + 1];
    ut0 = KA->ut_begin[wg];
    ut1 = KA->ut_begin[wg + 1];
  }
  HPair hcur = {0u, 0u};  // row scales of the first U group
  if (SINGLE && MODE != 1 && vt0 < vt1) {
    stage_u(pre_x, k ? pre_g1 : pre_g0, n1, dyn);  // the first unit's u
    LB_COUNT(11);
  }
  if (tid < DK_ARGS_BYTES / 16) reinterpret_cast<u32x4*>(sA_bytes)[tid] = acopy;
  lds_barrier_nf();  // the argument copy (and a single layer's first u) is complete
  LB_STAMP(1);
  if (SINGLE) wait_vmem_all();  // (the staging waited already: this tells the compiler so)

  if (SINGLE || MODE != 2) {
    if (!SINGLE) share1(rfl(A.vq), rfl(A.vr), wg, vt0, vt1);
    share1(rfl(A.uq), rfl(A.ur), wg, ut0, ut1);
  }
  if (MODE == 1) vt1 = vt0;
  if (MODE == 0) ut1 = ut0;
  // Layer records: a single layer's is read once here and kept (in scalar
  // registers); several layers' are read where they are needed.
  const SL L1 = SINGLE ? scalar_layer(A.L[0]) : SL{};
  auto layer_rec = [&](int li) { return SINGLE ? L1 : scalar_layer(A.L[li]); };
  // the first V unit's latent scales (and, for several layers, its sign
  // words): loaded ahead, like those of each next unit.  Thread i < 32
  // holds l of row i % 16 of tile T0 (i < 16) or T1.
  auto l_of = [&](const SL& L, int b, int t0, int t1) {
    return (uint32_t)L.l(b)[min(16 * (tid & 16 ? t1 : t0) + (tid & 15), L.r(b) - 1)];
  };
  uint32_t lcur = 0;
  if (vt0 < vt1) {
    int u = 0;
    if (!SINGLE) k = v_slot1<SINGLE>(A, vt0, u);
    const SL L = layer_rec(k >> 1);
    if (!SINGLE) {
      v_pair_tiles(u, (L.r(k & 1) + 15) >> 4, TPU, T0, T1);
      v = v_tile_geom(L.vb(k & 1), L.n, T0, T1);
      v_load_first<TPU>(v, w);
    }
    lcur = l_of(L, k & 1, T0, T1);
  }

  // ---------------- phase A
  struct GroupInfo {
    int li, tile, nt, b, p0, p1, nch;
  };
  auto group_at = [&](int t, const SL& L) {
    GroupInfo g;
    g.li = u_layer1<SINGLE>(A, t, g.tile);
    const int lend = SINGLE ? ut1 : min(ut1, rfl(A.ut_end[g.li]));
    g.nt = min(UTG, lend - t);
    u_role1(L, wave, g.b, g.p0, g.p1);
    g.nch = max(1, (g.p1 - g.p0 + DK_UPW - 1) / DK_UPW);
    return g;
  };
  auto layer_of_u = [&](int t) {
    int tile;
    return u_layer1<SINGLE>(A, t, tile);
  };
  // The first U group.  Its first block of sign words is copied straight
  // into LDS, and its row scales loaded, once the first V tile's loads are
  // issued (those complete first): the copy streams in during phase A while
  // holding no registers, and phase A's barriers do not wait for it.  A
  // workgroup without U tiles copies a stand-in (the start of the workspace
  // header, as one 16-row tile of one unit) instead: the loads stay
  // unconditional, which keeps the compiler's waits for earlier loads exact.
  UBlock<UTG> cur;
  const bool have_u = ut0 < ut1;
  SL uL = {};
  GroupInfo ug = {};
  if (have_u) {
    uL = layer_rec(layer_of_u(ut0));
    ug = group_at(ut0, uL);
  } else {
    uL.ub0 = uL.ub1 = sync;
    uL.h0 = uL.h1 = reinterpret_cast<const uint16_t*>(sync);
    uL.r0 = uL.r1 = 16;
    uL.m = uL.nb = 1;
    ug.nt = ug.p1 = 1;
  }
  auto issue_first_u = [&]() {
    if (MODE != 0) {
      compiler_memory_barrier();
      dma_ublock<UTG, PPT, CT>(uL, ug.b, ug.tile, ug.nt, ug.p0, ublk[wave]);
      hcur = load_group_h<UTG>(uL, ug.tile, ug.nt);
      compiler_memory_barrier();
    }
  };
  if (SINGLE || vt0 == vt1) issue_first_u();  // (a single layer staged its first u above)
  uint32_t tag = 0;
  bool tag_ready = MODE != 2;
  auto get_tag = [&]() {
    if (!tag_ready) {
      tag = call_tag(late(ctr));
      tag_ready = true;
    }
    return tag;
  };

  // one V tile (the first is its own copy of the code, so that no loop
  // boundary makes the compiler wait for the loads issued ahead)
  int staged = (SINGLE && vt0 < vt1) ? k : -1;  // the single-layer launch staged its first tile's u above
  auto v_step = [&](int t) {
    const SL L = layer_rec(k >> 1);
    const int b = k & 1;
    const int r = L.r(b);
    if (k != staged) {
      lds_barrier_nf();  // earlier readers of the staged u are done
      stage_u(L.x, L.g(b), L.n, dyn);
      LB_COUNT(11);
      staged = k;
      lds_barrier_nf();  // the staged u is complete
      LB_STAMP(7);
      if (t == vt0) wait_vmem_all();  // (staging waited already: this tells the compiler so)
      if (t == vt0) LB_STAMP(13);
    }
    // the next unit's sign words and latent scales
    int kn = k, Tn0 = T0, Tn1 = T1;
    VTile vn = v;
    VWords2 wn;
    uint32_t lnext = 0;
    if (t + 1 < vt1) {
      int un = 0;
      kn = v_slot1<SINGLE>(A, t + 1, un);
      const SL Ln = layer_rec(kn >> 1);
      v_pair_tiles(un, (Ln.r(kn & 1) + 15) >> 4, TPU, Tn0, Tn1);
      vn = v_tile_geom(Ln.vb(kn & 1), Ln.n, Tn0, Tn1);
      v_load_first<TPU>(vn, wn);
      lnext = l_of(Ln, kn & 1, Tn0, Tn1);
    }
    if (t == vt0) LB_STAMP(14);
    // the first U block after the next unit's words: loads complete in issue
    // order, so words issued after the 64 KB block would wait for all of it
    if (!SINGLE && t == vt0) issue_first_u();
    if (t == vt0) LB_STAMP(8);
    const f32x4 acc = v_tile_sums<TPU>(v, dyn, B, w);
    if (t == vt0) LB_STAMP(2);
    if (t == vt0) LB_WSTAMP(0);
    if ((lane & 15) < 2)  // column 0: tile T0, column 1: tile T1
#pragma unroll
      for (int q = 0; q < 4; ++q) vred[wave][16 * (lane & 15) + 4 * (lane >> 4) + q] = acc[q];
    lds_barrier_nf();
    if (t == vt0) LB_STAMP(15);
    if (tid < 32) {
      const int j = 16 * (tid & 16 ? T1 : T0) + (tid & 15);
      float s = 0.f;
#pragma unroll
      for (int w8 = 0; w8 < DK_WAVES; ++w8) s += vred[w8][tid];
      const f16 z = (j < r) ? (f16)(h2f((uint16_t)late(lcur)) * s) : (f16)0.f;
      zv[tid] = __builtin_bit_cast(uint16_t, z);
    }
    lds_barrier_nf();
    const uint32_t tg = get_tag();
    store_z_tile(L, b, T0, tg, zv);
    if (T1 != T0) store_z_tile(L, b, T1, tg, zv + 16);
    LB_STAMP(9);
    if (t + 1 < vt1) {
      k = kn;
      T0 = Tn0;
      T1 = Tn1;
      v = vn;
      lcur = lnext;
      w = wn;
    }
  };
  if (vt0 < vt1) v_step(vt0);
  for (int t = vt0 + 1; t < vt1; ++t) v_step(t);

  // ---------------- phase B
  // Groups of up to UTG tiles of one layer; each wave runs its pair range
  // [p0, p1) of its branch in blocks of DK_UPW pairs, whose sign words are
  // loaded one block ahead, with the group's row scales.
  //
  // The first group's z: its first round of polling loads, then (once the
  // LDS is free of phase A's u) the rest of the copy, and the first block's
  // words from the LDS copy.
  int zl_layer = -1, grp = 0;
  if (MODE != 0 && have_u) {
    ZCopy<8> zc0;
    const int nu0 = nunits(uL.r(ug.b));
    LB_STAMP(3);
    compiler_memory_barrier();
    zc_begin(zc0, uL, ug.b, min(2 * ug.p0, nu0), min(2 * ug.p1, nu0), dyn);
    get_tag();
    lds_barrier();  // phase A's readers of the LDS are done; the block copy has landed
    zc_finish(zc0, tag, MODE == 2, sync);
    zl_layer = ug.li;
    LB_STAMP(4);
    LB_STAMP(10);
    LB_COUNT(12);
    lds_ublock<UTG, PPT>(ublk[wave], ug.p0, nu0, cur);
  }
  get_tag();
  for (int t = ut0; t < ut1;) {
    const SL L = layer_rec(layer_of_u(t));
    const GroupInfo g = group_at(t, L);
    const int nu = nunits(L.r(g.b));
    if (g.li != zl_layer) {
      lds_barrier();  // earlier readers of the LDS (phase A's u, the previous layer's z) are done
      const int u0 = min(2 * g.p0, nu), u1 = min(2 * g.p1, nu);
      if (16 * (u1 - u0) <= 64 * 4)
        copy_z<4>(L, g.b, u0, u1, tag, MODE == 2, sync, dyn);
      else
        copy_z<16>(L, g.b, u0, u1, tag, MODE == 2, sync, dyn);
      zl_layer = g.li;
      LB_STAMP(10);
      LB_COUNT(12);
    }
    const uint16_t* zb = dyn + L.zoff(g.b);
    const HPair hg = hcur;  // this group's row scales (loaded with its first block)
    f32x4 acc[UTG / 2], acc1[UTG / 2];  // tile pairs (2j, 2j + 1)
#pragma unroll
    for (int j = 0; j < UTG / 2; ++j) acc[j] = acc1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < g.nch; ++c) {
      // the next block's words: this group's next chunk, or the next group's first
      UBlock<UTG> nxt;
      bool more = false;
      if (c + 1 < g.nch) {
        load_ublock(L, g.b, g.tile, g.nt, g.p0 + (c + 1) * DK_UPW, g.p1, nxt);
        more = true;
      } else if (t + g.nt < ut1) {
        const SL Ln = layer_rec(layer_of_u(t + g.nt));
        const GroupInfo h = group_at(t + g.nt, Ln);
        load_ublock(Ln, h.b, h.tile, h.nt, h.p0, h.p1, nxt);
        hcur = load_group_h<UTG>(Ln, h.tile, h.nt);  // the next group's
        more = true;
      }
      const int pc = g.p0 + c * DK_UPW;
#pragma unroll
      for (int i = 0; i < DK_UPW; ++i) {
        const int p = pc + i;
        if (p < g.p1) {
          const bool two = 2 * p + 1 < nu;
          const PairAct za = load_pair_act(zb + 128 * p, two);
#pragma unroll
          for (int j = 0; j < UTG / 2; ++j)
            if (2 * j < g.nt)  // (for an odd count the last tile pairs with itself: load_ublock clamps)
              pair_products2(za, pair_bits(late(cur.w[2 * j][i]), two), pair_bits(late(cur.w[2 * j + 1][i]), two), two,
                             B, acc[j], acc1[j]);
        }
      }
      if (more) cur = nxt;
    }
#pragma unroll
    for (int j = 0; j < UTG / 2; ++j) acc[j] += acc1[j];
    if (t == ut0) LB_STAMP(5);
    if (t == ut0) LB_WSTAMP(1);
    u_epilogue<UTG>(L, g.tile, g.nt, acc, ured[grp & 1], late(hg.h0), late(hg.h1));
    ++grp;
    t += g.nt;
  }
  LB_STAMP(6);
  LB_STAMP_WRITE();
  // this workgroup's call is done: the next call's tag is one higher
  if (MODE == 2 && tid == 0) add64c_noret(sync + LB_SYNC_CTR + 8 * wg, 1ull);
}

// Dynamic LDS of a one-token launch: u of the largest input size in sparse
// order, or the z row of the largest layer.
size_t lb_decode1_lds_bytes(const LbDecodeArgs& a) {
  size_t m = 0;
  for (int i = 0; i < a.nlayers; ++i) {
    const size_t u = (size_t)64 * nunits(a.L[i].n) * 2, z = (size_t)a.L[i].zs * 2;
    m = u > m ? u : m;
    m = z > m ? z : m;
  }
  return m;
}

typedef void (*Decode1Kernel)(const uint8_t*, const uint8_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                             uint8_t*, int, uint32_t, LbDecodeArgs);

// The instantiation for a launch: one or several layers, one or two V tiles
// per unit, U groups of 4 tiles (small: no workgroup holds more than 4 U
// tiles) or 8.
template <int MODE, int UTG, int PPT, int CT = UTG>
Decode1Kernel decode1_pick(bool single, bool one) {
  if (single)
    return one ? lb_decode1_kernel<MODE, true, 1, UTG, PPT, CT> : lb_decode1_kernel<MODE, true, 2, UTG, PPT, CT>;
  return one ? lb_decode1_kernel<MODE, false, 1, UTG, PPT, CT> : lb_decode1_kernel<MODE, false, 2, UTG, PPT, CT>;
}

// The instantiation for a launch: one or several layers, one or two V tiles
// per unit, U groups of 4 tiles (small: no workgroup holds more than 4 U
// tiles) or 8, first-block copies of 2 pairs per tile (narrow: no wave's
// range is longer) or 4, of 7 tiles of a group of 8 (seven: no workgroup
// holds 8 U tiles).
template <int MODE>
Decode1Kernel decode1_variant(bool single, bool one, bool small = false, bool narrow = false, bool seven = false) {
  if constexpr (MODE != 0) {
    if (small) return narrow ? decode1_pick<MODE, 4, 2>(single, one) : decode1_pick<MODE, 4, DK_UPW>(single, one);
    if (narrow) return decode1_pick<MODE, DK_UTG, 2>(single, one);
    if (seven) return decode1_pick<MODE, DK_UTG, DK_UPW, DK_UTG - 1>(single, one);
  }
  return decode1_pick<MODE, DK_UTG, DK_UPW>(single, one);
}

// Whether no wave's phase-B pair range exceeds 2 pairs in any layer
// (u_role1: quarters of a branch's pairs with two branches, eighths with one).
static bool decode1_narrow(const LbDecodeArgs& a) {
  for (int i = 0; i < a.nlayers; ++i)
    for (int b = 0; b < a.L[i].nb; ++b) {
      const int np = (nunits(a.L[i].br[b].r) + 1) >> 1;
      if (np > (a.L[i].nb == 2 ? 8 : 16)) return false;
    }
  return true;
}

// The most U tiles a workgroup holds: q + (r > 0) for an even split, or the
// largest range of a cost-balanced one.
static int decode1_max_utiles(const LbDecodeArgs& a, int G, bool single) {
  if (single || G == 0) return a.uq + (a.ur > 0 ? 1 : 0);
  int mx = 0;
  for (int w = 0; w < G; ++w) mx = a.ut_begin[w + 1] - a.ut_begin[w] > mx ? a.ut_begin[w + 1] - a.ut_begin[w] : mx;
  return mx;
}

// Workgroups of a single launch that fit at once, for the given dynamic LDS
// (the lower count of the two V unit sizes).
hipError_t lb_decode1_occupancy(bool single, size_t lds, int& occ) {
  int o[10] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  hipError_t e = hipSuccess;
  for (int i = 0; i < 10 && e == hipSuccess; ++i)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &o[i], decode1_variant<2>(single, (i & 1) != 0, i < 8 && (i & 2) != 0, i < 8 && (i & 4) != 0, i >= 8),
        DK_THREADS, lds);
  occ = o[0];
  for (int i = 1; i < 10; ++i) occ = o[i] < occ ? o[i] : occ;
  return e;
}

// Launches for one token.  a.vt_end / a.nvt count V units (a.vtpu 16-rank
// tiles of a branch each).  G > 0: one launch of G workgroups (the caller has
// checked that G are resident at once, and a.vt_begin / a.ut_begin hold the
// ranges of a multi-layer call); G == 0: the two launches.
hipError_t lb_launch_decode1(const LbDecodeArgs& args, int G, void* sync, hipStream_t stream) {
  const size_t lds = lb_decode1_lds_bytes(args);
  const bool single = args.nlayers == 1;
  LbDecodeArgs a = args;
  // preloaded copies of the single layer's phase-A fields
  const LbLayerArgs& L0 = args.L[0];
  const uint8_t* vb0 = single ? L0.br[0].vbits : nullptr;
  const uint8_t* vb1 = single ? L0.br[1].vbits : nullptr;
  const uint16_t* px = single ? L0.x : nullptr;
  const uint16_t* g0 = single ? L0.br[0].g : nullptr;
  const uint16_t* g1 = single ? L0.br[1].g : nullptr;
  // n, the branches' V tile counts and the tiles per V unit ride in the
  // high bits of pre_n and pre_misc
  const int ntv0 = single ? (L0.br[0].r + 15) / 16 : 0;
  const int ntv1 = single && L0.nb == 2 ? (L0.br[1].r + 15) / 16 : 0;
  if (single && (L0.n > 0xFFFF || ntv0 > 0xFFFF || ntv1 > 0x7FFF)) return hipErrorInvalidValue;
  if (args.vtpu != 1 && args.vtpu != 2) return hipErrorInvalidValue;
  const int pn = single ? (int)((uint32_t)L0.n | ((uint32_t)ntv0 << 16)) : 0;
  uint8_t* sy = static_cast<uint8_t*>(sync);
  auto misc = [&](int vq, int vr) { return (uint32_t)vq | ((uint32_t)vr << 8) | ((uint32_t)ntv1 << 17); };
  const bool one = args.vtpu == 1;
  if (G > 0) {
    a.vq = a.nvt / G;
    a.vr = a.nvt % G;
    a.uq = a.nut / G;
    a.ur = a.nut % G;
    if (a.vq > 255 || a.vr > 255) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decode1_variant<2>(single, one, decode1_max_utiles(a, G, single) <= 4, decode1_narrow(a),
                                          decode1_max_utiles(a, G, single) <= DK_UTG - 1), dim3(G), dim3(DK_THREADS),
                       lds, stream, vb0, vb1, px, g0, g1, sy, pn, single ? misc(a.vq, a.vr) : 0u, a);
    return hipGetLastError();
  }
  a.vq = 1;
  a.vr = 0;
  a.uq = 0;
  a.ur = 0;
  hipLaunchKernelGGL(decode1_variant<0>(single, one), dim3(a.nvt), dim3(DK_THREADS), lds, stream, vb0, vb1, px, g0,
                     g1, sy, pn, single ? misc(1, 0) : 0u, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int gb = a.nut < 1024 ? a.nut : 1024;
  a.vq = 0;
  a.vr = 0;
  a.uq = a.nut / gb;
  a.ur = a.nut % gb;
  // (the U launch does no V work: one instantiation per layer count)
  hipLaunchKernelGGL(decode1_variant<1>(single, false, decode1_max_utiles(a, 0, true) <= 4, decode1_narrow(a),
                                        decode1_max_utiles(a, 0, true) <= DK_UTG - 1), dim3(gb), dim3(DK_THREADS),
                     lds, stream, vb0, vb1, px, g0, g1,
                     sy, pn, single ? misc(0, 0) : 0u, a);
  return hipGetLastError();
}
