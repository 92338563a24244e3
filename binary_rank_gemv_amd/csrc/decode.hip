// Decode path (1..16 tokens) of the LittleBit layer on gfx950 matrix cores.
//
// Per branch (explainx.ai explainer, "How it works" items 1-3):
//   u = g*x (fp16), t = sign(V)^T u, z = l*t (fp16), s = sign(U) z, y = sum_b h_b*s_b.
// Each 16-row tile of a packed factor is a stream of 16x16x32 matrix-core
// steps: tokens fill the 16 columns, the signs are expanded in registers to
// exact +-1.0 by lb16_step_operand_val (one shift and one and-or per two
// values).  Operand columns of absent tokens read the last token's data;
// those output columns are never stored, so operand loads are unconditional.
//
// One call = phase A (V pass over every 16-row tile of every sign(V)^T,
// giving z) then phase B (U pass over every 16-row output tile, giving y).
// Phase B needs all of z.  Either the phases are two launches, or one launch
// of exactly as many 512-thread workgroups as are resident at once: then z
// is stored as 64-bit words [32-bit call tag | two fp16 values] with
// device-coherent stores, and phase B polls its z words until every tag
// equals this call's tag, so there is no separate grid barrier.  The tag is
// one more than a per-workgroup call counter in the workspace header (never
// 0), read at kernel start and incremented by the workgroup as its last action
// (calls on one stream run one after another, so every workgroup reads the
// same value).  The two-launch path stores z with tag 0, so a later single
// launch never accepts its words.
// Every word a call polls is written by that same call, so a stale word could
// only pass if its address went unwritten for a multiple of 2^32 - 1 calls.  Each
// workgroup issues the loads of its phase-B sign words and row scales during
// phase A, so their latency overlaps phase A.
#include "lb_common.h"
#include "lb_sync.h"

#include <type_traits>
#include <vector>

// Phase timestamps, in an instrumented build only (-DLB_PHASE_STAMPS; the
// regular library has none of this): thread 0 of each workgroup stores the
// 100 MHz real-time counter at fixed points of a call to the device buffer
// given to littlebit_phase_stamps_multi_set, slot 16 w + i for workgroup w
// and point i (0 start, 10 / 13 / 14 pair slot 0 / 3 / 7 of the first V
// batch done, 1 phase-B loads issued, 3 V products done, 2 first V tile done,
// 9 last V tile done, 4 z copy done (the last layer entered), 5 first U
// group done, 8 / 7 a U group begun / its products issued, 6 end; each
// stamp holds its last time); lane 0 of every wave
// stores its z copy's end at slot 16 (256 + w) + wave.
#ifdef LB_PHASE_STAMPS
__device__ uint64_t* g_phase_stamps_multi;
#define LB_MSTAMP(i)                                                                 \
  do {                                                                               \
    uint64_t* sp_ = g_phase_stamps_multi;                                            \
    if (threadIdx.x == 0 && sp_) sp_[16 * blockIdx.x + (i)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define LB_MWSTAMP()                                                                 \
  do {                                                                               \
    uint64_t* sp_ = g_phase_stamps_multi;                                            \
    if ((threadIdx.x & 63) == 0 && sp_ && blockIdx.x < 256)                          \
      sp_[16 * (256 + blockIdx.x) + (threadIdx.x >> 6)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
extern "C" int littlebit_phase_stamps_multi_set(void* p) {
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_phase_stamps_multi), &p, sizeof(p));
}
#else
#define LB_MSTAMP(i) ((void)0)
#define LB_MWSTAMP() ((void)0)
#endif

#define LB_WAVES 8                    // waves per workgroup (2 per SIMD)
#define LB_THREADS (64 * LB_WAVES)
#define LB_MAXPV 8                    // V-pass pairs per wave held in registers
#define LB_MAXT 3                     // phase-B tiles whose sign words are prefetched
#define LB_MAXPW 3                    // phase-B pairs per wave held in registers (1-token kernels)
#define LB_MAXPW_MULTI 4              // the same, kernels for up to LB_MAX_BATCH tokens
#define LB_UPRE_BYTES (64 * 1024)     // LDS for a workgroup's phase-B sign bytes (single launch)
#define LB_UPRE_OPS 8                 // 1 KB global-to-LDS loads per wave filling it
#define LB_UPRE_HROWS 512             // row scales of the copied tiles (an LDS table)
// dynamic LDS a launch of that variant may take: what the static arrays
// (partial sums 24 KB, two z tiles 1 KB, the copy, the row-scale table) leave of 160 KB
#define LB_UPRE_DYN_MAX (160 * 1024 - LB_MAXT * LB_WAVES * 256 * 4 - 1024 - LB_UPRE_BYTES - 2 * LB_UPRE_HROWS)
#define LB_MAX_BATCH 16               // tokens of a decode call (phase-A kernels for 1 and for up to 16)

namespace {

// The decode kernel's explicit arguments in order, as laid out in the kernel
// argument segment (each at its natural alignment, as in a struct).
struct LbDecodeKernargs {
  const uint8_t *pre_vb0, *pre_vb1;
  const uint16_t *pre_x, *pre_g0, *pre_g1;
  int pre_n, pre_ldx, pre_vsplit;
  uint32_t pre_misc;
  LbDecodeArgs A;
  uint8_t* sync;
};

// The argument block A of the decode kernel, read through a pointer the
// compiler cannot see through, so no load of its fields is placed above the
// call.  (Taking the parameter's address instead would copy it to scratch.)
__device__ __forceinline__ const LbDecodeArgs& kernarg_barrier() {
  typedef const __attribute__((address_space(4))) char* KBytes;
  typedef const __attribute__((address_space(4))) LbDecodeArgs* KPtr;
  KPtr p = (KPtr)((KBytes)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(LbDecodeKernargs, A));
  __asm__ volatile("" : "+s"(p));
  return *(const LbDecodeArgs*)p;
}

// Flattened view of one layer: branch fields are selected with `b ? x1 : x0`
// so no per-branch array is indexed at run time.
struct LayerView {
  const uint8_t *vb0, *vb1, *ub0, *ub1;
  const uint16_t *h0, *h1, *l0, *l1, *g0, *g1;
  int r0, r1, zoff0, zoff1;
  int nb, m, n, zs;
  const uint16_t* x;
  long ldx;
  uint16_t* y;
  long ldy;
  uint64_t* z;
};

__device__ __forceinline__ LayerView layer_view(const LbLayerArgs& L) {
  LayerView v;
  v.vb0 = L.br[0].vbits; v.vb1 = L.br[1].vbits;
  v.ub0 = L.br[0].ubits; v.ub1 = L.br[1].ubits;
  v.h0 = L.br[0].h; v.h1 = L.br[1].h;
  v.l0 = L.br[0].l; v.l1 = L.br[1].l;
  v.g0 = L.br[0].g; v.g1 = L.br[1].g;
  v.r0 = L.br[0].r; v.r1 = L.br[1].r;
  v.zoff0 = L.br[0].zoff; v.zoff1 = L.br[1].zoff;
  v.nb = L.nb; v.m = L.m; v.n = L.n; v.zs = L.zs;
  v.x = L.x; v.ldx = L.ldx; v.y = L.y; v.ldy = L.ldy; v.z = L.z;
  return v;
}

// Mapping of global tile indices to layers: the cumulative tile counts are
// read from the argument block where needed (scalar loads, wave-uniform
// indices), not copied into a per-thread array the compiler could only
// index through scratch memory.
struct TileMap {
  const LbDecodeArgs* A;
};

__device__ __forceinline__ void load_map(const LbDecodeArgs& A, TileMap& M) { M.A = &A; }

// Layer of global U tile t (tile index inside the layer in `tile`).
template <bool SINGLE>
__device__ __forceinline__ int u_layer(const TileMap& M, int t, int& tile) {
  if (SINGLE) {
    tile = t;
    return 0;
  }
  const LbDecodeArgs& A = *M.A;
  int li = 0;
#pragma unroll
  for (int i = 0; i < LB_MAX_LAYERS - 1; ++i)
    if (i < A.nlayers - 1 && t >= A.ut_end[i]) li = i + 1;
  li = __builtin_amdgcn_readfirstlane(li);
  tile = t - (li > 0 ? A.ut_end[li - 1] : 0);
  return li;
}

// End (exclusive) of layer li's global U tiles.
__device__ __forceinline__ int layer_u_end(const TileMap& M, int li) {
  return M.A->ut_end[__builtin_amdgcn_readfirstlane(li)];
}

// Slot 2*layer + branch of global V tile t (one layer: `vsplit` = tiles of
// branch 0).
template <bool SINGLE>
__device__ __forceinline__ int v_slot(const TileMap& M, int vsplit, int t, int& tile) {
  if (SINGLE) {
    const int k = t >= vsplit ? 1 : 0;
    tile = t - (k ? vsplit : 0);
    return k;
  }
  const LbDecodeArgs& A = *M.A;
  int k = 0;
#pragma unroll
  for (int q = 0; q < 2 * LB_MAX_LAYERS - 1; ++q)
    if (q < 2 * A.nlayers - 1 && t >= A.vt_end[q]) k = q + 1;
  k = __builtin_amdgcn_readfirstlane(k);
  tile = t - (k > 0 ? A.vt_end[k - 1] : 0);
  return k;
}

// Contiguous share [beg, end) of part i: q items each, one more for parts < r.
__device__ inline void share(int q, int r, int i, int& beg, int& end) {
  beg = i * q + min(i, r);
  end = beg + q + (i < r ? 1 : 0);
}

// Phase-B role of wave `wave` (scalar): branch and pair range.
__device__ inline void u_role(const LayerView& L, int wave, int& b, int& p0, int& p1) {
  if (L.nb == 2) {
    b = wave >> 2;
    const int np = (lb16_units(b ? L.r1 : L.r0) + 1) >> 1, w = wave & 3;
    p0 = (np * w) >> 2;
    p1 = (np * (w + 1)) >> 2;
  } else {
    b = 0;
    const int np = (lb16_units(L.r0) + 1) >> 1;
    p0 = (np * wave) >> 3;
    p1 = (np * (wave + 1)) >> 3;
  }
}

// ------------------------------------------------------------------ phase A
// One 16-row tile of sign(V)^T of branch b of layer L: t = sum_k s_k g_k x_k
// per token, then z = fp16(l*t), stored as tagged words.  The matrix core
// forms each product g_k x_k exactly: its A operand is +-g_k (g's fp16 sign
// bit flipped by the weight's sign bit, as in the prefill GEMMs) and its B
// operand the token's x, so no scaled copy of x is made.  Wave w sums pairs
// w, w + 8, w + 16, ... (128 inputs each, four 32-input matrix steps), in
// order; the sign words of a batch of LB_WAVES * LB_MAXPV pairs are loaded
// together.  Every lane loads its own token's x (and a share of g) of a pair
// straight into the operand registers, two pairs ahead of the products: x
// is read once per workgroup and nothing is staged in LDS.
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Geometry of this thread's part of the V pass over one 16-row tile of
// branch b of layer L.
struct VGeom {
  const uint16_t* x;        // token t's activations at x + t * ldx
  const uint16_t* g;
  const uint8_t* tile_ptr;  // the tile's packed sign words
  long ldx;
  int n, nu, np;
};

// Reads only the fields a caller may know before the rest of the arguments:
// the factor's sign words (vb0, vb1), x, ldx, g0, g1 and n.
__device__ __forceinline__ VGeom v_geom(const LayerView& L, int b, int tile) {
  VGeom G;
  G.n = L.n;
  G.g = b ? L.g1 : L.g0;
  G.nu = lb16_units(G.n);
  G.np = (G.nu + 1) >> 1;
  G.tile_ptr = (b ? L.vb1 : L.vb0) + (long)tile * lb16_tile_bytes(G.n);
  G.x = L.x;
  G.ldx = L.ldx;
  return G;
}

// Inputs k..k+7 of a row of x or of g: with 16-byte loads (FAST: x 16-byte
// aligned, ldx and n multiples of 8, so a group of 8 inputs lies wholly below
// n or wholly at/after it) from an always-valid address, zeroed by the
// caller when k >= n; else one by one, zero at and beyond n.  FAST is a
// template argument of the kernel, chosen by the host: as a run-time flag
// both forms sat around every load, and the compiler's waits at their joins
// took no account of the loads issued ahead.
template <bool FAST>
__device__ __forceinline__ uint4 v_load8(const VGeom& G, const uint16_t* row, int k) {
  if (FAST) return *reinterpret_cast<const uint4*>(row + min(k, G.n - 8));
  uint16_t e8[8];
  for (int e = 0; e < 8; ++e) e8[e] = (k + e < G.n) ? row[k + e] : (uint16_t)0;
  return *reinterpret_cast<uint4*>(e8);
}

// One pair's operands of this lane: its token's x (B operands of the four
// steps, inputs 128 p + 32 s + 8 grp .. + 7 of step s) and one 32-bit pair
// of g.  Lane r of row grp holds g of inputs 128 p + 32 (r / 4) + 8 grp +
// 2 (r % 4) and + 1, i.e. dword r % 4 of step r / 4 of its row's operand, so
// each g value is loaded once per wave and reaches the lanes of its row by
// a row broadcast (v_pair_g); loading every lane's operand would move 16
// times the bytes of g through the L1 cache, as much as x itself.
struct VPairAct {
  uint4 x[4];
  uint32_t g;
};

// Loads pair p's operands (token row `trow`).  Unconditional (a pair past
// the share is loaded from the clamped pair, never used), so wait counts stay
// exact; g at and beyond n reads as zero.
template <bool FAST>
__device__ __forceinline__ void v_load_pair(const VGeom& G, int p, int trow, VPairAct& a) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, r = lane & 15;
  const uint16_t* xr = G.x + (long)trow * G.ldx;
#pragma unroll
  for (int s = 0; s < 4; ++s) a.x[s] = v_load8<FAST>(G, xr, 128 * p + 32 * s + 8 * grp);
  const int kg = 128 * p + 32 * (r >> 2) + 8 * grp + 2 * (r & 3);
  if (FAST) {
    // n % 8 == 0: both inputs of the pair lie below n or neither does
    const uint32_t v = *reinterpret_cast<const uint32_t*>(G.g + min(kg, G.n - 2));
    a.g = kg < G.n ? v : 0u;
  } else {
    const uint32_t lo = kg < G.n ? G.g[kg] : 0u, hi = kg + 1 < G.n ? G.g[kg + 1] : 0u;
    a.g = lo | (hi << 16);
  }
}

// Dword dd (inputs 2 dd, 2 dd + 1 of the lane's 8) of step S's g operand:
// from lane 4 S + dd of the row (every lane of the row is written, so the
// move needs no prior value).
template <int S>
__device__ __forceinline__ u32x4 v_pair_g(uint32_t gw) {
  u32x4 q;
  q[0] = (uint32_t)__builtin_amdgcn_mov_dpp((int)gw, 0x150 + 4 * S + 0, 0xF, 0xF, false);
  q[1] = (uint32_t)__builtin_amdgcn_mov_dpp((int)gw, 0x150 + 4 * S + 1, 0xF, 0xF, false);
  q[2] = (uint32_t)__builtin_amdgcn_mov_dpp((int)gw, 0x150 + 4 * S + 2, 0xF, 0xF, false);
  q[3] = (uint32_t)__builtin_amdgcn_mov_dpp((int)gw, 0x150 + 4 * S + 3, 0xF, 0xF, false);
  return q;
}

// The loads that open a batch of V pairs starting at pair wb of a tile: the
// wave's sign words (pair wb + wave + 8 i in slot i), then its first pair's
// operands.
struct VLoads {
  uint32_t words[LB_MAXPV];
  VPairAct act;
};

template <bool FAST>
__device__ __forceinline__ void v_issue(const VGeom& G, int wb, int batch, VLoads& R) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  // unconditional loads (clamped to the tile's last pair) keep the wait
  // counts exact; slots beyond the tile are never used
#pragma unroll
  for (int i = 0; i < LB_MAXPV; ++i)
    R.words[i] = lb16_load_pair(G.tile_ptr, min(wb + wave + 8 * i, G.np - 1), lane, G.nu);
  v_load_pair<FAST>(G, min(wb + wave, G.np - 1), min(lane & 15, batch - 1), R.act);
}

// Stores one V tile's z (zstage: [token][16 rows] fp16, in LDS) as tagged
// words [tag | z(2q) | z(2q+1)], 8 words per token for the 16 rows; the
// branch's last tile also writes the zero words between 16*ceil(r/16) and
// 64*ceil(r/64).
__device__ __forceinline__ void v_store_z(const LayerView& L, int batch, int b, int tile, uint32_t tag,
                                          const uint32_t* zstage) {
  const int tid = threadIdx.x;
  const int r = b ? L.r1 : L.r0;
  uint64_t* __restrict__ zw = L.z;
  const int zrow = L.zs >> 1, zoff = (b ? L.zoff1 : L.zoff0) >> 1;
  if (tid < 8 * batch) {
    const int q = tid & 7, tt = tid >> 3;
    const uint32_t v = zstage[tt * 8 + q];
    st64c(zw + (long)tt * zrow + zoff + 8 * tile + q, (uint64_t)tag | ((uint64_t)v << 32));
  }
  const int ntv = (r + 15) >> 4;
  if (tile == ntv - 1) {
    const int w0 = 8 * ntv, w1 = 32 * lb16_units(r);
    const int nw = w1 - w0;
    for (int i = tid; i < nw * batch; i += LB_THREADS) {
      const int tt = i / nw, ww = w0 + i % nw;
      st64c(zw + (long)tt * zrow + zoff + ww, (uint64_t)tag);
    }
  }
}

// V pass over one 16-row tile of branch b of layer L, then z = l*t of the
// tile's rows stored as tagged words.  R holds the first batch's loads
// (v_issue with this geometry, issued by the caller: EARLY, or here).
// HOOK: hook() runs after the last pair's loads are issued (its loads then
// queue behind this tile's, which complete first).  DEFER: z is left in
// zstage for the caller to store (v_store_z).
template <int MAXB, bool FAST, bool HOOK, bool EARLY, bool DEFER = false, class Hook>
__device__ __forceinline__ void v_tile(const LayerView& L, int batch, int b, int tile, const uint32_t& tag,
                                       const LbSignConsts& sc, float (*red)[256], uint32_t* zstage, Hook&& hook,
                                       const VLoads& early) {
  const VGeom G = v_geom(L, b, tile);
  const int np = G.np, nu = G.nu;
  const int r = b ? L.r1 : L.r0;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int tok = lane & 15, grp = lane >> 4;
  const int trow = min(tok, batch - 1);      // operand row read by this lane
  const int rho = tid & 15, tk = (tid >> 4) & 15;  // epilogue role (threads < 256)
  const int j = 16 * tile + rho;
  // l[j] (from an always-valid index; converted at use in the epilogue)
  const uint32_t lj_raw = (b ? L.l1 : L.l0)[min(j, r - 1)];

  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  // the products of one pair: A = +-g (sign bit of the weight xor that of
  // g), B = x, four steps alternating between two accumulators
  auto step = [&](auto S, uint32_t reg, const uint4& x, uint32_t gw) {
    constexpr int s = decltype(S)::value;
    const u32x4 gq = v_pair_g<s>(gw);
    u32x4 d;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) d[dd] = ((reg << (4 * s + dd)) & sc.sign_mask) ^ gq[dd];
    f32x4& ac = (s & 1) ? acc1 : acc;
    ac = mfma16(__builtin_bit_cast(f16x8, d), __builtin_bit_cast(f16x8, x), ac);
  };
  auto pair_products = [&](uint32_t word, int p, const VPairAct& a) {
    // Inputs at and beyond n: g reads as zero there, so their A operands are
    // +-0 and their products vanish (x itself came from a clamped, valid
    // address: finite activations, as the layer's inputs are).
    // late(): the expansion is not hoisted above this point (it would hold
    // registers and wait for the load early)
    const uint32_t reg = lb16_reg_word(late(word), lb16_pair_sel(p, lane, nu));
    const uint32_t gw = late(a.g);
    step(std::integral_constant<int, 0>(), reg, a.x[0], gw);
    step(std::integral_constant<int, 1>(), reg, a.x[1], gw);
    step(std::integral_constant<int, 2>(), reg, a.x[2], gw);
    step(std::integral_constant<int, 3>(), reg, a.x[3], gw);
  };
  constexpr int WB = LB_WAVES * LB_MAXPV;
  VLoads R;
  if constexpr (EARLY) R = early;
  else v_issue<FAST>(G, 0, batch, R);
  for (int wb = 0; wb < np; wb += WB) {
    if (wb != 0) v_issue<FAST>(G, wb, batch, R);
    // operands two pairs ahead of the products (8 KB per wave in flight)
    VPairAct cur = R.act, nx1;
    v_load_pair<FAST>(G, min(wb + wave + 8, np - 1), trow, nx1);
    const int pend = min(np, wb + WB);
#pragma unroll
    for (int i = 0; i < LB_MAXPV; ++i) {
      const int p = wb + wave + 8 * i;
      // the operands of the pair after next first (clamped: always issued)
      VPairAct nx2;
      v_load_pair<FAST>(G, min(p + 16, np - 1), trow, nx2);
      if (p < pend) pair_products(R.words[i], p, cur);
      if (wb == 0 && i == 0) LB_MSTAMP(10);
      if (wb == 0 && i == 3) LB_MSTAMP(13);
      if (wb == 0 && i == 7) LB_MSTAMP(14);
      cur = nx1;
      nx1 = nx2;
    }
  }
  if constexpr (HOOK) {
    hook();
    LB_MSTAMP(1);
  }
  acc += acc1;
  LB_MSTAMP(3);

#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(4 * grp + i) * 16 + tok] = acc[i];
  __syncthreads();

  if (tid < 256) {
    const int e = rho * 16 + tk;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < LB_WAVES; ++w) t += red[w][e];
    const f16 zv = (j < r) ? (f16)(h2f((uint16_t)late(lj_raw)) * t) : (f16)0.f;
    reinterpret_cast<uint16_t*>(zstage)[tk * 16 + rho] = __builtin_bit_cast(uint16_t, zv);
  }
  __syncthreads();
  if constexpr (!DEFER) v_store_z(L, batch, b, tile, late(tag), zstage);
}

// ------------------------------------------------------------------ phase B
// Prefetched per-tile data: this wave's sign words.
template <int NPW>
struct UTilePre {
  uint32_t w[NPW];
};

// Row scales (h of both branches, fp16 bits: converting here would wait for
// the load) of the two epilogue entries of a thread in a tile group: entry j
// belongs to tile (wave >> 2) + 2 j of the group and row (tid & 15).
struct HPre {
  uint32_t h0[2], h1[2];
};

// Loads entry j's row scales: row 16*tile + (tid & 15) of layer L (a row
// beyond m loads row m - 1; such entries are never stored).
__device__ __forceinline__ void load_h(const LayerView& L, int tile, HPre& H, int j) {
  const int i = min(16 * tile + (int)(threadIdx.x & 15), L.m - 1);
  H.h0[j] = L.h0[i];
  H.h1[j] = (L.nb == 2 ? L.h1 : L.h0)[i];
}

template <int NPW>
__device__ __forceinline__ void u_prefetch(const LayerView& L, int tile, UTilePre<NPW>& P) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  int b, p0, p1;
  u_role(L, wave, b, p0, p1);
  const int r = b ? L.r1 : L.r0;
  const int nu = lb16_units(r);
  const uint8_t* tp = (b ? L.ub1 : L.ub0) + (long)tile * lb16_tile_bytes(r);
  const int plast = max(p1 - 1, 0);
#pragma unroll
  for (int i = 0; i < NPW; ++i) P.w[i] = lb16_load_pair(tp, min(p0 + i, plast), lane, nu);
}

// Phase-B role of a wave for the layer whose z is staged in LDS.
struct UState {
  int li;              // layer whose z is in LDS (-1: none)
  int b, p0, p1, nu;
};

// 16-byte loads per lane in flight per pass of the z poll: 24 at larger
// batches, 8 (fewer registers to set up) when the range is at most that
#define LB_POLL_LOADS 24
#define LB_POLL_LOADS_SMALL 8
#define LB_POLL_LOADS_MULTI 32  // multi-token kernels

// Copies the steps [s0, s1) of a wave's range of layer L's z into LDS (zl:
// [token][zs + 8] fp16), polling (check) until every word carries this call's
// tag.  The range (128 bytes per step and token) is cut into 16-byte chunks
// (two tagged words, four values) dealt to the lanes in order: chunk
// lane + 64 j is load j of the lane, so no two lanes load the same bytes (at
// batch 1 a range of 12 steps is two loads per lane).  Up to NL loads per
// lane are issued before any result is examined, so a pass costs one
// memory round trip; a later pass re-reads only the loads whose chunks were
// not all tagged.  A wave later reads only the range it copied, so no barrier
// follows the copy; the barrier in front keeps the previous layer's readers
// safe.
template <int NL>
__device__ __forceinline__ void u_copy_z(const LayerView& L, int batch, uint32_t tag, bool check, uint8_t* sync,
                                         const UState& S, uint16_t* zl, int s0, int s1) {
  const int lane = threadIdx.x & 63;
  const int zoff = S.b ? L.zoff1 : L.zoff0;
  const int oob = batch * L.zs * 4;  // a load at this offset returns zeros and marks an idle lane
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(L.z, oob);
  const int per_tok = 8 * (s1 - s0);              // chunks per token
  const int nload = (batch * per_tok + 63) >> 6;  // loads per lane
  // position of this lane's next chunk: token t, chunk w of the token, and
  // its byte offset in z (g) and element offset in zl (l).  A load moves 64
  // chunks on: dq tokens and dr chunks, with a carry into the next token when
  // the chunk index passes per_tok.
  int t = 0, w = lane;
  while (w >= per_tok) {
    w -= per_tok;
    ++t;
  }
  const int dq = 64 / per_tok, dr = 64 - dq * per_tok;
  const int zsb = 4 * L.zs, zsl = L.zs + 8;
  int g = t * zsb + 4 * zoff + 128 * s0 + 16 * w;
  int l = t * zsl + zoff + 32 * s0 + 4 * w;
  const int dg = dq * zsb + 16 * dr, dl = dq * zsl + 4 * dr;
  const int cg = zsb - 16 * per_tok, cl = zsl - 4 * per_tok;  // the carry's offset changes
  for (int jb = 0; jb < nload; jb += NL) {
    const int nj = min(NL, nload - jb);
    int goff[NL], loff[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if (i < nj) {
        goff[i] = t < batch ? g : oob;
        loff[i] = l;
        w += dr;
        t += dq;
        g += dg;
        l += dl;
        if (w >= per_tok) {
          w -= per_tok;
          ++t;
          g += cg;
          l += cl;
        }
      }
    }
    static_assert(NL <= 32, "one bit per load");
    uint32_t todo = nj >= 32 ? ~0u : (1u << nj) - 1u;  // loads of this batch still to read
    u32x4 q[NL];
    int spins = 0;
    for (;;) {
      compiler_memory_barrier();  // every pass re-reads the words
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (todo & (1u << i)) q[i] = ld_tagged2(rs, goff[i]);
      if (check) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          if (todo & (1u << i)) {
            const bool ok = (goff[i] == oob) | ((q[i][0] == tag) & (q[i][2] == tag));
            if (__all(ok)) todo &= ~(1u << i);
          }
        }
      } else {
        todo = 0;
      }
      if (todo == 0) break;
      if (++spins > LB_SPIN_LIMIT) {
        st32c(sync + LB_SYNC_ERR, 1u);
        break;
      }
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if (i < nj && goff[i] != oob) {
        uint2 d;
        d.x = q[i][1];
        d.y = q[i][3];
        *reinterpret_cast<uint2*>(zl + loff[i]) = d;
      }
    }
  }
}

// Copies this wave's range of layer L's z into LDS (u_copy_z), after taking
// the wave's phase-B role for the layer.  NLB: loads per lane per pass for a
// large range (the multi-token kernels take more, so 16 tokens of a 4-pair
// range need one pass batch, not two).
template <int NLB = LB_POLL_LOADS>
__device__ __forceinline__ void u_enter_layer(const LayerView& L, int li, int batch, uint32_t tag, bool check,
                                              uint8_t* sync, UState& S, uint16_t* zl) {
  const int wave = wave_id();
  tag = late(tag);
  __syncthreads();  // earlier readers of zl (previous layer, or phase A's u) are done
  S.li = li;
  u_role(L, wave, S.b, S.p0, S.p1);
  S.nu = lb16_units(S.b ? L.r1 : L.r0);
  const int s0 = 4 * S.p0;
  const int s1 = min(4 * S.p1, 2 * S.nu);  // steps of this wave's range that hold data
  if (s1 <= s0) return;
  // without polling (z written by an earlier launch) a pass never repeats, so
  // the small variant (batches of loads one after another) is enough
  if (!check || batch * 8 * (s1 - s0) <= 64 * LB_POLL_LOADS_SMALL)
    u_copy_z<LB_POLL_LOADS_SMALL>(L, batch, tag, check, sync, S, zl, s0, s1);
  else
    u_copy_z<NLB>(L, batch, tag, check, sync, S, zl, s0, s1);
  LB_MSTAMP(4);
  LB_MWSTAMP();
}

// ---------------------------------------------- phase-B sign bytes in LDS
// A workgroup's U tiles [ut0, ut1) are, per layer and branch, one contiguous
// run of packed bytes.  The single launch copies the runs of (at most) its
// first two layers into LDS while phase A runs: a stream of up to
// LB_UPRE_BYTES, cut into 1 KB global-to-LDS loads, LB_UPRE_OPS per wave, a
// fixed count (loads past the stream's end repeat its last 16 bytes into
// unused LDS), so the compiler's wait counts stay exact.  Tiles [ut0, cover)
// are in LDS; a tile's bytes keep the global layout (pair p at 256 p, an odd
// last unit alone at 256 (NU/2), 2 bytes per lane).
struct UPrePlan {
  int split;    // first global tile of the second layer (ut1 when none)
  int cover;    // tiles [ut0, cover) are in LDS
  int off[4];   // LDS byte offset of run (layer slot s, branch b) = 2 s + b
};

__device__ __forceinline__ int tile_bytes_b(const LayerView& L, int b) {
  return (int)lb16_tile_bytes(b ? L.r1 : L.r0);
}

// Plans and issues the copy (all values wave-uniform but the addresses), and
// loads this thread's row scale for the LDS table of the covered tiles:
// thread (local tile tid / 32, branch (tid / 16) % 2, row tid % 16).
template <bool SINGLE>
__device__ __forceinline__ void upre_issue(const LbDecodeArgs& A, const TileMap& M, int ut0, int ut1,
                                           int max_tiles, uint8_t* lds, UPrePlan& P, uint32_t& hval) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  int tile0;
  const int li0 = u_layer<SINGLE>(M, min(ut0, A.nut - 1), tile0);
  const int end0 = SINGLE ? ut1 : min(ut1, layer_u_end(M, li0));
  const int li1 = SINGLE ? li0 : min(li0 + 1, A.nlayers - 1);
  const int end1 = SINGLE ? ut1 : min(ut1, layer_u_end(M, li1));
  const LayerView L0 = layer_view(A.L[li0]);
  const LayerView L1 = layer_view(A.L[li1]);
  // whole tiles, as many as fit: the first layer's, then the second's
  const int pt0 = tile_bytes_b(L0, 0) + (L0.nb == 2 ? tile_bytes_b(L0, 1) : 0);
  const int pt1 = tile_bytes_b(L1, 0) + (L1.nb == 2 ? tile_bytes_b(L1, 1) : 0);
  const int n0a = max(end0 - ut0, 0), n1a = (SINGLE || li1 == li0) ? 0 : max(end1 - end0, 0);
  const int n0 = min(min(n0a, max_tiles), LB_UPRE_BYTES / pt0);
  const int n1 = n0 < n0a ? 0 : min(min(n1a, max_tiles - n0), (LB_UPRE_BYTES - n0 * pt0) / pt1);
  const int b00 = n0 * tile_bytes_b(L0, 0), b01 = L0.nb == 2 ? n0 * tile_bytes_b(L0, 1) : 0;
  const int b10 = n1 * tile_bytes_b(L1, 0), b11 = L1.nb == 2 ? n1 * tile_bytes_b(L1, 1) : 0;
  const int total = b00 + b01 + b10 + b11;
  P.split = end0;
  P.cover = n1 > 0 ? end0 + n1 : ut0 + n0;
  P.off[0] = 0;
  P.off[1] = b00;
  P.off[2] = b00 + b01;
  P.off[3] = b00 + b01 + b10;
  const uint8_t* src0 = L0.ub0 + (long)tile0 * tile_bytes_b(L0, 0);
  const uint8_t* src1 = (L0.nb == 2 ? L0.ub1 : L0.ub0) + (long)tile0 * tile_bytes_b(L0, L0.nb == 2 ? 1 : 0);
  const uint8_t* src2 = L1.ub0;
  const uint8_t* src3 = L1.nb == 2 ? L1.ub1 : L1.ub0;
#pragma unroll
  for (int j = 0; j < LB_UPRE_OPS; ++j) {
    const int i = wave * LB_UPRE_OPS + j;
    // stream offset of this lane's 16 bytes (past the end: the last 16)
    const int o = min(1024 * i + 16 * lane, max(total - 16, 0));
    const uint8_t* src = o >= P.off[3] && P.off[3] < total ? src3 + (o - P.off[3])
                         : o >= P.off[2] && P.off[2] < total ? src2 + (o - P.off[2])
                         : o >= P.off[1] && P.off[1] < total ? src1 + (o - P.off[1])
                                                              : src0 + o;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds + 1024 * i), 16, 0, 0);
  }
  {
    // row scale (an always-valid row: tiles past the covered ones load row 0)
    const int tid = threadIdx.x;
    const int t = ut0 + (tid >> 5), hb = (tid >> 4) & 1;
    const bool in = t < P.cover;
    const bool second = t >= P.split;
    const LayerView& L = second ? L1 : L0;
    const int tl = in ? (second ? t - P.split : tile0 + t - ut0) : 0;
    const uint16_t* h = (hb && L.nb == 2) ? L.h1 : L.h0;
    hval = h[min(16 * tl + (tid & 15), L.m - 1)];
  }
}

// The fp16 outputs an epilogue thread still has to store (p == nullptr: none).
// Stores are held back until the next group's sign words are requested: a
// store counts in the same in-order counter as the loads, so a wait for a
// later load would also wait for the store to reach memory.
struct YOut {
  uint16_t* p[2];
  uint16_t v[2];
};

__device__ __forceinline__ void store_y(const YOut& o) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (o.p[j]) *o.p[j] = o.v[j];
}

// Cross-wave sums of nt <= LB_MAXT tiles' accumulators and the epilogue:
// y = sum_b h_b * s_b for the entries of this thread (stores held back).
__device__ __forceinline__ YOut u_finish(const LayerView& L, int batch, int tile0, int nt, const f32x4 (&acc)[LB_MAXT],
                                         const HPre& H, float (*red)[LB_WAVES][256]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int tok = lane & 15, grp = lane >> 4;
  __syncthreads();  // previous users of red are done
#pragma unroll
  for (int k = 0; k < LB_MAXT; ++k)
    if (k < nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[k][wave][(4 * grp + q) * 16 + tok] = acc[k][q];
  __syncthreads();

  // thread tid finishes entries tid and tid + 512 of (tile, row, token); its
  // row 16*tile + (tid & 15) is the one whose scales it prefetched
  static_assert(LB_MAXT == 3 && LB_THREADS == 512, "epilogue mapping");
  const int rho = tid & 15, tk = (tid >> 4) & 15;
  YOut out;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    out.p[j] = nullptr;
    out.v[j] = 0;
    const int k = (wave >> 2) + 2 * j;  // tile of entry tid + 512 j (wave-uniform)
    const int i = 16 * (tile0 + k) + rho;
    if (k < nt && tk < batch && i < L.m) {
      const int e = rho * 16 + tk;
      const uint32_t h0 = H.h0[j], h1 = H.h1[j];
      float y;
      if (L.nb == 2) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int w = 0; w < LB_WAVES / 2; ++w) {
          s0 += red[k][w][e];
          s1 += red[k][w + LB_WAVES / 2][e];
        }
        y = fmaf(h2f((uint16_t)late(h0)), s0, h2f((uint16_t)late(h1)) * s1);  // one rounding order in every path
      } else {
        float s0 = 0.f;
#pragma unroll
        for (int w = 0; w < LB_WAVES; ++w) s0 += red[k][w][e];
        y = h2f((uint16_t)late(h0)) * s0;
      }
      out.p[j] = L.y + (long)tk * L.ldy + i;
      out.v[j] = f2h(y);
    }
  }
  return out;
}


// Phase B for nt <= LB_MAXT consecutive U tiles (from tile0) of layer L, whose
// sign words and row scales are in P[0..nt): the matrix steps of all tiles
// run interleaved, then one epilogue (one pair of barriers) finishes them all.
// NPW pairs per wave are in registers; any further pairs are loaded here.
template <int NPW>
__device__ __forceinline__ YOut u_group(const LayerView& L, int li, int batch, int tile0, int nt,
                                        const UTilePre<NPW> (&P)[LB_MAXT], const HPre& H, uint32_t tag, bool check,
                                        uint8_t* sync,
                                        const LbSignConsts& sc, UState& S, uint16_t* zl,
                                        float (*red)[LB_WAVES][256]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int tok = lane & 15, grp = lane >> 4;
  if (li != S.li) u_enter_layer<(NPW == LB_MAXPW ? LB_POLL_LOADS : LB_POLL_LOADS_MULTI)>(L, li, batch, tag, check, sync, S, zl);
  LB_MSTAMP(8);
  // operand rows: absent tokens read the last token's row (never stored)
  const uint16_t* zb = zl + min(tok, batch - 1) * (L.zs + 8) + (S.b ? L.zoff1 : L.zoff0) + 8 * grp;
  const int s1 = 2 * S.nu;  // steps of the branch that hold data

  f32x4 acc[LB_MAXT];
#pragma unroll
  for (int k = 0; k < LB_MAXT; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int p = S.p0 + i;
    if (p < S.p1) {
      const uint32_t sel = lb16_pair_sel(p, lane, S.nu);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (4 * p + st < s1) {  // an odd last unit has two steps
          const f16x8 bv = *reinterpret_cast<const f16x8*>(zb + 32 * (4 * p + st));
#pragma unroll
          for (int k = 0; k < LB_MAXT; ++k) {
            if (k < nt) {
              // late(): the expansion is not hoisted above this point
              const uint32_t reg = lb16_reg_word(late(P[k].w[i]), sel);
              acc[k] = mfma16(lb16_step_operand_val(reg, st, sc.sign_mask, sc.one_pair), bv, acc[k]);
            }
          }
        }
      }
    }
  }
  // pairs beyond the register window (ranks above 64 * 4 * NPW per wave)
  if (S.p1 > S.p0 + NPW) {
    const int r = S.b ? L.r1 : L.r0;
    for (int p = S.p0 + NPW; p < S.p1; ++p) {
      const uint32_t sel = lb16_pair_sel(p, lane, S.nu);
      uint32_t w[LB_MAXT];
#pragma unroll
      for (int k = 0; k < LB_MAXT; ++k) {
        const uint8_t* tp = (S.b ? L.ub1 : L.ub0) + (long)(tile0 + min(k, nt - 1)) * lb16_tile_bytes(r);
        w[k] = lb16_load_pair(tp, p, lane, S.nu);
      }
      for (int st = 0; st < 4; ++st) {
        if (4 * p + st < s1) {
          const f16x8 bv = *reinterpret_cast<const f16x8*>(zb + 32 * (4 * p + st));
#pragma unroll
          for (int k = 0; k < LB_MAXT; ++k) {
            if (k < nt) {
              const uint32_t reg = lb16_reg_word(w[k], sel);
              acc[k] = mfma16(lb16_step_operand_val(reg, st, sc.sign_mask, sc.one_pair), bv, acc[k]);
            }
          }
        }
      }
    }
  }
  LB_MSTAMP(7);
  return u_finish(L, batch, tile0, nt, acc, H, red);
}

// Phase B for the copied tiles [tile0, tile0 + T) of layer L (T <= span_max,
// their sign bytes in LDS: w0/w1 = tile tile0's bytes of branch 0/1, tb0/tb1
// = bytes per tile; their row scales in hl: 32 per tile, branch 0 then 1).
// Each wave runs its pair range (u_role) over every tile, four tiles at a
// time, and leaves its sums in `part` ([wave][tile][row][token], no barrier);
// one barrier, then every output is y = h_0 * (sum over branch-0 waves) +
// h_1 * (sum over branch-1 waves), the sums taken in wave order as in u_group.
// NLB: as for u_enter_layer.
template <int NLB>
__device__ __forceinline__ void u_span_lds(const LayerView& L, int li, int batch, int tile0, int T, int span_max,
                                           const uint8_t* w0, const uint8_t* w1, int tb0, int tb1, const uint16_t* hl,
                                           uint32_t tag, bool check, uint8_t* sync, const LbSignConsts& sc, UState& S,
                                           uint16_t* zl, float* part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int tok = lane & 15, grp = lane >> 4;
  if (li != S.li) u_enter_layer<NLB>(L, li, batch, tag, check, sync, S, zl);
  const uint16_t* zb = zl + min(tok, batch - 1) * (L.zs + 8) + (S.b ? L.zoff1 : L.zoff0) + 8 * grp;
  const int s1 = 2 * S.nu;  // steps of the branch that hold data
  const uint8_t* wb = S.b ? w1 : w0;
  const int tb = S.b ? tb1 : tb0;
  for (int k0 = 0; k0 < T; k0 += 4) {
    f32x4 acc[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p = S.p0; p < S.p1; ++p) {
      const uint32_t sel = lb16_pair_sel(p, lane, S.nu);
      const int woff = 256 * p + ((2 * p + 1 < S.nu) ? 4 * lane : 4 * (lane >> 1));
      uint32_t reg[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        reg[kk] = lb16_reg_word(*reinterpret_cast<const uint32_t*>(wb + min(k0 + kk, T - 1) * tb + woff), sel);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (4 * p + st < s1) {  // an odd last unit has two steps
          const f16x8 bv = *reinterpret_cast<const f16x8*>(zb + 32 * (4 * p + st));
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            if (k0 + kk < T)
              acc[kk] = mfma16(lb16_step_operand_val(reg[kk], st, sc.sign_mask, sc.one_pair), bv, acc[kk]);
        }
      }
    }
    if (tok < batch) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        if (k0 + kk < T)
#pragma unroll
          for (int q = 0; q < 4; ++q) part[((wave * span_max + k0 + kk) * 16 + 4 * grp + q) * batch + tok] = acc[kk][q];
    }
  }
  __syncthreads();
  const int nout = T * 16 * batch;
  for (int e = tid; e < nout; e += LB_THREADS) {
    const int k = e / (16 * batch), rem = e - k * 16 * batch;
    const int row = rem / batch, tk = rem - row * batch;
    const int i = 16 * (tile0 + k) + row;
    if (i >= L.m) continue;
    const int o = (k * 16 + row) * batch + tk, ws = span_max * 16 * batch;
    float y;
    if (L.nb == 2) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int w = 0; w < LB_WAVES / 2; ++w) {
        a0 += part[w * ws + o];
        a1 += part[(w + LB_WAVES / 2) * ws + o];
      }
      y = fmaf(h2f(hl[32 * k + row]), a0, h2f(hl[32 * k + 16 + row]) * a1);
    } else {
      float a0 = 0.f;
#pragma unroll
      for (int w = 0; w < LB_WAVES; ++w) a0 += part[w * ws + o];
      y = h2f(hl[32 * k + row]) * a0;
    }
    L.y[(long)tk * L.ldy + i] = f2h(y);
  }
}

}  // namespace

// -------------------------------------------------------------- kernels

// MODE 0: phase A only; 1: phase B only; 2: both in one launch (z tagged and
// polled).  SINGLE: one layer.  Workgroup w takes a contiguous range of the V
// tiles and of the U tiles.  MAXB: the most tokens a phase A handles
// (LB_MAX_BATCH; calls of one token run decode1.hip's kernels); the
// phase-B-only kernel (MODE 1) takes any batch with the default.
//
// The leading arguments are preloaded into scalar registers by the dispatch
// (kernel-argument preloading), so a single-layer kernel issues its first
// sign-word and activation loads without waiting for a kernel-argument fetch.
// They repeat fields of A.L[0]; the multi-layer kernel ignores them.
//   misc = vq | vr << 8 | batch << 16  (V tiles of
//          workgroup w: vq + (w < vr), contiguous)
template <int MODE, bool SINGLE, bool UPRE, int MAXB = 1, bool FAST = true>
__global__ __launch_bounds__(LB_THREADS) void lb_decode_kernel(
    const uint8_t* pre_vb0, const uint8_t* pre_vb1, const uint16_t* pre_x, const uint16_t* pre_g0,
    const uint16_t* pre_g1, int pre_n, int pre_ldx, int pre_vsplit, uint32_t pre_misc,
    LbDecodeArgs, uint8_t* sync) {
  extern __shared__ __align__(16) uint16_t u_lds[];
  __shared__ __align__(16) float red[LB_MAXT][LB_WAVES][256];  // cross-wave partial sums
  // z of a V tile (16 tokens x 16 rows of fp16); two, so a multi-layer
  // launch stores a tile's z during the next tile
  __shared__ __align__(16) uint32_t zst[2][128];
  uint32_t* zstage = zst[0];
  __shared__ __align__(16) uint8_t upre_lds[UPRE ? LB_UPRE_BYTES : 16];  // phase-B sign bytes
  __shared__ uint16_t hl_lds[UPRE ? LB_UPRE_HROWS : 1];                  // and row scales
  static_assert(!UPRE || MODE == 2, "the sign-byte copy belongs to the single launch");

  const int wg = blockIdx.x;
  LB_MSTAMP(0);
  // single launch of one layer: the first V tile's first loads need only the
  // preloaded arguments, so they are issued before anything else
  constexpr bool EARLY = SINGLE && MODE == 2;
  VLoads early;
  int vt0 = 0, vt1 = 0;
  if (SINGLE) {
    share((int)(pre_misc & 255u), (int)((pre_misc >> 8) & 255u), wg, vt0, vt1);
    if (EARLY && vt0 < vt1) {
      LayerView P;  // the fields v_geom reads
      P.vb0 = pre_vb0;
      P.vb1 = pre_vb1;
      P.x = pre_x;
      P.g0 = pre_g0;
      P.g1 = pre_g1;
      P.n = pre_n;
      P.ldx = pre_ldx;
      const int b = vt0 >= pre_vsplit ? 1 : 0;
      v_issue<FAST>(v_geom(P, b, vt0 - (b ? pre_vsplit : 0)), 0, (int)((pre_misc >> 16) & 31u), early);
    }
  }
  // the remaining arguments are read from here on (their loads, and register
  // spills that wait for them, stay behind the loads above)
  const LbDecodeArgs& A = kernarg_barrier();
  const int batch = SINGLE ? (int)((pre_misc >> 16) & 31u) : A.batch;
  const LbSignConsts sc = lb16_sign_consts();
  TileMap M;
  load_map(A, M);
  LayerView V0;
  if (SINGLE) {
    V0 = layer_view(A.L[0]);
    V0.vb0 = pre_vb0;
    V0.vb1 = pre_vb1;
    V0.x = pre_x;
    V0.g0 = pre_g0;
    V0.g1 = pre_g1;
    V0.n = pre_n;
    V0.ldx = pre_ldx;
  }

  int ut0 = 0, ut1 = 0;
  if (!SINGLE) {
    if (MODE == 2) {
      vt0 = A.vt_begin[wg];
      vt1 = A.vt_begin[wg + 1];
    } else {
      share(A.vq, A.vr, wg, vt0, vt1);
    }
  }
  if (MODE == 1) vt1 = vt0;
  // this call's z tag (single launch only): call_tag of the workgroup's call
  // counter, loaded (load_ctr) once the first V tile's sign words have
  // landed, before that tile's z store, so waiting for the words never waits
  // for it.  The two-launch path keeps tag 0, which no poll accepts.
  uint32_t tag = 0;
  auto load_ctr = [&]() {
    if (MODE == 2) tag = call_tag(ld32c(sync + LB_SYNC_CTR + 8 * wg));
  };
  // phase-B pairs per wave in registers
  constexpr int NPW = MAXB > 1 ? LB_MAXPW_MULTI : LB_MAXPW;
  UTilePre<NPW> pre[LB_MAXT];
  HPre hpre;
  UPrePlan plan;
  plan.split = plan.cover = 0;
  uint32_t hval = 0;
  // copied tiles per workgroup: the row-scale table's 16, and partial sums
  // [wave][tile][row][token] within the 6144 floats of red
  const int span_max = min(LB_UPRE_HROWS / 32, (LB_MAXT * LB_WAVES * 256) / (LB_WAVES * 16 * batch));
  // every load is issued (tiles clamped to a valid one), which keeps the
  // wait counts exact; tiles beyond ut1 are never used
  auto prefetch = [&]() {
    if (SINGLE) {
      share(A.uq, A.ur, wg, ut0, ut1);
    } else {
      ut0 = A.ut_begin[wg];
      ut1 = A.ut_begin[wg + 1];
    }
    const int nut = A.nut;
    if (UPRE) {
      upre_issue<SINGLE>(A, M, ut0, ut1, span_max, upre_lds, plan, hval);
    } else {
#pragma unroll
      for (int k = 0; k < LB_MAXT; ++k) {
        int tile;
        const int li = u_layer<SINGLE>(M, min(ut0 + k, nut - 1), tile);
        u_prefetch(SINGLE ? V0 : layer_view(A.L[li]), tile, pre[k]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int tile;
      const int li = u_layer<SINGLE>(M, min(ut0 + (wave_id() >> 2) + 2 * j, nut - 1), tile);
      load_h(SINGLE ? V0 : layer_view(A.L[li]), tile, hpre, j);
    }
  };
  // V tiles, then phase B.  Phase-B loads (prefetch) are issued during phase
  // A, after the sign words they would otherwise delay (loads complete in
  // issue order), or after a pause by a workgroup without V tiles (letting
  // the V-tile workgroups' sign words go to memory first).
  if (vt0 < vt1 && SINGLE) {
    // one layer: the first tile's loads came from the early issue (single
    // launch) or are issued in v_tile; phase-B loads follow its sign words
    int tile;
    const int k = v_slot<SINGLE>(M, pre_vsplit, vt0, tile);
    auto first_hook = [&]() {
      load_ctr();
      prefetch();
    };
    v_tile<MAXB, FAST, MODE == 2, EARLY>(V0, batch, k & 1, tile, tag, sc, red[0], zstage, first_hook, early);
    __syncthreads();
    LB_MSTAMP(2);
    for (int t = vt0 + 1; t < vt1; ++t) {
      const int kt = v_slot<SINGLE>(M, pre_vsplit, t, tile);
      v_tile<MAXB, FAST, false, false>(V0, batch, kt & 1, tile, tag, sc, red[0], zstage, prefetch, early);
      __syncthreads();
    }
    LB_MSTAMP(9);
  } else if (vt0 < vt1) {
    // several layers: a tile's first loads are issued at the end of the
    // previous tile's products, and the previous tile's z is stored then (so
    // no wait for a tile's words also waits for the stores before them).
    // The phase-B loads go out with the last tile's hook, after every V
    // word.
    int tile;
    int k = v_slot<SINGLE>(M, pre_vsplit, vt0, tile);
    VLoads cur;
    v_issue<FAST>(v_geom(layer_view(A.L[k >> 1]), k & 1, tile), 0, batch, cur);
    int prev_k = -1, prev_tile = 0;
    for (int t = vt0; t < vt1; ++t) {
      int ntile = 0;
      const int nk = t + 1 < vt1 ? v_slot<SINGLE>(M, pre_vsplit, t + 1, ntile) : -1;
      VLoads nxt;
      auto hook = [&]() {
        if (nk >= 0) v_issue<FAST>(v_geom(layer_view(A.L[nk >> 1]), nk & 1, ntile), 0, batch, nxt);
        if (t == vt0) load_ctr();
        if (prev_k >= 0)
          v_store_z(layer_view(A.L[prev_k >> 1]), batch, prev_k & 1, prev_tile, late(tag), zst[(t - vt0 + 1) & 1]);
        if (MODE == 2 && t == vt1 - 1) prefetch();
      };
      const LayerView L = layer_view(A.L[k >> 1]);
      v_tile<MAXB, FAST, true, true, true>(L, batch, k & 1, tile, tag, sc, red[0], zst[(t - vt0) & 1], hook, cur);
      __syncthreads();
      if (t == vt0) LB_MSTAMP(2);
      prev_k = k;
      prev_tile = tile;
      k = nk;
      tile = ntile;
      cur = nxt;
    }
    v_store_z(layer_view(A.L[prev_k >> 1]), batch, prev_k & 1, prev_tile, late(tag), zst[(vt1 - 1 - vt0) & 1]);
    LB_MSTAMP(9);
  } else if (MODE == 2) {
    for (int i = 0; i < 3; ++i) __builtin_amdgcn_s_sleep(24);
    load_ctr();
    prefetch();
  }
  if (MODE == 1) share(A.uq, A.ur, wg, ut0, ut1);
  if (MODE != 0) {
    const bool check = MODE == 2;
    UState S;
    S.li = -1;
    // U tiles in groups of up to LB_MAXT tiles of one layer; the first group
    // uses the sign words prefetched during phase A (single launch)
    YOut yo;
    yo.p[0] = yo.p[1] = nullptr;
    yo.v[0] = yo.v[1] = 0;
    int t = ut0;
    // sign bytes copied to LDS: every wave's copies have landed (a wait for
    // all of this wave's loads, then the barrier in front of the z copy)
    if (UPRE) {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
      hl_lds[threadIdx.x] = (uint16_t)hval;
      __syncthreads();
    }
    if (UPRE) {
      // the copied prefix [ut0, cover), one span per layer, then the rest
      // from memory (separate loops: no register of one path waits on the
      // other's loads)
      while (t < plan.cover) {
        int tile;
        const int li = u_layer<SINGLE>(M, t, tile);
        const int lend = SINGLE ? ut1 : min(ut1, layer_u_end(M, li));
        const int T = min(lend, plan.cover) - t;
        const LayerView L = SINGLE ? V0 : layer_view(A.L[li]);
        const int slot = t >= plan.split ? 1 : 0;
        const int first = slot ? plan.split : ut0;
        const int tb0 = tile_bytes_b(L, 0), tb1 = tile_bytes_b(L, L.nb == 2 ? 1 : 0);
        const uint8_t* w0 = upre_lds + (slot ? plan.off[2] : plan.off[0]) + (t - first) * tb0;
        const uint8_t* w1 = upre_lds + (slot ? plan.off[3] : plan.off[1]) + (t - first) * tb1;
        u_span_lds<(MAXB > 1 ? LB_POLL_LOADS_MULTI : LB_POLL_LOADS)>(L, li, batch, tile, T, span_max, w0, w1, tb0, tb1, hl_lds + 32 * (t - ut0), tag, check, sync, sc, S,
                   u_lds, &red[0][0][0]);
        if (t == ut0) LB_MSTAMP(5);
        t += T;
      }
    }
    // Groups of up to LB_MAXT tiles of one layer from registers.  A group's
    // sign words and row scales are loaded while the group before it runs
    // (the single launch's first group: during phase A), so no group waits
    // a memory round trip for them.  The loads are unconditional (the group
    // after the last repeats the last group's tiles, never used), which
    // keeps the compiler's wait counts exact.
    auto group_of = [&](int tg, int& tile, int& nt) {
      const int li = u_layer<SINGLE>(M, tg, tile);
      const int lend = SINGLE ? ut1 : min(ut1, layer_u_end(M, li));
      nt = min(LB_MAXT, lend - tg);
      return li;
    };
    auto load_group = [&](int tg, UTilePre<NPW> (&p)[LB_MAXT], HPre& h) {
      int tile, nt;
      const int li = group_of(tg, tile, nt);
      const LayerView L = SINGLE ? V0 : layer_view(A.L[li]);
#pragma unroll
      for (int k = 0; k < LB_MAXT; ++k) u_prefetch(L, tile + min(k, nt - 1), p[k]);
#pragma unroll
      for (int j = 0; j < 2; ++j) load_h(L, tile + min((wave_id() >> 2) + 2 * j, nt - 1), h, j);
    };
    UTilePre<NPW> cur[LB_MAXT];
    HPre hc;
    if (MODE == 2 && !UPRE) {
#pragma unroll
      for (int k = 0; k < LB_MAXT; ++k) cur[k] = pre[k];
      hc = hpre;
    } else if (t < ut1) {
      load_group(t, cur, hc);
    }
    bool first_group = true;
    while (t < ut1) {
      int tile, nt;
      const int li = group_of(t, tile, nt);
      UTilePre<NPW> nxt[LB_MAXT];
      HPre hn;
      load_group(min(t + nt, ut1 - 1), nxt, hn);
      store_y(yo);
      yo = u_group(SINGLE ? V0 : layer_view(A.L[li]), li, batch, tile, nt, cur, hc, tag, check, sync, sc, S, u_lds,
                   red);
      if (first_group) LB_MSTAMP(5);
      first_group = false;
      t += nt;
#pragma unroll
      for (int k = 0; k < LB_MAXT; ++k) cur[k] = nxt[k];
      hc = hn;
    }
    store_y(yo);
  }
  LB_MSTAMP(6);
  // this workgroup's call is done: the next call's tag is one higher
  if (MODE == 2 && threadIdx.x == 0) add64c_noret(sync + LB_SYNC_CTR + 8 * wg, 1ull);
}

// Copies the workspace's poll error word to *out and clears it (one thread;
// a kernel rather than a copy call, so it can sit in a captured graph).
__global__ void lb_take_error_kernel(uint8_t* sync, uint32_t* out) {
  if (threadIdx.x == 0) {
    uint32_t* e = reinterpret_cast<uint32_t*>(sync + LB_SYNC_ERR);
    *out = ld32c(e);
    st32c(e, 0u);
  }
}

hipError_t lb_launch_take_error(void* sync, uint32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(lb_take_error_kernel, dim3(1), dim3(64), 0, stream, (uint8_t*)sync, out);
  return hipGetLastError();
}

static int g_fused_grid[64];  // per device: workgroups of the single-launch kernel (0: unknown, -1: none)

// Dynamic LDS of a decode launch: phase B stages z (zs + 8 halves per token)
// of the largest layer (phase A keeps its operands in registers).
size_t lb_decode_lds_bytes(const LbDecodeArgs& a) {
  int zs = 0;
  for (int i = 0; i < a.nlayers; ++i) zs = a.L[i].zs > zs ? a.L[i].zs : zs;
  return (size_t)a.batch * (zs + 8) * sizeof(uint16_t);
}

// Splits costs c[0..n) into G contiguous ranges, begin[0..G], whose largest
// total is the smallest possible: a binary search on that total, each trial
// filling ranges greedily; ranges past the last tile are empty.
static void balanced_split(const int64_t* c, int n, int G, int* begin) {
  int64_t lo = 0, hi = 0;
  for (int i = 0; i < n; ++i) {
    lo = c[i] > lo ? c[i] : lo;
    hi += c[i];
  }
  auto parts = [&](int64_t cap) {
    int k = n > 0 ? 1 : 0;
    int64_t sum = 0;
    for (int i = 0; i < n; ++i) {
      if (sum > 0 && sum + c[i] > cap) {
        ++k;
        sum = 0;
      }
      sum += c[i];
    }
    return k;
  };
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (parts(mid) <= G) hi = mid; else lo = mid + 1;
  }
  int w = 0;
  int64_t sum = 0;
  begin[0] = 0;
  for (int i = 0; i < n; ++i) {
    if (sum > 0 && sum + c[i] > lo) {
      begin[++w] = i;
      sum = 0;
    }
    sum += c[i];
  }
  while (w < G) begin[++w] = n;
}

// Cost-balanced tile ranges of a multi-layer single launch.  A V tile costs
// its reduction length plus a fixed share (u staging, cross-wave sums, z
// store, about a 4096-input pass); a U tile its two branches' ranks plus a
// smaller fixed share.
static void cost_split(LbDecodeArgs& a, int G, int vrows = 16) {
  std::vector<int64_t> c;
  c.reserve(a.nvt > a.nut ? a.nvt : a.nut);
  for (int li = 0; li < a.nlayers; ++li)
    for (int b = 0; b < a.L[li].nb; ++b)
      for (int t = 0; t < (a.L[li].br[b].r + vrows - 1) / vrows; ++t) c.push_back(a.L[li].n + 4096);
  balanced_split(c.data(), (int)c.size(), G, a.vt_begin);
  c.clear();
  for (int li = 0; li < a.nlayers; ++li) {
    const int64_t k = a.L[li].br[0].r + (a.L[li].nb == 2 ? a.L[li].br[1].r : 0) + 512;
    for (int t = 0; t < (a.L[li].m + 15) / 16; ++t) c.push_back(k);
  }
  balanced_split(c.data(), (int)c.size(), G, a.ut_begin);
}

// Smallest per-CU occupancy of the single-launch kernels of one token limit
// and one form of the activation loads.
template <int MAXB, bool FAST>
static hipError_t fused_occupancy_f(int& occ) {
  int o[4] = {0, 0, 0, 0};
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o[0], lb_decode_kernel<2, true, false, MAXB, FAST>,
                                                              LB_THREADS, LB_DECODE_LDS_MAX);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o[1], lb_decode_kernel<2, false, false, MAXB, FAST>, LB_THREADS,
                                                     LB_DECODE_LDS_MAX);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o[2], lb_decode_kernel<2, true, true, MAXB, FAST>, LB_THREADS,
                                                     LB_UPRE_DYN_MAX);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o[3], lb_decode_kernel<2, false, true, MAXB, FAST>, LB_THREADS,
                                                     LB_UPRE_DYN_MAX);
  occ = o[0];
  for (int i = 1; i < 4; ++i) occ = o[i] < occ ? o[i] : occ;
  return e;
}

// Smallest per-CU occupancy of the single-launch kernels of one token limit
// (both forms of the activation loads).
template <int MAXB>
static hipError_t fused_occupancy(int& occ) {
  int a = 0, b = 0;
  hipError_t e = fused_occupancy_f<MAXB, true>(a);
  if (e == hipSuccess) e = fused_occupancy_f<MAXB, false>(b);
  occ = a < b ? a : b;
  return e;
}

// The multi-token V pass takes 16-byte loads of x and g when every layer's x
// is 16-byte aligned with ldx and n multiples of 8 (g is 16-byte aligned by
// contract).
static bool decode_fast_loads(const LbDecodeArgs& a) {
  for (int i = 0; i < a.nlayers; ++i) {
    const LbLayerArgs& L = a.L[i];
    if ((((uintptr_t)L.x) & 15) != 0 || (L.ldx & 7) != 0 || (L.n & 7) != 0) return false;
  }
  return true;
}

hipError_t lb_decode1_occupancy(bool single, size_t lds, int& occ);
size_t lb_decode1_lds_bytes(const LbDecodeArgs& a);
hipError_t lb_launch_decode1(const LbDecodeArgs& args, int G, void* sync, hipStream_t stream);

// Workgroups of a single launch on this device (0: none fits).  Every single
// launch, of any decode kernel, uses this one grid, so that every workgroup's
// call counter in a workspace advances by one per call.
static hipError_t fused_grid(int& G) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  G = 0;
  if (dev < 0 || dev >= 64) return hipSuccess;
  if (g_fused_grid[dev] == 0) {
    int ncu = 0, occb = 0, occ1 = 0, occ2 = 0;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // every workgroup of the single launch must be resident at once: size
    // the grid for the largest dynamic LDS a launch may request (one token
    // runs decode1.hip's kernels, two to LB_MAX_BATCH these)
    e = fused_occupancy<LB_MAX_BATCH>(occb);
    if (e != hipSuccess) return e;
    e = lb_decode1_occupancy(true, LB_DECODE1_LDS_MAX, occ1);
    if (e != hipSuccess) return e;
    e = lb_decode1_occupancy(false, LB_DECODE1_LDS_MAX, occ2);
    if (e != hipSuccess) return e;
    g_fused_grid[dev] = (occb >= 1 && occ1 >= 1 && occ2 >= 1) ? (ncu < LB_MAX_GRID ? ncu : LB_MAX_GRID) : -1;
  }
  G = g_fused_grid[dev] > 0 ? g_fused_grid[dev] : 0;
  return hipSuccess;
}

template <bool SINGLE, int MAXB, bool FAST>
static hipError_t launch_decode_f(const LbDecodeArgs& args, void* sync, int allow_fused,
                                  hipStream_t stream) {
  const size_t lds = lb_decode_lds_bytes(args);
  if (lds > LB_DECODE_LDS_MAX) return hipErrorInvalidValue;  // the host routes such calls elsewhere
  hipError_t e = hipSuccess;
  // preloaded copies of layer 0's phase-A fields (single-layer kernels)
  const LbLayerArgs& L0 = args.L[0];
  const uint8_t* vb0 = SINGLE ? L0.br[0].vbits : nullptr;
  const uint8_t* vb1 = SINGLE ? L0.br[1].vbits : nullptr;
  const uint16_t* px = SINGLE ? L0.x : nullptr;
  const uint16_t* g0 = SINGLE ? L0.br[0].g : nullptr;
  const uint16_t* g1 = SINGLE ? L0.br[1].g : nullptr;
  const int pn = SINGLE ? L0.n : 0, pldx = SINGLE ? (int)L0.ldx : 0, vsplit = SINGLE ? args.vt_end[0] : 0;
  auto misc = [&](const LbDecodeArgs& a) {
    return (uint32_t)a.vq | ((uint32_t)a.vr << 8) | ((uint32_t)a.batch << 16);
  };
  if (allow_fused) {
    int G = 0;
    e = fused_grid(G);
    if (e != hipSuccess) return e;
    if (G > 0) {
      LbDecodeArgs a = args;
      a.vq = a.nvt / G; a.vr = a.nvt % G;
      a.uq = a.nut / G; a.ur = a.nut % G;
      if (!SINGLE) cost_split(a, G);
      // the variant that copies phase B's sign bytes to LDS during phase A,
      // when the dynamic LDS leaves room for the copy and a workgroup's U
      // tiles are more than the register prefetch holds (one group of
      // LB_MAXT tiles of one layer, LB_MAXPW pairs per wave: the 1-token
      // window, which the multi-token kernels' window contains)
      bool regs_hold = SINGLE && (a.nut + G - 1) / G <= LB_MAXT;
      for (int b = 0; b < args.L[0].nb && regs_hold; ++b) {
        const int np = (lb16_units(args.L[0].br[b].r) + 1) >> 1;
        regs_hold = (np + (args.L[0].nb == 2 ? 3 : 7)) / (args.L[0].nb == 2 ? 4 : 8) <= LB_MAXPW;
      }
      if (lds <= LB_UPRE_DYN_MAX && !regs_hold)
        hipLaunchKernelGGL((lb_decode_kernel<2, SINGLE, true, MAXB, FAST>), dim3(G), dim3(LB_THREADS), lds, stream, vb0, vb1, px,
                           g0, g1, pn, pldx, vsplit, misc(a), a, (uint8_t*)sync);
      else
        hipLaunchKernelGGL((lb_decode_kernel<2, SINGLE, false, MAXB, FAST>), dim3(G), dim3(LB_THREADS), lds, stream, vb0, vb1, px,
                           g0, g1, pn, pldx, vsplit, misc(a), a, (uint8_t*)sync);
      return hipGetLastError();
    }
  }
  LbDecodeArgs a = args;
  a.vq = 1; a.vr = 0;
  hipLaunchKernelGGL((lb_decode_kernel<0, SINGLE, false, MAXB, FAST>), dim3(a.nvt), dim3(LB_THREADS), lds, stream, vb0, vb1, px, g0,
                     g1, pn, pldx, vsplit, misc(a), a, (uint8_t*)sync);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int gb = a.nut < 1024 ? a.nut : 1024;
  a.uq = a.nut / gb; a.ur = a.nut % gb;
  hipLaunchKernelGGL((lb_decode_kernel<1, SINGLE, false>), dim3(gb), dim3(LB_THREADS), lds, stream, vb0, vb1, px, g0, g1,
                     pn, pldx, vsplit, misc(a), a, (uint8_t*)sync);
  return hipGetLastError();
}

template <bool SINGLE, int MAXB>
static hipError_t launch_decode_t(const LbDecodeArgs& args, void* sync, int allow_fused,
                                  hipStream_t stream) {
  return decode_fast_loads(args) ? launch_decode_f<SINGLE, MAXB, true>(args, sync, allow_fused, stream)
                                 : launch_decode_f<SINGLE, MAXB, false>(args, sync, allow_fused, stream);
}

hipError_t lb_launch_decode(const LbDecodeArgs& args, void* sync, int allow_fused,
                            hipStream_t stream) {
  if (args.batch == 1) {
    // one token: the sparse-instruction kernels of decode1.hip
    if (lb_decode1_lds_bytes(args) > LB_DECODE1_LDS_MAX) return hipErrorInvalidValue;
    int G = 0;
    if (allow_fused) {
      hipError_t e = fused_grid(G);
      if (e != hipSuccess) return e;
    }
    // its V work comes in units of one or two 16-rank tiles of a branch:
    // two (one instruction serves both) when there are more tiles than
    // workgroups, one otherwise (every workgroup then has at most one tile,
    // and a second would only lengthen the busy ones)
    LbDecodeArgs a = args;
    int tiles = 0;
    for (int i = 0; i < a.nlayers; ++i)
      for (int b = 0; b < a.L[i].nb; ++b) tiles += (a.L[i].br[b].r + 15) / 16;
    a.vtpu = tiles > LB_MAX_GRID ? 2 : 1;
    int vu = 0;
    for (int i = 0; i < a.nlayers; ++i)
      for (int b = 0; b < 2; ++b) {
        if (b < a.L[i].nb) vu += ((a.L[i].br[b].r + 15) / 16 + a.vtpu - 1) / a.vtpu;
        a.vt_end[2 * i + b] = vu;
      }
    a.nvt = vu;
    if (G > 0 && a.nlayers > 1) cost_split(a, G, 16 * a.vtpu);
    return lb_launch_decode1(a, G, sync, stream);
  }
  return args.nlayers == 1 ? launch_decode_t<true, LB_MAX_BATCH>(args, sync, allow_fused, stream)
                           : launch_decode_t<false, LB_MAX_BATCH>(args, sync, allow_fused, stream);
}
