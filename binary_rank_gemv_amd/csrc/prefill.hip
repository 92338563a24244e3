// Prefill path (many tokens) of the LittleBit layer: two matrix-core GEMMs.
//
// Per branch b (explainx.ai explainer, "How it works" items 1-3):
//   GEMM 1:  T_b = sign(V_b)^T (g_b * X)^T     rows j < r_b, one column per token
//            Z_b = fp16(l_b * T_b), stored token-major as z[token][zoff_b + j]
//   GEMM 2:  Y^T = sum_b diag(h_b) sign(U_b) Z_b^T   rows i < m, one column per token
// The sign factors stay packed (LB16); each 16x32 operand fragment is
// expanded in registers to exact values, +-1.0 in GEMM 1 and +-h_b[i] in
// GEMM 2 (lb16_step_operand_val), and reused for four token tiles; so GEMM 2
// sums both branches in one set of accumulators.  The activation operand (g*x, or z) is staged
// through LDS in chunks of 128 inputs x 128 tokens, double buffered, and read
// as 16x32 fragments.  Accumulation is fp32; g*x and l*t are rounded to fp16
// (the same roundings as the decode path); y is rounded to fp16 once.
//
// Workgroup = 4 waves, 128 rows x 128 tokens; wave (wr, wc) owns 64 rows
// (4 tiles) x 64 tokens (4 tiles) = 16 accumulators of 16x16.
#include <type_traits>

#include "lb_common.h"

#define PF_THREADS 256
#define PF_BM 128   // rows per workgroup (8 tiles of 16)
#define PF_BN 128   // tokens per workgroup
#define PF_ROW 136  // halves per staged token row: 128 inputs + 8 (staggers LDS banks)

namespace {

__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

typedef f16 h2 __attribute__((ext_vector_type(2)));

// One segment of the reduction: a packed sign factor (rows in tiles of 16,
// reduction length K) against an activation source with `kvalid` usable
// inputs per token (zero beyond).
struct Seg {
  const uint8_t* bits;  // LB16 factor
  int K;                // reduction length of the packed factor
  int ntiles;           // row tiles of the factor
  const uint16_t* src;  // activations: src[token * ld + k]
  long ld;
  int kvalid;           // inputs k < kvalid are read; others are zero
  const uint16_t* g;    // per-input scale (GEMM 1) or nullptr
};

// Staged registers of one chunk: thread t holds segments t + 256 i (i < 8),
// i.e. token (t >> 4) + 16 i, inputs 8 (t & 15) .. +7 of the chunk.
struct Chunk {
  uint4 v[8];
  uint4 gv;
};

// FAST: 16-byte loads (src and ld aligned, kvalid % 8 == 0).  Addresses are
// clamped to valid ones; out-of-range values are zeroed at the store.
template <bool FAST>
__device__ __forceinline__ void chunk_load(const Seg& S, int M, int tok0, int k0, Chunk& C) {
  const int tid = threadIdx.x;
  const int k = k0 + 8 * (tid & 15);
  if (FAST) {
    const int kc = min(k, S.kvalid - 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = min(tok0 + (tid >> 4) + 16 * i, M - 1);
      C.v[i] = *reinterpret_cast<const uint4*>(S.src + (long)tok * S.ld + kc);
    }
    if (S.g) C.gv = *reinterpret_cast<const uint4*>(S.g + kc);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = min(tok0 + (tid >> 4) + 16 * i, M - 1);
      uint16_t e[8];
      for (int q = 0; q < 8; ++q) e[q] = (k + q < S.kvalid) ? S.src[(long)tok * S.ld + k + q] : (uint16_t)0;
      C.v[i] = *reinterpret_cast<uint4*>(e);
    }
    if (S.g) {
      uint16_t e[8];
      for (int q = 0; q < 8; ++q) e[q] = (k + q < S.kvalid) ? S.g[k + q] : (uint16_t)0;
      C.gv = *reinterpret_cast<uint4*>(e);
    }
  }
}

__device__ __forceinline__ void chunk_store(const Seg& S, int M, int tok0, int k0, const Chunk& C,
                                            uint16_t* buf) {
  const int tid = threadIdx.x;
  const int k = k0 + 8 * (tid & 15);
  const bool kin = k < S.kvalid;  // a group of 8 is wholly in or out (kvalid % 8 == 0 on the fast path;
                                  // the element-wise path zeroed its own tail)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = (tid >> 4) + 16 * i;
    uint4 v = C.v[i];
    if (S.g) {
      // g*x rounded to fp16 (one correctly rounded product per value)
      h2 p[4];
      const h2* xv = reinterpret_cast<const h2*>(&v);
      const h2* gv = reinterpret_cast<const h2*>(&C.gv);
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = xv[q] * gv[q];
      v = *reinterpret_cast<uint4*>(p);
    }
    if (!kin || tok0 + t >= M) v = make_uint4(0u, 0u, 0u, 0u);
    uint16_t* dst = static_cast<uint16_t*>(__builtin_assume_aligned(buf + t * PF_ROW + 8 * (tid & 15), 16));
    *reinterpret_cast<uint4*>(dst) = v;
  }
}

// One reduction segment added into acc[4][4].  Row tile rt's operand values
// are +-v with v from vpair[rt] (fp16 bits of |v| in both halves); flip[rt]
// is all ones where v < 0.
template <bool FAST>
__device__ __forceinline__ void run_segment(const Seg& S, int M, int tok0, int tile0, const LbSignConsts& sc,
                                            const uint32_t (&vpair)[4], const uint32_t (&flip)[4],
                                            uint16_t (*bs)[PF_BN * PF_ROW], f32x4 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wc = wave & 1;
  const int grp = lane >> 4, col = lane & 15;
  const int nu = lb16_units(S.K), np = (nu + 1) >> 1;
  const long tbytes = lb16_tile_bytes(S.K);
  const uint8_t* tp[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) tp[rt] = S.bits + (long)min(tile0 + rt, S.ntiles - 1) * tbytes;

  Chunk C;
  __syncthreads();  // previous users of the staging buffers are done
  chunk_load<FAST>(S, M, tok0, 0, C);
  chunk_store(S, M, tok0, 0, C, bs[0]);
  uint32_t w[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) w[rt] = lb16_load_pair(tp[rt], 0, lane, nu);
  __syncthreads();

  for (int p = 0; p < np; ++p) {
    // next chunk and sign words: issued unconditionally (the last chunk is
    // re-read at the end) so the wait counts below stay exact
    const int pn = min(p + 1, np - 1);
    Chunk N;
    chunk_load<FAST>(S, M, tok0, 128 * pn, N);
    uint32_t wn[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) wn[rt] = lb16_load_pair(tp[rt], pn, lane, nu);
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the matrix work

    const uint32_t sel = lb16_pair_sel(p, lane, nu);
    uint32_t reg[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) reg[rt] = lb16_reg_word(w[rt], sel) ^ flip[rt];
    const uint16_t* bb = bs[p & 1] + (64 * wc + col) * PF_ROW + 8 * grp;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      f16x8 b[4], a[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) b[tt] = *reinterpret_cast<const f16x8*>(bb + 16 * tt * PF_ROW + 32 * st);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) a[rt] = lb16_step_operand_val(reg[rt], st, sc.sign_mask, vpair[rt]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[rt][tt] = mfma16(a[rt], b[tt], acc[rt][tt]);
    }
    // unconditional (after the last chunk it refills the idle buffer), so the
    // loads above are not sunk into a branch behind the matrix work
    chunk_store(S, M, tok0, 128 * pn, N, bs[(p + 1) & 1]);
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) w[rt] = wn[rt];
  }
}

}  // namespace

// MODE 1: GEMM 1 for branch blockIdx.z.  MODE 2: GEMM 2 over all branches.
// blockIdx.x: 128-row block, blockIdx.y: 128-token block.
template <int MODE, bool FAST>
__global__ __launch_bounds__(PF_THREADS, 2) void lb_prefill_kernel(LbPrefillArgs A) {
  __shared__ __align__(16) uint16_t bs[2][PF_BN * PF_ROW];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wr = wave >> 1, wc = wave & 1;
  const int grp = lane >> 4, col = lane & 15;
  const int tok0 = blockIdx.y * PF_BN;
  const int tile0 = 8 * blockIdx.x + 4 * wr;  // first row tile of this wave
  const int M = A.M;
  const LbSignConsts sc = lb16_sign_consts();
  f32x4 acc[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (MODE == 1) {
    const int b = blockIdx.z;
    const LbBranchArgs& B = A.br[b];
    const int ntiles = (B.r + 15) >> 4;
    if (8 * (int)blockIdx.x >= ntiles) return;  // block beyond this branch's rows (uniform)
    Seg S{B.vbits, A.n, ntiles, A.x, A.ldx, A.n, B.g};
    const uint32_t one[4] = {sc.one_pair, sc.one_pair, sc.one_pair, sc.one_pair}, none[4] = {0u, 0u, 0u, 0u};
    run_segment<FAST>(S, M, tok0, tile0, sc, one, none, bs, acc);

    // z = fp16(l * t), token-major; rows j >= r are stored as zero
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int tile = tile0 + rt;
      if (tile >= ntiles) continue;
      const int j0 = 16 * tile + 4 * grp;
      float lq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) lq[q] = (j0 + q < B.r) ? h2f(B.l[j0 + q]) : 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int tok = tok0 + 64 * wc + 16 * tt + col;
        if (tok >= M) continue;
        uint16_t zq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) zq[q] = f2h(lq[q] * acc[rt][tt][q]);
        *reinterpret_cast<uint2*>(A.z + (long)tok * A.zs + B.zoff + j0) = *reinterpret_cast<uint2*>(zq);
      }
    }
    // the block holding the last row tile also zeroes this token block's
    // z entries between 16*ceil(r/16) and 128*ceil(r/128)
    if ((int)blockIdx.x == (ntiles - 1) >> 3) {
      const int j0 = 16 * ntiles, nz = 128 * ((B.r + 127) / 128) - j0;  // a multiple of 16
      const int per_tok = nz >> 2;                                 // 8-byte stores per token
      for (int e = threadIdx.x; e < per_tok * PF_BN; e += PF_THREADS) {
        const int tok = tok0 + e / per_tok;
        if (tok < M) *reinterpret_cast<uint2*>(A.z + (long)tok * A.zs + B.zoff + j0 + 4 * (e % per_tok)) = make_uint2(0u, 0u);
      }
    }
  } else {
    const int ntiles = (A.m + 15) >> 4;
    for (int b = 0; b < A.nb; ++b) {
      const LbBranchArgs& B = A.br[b];
      Seg S{B.ubits, B.r, ntiles, A.z + B.zoff, A.zs, 64 * lb16_units(B.r), nullptr};
      // operand values +-h_b[i] for the lane's row i (rows >= m read row m-1; never stored)
      uint32_t hv[4], fl[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const uint32_t hb = B.h[min(16 * (tile0 + rt) + col, A.m - 1)];
        hv[rt] = (hb & 0x7FFFu) * 0x10001u;
        fl[rt] = (hb & 0x8000u) ? 0xFFFFFFFFu : 0u;
      }
      run_segment<true>(S, M, tok0, tile0, sc, hv, fl, bs, acc);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int tile = tile0 + rt;
      if (tile >= ntiles) continue;
      const int i0 = 16 * tile + 4 * grp;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int tok = tok0 + 64 * wc + 16 * tt + col;
        if (tok >= M) continue;
        uint16_t* yp = A.y + (long)tok * A.ldy + i0;
        uint16_t yq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) yq[q] = f2h(acc[rt][tt][q]);
        if (i0 + 3 < A.m && ((uintptr_t)yp & 7) == 0) {
          *reinterpret_cast<uint2*>(yp) = *reinterpret_cast<uint2*>(yq);
        } else {
          for (int q = 0; q < 4; ++q)
            if (i0 + q < A.m) yp[q] = yq[q];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ v2
// The main prefill kernels, for n % 128 == 0 and 16-byte aligned x rows.
// Workgroup tile: 256 rows x 128 tokens, 8 waves, two on each SIMD.  Wave w
// owns the 64 rows of row group w % 4 (4 tiles) and all 128 tokens (8
// tiles), so each expanded sign fragment feeds 8 matrix-core steps; the two
// waves of a SIMD (w and w + 4) take the two halves of every 128-input chunk
// (steps 0-1 and 2-3), so one issues while the other waits, and their
// accumulators are summed through LDS at the end.  Activation chunks (128
// inputs x 128 tokens = 32 KB) go from memory straight to LDS with 16-byte
// global-to-LDS loads, no registers involved.  In LDS the 8 inputs q (of 16)
// of token t sit in 16-byte slot 16 t + (q ^ (t & 15)): the 16 lanes reading
// one fragment row (same q, 16 tokens) then hit 16 distinct bank groups, and
// the 16 lanes loading one token still read one contiguous 256-byte row
// segment.  GEMM 1 folds g into the sign operand (exact +-g_k, by XOR of the
// sign bit), GEMM 2 folds h (exact +-h_i).  Tokens beyond M load the last
// token's row (outputs never stored).
// Three stages, so a chunk's loads are started two chunks ahead.  Each stage
// is a __shared__ array of its own: the compiler tells the arrays'
// global-to-LDS writes apart and adds no wait of its own before reads of the
// stage being consumed; the waits that order the stages are explicit.
#define P2_WAVES 8
#define P2_STAGES 3
#define P2_CHUNK 32768
// stage layout: activations, then the sign bytes of the chunk's pair
// [row group][row tile][256 bytes], then g (256 bytes used of 1 KB)
#define P2_WORDS_OFF P2_CHUNK
#define P2_G_OFF (P2_CHUNK + 4 * 4 * 256)
#define P2_STAGE_BYTES (P2_G_OFF + 1024)

// Tile of a workgroup of the one-dimensional grid: 256-row block bx, token
// block by, branch bz (GEMM 1).  Workgroups go to the 8 XCDs (each with its
// own L2) round-robin by index; XCD x takes a contiguous run of tiles in
// token-block-major order, so that the activations of a token block (g*x,
// or z) are fetched into one L2 and its workgroups share them there.
struct P2Tile {
  int bx, by, bz;
};

__device__ __forceinline__ P2Tile p2_tile(int rb, int tb, int nbz) {
  const int n = rb * tb * nbz, L = (int)blockIdx.x;
  const int xcd = L & 7, idx = L >> 3, per = n >> 3, rem = n & 7;
  const int P = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  P2Tile t;
  t.by = P / (rb * nbz);
  const int q = P - t.by * rb * nbz;
  t.bz = q / rb;
  t.bx = q - t.bz * rb;
  return t;
}

// Row tiles of GEMM `mode` (the largest branch's for GEMM 1), and the
// 64 * rowt-row blocks that cover them.
__host__ __device__ inline int p2_row_tiles(const LbPrefillArgs& a, int mode) {
  int t = 0;
  if (mode == 1)
    for (int b = 0; b < a.nb; ++b) t = max(t, (a.br[b].r + 15) >> 4);
  else
    t = (a.m + 15) >> 4;
  return t;
}

__host__ __device__ inline int p2_row_blocks(const LbPrefillArgs& a, int mode, int rowt) {
  return (p2_row_tiles(a, mode) + 4 * rowt - 1) / (4 * rowt);
}

// ROWT: row tiles per wave (4, or 3 where 192-row blocks fill the machine
// in fewer rounds of workgroups).  The launch covers row tiles tile_base..
// in row_blocks blocks of 4 * ROWT tiles (a GEMM may be split into a launch
// of 256-row blocks and one of 192-row blocks for the last round).
template <int MODE, int ROWT>
__global__ __launch_bounds__(64 * P2_WAVES, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void
lb_prefill2_kernel(LbPrefillArgs A, int tile_base, int row_blocks) {
  static_assert(ROWT == 3 || ROWT == 4, "3 or 4 row tiles per wave");
  __shared__ __align__(16) uint8_t stage0[P2_STAGE_BYTES];
  __shared__ __align__(16) uint8_t stage1[P2_STAGE_BYTES];
  __shared__ __align__(16) uint8_t stage2[P2_STAGE_BYTES];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int rg = wave & 3, kh = wave >> 2;  // row group, half of each chunk
  const int grp = lane >> 4, col = lane & 15;
  const int M = A.M;
  const P2Tile bt = p2_tile(row_blocks, (M + PF_BN - 1) / PF_BN, MODE == 1 ? A.nb : 1);
  const int tok0 = bt.by * PF_BN;
  const int blk0 = tile_base + 4 * ROWT * bt.bx;  // first row tile of this workgroup
  const int tile0 = blk0 + ROWT * rg;             // first row tile of this wave
  const LbSignConsts sc = lb16_sign_consts();

  // the reduction as a sequence of 128-input chunks over one or two segments
  const int b1 = MODE == 1 ? bt.bz : 0;
  const LbBranchArgs& B0 = A.br[b1];
  const LbBranchArgs& B1 = A.br[MODE == 2 && A.nb == 2 ? 1 : b1];
  const int ntiles = MODE == 1 ? (B0.r + 15) >> 4 : (A.m + 15) >> 4;
  if (blk0 >= ntiles) return;  // rows beyond this branch (uniform)
  const int K0 = MODE == 1 ? A.n : B0.r, K1 = MODE == 1 ? A.n : B1.r;
  const int nu0 = lb16_units(K0), nu1 = lb16_units(K1);
  const int np0 = MODE == 1 ? A.n / 128 : (nu0 + 1) >> 1;
  const int np1 = MODE == 2 && A.nb == 2 ? (nu1 + 1) >> 1 : 0;
  const int C = np0 + np1;
  const uint8_t* bits0 = MODE == 1 ? B0.vbits : B0.ubits;
  const uint8_t* bits1 = MODE == 1 ? B1.vbits : B1.ubits;
  const uint16_t* src0 = MODE == 1 ? A.x : A.z + B0.zoff;
  const uint16_t* src1 = MODE == 1 ? A.x : A.z + B1.zoff;
  const long ld = MODE == 1 ? A.ldx : A.zs;
  const uint16_t* gsrc = B0.g;

  // GEMM 2: h_b[i] of the lane's row i of each tile, branch 0 in the low and
  // branch 1 in the high half
  uint32_t hraw[ROWT];
#pragma unroll
  for (int rt = 0; rt < ROWT; ++rt) {
    hraw[rt] = 0u;
    if (MODE == 2) {
      const int i = min(16 * (tile0 + rt) + col, A.m - 1);
      hraw[rt] = (uint32_t)B0.h[i] | ((uint32_t)B1.h[i] << 16);
    }
  }

  // per-lane byte offsets of the loads, the same for every chunk (the launch
  // guarantees that they fit 32 bits): activation slot i; sign bytes of row
  // tile lane/16 of the row group for segment sg (with 3 tiles per wave,
  // lanes 48.. load a tile nobody reads), 16 per lane, for a full
  // pair (256 bytes per tile) and for a pair of one unit (128 bytes, each
  // half-row loaded twice so that the LDS copy keeps the full pair's
  // addressing: byte 4j of a lane's word sits at 4*(lane/2)); g.  Wave
  // (rg, kh) loads activation slots 8 rg + 4 kh + i (i < 4), tokens
  // 32 rg + 16 kh .. + 15 of the block (past the last token: the last token)
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = (rg * 8 + 4 * kh + i) * 64 + lane;
    const int t = u >> 4, q = (u & 15) ^ (t & 15);
    aoff[i] = (uint32_t)(((long)min(tok0 + t, M - 1) * ld + 8 * q) * 2);
  }
  const uint32_t row0 = (uint32_t)(min(tile0 + (lane >> 4), ntiles - 1) * lb16_tile_bytes(K0));
  const uint32_t row1 = (uint32_t)(min(tile0 + (lane >> 4), ntiles - 1) * lb16_tile_bytes(K1));

  // loads of chunk c into stage S (all global-to-LDS), shared by all waves
  // so that no wave's matrix steps wait much longer on the memory queue
  // than its partner's on the SIMD: 4 KB of activations each, the sign bytes
  // of row group rg (first-half waves) and (GEMM 1, second-half waves) g
  // (lanes 16.. repeat lanes 0..15; four waves write the same bytes).
  auto issue = [&](auto khc, int c, uint8_t* S) {
    constexpr int KH = decltype(khc)::value;
    const int sg = c >= np0 ? 1 : 0;
    const int p = c - (sg ? np0 : 0);
    const uint8_t* src = reinterpret_cast<const uint8_t*>(sg ? src1 : src0) + 256 * p;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(src + aoff[i], (__attribute__((address_space(3))) void*)(S + (rg * 8 + 4 * KH + i) * 1024),
                                       16, 0, 0);
    if (KH == 0) {
      const bool full = 2 * p + 1 < (sg ? nu1 : nu0);
      const uint8_t* wsrc = (sg ? bits1 : bits0) + 256 * p + (sg ? row1 : row0) + 16 * (lane & (full ? 15 : 7));
      __builtin_amdgcn_global_load_lds(wsrc, (__attribute__((address_space(3))) void*)(S + P2_WORDS_OFF + rg * 1024), 16,
                                       0, 0);
    } else if (MODE == 1) {
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(gsrc) + 256 * p + 16 * (lane & 15),
                                       (__attribute__((address_space(3))) void*)(S + P2_G_OFF), 16, 0, 0);
    }
  };

  f32x4 acc[ROWT][8];
#pragma unroll
  for (int rt = 0; rt < ROWT; ++rt)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per chunk c (stage S) a wave runs its two matrix steps, 2kh and 2kh+1, or,
  // for a pair made of one unit (2 steps), step kh alone.  The barrier that
  // makes chunk c + 1 visible sits between the two steps: after it the wave
  // reads chunk c + 1's first-step B fragments and sign words, which land
  // while its second step of chunk c runs, so no chunk opens with the matrix
  // core waiting for LDS.  Everything a wave reads of stage S (both steps' B
  // fragments and g) is read before that barrier and waited for, so the
  // stage may be refilled once every wave has passed it.  The loads of chunk
  // c + 2 into stage `ahead` (the stage of chunk c - 1, free since the
  // barrier before) are issued between the first step's products, where a
  // wave stalled on a full memory queue leaves the matrix core to the other
  // wave of its SIMD.
  auto pair_of = [&](int c, int& sg, int& p, bool& full) {
    sg = c >= np0 ? 1 : 0;
    p = c - (sg ? np0 : 0);
    full = 2 * p + 1 < (sg ? nu1 : nu0);
  };
  // the lane's column, opaque here so that the fragment addresses are formed
  // per chunk instead of being held in registers across the loop
  auto read_b = [&](const uint8_t* S, int st, f16x8* dst) {
    int colx = col;
    __asm__ volatile("" : "+v"(colx));
    const int q = 4 * st + grp;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
      dst[tt] = *reinterpret_cast<const f16x8*>(S + 16 * (16 * (16 * tt + colx) + (q ^ colx)));
  };
  // GEMM 2: h_b[i] of segment (branch) sg in both halves of a word, for the
  // lane's row of each tile
  auto hpairs = [&](int sg, uint32_t* hp) {
#pragma unroll
    for (int rt = 0; rt < ROWT; ++rt) hp[rt] = __builtin_amdgcn_perm(hraw[rt], hraw[rt], sg ? 0x03020302u : 0x01000100u);
  };
  // chunk c's first-step B fragments and its sign words, from stage S
  auto head = [&](int c, const uint8_t* S, f16x8* b0, uint32_t* reg) {
    int sg, p;
    bool full;
    pair_of(c, sg, p, full);
    const int st0 = full ? 2 * kh : kh;
    const uint32_t sel = lb16_pair_sel(p, lane, sg ? nu1 : nu0);
    const uint32_t* words = reinterpret_cast<const uint32_t*>(S + P2_WORDS_OFF) + rg * 256 + (full ? lane : lane >> 1);
    read_b(S, st0, b0);
#pragma unroll
    for (int rt = 0; rt < ROWT; ++rt)
      reg[rt] = lb16_reg_word(words[64 * rt], sel);
  };
  // The A operand of step st: the weight's sign bit XORed into the scale's
  // fp16 bits, +-g_k (GEMM 1: gq, per input) or +-h_i (GEMM 2: hp, per row).
  auto mstep = [&](auto khc, int c, int st, const f16x8* bb, const uint32_t* reg, const u32x4& gq, const uint32_t* hp,
                   uint8_t* ahead, bool with_loads) {
    if (with_loads) issue(khc, min(c + P2_STAGES - 1, C - 1), ahead);
#pragma unroll
    for (int rt = 0; rt < ROWT; ++rt) {
      u32x4 d;
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) d[dd] = ((reg[rt] << (4 * st + dd)) & sc.sign_mask) ^ (MODE == 1 ? gq[dd] : hp[rt]);
      const f16x8 a = __builtin_bit_cast(f16x8, d);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) acc[rt][tt] = mfma16(a, bb[tt], acc[rt][tt]);
    }
    // issue order: the first operand, then each later operand's ALU work
    // (and the loads) spread between the products of the one before
    __builtin_amdgcn_sched_group_barrier(0x2, 8, 0);
#pragma unroll
    for (int i = 0; i < 8 * (ROWT - 1); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x2, 1, 0);
      if (with_loads && (i & 3) == 3 && i < 20) __builtin_amdgcn_sched_group_barrier(0x10, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x8, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // A wave waits until its loads of the next chunk and its LDS reads have
  // landed (its loads of the chunk after may still be in flight); then all
  // meet (the empty asm keeps LDS reads below the barrier).  Every first step
  // issues loads, past the end as repeats of the last chunk into a stage
  // nobody reads again, so the wait count is a constant; the two halves'
  // waves (different loads) run separate copies of the loop, so that no
  // branch separates a load from its waits.
  auto run = [&](auto khc) __attribute__((always_inline)) {
    constexpr int KH = decltype(khc)::value;
    // global-to-LDS loads per chunk of this wave: 4 of activations, the sign
    // bytes (first half) or g (second half, GEMM 1)
    constexpr int kOps = 4 + (KH == 0 || MODE == 1 ? 1 : 0);
    constexpr int kWait = kOps * (P2_STAGES - 2);
    auto sync = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt((kWait & 15) | ((kWait >> 4) << 14) | (7 << 4));
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    };
    f16x8 b0[8], b1[8];
    uint32_t reg[ROWT], regn[ROWT] = {};
    auto body = [&](int c, const uint8_t* S, const uint8_t* Snext, uint8_t* ahead) __attribute__((always_inline)) {
      int sg, p;
      bool full;
      pair_of(c, sg, p, full);
      const int st0 = full ? 2 * kh : kh;
      read_b(S, st0 + 1, b1);
      u32x4 gq0 = u32x4{0u, 0u, 0u, 0u}, gq1 = gq0;
      if (MODE == 1) {
        gq0 = *reinterpret_cast<const u32x4*>(S + P2_G_OFF + 2 * (32 * st0 + 8 * grp));
        gq1 = *reinterpret_cast<const u32x4*>(S + P2_G_OFF + 2 * (32 * (st0 + 1) + 8 * grp));
      }
      uint32_t hp[ROWT];
      if (MODE == 2) hpairs(sg, hp);
      __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of the first step's products
      mstep(khc, c, st0, b0, reg, gq0, hp, ahead, true);
      // unconditional (after the last chunk it rereads that chunk's copy in
      // a stage nobody needs), so that every path to a read of a stage has
      // passed the same waits
      sync();
      head(min(c + 1, C - 1), Snext, b0, regn);
      if (full) mstep(khc, c, st0 + 1, b1, reg, gq1, hp, ahead, false);
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) reg[rt] = regn[rt];
    };
    issue(khc, 0, stage0);
    issue(khc, min(1, C - 1), stage1);
    sync();
    head(0, stage0, b0, reg);
    int c = 0;
    for (; c + P2_STAGES <= C; c += P2_STAGES) {
      body(c, stage0, stage1, stage2);
      body(c + 1, stage1, stage2, stage0);
      body(c + 2, stage2, stage0, stage1);
    }
    if (c < C) body(c, stage0, stage1, stage2);
    if (c + 1 < C) body(c + 1, stage1, stage2, stage0);
  };
  if (kh == 0)
    run(std::integral_constant<int, 0>());
  else
    run(std::integral_constant<int, 1>());
  // every load has landed and every wave is past its reads: the stages are free
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  __syncthreads();

  // the second-half waves hand their sums to the first-half waves: row tiles
  // 0..2 through the three stages, then (4 tiles per wave) row tile 3
  // through the first
  {
    f32x4* red0 = reinterpret_cast<f32x4*>(stage0) + rg * 512 + lane;
    f32x4* red1 = reinterpret_cast<f32x4*>(stage1) + rg * 512 + lane;
    f32x4* red2 = reinterpret_cast<f32x4*>(stage2) + rg * 512 + lane;
    if (kh == 1) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        red0[64 * tt] = acc[0][tt];
        red1[64 * tt] = acc[1][tt];
        red2[64 * tt] = acc[2][tt];
      }
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        acc[0][tt] += red0[64 * tt];
        acc[1][tt] += red1[64 * tt];
        acc[2][tt] += red2[64 * tt];
      }
    }
    if constexpr (ROWT == 4) {
      __syncthreads();
      if (kh == 1) {
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) red0[64 * tt] = acc[ROWT - 1][tt];
      }
      __syncthreads();
      if (kh == 0) {
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) acc[ROWT - 1][tt] += red0[64 * tt];
      }
    }
  }

  // Blocks wholly inside the rows (m, or the branch's r in GEMM 1), with the
  // output and its row pitch 16-byte aligned, store through LDS
  // (workgroup-uniform): the first-half waves place their rows of every
  // token (fp16) in a token-major tile, tokens 0..63 in stage 0 and 64..127
  // in stage 1, then all waves store whole 16-byte pieces of each token's
  // contiguous run of rows, instead of 8-byte pieces 16 tokens apart.
  uint16_t* const out = MODE == 1 ? A.z + B0.zoff : A.y;
  const long ldo = MODE == 1 ? A.zs : A.ldy;
  const bool whole_rows = blk0 + 4 * ROWT <= ntiles && 16 * blk0 + 64 * ROWT <= (MODE == 1 ? B0.r : A.m) &&
                          (ldo & 7) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  constexpr int RS = 64 * ROWT + 8;  // halves per staged token (16 more: banks staggered)
  static_assert(64 * RS * 2 <= P2_STAGE_BYTES, "half the staged tile fits a stage");
  auto store_staged = [&](auto value) {
    __syncthreads();  // every reader of the reduction buffers is done
    if (kh == 0) {
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) {
        const int lr = 16 * (ROWT * rg + rt) + 4 * grp;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          uint16_t v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = value(rt, tt, q);
          uint8_t* st = tt < 4 ? stage0 : stage1;
          *reinterpret_cast<uint2*>(st + 2 * ((16 * (tt & 3) + col) * RS + lr)) = *reinterpret_cast<uint2*>(v);
        }
      }
    }
    __syncthreads();
    constexpr int CPT = 8 * ROWT;  // 16-byte pieces per token
    const int row0 = 16 * blk0;
    for (int e = threadIdx.x; e < PF_BN * CPT; e += 64 * P2_WAVES) {
      const int t = e / CPT, j = e - t * CPT;
      if (tok0 + t < M) {
        const uint8_t* st = t < 64 ? stage0 : stage1;
        *reinterpret_cast<uint4*>(out + (long)(tok0 + t) * ldo + row0 + 8 * j) =
            *reinterpret_cast<const uint4*>(st + 2 * ((t & 63) * RS + 8 * j));
      }
    }
  };
  if (MODE == 1 && whole_rows)
    store_staged([&](int rt, int tt, int q) { return f2h(h2f(B0.l[16 * (tile0 + rt) + 4 * grp + q]) * acc[rt][tt][q]); });
  if (MODE == 1) {
    const LbBranchArgs& B = B0;
    if (kh == 0 && !whole_rows) {
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) {
        const int tile = tile0 + rt;
        if (tile >= ntiles) continue;
        const int j0 = 16 * tile + 4 * grp;
        float lq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) lq[q] = (j0 + q < B.r) ? h2f(B.l[j0 + q]) : 0.f;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const int tok = tok0 + 16 * tt + col;
          if (tok >= M) continue;
          uint16_t zq[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) zq[q] = f2h(lq[q] * acc[rt][tt][q]);
          *reinterpret_cast<uint2*>(A.z + (long)tok * A.zs + B.zoff + j0) = *reinterpret_cast<uint2*>(zq);
        }
      }
    }
    // the block holding the last row tile also zeroes this token block's
    // z entries between 16*ceil(r/16) and 128*ceil(r/128)
    if (blk0 <= ntiles - 1 && ntiles - 1 < blk0 + 4 * ROWT) {
      const int j0 = 16 * ntiles, nz = 128 * ((B.r + 127) / 128) - j0;
      const int per_tok = nz >> 2;
      for (int e = threadIdx.x; e < per_tok * PF_BN; e += 64 * P2_WAVES) {
        const int tok = tok0 + e / per_tok;
        if (tok < M)
          *reinterpret_cast<uint2*>(A.z + (long)tok * A.zs + B.zoff + j0 + 4 * (e % per_tok)) = make_uint2(0u, 0u);
      }
    }
  } else if (whole_rows) {
    store_staged([&](int rt, int tt, int q) { return f2h(acc[rt][tt][q]); });
  } else if (kh == 0) {
#pragma unroll
    for (int rt = 0; rt < ROWT; ++rt) {
      const int tile = tile0 + rt;
      if (tile >= ntiles) continue;
      const int i0 = 16 * tile + 4 * grp;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int tok = tok0 + 16 * tt + col;
        if (tok >= M) continue;
        uint16_t* yp = A.y + (long)tok * A.ldy + i0;
        uint16_t yq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) yq[q] = f2h(acc[rt][tt][q]);
        if (i0 + 3 < A.m && ((uintptr_t)yp & 7) == 0) {
          *reinterpret_cast<uint2*>(yp) = *reinterpret_cast<uint2*>(yq);
        } else {
          for (int q = 0; q < 4; ++q)
            if (i0 + q < A.m) yp[q] = yq[q];
        }
      }
    }
  }
}

static int p2_cu_count() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    return 0;
  return ncu;
}

// Row geometry of lb_prefill2_kernel for GEMM `mode`: the first `split`
// row tiles (a multiple of 16) in 256-row blocks (4 tiles per wave), the
// rest in 192-row blocks (3 tiles per wave), chosen to minimise the rounds
// of one workgroup per compute unit weighted by rows per block.  Workgroups
// of the same height take about the same time, and each launch's
// workgroups start together, so a launch costs rounds x height.  E.g. the
// 7B layer's GEMM 1 (2 x 92 tiles, 16 token blocks): all in 192-row blocks,
// 256 workgroups, one round of 3 (against 192 workgroups, one round of 4);
// its GEMM 2 (688 tiles): 512 tiles in 256-row blocks (2 rounds of 4), 176
// in 192-row blocks (240 workgroups, 1 round of 3), against 3 rounds of 4.
// GEMM 1 is never split (its last block also clears z's padding).
static int p2_split(const LbPrefillArgs& a, int mode, unsigned tb) {
  const int T = p2_row_tiles(a, mode), ncu = p2_cu_count();
  const long nz = mode == 1 ? a.nb : 1;
  if (ncu == 0) return T;
  auto rounds = [&](long wgs) { return (wgs + ncu - 1) / ncu; };
  auto cost = [&](int split) {
    const long b4 = (split + 15) / 16, b3 = (T - split + 11) / 12;
    return rounds(b4 * tb * nz) * 4 + rounds(b3 * tb * nz) * 3;
  };
  int best = T;  // all in 256-row blocks
  long bc = cost(T);
  if (cost(0) < bc) best = 0, bc = cost(0);
  if (mode == 2)
    for (int sp = 16; sp < T; sp += 16)
      if (cost(sp) < bc) best = sp, bc = cost(sp);
  return best;
}

hipError_t lb_launch_prefill(const LbPrefillArgs& a, hipStream_t stream) {
  const unsigned tb = (unsigned)((a.M + PF_BN - 1) / PF_BN);
  int maxt = 0;
  for (int b = 0; b < a.nb; ++b) maxt = max(maxt, (a.br[b].r + 15) >> 4);
  const bool aligned_x = (((uintptr_t)a.x & 15) == 0) && (a.ldx % 8 == 0);
  // v2 addresses a token row by a 32-bit byte offset
  // (with 16 rows of slack: a slot offset is formed 16 rows ahead before its
  // range check)
  auto fits32 = [&](long ld, long width) { return ((long)(a.M + 16) * ld + width) * 2 < (1l << 32); };
  hipError_t e;
  if (aligned_x && a.n % 128 == 0 && fits32(a.ldx, a.n)) {
    // v2: GEMM 1 over both branches, then GEMM 2 (one-dimensional grids, see p2_tile)
    if (p2_split(a, 1, tb) == 0) {
      const int rb = p2_row_blocks(a, 1, 3);
      hipLaunchKernelGGL((lb_prefill2_kernel<1, 3>), dim3((unsigned)(rb * tb * a.nb)), dim3(64 * P2_WAVES), 0, stream,
                         a, 0, rb);
    } else {
      const int rb = p2_row_blocks(a, 1, 4);
      hipLaunchKernelGGL((lb_prefill2_kernel<1, 4>), dim3((unsigned)(rb * tb * a.nb)), dim3(64 * P2_WAVES), 0, stream,
                         a, 0, rb);
    }
  } else {
    const dim3 g1((unsigned)((maxt + 7) / 8), tb, (unsigned)a.nb);
    if (a.n % 8 == 0 && aligned_x)
      hipLaunchKernelGGL((lb_prefill_kernel<1, true>), g1, dim3(PF_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((lb_prefill_kernel<1, false>), g1, dim3(PF_THREADS), 0, stream, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // GEMM 2 reads z (always 16-byte aligned, zero-padded to whole chunks)
  const int mt = (a.m + 15) >> 4;
  if (fits32(a.zs, a.zs)) {
    const int T = p2_row_tiles(a, 2), split = p2_split(a, 2, tb);
    if (split > 0) {
      const int rb = (split + 15) / 16;
      hipLaunchKernelGGL((lb_prefill2_kernel<2, 4>), dim3((unsigned)(rb * tb)), dim3(64 * P2_WAVES), 0, stream, a, 0,
                         rb);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (split < T) {
      const int rb = (T - split + 11) / 12;
      hipLaunchKernelGGL((lb_prefill2_kernel<2, 3>), dim3((unsigned)(rb * tb)), dim3(64 * P2_WAVES), 0, stream, a,
                         split, rb);
    }
  } else
    hipLaunchKernelGGL((lb_prefill_kernel<2, true>), dim3((unsigned)((mt + 7) / 8), tb, 1), dim3(PF_THREADS), 0,
                       stream, a);
  return hipGetLastError();
}
