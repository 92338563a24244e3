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
    // z entries between 16*ceil(r/16) and 64*ceil(r/64)
    if ((int)blockIdx.x == (ntiles - 1) >> 3) {
      const int j0 = 16 * ntiles, nz = 64 * lb16_units(B.r) - j0;  // a multiple of 16
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

hipError_t lb_launch_prefill(const LbPrefillArgs& a, hipStream_t stream) {
  const unsigned tb = (unsigned)((a.M + PF_BN - 1) / PF_BN);
  int maxt = 0;
  for (int b = 0; b < a.nb; ++b) maxt = max(maxt, (a.br[b].r + 15) >> 4);
  const bool fast = (a.n % 8 == 0) && (((uintptr_t)a.x & 15) == 0) && (a.ldx % 8 == 0);
  const dim3 g1((unsigned)((maxt + 7) / 8), tb, (unsigned)a.nb);
  if (fast)
    hipLaunchKernelGGL((lb_prefill_kernel<1, true>), g1, dim3(PF_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((lb_prefill_kernel<1, false>), g1, dim3(PF_THREADS), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2((unsigned)((((a.m + 15) >> 4) + 7) / 8), tb, 1);
  hipLaunchKernelGGL((lb_prefill_kernel<2, true>), g2, dim3(PF_THREADS), 0, stream, a);
  return hipGetLastError();
}
