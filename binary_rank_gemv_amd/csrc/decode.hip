// Decode path (1..16 tokens) of the LittleBit layer on gfx950 matrix cores.
//
// Per branch (explainx.ai explainer, "How it works" items 1-3):
//   u = g*x (fp16), t = sign(V)^T u, z = l*t (fp16), s = sign(U) z, y = sum_b h_b*s_b.
// Each 16-row tile of a packed factor is one 16x16x32 matrix-core operand
// stream: tokens fill the 16 columns, 4 waves split the reduction, and the
// signs are expanded in registers by lb16_step_operand (one shift and one mask
// per two values).  Activations in the "negated class" (k & 2) are stored
// negated and their per-token sum is added back (t = acc + C_u, s = acc + D).
#include "lb_common.h"

namespace {

__device__ inline void find_vtile(const LbDecodeArgs& A, int t, int& li, int& b, int& tile) {
  li = 0; b = 0; tile = 0;
  for (int i = 0; i < A.nlayers; ++i)
    for (int bb = 0; bb < A.L[i].nb; ++bb) {
      const int nt = (A.L[i].br[bb].r + 15) >> 4;
      const int beg = A.L[i].vt_begin[bb];
      if (t >= beg && t < beg + nt) { li = i; b = bb; tile = t - beg; return; }
    }
}

__device__ inline void find_utile(const LbDecodeArgs& A, int t, int& li, int& tile) {
  li = 0; tile = 0;
  for (int i = 0; i < A.nlayers; ++i) {
    const int nt = (A.L[i].m + 15) >> 4;
    if (t >= A.L[i].ut_begin && t < A.L[i].ut_begin + nt) { li = i; tile = t - A.L[i].ut_begin; return; }
  }
}

// Sum over the `width` consecutive lanes that share a value (width = 1..64, power of 2).
__device__ inline float seg_sum(float v, int width) {
  for (int off = 1; off < width; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace

// --------------------------------------------------------------------- V pass
// One workgroup per 16-row tile of sign(V)^T of one branch; the reduction over
// the n inputs is cut into LDS chunks of `chunk_units` * 64 columns.
__global__ __launch_bounds__(256) void lb_decode_vpass(LbDecodeArgs A, int chunk_units) {
  extern __shared__ __align__(16) uint16_t u_lds[];
  __shared__ float red[4][256];
  __shared__ float part[256];
  __shared__ float cu[16];
  __shared__ float cs[256];

  int li, b, tile;
  find_vtile(A, blockIdx.x, li, b, tile);
  const int batch = A.batch;
  const int n = A.L[li].n;
  const long ldx = A.L[li].ldx;
  const uint16_t* __restrict__ x = A.L[li].x;
  const uint16_t* __restrict__ g = A.L[li].br[b].g;
  const uint16_t* __restrict__ l = A.L[li].br[b].l;
  const int r = A.L[li].br[b].r;
  const int nu = lb16_units(n);
  const uint8_t* __restrict__ tile_ptr = A.L[li].br[b].vbits + (long)tile * lb16_tile_bytes(n);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok = lane & 15, grp = lane >> 4;

  // threads per token for building u (power of two, >= 16)
  int lb = 0;
  while ((1 << lb) < batch) ++lb;
  const int tpt = 256 >> lb;
  const int my_tok = tid / tpt, my_sub = tid % tpt;
  float csum_u = 0.f;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int u0 = 0; u0 < nu; u0 += chunk_units) {
    const int u1 = min(nu, u0 + chunk_units);
    const int k0 = 64 * u0, kc = 64 * (u1 - u0);
    const int rowh = kc + 8;
    __syncthreads();
    // u = fp16(g*x), negated class stored negated, zero beyond n
    if (my_tok < batch) {
      for (int k8 = my_sub; k8 < (kc >> 3); k8 += tpt) {
        const int k = k0 + 8 * k8;
        uint16_t vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kk = k + e;
          float v = 0.f;
          if (kk < n) v = h2f(g[kk]) * h2f(x[(long)my_tok * ldx + kk]);
          const f16 hv = (f16)v;
          if (lb16_negated_class(kk)) {
            csum_u += (float)hv;
            vals[e] = __builtin_bit_cast(uint16_t, (f16)(-hv));
          } else {
            vals[e] = __builtin_bit_cast(uint16_t, hv);
          }
        }
        uint16_t* dst = u_lds + my_tok * rowh + 8 * k8;
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = vals[e];
      }
    }
    __syncthreads();
    // this wave's pairs of the chunk
    const int pb = u0 >> 1, pe = (u1 + 1) >> 1, np = pe - pb;
    const int p0 = pb + (wave * np) / 4, p1 = pb + ((wave + 1) * np) / 4;
    for (int p = p0; p < p1; ++p) {
      const uint32_t reg = lb16_reg_word(lb16_load_pair(tile_ptr, p, lane, nu));
      const int nsteps = (2 * p + 1 < nu) ? 4 : 2;
      for (int st = 0; st < nsteps; ++st) {
        const f16x8 av = lb16_step_operand(reg, st);
        f16x8 bv = {0, 0, 0, 0, 0, 0, 0, 0};
        if (tok < batch)
          bv = *reinterpret_cast<const f16x8*>(u_lds + tok * rowh + (32 * (4 * p + st) - k0) + 8 * grp);
        acc = mfma16(av, bv, acc);
      }
    }
  }
  // per-token sum of the negated-class u values (deterministic tree)
  part[tid] = seg_sum(csum_u, min(tpt, 64));
  __syncthreads();
  if (tid < 16) {
    float s = 0.f;
    if (tid < batch) {
      const int first = tid * tpt;
      for (int w = 0; w < tpt; w += 64) s += part[first + w];
    }
    cu[tid] = s;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(4 * grp + i) * 16 + tok] = acc[i];
  __syncthreads();

  // thread -> (row rho, token tk); rho fastest for contiguous z rows
  const int rho = tid & 15, tk = tid >> 4;
  const int j = 16 * tile + rho;
  const float t = red[0][rho * 16 + tk] + red[1][rho * 16 + tk] + red[2][rho * 16 + tk] +
                  red[3][rho * 16 + tk] + cu[tk];
  f16 zv = (f16)0.f;
  if (j < r) zv = (f16)(h2f(l[j]) * t);
  uint16_t* __restrict__ z = A.L[li].z;
  const int zs = A.L[li].zs, zoff = A.L[li].br[b].zoff;
  if (tk < batch)
    z[(long)tk * zs + zoff + j] = __builtin_bit_cast(uint16_t, lb16_negated_class(j) ? (f16)(-zv) : zv);
  cs[tk * 16 + rho] = (j < r && lb16_negated_class(j)) ? (float)zv : 0.f;
  __syncthreads();
  if (tid < 16) {
    float s = 0.f;
    for (int q = 0; q < 16; ++q) s += cs[tid * 16 + q];
    A.L[li].csum[A.L[li].br[b].csum_off + tile * 16 + tid] = s;
  }
  // the last tile also clears the z columns between 16*ceil(r/16) and 64*ceil(r/64)
  const int ntv = (r + 15) >> 4;
  if (tile == ntv - 1) {
    const int rp = 16 * ntv, kpu = 64 * lb16_units(r);
    const int cnt = (kpu - rp) * batch;
    for (int e = tid; e < cnt; e += 256) {
      const int tt = e / (kpu - rp), jj = rp + e % (kpu - rp);
      z[(long)tt * zs + zoff + jj] = 0;
    }
  }
}

// --------------------------------------------------------------------- U pass
// One workgroup per 16-row tile of the outputs of one layer; waves 0-1 take
// the primary branch and waves 2-3 the residual one (all four with one branch).
__global__ __launch_bounds__(256) void lb_decode_upass(LbDecodeArgs A) {
  __shared__ float red[4][256];
  __shared__ float dsum[2][16];

  int li, tile;
  find_utile(A, blockIdx.x, li, tile);
  const int batch = A.batch;
  const int nb = A.L[li].nb;
  const int m = A.L[li].m;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok = lane & 15, grp = lane >> 4;
  const uint16_t* __restrict__ z = A.L[li].z;
  const int zs = A.L[li].zs;

  // D_b[tok] = sum of the negated-class z of branch b (from the V-pass tile sums)
  if (wave == 0) {
    for (int bb = 0; bb < nb; ++bb) {
      const int ntv = (A.L[li].br[bb].r + 15) >> 4;
      const float* cs = A.L[li].csum + A.L[li].br[bb].csum_off;
      float s = 0.f;
      for (int T = grp; T < ntv; T += 4) s += cs[T * 16 + tok];
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      if (lane < 16) dsum[bb][lane] = s;
    }
  }

  const int b = (nb == 2) ? (wave >> 1) : 0;
  const int wsub = (nb == 2) ? (wave & 1) : wave;
  const int nsub = (nb == 2) ? 2 : 4;
  const int r = A.L[li].br[b].r;
  const int nu = lb16_units(r);
  const int np = (nu + 1) >> 1;
  const int p0 = (wsub * np) / nsub, p1 = ((wsub + 1) * np) / nsub;
  const uint8_t* __restrict__ tile_ptr = A.L[li].br[b].ubits + (long)tile * lb16_tile_bytes(r);
  const uint16_t* __restrict__ zrow = z + (long)tok * zs + A.L[li].br[b].zoff + 8 * grp;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int p = p0; p < p1; ++p) {
    const uint32_t reg = lb16_reg_word(lb16_load_pair(tile_ptr, p, lane, nu));
    const int nsteps = (2 * p + 1 < nu) ? 4 : 2;
    for (int st = 0; st < nsteps; ++st) {
      const f16x8 av = lb16_step_operand(reg, st);
      f16x8 bv = {0, 0, 0, 0, 0, 0, 0, 0};
      if (tok < batch) bv = *reinterpret_cast<const f16x8*>(zrow + 32 * (4 * p + st));
      acc = mfma16(av, bv, acc);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(4 * grp + i) * 16 + tok] = acc[i];
  __syncthreads();

  const int rho = tid & 15, tk = tid >> 4;
  const int i = 16 * tile + rho;
  if (tk < batch && i < m) {
    const int e = rho * 16 + tk;
    float y;
    if (nb == 2) {
      const float s0 = red[0][e] + red[1][e] + dsum[0][tk];
      const float s1 = red[2][e] + red[3][e] + dsum[1][tk];
      y = h2f(A.L[li].br[0].h[i]) * s0 + h2f(A.L[li].br[1].h[i]) * s1;
    } else {
      const float s0 = red[0][e] + red[1][e] + red[2][e] + red[3][e] + dsum[0][tk];
      y = h2f(A.L[li].br[0].h[i]) * s0;
    }
    A.L[li].y[(long)tk * A.L[li].ldy + i] = f2h(y);
  }
}

hipError_t lb_launch_decode(const LbDecodeArgs& args, int chunk_units, hipStream_t stream) {
  const size_t lds = (size_t)args.batch * (64 * chunk_units + 8) * sizeof(uint16_t);
  hipLaunchKernelGGL(lb_decode_vpass, dim3(args.nvt), dim3(256), lds, stream, args, chunk_units);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lb_decode_upass, dim3(args.nut), dim3(256), 0, stream, args);
  return hipGetLastError();
}
