// LB16 packing of latent signs (explainx.ai explainer, "How it works" item 1:
// inference keeps only the signs of the thin factors, one bit per entry).
// One thread builds one 32-bit pair word (or the odd last 16-bit unit) of one
// lane of one tile.
#include "lb_common.h"

template <typename T>
__device__ inline bool lb_is_negative(T v) {
  return (float)v < 0.0f;  // +0, -0 and NaN are not negative
}

template <typename T>
__global__ __launch_bounds__(256) void lb_pack_kernel(const T* __restrict__ latent, long ld,
                                                      int transpose, int R, int K,
                                                      uint8_t* __restrict__ dst) {
  const int nu = lb16_units(K);
  const int npairs = (nu + 1) >> 1;
  const long per_tile = 64L * npairs;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int ntiles = (R + 15) >> 4;
  if (gid >= per_tile * ntiles) return;
  const int tile = (int)(gid / per_tile);
  const int rem = (int)(gid - (long)tile * per_tile);
  const int p = rem >> 6;       // pair index
  const int lane = rem & 63;
  const int row = 16 * tile + (lane & 15);
  const int grp = lane >> 4;

  uint32_t word = 0;
  const int nunits = (2 * p + 1 < nu) ? 2 : 1;
  for (int half = 0; half < nunits; ++half) {
    const int u = 2 * p + half;
    uint32_t unit = 0;
    for (int q = 0; q < 2; ++q) {
      const int step = 2 * u + q;
      for (int e = 0; e < 8; ++e) {
        const int k = 32 * step + 8 * grp + e;
        bool neg = false;
        if (row < R && k < K) {
          const T v = transpose ? latent[(long)k * ld + row] : latent[(long)row * ld + k];
          neg = lb_is_negative(v);
        }
        if (neg) unit |= 1u << (8 * (e & 1) + 7 - (4 * q + (e >> 1)));
      }
    }
    word |= unit << (16 * half);
  }
  uint8_t* tile_ptr = dst + (long)tile * lb16_tile_bytes(K);
  const int off = 256 * p + (nunits == 2 ? 4 : 2) * lane;
  if (nunits == 2)
    *reinterpret_cast<uint32_t*>(tile_ptr + off) = word;
  else
    *reinterpret_cast<uint16_t*>(tile_ptr + off) = (uint16_t)word;
}

hipError_t lb_launch_pack(const void* latent, int is_f16, long ld, int transpose, int R, int K,
                          void* dst, hipStream_t stream) {
  const int nu = lb16_units(K);
  const long threads = 64L * ((nu + 1) >> 1) * ((R + 15) >> 4);
  const long blocks = (threads + 255) / 256;
  if (is_f16)
    hipLaunchKernelGGL(lb_pack_kernel<f16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const f16*)latent, ld, transpose, R, K, (uint8_t*)dst);
  else
    hipLaunchKernelGGL(lb_pack_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const float*)latent, ld, transpose, R, K, (uint8_t*)dst);
  return hipGetLastError();
}

// ------------------------------------------------------------------ transpose
// The packing of the K x R transpose of a packed R x K factor (the
// backward-input product of quantization-aware training, explainx.ai
// explainer, "How it works" item 3, runs the layer transposed: sign(U) in
// the V role and sign(V) in the U role).  One thread builds one output pair
// word (or odd unit) from single-bit reads of the input.

// Bit (row, k) of a packed factor with reduction length K (1 = negative).
__device__ inline uint32_t lb16_read_bit(const uint8_t* __restrict__ src, int K, int row, int k) {
  const int nu = lb16_units(K);
  const int s = k >> 5, grp = (k >> 3) & 3, e = k & 7;
  const int lane = (row & 15) + 16 * grp;
  const int u = s >> 1, q = s & 1, p = u >> 1;
  const uint8_t* tp = src + (long)(row >> 4) * lb16_tile_bytes(K);
  uint32_t unit;
  if (2 * p + 1 < nu) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(tp + 256 * p + 4 * lane);
    unit = (u & 1) ? (w >> 16) : (w & 0xFFFFu);
  } else {
    unit = *reinterpret_cast<const uint16_t*>(tp + 256 * p + 2 * lane);
  }
  return (unit >> (8 * (e & 1) + 7 - (4 * q + (e >> 1)))) & 1u;
}

__global__ __launch_bounds__(256) void lb_transpose_kernel(const uint8_t* __restrict__ src, int R, int K,
                                                           uint8_t* __restrict__ dst) {
  // output factor: R' = K rows, reduction length K' = R
  const int Ro = K, Ko = R;
  const int nu = lb16_units(Ko);
  const int npairs = (nu + 1) >> 1;
  const long per_tile = 64L * npairs;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int ntiles = (Ro + 15) >> 4;
  if (gid >= per_tile * ntiles) return;
  const int tile = (int)(gid / per_tile);
  const int rem = (int)(gid - (long)tile * per_tile);
  const int p = rem >> 6;
  const int lane = rem & 63;
  const int row = 16 * tile + (lane & 15);
  const int grp = lane >> 4;

  uint32_t word = 0;
  const int nunits = (2 * p + 1 < nu) ? 2 : 1;
  for (int half = 0; half < nunits; ++half) {
    const int u = 2 * p + half;
    uint32_t unit = 0;
    for (int q = 0; q < 2; ++q) {
      const int step = 2 * u + q;
      for (int e = 0; e < 8; ++e) {
        const int k = 32 * step + 8 * grp + e;
        if (row < Ro && k < Ko && lb16_read_bit(src, K, k, row))
          unit |= 1u << (8 * (e & 1) + 7 - (4 * q + (e >> 1)));
      }
    }
    word |= unit << (16 * half);
  }
  uint8_t* tile_ptr = dst + (long)tile * lb16_tile_bytes(Ko);
  const int off = 256 * p + (nunits == 2 ? 4 : 2) * lane;
  if (nunits == 2)
    *reinterpret_cast<uint32_t*>(tile_ptr + off) = word;
  else
    *reinterpret_cast<uint16_t*>(tile_ptr + off) = (uint16_t)word;
}

hipError_t lb_launch_transpose_packed(const void* src, int R, int K, void* dst, hipStream_t stream) {
  const int nu = lb16_units(R);  // the output's reduction length is R
  const long threads = 64L * ((nu + 1) >> 1) * ((K + 15) >> 4);
  const long blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(lb_transpose_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint8_t*)src, R, K,
                     (uint8_t*)dst);
  return hipGetLastError();
}
