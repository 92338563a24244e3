// Dual-SVID initialization of a layer's branches from a dense weight, on the
// GPU (liblittlebit_init.so, an offline library of its own) (the step before the layer; explainx.ai explainer, "How it works"
// item 3: a truncated SVD of the weights, its signs and magnitudes mapped
// into the parameters, and a residual branch fitted to what the first leaves).
//
// Per branch, with R the matrix to approximate (W, then the residual):
//   1. Gram matrix of R on its smaller side (rocBLAS dgemm) and its
//      eigendecomposition (rocSOLVER dsyevd): the top r eigenpairs give the
//      singular vectors on that side and the singular values;
//   2. the other side's vectors from R times those vectors; latent factors
//      U' = P S^(1/2), V' = Q S^(1/2); each component oriented so that the
//      largest-magnitude entry of its V' column (first index on ties) is
//      positive;
//   2b. optionally, a Joint-ITQ rotation of both latent factors (LittleBit-2
//      paragraph of the explainer: the latent factors aligned with the binary
//      hypercube before training), which leaves U' V'^T unchanged;
//   3. sign-value split of U' and of V': the rank-1 approximation a b^T of
//      |U'| (and of |V'|) by power iteration (non-negative leading singular
//      vectors), a = sqrt(sigma) p, b = sqrt(sigma) q; h = a_U, g = a_V,
//      l = b_U * b_V, rounded to fp16;
//   4. the residual R -= diag(h) sign(U') diag(l) sign(V')^T diag(g) with the
//      fp16 scales (the deployed branch).
// Everything runs in float64 on the device.  R is kept row-major m x n, which
// is column-major n x m (X = R^T) for rocBLAS.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <rocsolver/rocsolver.h>

#include <math.h>
#include <stdint.h>

#include <string>
#include <vector>

#include <stdarg.h>
#include <stdio.h>

#include "littlebit_init.h"

namespace {

constexpr int kThreads = 256;
constexpr int kPowerIters = 500;  // upper bound; stops when the singular value settles

__global__ void to_f64_kernel(const float* __restrict__ W, int64_t m, int64_t n, int64_t ldw,
                              double* __restrict__ X) {
  const int64_t total = m * n;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / n, k = e - i * n;
    X[e] = (double)W[i * ldw + k];
  }
}

// Y (k x r, column-major) column j = eigenvector of the (j+1)-th largest
// eigenvalue (columns of E, ascending); sig[j] = sqrt(max(lambda, 0)).
__global__ void take_top_kernel(const double* __restrict__ E, const double* __restrict__ D, int k, int r,
                                double* __restrict__ Y, double* __restrict__ sig) {
  const int j = blockIdx.x;
  const int src = k - 1 - j;
  for (int i = threadIdx.x; i < k; i += blockDim.x) Y[(int64_t)j * k + i] = E[(int64_t)src * k + i];
  if (threadIdx.x == 0) sig[j] = sqrt(fmax(D[src], 0.0));
}

// Column j of A (rows x r, column-major) times sig[j]^power (power +-0.5);
// a zero singular value gives a zero column.
__global__ void scale_cols_kernel(double* __restrict__ A, int64_t rows, int r, const double* __restrict__ sig,
                                  double power) {
  const int j = blockIdx.y;
  const double s = sig[j];
  const double f = s > 0.0 ? pow(s, power) : 0.0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += (int64_t)gridDim.x * blockDim.x)
    A[(int64_t)j * rows + i] *= f;
}

// Orientation of component j: the largest-magnitude entry of V' column j
// (first index on ties) becomes positive; U' column j follows.
__global__ void orient_kernel(double* __restrict__ U, int64_t m, double* __restrict__ V, int64_t n) {
  const int j = blockIdx.x;
  double* v = V + (int64_t)j * n;
  __shared__ double best[kThreads];
  __shared__ int64_t bidx[kThreads];
  double b = -1.0;
  int64_t bi = 0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const double a = fabs(v[i]);
    if (a > b) {
      b = a;
      bi = i;
    }
  }
  best[threadIdx.x] = b;
  bidx[threadIdx.x] = bi;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      const double o = best[threadIdx.x + s];
      const int64_t oi = bidx[threadIdx.x + s];
      if (o > best[threadIdx.x] || (o == best[threadIdx.x] && oi < bidx[threadIdx.x])) {
        best[threadIdx.x] = o;
        bidx[threadIdx.x] = oi;
      }
    }
    __syncthreads();
  }
  const bool flip = v[bidx[0]] < 0.0;
  __syncthreads();
  if (flip) {
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) v[i] = -v[i];
    double* u = U + (int64_t)j * m;
    for (int64_t i = threadIdx.x; i < m; i += blockDim.x) u[i] = -u[i];
  }
}

__global__ void abs_kernel(const double* __restrict__ A, int64_t total, double* __restrict__ B) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x)
    B[e] = fabs(A[e]);
}

__global__ void fill_kernel(double* __restrict__ a, int64_t count, double v) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count; e += (int64_t)gridDim.x * blockDim.x)
    a[e] = v;
}

// fp16 bits of x, rounded to nearest even from float64 (one rounding).
__device__ uint16_t f64_to_f16_bits(double x) {
  const uint16_t sgn = signbit(x) ? 0x8000u : 0u;
  double a = fabs(x);
  if (isnan(a)) return (uint16_t)(sgn | 0x7E00u);
  if (a >= 65520.0) return (uint16_t)(sgn | 0x7C00u);  // rounds to infinity
  if (a < 6.103515625e-05) {                           // below the smallest normal, 2^-14
    const double q = rint(a * 16777216.0);               // units of 2^-24, exact product
    return (uint16_t)(sgn | (uint16_t)q);                // q == 1024 is the smallest normal
  }
  int e;
  const double f = frexp(a, &e);  // a = f 2^e, f in [0.5, 1)
  double q = rint((2.0 * f - 1.0) * 1024.0);
  int ex = e - 1;
  if (q >= 1024.0) {
    q = 0.0;
    ex += 1;
  }
  if (ex > 15) return (uint16_t)(sgn | 0x7C00u);
  return (uint16_t)(sgn | (uint16_t)((ex + 15) << 10) | (uint16_t)q);
}

__device__ double f16_bits_to_f64(uint16_t b) { return (double)__builtin_bit_cast(_Float16, b); }

// Scales of one factor from the power iteration: out[i] = fp16(sqrt(s) v[i]).
__global__ void scale_out_kernel(const double* __restrict__ v, int64_t count, double s, uint16_t* __restrict__ out) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count; e += (int64_t)gridDim.x * blockDim.x)
    out[e] = f64_to_f16_bits(sqrt(s) * v[e]);
}

// l = fp16(sqrt(sU) qU[j] * sqrt(sV) qV[j])
__global__ void l_out_kernel(const double* __restrict__ qU, double sU, const double* __restrict__ qV, double sV, int r,
                             uint16_t* __restrict__ l) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < r; j += gridDim.x * blockDim.x)
    l[j] = f64_to_f16_bits((sqrt(sU) * qU[j]) * (sqrt(sV) * qV[j]));
}

// Latent output: dst (rows x r, row-major fp32) from src (column-major f64).
__global__ void latent_out_kernel(const double* __restrict__ src, int64_t rows, int r, float* __restrict__ dst) {
  const int64_t total = rows * r;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / r, j = e - i * r;
    dst[e] = (float)src[(int64_t)j * rows + i];
  }
}

// The deployed branch's factors for the residual update, from the fp32
// latents (the signs the layer packs) and the fp16 scales:
// A[i, j] = h_i s^U_ij l_j (m x r), B[k, j] = g_k s^V_kj (n x r), column-major.
__global__ void deployed_factors_kernel(const float* __restrict__ Ul, const uint16_t* __restrict__ h,
                                        const uint16_t* __restrict__ l, int64_t m, const float* __restrict__ Vl,
                                        const uint16_t* __restrict__ g, int64_t n, int r, double* __restrict__ A,
                                        double* __restrict__ B) {
  const int64_t ta = m * r, tb = n * r;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < ta + tb; e += (int64_t)gridDim.x * blockDim.x) {
    if (e < ta) {
      const int64_t j = e / m, i = e - j * m;
      const double s = Ul[i * r + j] < 0.f ? -1.0 : 1.0;
      A[e] = f16_bits_to_f64(h[i]) * s * f16_bits_to_f64(l[j]);
    } else {
      const int64_t f = e - ta;
      const int64_t j = f / n, k = f - j * n;
      const double s = Vl[k * r + j] < 0.f ? -1.0 : 1.0;
      B[f] = f16_bits_to_f64(g[k]) * s;
    }
  }
}

__global__ void identity_kernel(double* __restrict__ R, int r) {
  const int64_t total = (int64_t)r * r;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x)
    R[e] = (e / r == e % r) ? 1.0 : 0.0;
}

// A = sign(A) as +-1 (-1 iff < 0), in place
__global__ void sign_kernel(double* __restrict__ A, int64_t total) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x)
    A[e] = A[e] < 0.0 ? -1.0 : 1.0;
}

int grid_for(int64_t total) {
  const int64_t g = (total + kThreads - 1) / kThreads;
  return (int)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};

}  // namespace

// Leading singular triplet of the non-negative matrix M (rows x r,
// column-major) by power iteration from the all-ones direction: q unit (r),
// p unit (rows), returns sigma.  p and q stay non-negative.
static int power_rank1(rocblas_handle hb, hipStream_t stream, const double* M, int64_t rows, int r, double* p,
                       double* q, double& sigma, std::string& err) {
  hipLaunchKernelGGL(fill_kernel, dim3(grid_for(r)), dim3(kThreads), 0, stream, q, (int64_t)r, 1.0 / sqrt((double)r));
  double prev = -1.0;
  sigma = 0.0;
  const double one = 1.0, zero = 0.0;
  for (int it = 0; it < kPowerIters; ++it) {
    double np = 0.0, nq = 0.0;
    if (rocblas_dgemv(hb, rocblas_operation_none, (rocblas_int)rows, r, &one, M, (rocblas_int)rows, q, 1, &zero, p, 1) !=
            rocblas_status_success ||
        rocblas_dnrm2(hb, (rocblas_int)rows, p, 1, &np) != rocblas_status_success) {
      err = "rocBLAS dgemv/dnrm2 failed in the rank-1 fit";
      return LB_ERR_HIP;
    }
    if (!(np > 0.0)) {  // M is zero: every scale is zero
      sigma = 0.0;
      return 0;
    }
    const double inv_p = 1.0 / np;
    if (rocblas_dscal(hb, (rocblas_int)rows, &inv_p, p, 1) != rocblas_status_success ||
        rocblas_dgemv(hb, rocblas_operation_transpose, (rocblas_int)rows, r, &one, M, (rocblas_int)rows, p, 1, &zero, q,
                      1) != rocblas_status_success ||
        rocblas_dnrm2(hb, r, q, 1, &nq) != rocblas_status_success) {
      err = "rocBLAS dscal/dgemv/dnrm2 failed in the rank-1 fit";
      return LB_ERR_HIP;
    }
    const double inv_q = 1.0 / nq;
    if (rocblas_dscal(hb, r, &inv_q, q, 1) != rocblas_status_success) {
      err = "rocBLAS dscal failed in the rank-1 fit";
      return LB_ERR_HIP;
    }
    sigma = nq;
    if (fabs(sigma - prev) <= 1e-15 * sigma) break;
    prev = sigma;
  }
  return 0;
}

static int lb_run_dual_svid(const float* W, int64_t m, int64_t n, int64_t ldw, int r, int nbranches, int itq_iters,
                     const lb_init_branch* out, hipStream_t stream, std::string& err) {
  const int64_t k = m < n ? m : n;
  const bool gram_on_n = n <= m;  // eigenvectors on the input side (V) when n <= m
  auto alloc = [&](DevBuf& b, size_t bytes) {
    return hipMalloc(&b.p, bytes > 0 ? bytes : 8) == hipSuccess;
  };
  DevBuf X, G, D, E, Y, sig, Ud, Vd, Mabs, p, q, qU, A, B, info, Rm, Mm, Su, Svt, Sv, Ee;
  const size_t dz = sizeof(double);
  const int64_t mr = (m > n ? m : n) * (int64_t)r;
  if (!alloc(X, (size_t)(m * n) * dz) || !alloc(G, (size_t)(k * k) * dz) || !alloc(D, (size_t)k * dz) ||
      !alloc(E, (size_t)k * dz) || !alloc(Y, (size_t)(k * r) * dz) || !alloc(sig, (size_t)r * dz) ||
      !alloc(Ud, (size_t)(m * r) * dz) || !alloc(Vd, (size_t)(n * r) * dz) || !alloc(Mabs, (size_t)mr * dz) ||
      !alloc(p, (size_t)(m > n ? m : n) * dz) || !alloc(q, (size_t)r * dz) || !alloc(qU, (size_t)r * dz) ||
      !alloc(A, (size_t)(m * r) * dz) || !alloc(B, (size_t)(n * r) * dz) || !alloc(info, sizeof(rocblas_int)) ||
      !alloc(Rm, itq_iters > 0 ? (size_t)r * r * dz : 8) || !alloc(Mm, itq_iters > 0 ? (size_t)r * r * dz : 8) ||
      !alloc(Su, itq_iters > 0 ? (size_t)r * r * dz : 8) || !alloc(Svt, itq_iters > 0 ? (size_t)r * r * dz : 8) ||
      !alloc(Sv, itq_iters > 0 ? (size_t)r * dz : 8) || !alloc(Ee, itq_iters > 0 ? (size_t)r * dz : 8)) {
    err = "device allocation for the initialization failed";
    return LB_ERR_HIP;
  }
  rocblas_handle hb = nullptr;
  if (rocblas_create_handle(&hb) != rocblas_status_success) {
    err = "rocblas_create_handle failed";
    return LB_ERR_HIP;
  }
  struct HandleGuard {
    rocblas_handle h;
    ~HandleGuard() { rocblas_destroy_handle(h); }
  } guard{hb};
  if (rocblas_set_stream(hb, stream) != rocblas_status_success ||
      rocblas_set_pointer_mode(hb, rocblas_pointer_mode_host) != rocblas_status_success) {
    err = "rocblas stream/pointer-mode setup failed";
    return LB_ERR_HIP;
  }
  double* Xd = (double*)X.p;
  double* Gd = (double*)G.p;
  double* Yd = (double*)Y.p;
  double* Ub = (double*)Ud.p;
  double* Vb = (double*)Vd.p;
  double* sg = (double*)sig.p;
  hipLaunchKernelGGL(to_f64_kernel, dim3(grid_for(m * n)), dim3(kThreads), 0, stream, W, m, n, ldw, Xd);
  const double one = 1.0, zero = 0.0, minus_one = -1.0;
  for (int b = 0; b < nbranches; ++b) {
    // 1. Gram matrix of the smaller side and its eigenpairs
    rocblas_status st;
    if (gram_on_n)
      st = rocblas_dgemm(hb, rocblas_operation_none, rocblas_operation_transpose, (rocblas_int)n, (rocblas_int)n,
                         (rocblas_int)m, &one, Xd, (rocblas_int)n, Xd, (rocblas_int)n, &zero, Gd, (rocblas_int)n);
    else
      st = rocblas_dgemm(hb, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)m, (rocblas_int)m,
                         (rocblas_int)n, &one, Xd, (rocblas_int)n, Xd, (rocblas_int)n, &zero, Gd, (rocblas_int)m);
    if (st != rocblas_status_success) {
      err = "rocBLAS dgemm (Gram matrix) failed";
      return LB_ERR_HIP;
    }
    st = rocsolver_dsyevd(hb, rocblas_evect_original, rocblas_fill_upper, (rocblas_int)k, Gd, (rocblas_int)k,
                          (double*)D.p, (double*)E.p, (rocblas_int*)info.p);
    rocblas_int hinfo = 0;
    if (st != rocblas_status_success ||
        hipMemcpyAsync(&hinfo, info.p, sizeof hinfo, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess || hinfo != 0) {
      err = "rocSOLVER dsyevd failed (status " + std::to_string((int)st) + ", info " + std::to_string((int)hinfo) + ")";
      return LB_ERR_HIP;
    }
    hipLaunchKernelGGL(take_top_kernel, dim3(r), dim3(kThreads), 0, stream, Gd, (const double*)D.p, (int)k, r, Yd, sg);
    // 2. latent factors, oriented
    if (gram_on_n) {
      // V side: Y (n x r); U' = R Y S^(-1/2) = X^T Y S^(-1/2); V' = Y S^(1/2)
      st = rocblas_dgemm(hb, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)m, r, (rocblas_int)n,
                         &one, Xd, (rocblas_int)n, Yd, (rocblas_int)n, &zero, Ub, (rocblas_int)m);
      if (hipMemcpyAsync(Vb, Yd, (size_t)(n * r) * dz, hipMemcpyDeviceToDevice, stream) != hipSuccess) {
        err = "device copy failed";
        return LB_ERR_HIP;
      }
      hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for(m) < 64 ? grid_for(m) : 64, r), dim3(kThreads), 0, stream, Ub,
                         m, r, (const double*)sg, -0.5);
      hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for(n) < 64 ? grid_for(n) : 64, r), dim3(kThreads), 0, stream, Vb,
                         n, r, (const double*)sg, 0.5);
    } else {
      // U side: Y (m x r); V' = R^T Y S^(-1/2) = X Y S^(-1/2); U' = Y S^(1/2)
      st = rocblas_dgemm(hb, rocblas_operation_none, rocblas_operation_none, (rocblas_int)n, r, (rocblas_int)m, &one, Xd,
                         (rocblas_int)n, Yd, (rocblas_int)m, &zero, Vb, (rocblas_int)n);
      if (hipMemcpyAsync(Ub, Yd, (size_t)(m * r) * dz, hipMemcpyDeviceToDevice, stream) != hipSuccess) {
        err = "device copy failed";
        return LB_ERR_HIP;
      }
      hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for(n) < 64 ? grid_for(n) : 64, r), dim3(kThreads), 0, stream, Vb,
                         n, r, (const double*)sg, -0.5);
      hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for(m) < 64 ? grid_for(m) : 64, r), dim3(kThreads), 0, stream, Ub,
                         m, r, (const double*)sg, 0.5);
    }
    if (st != rocblas_status_success) {
      err = "rocBLAS dgemm (second factor) failed";
      return LB_ERR_HIP;
    }
    hipLaunchKernelGGL(orient_kernel, dim3(r), dim3(kThreads), 0, stream, Ub, m, Vb, n);
    // 2b. Joint-ITQ rotation shared by both factors (the product U' V'^T is
    // unchanged): from R = I, B = sign([U'; V'] R), then R = P Q^T for the
    // SVD P S Q^T of M = U'^T B_U + V'^T B_V (taken as the polar factor
    // M (M^T M)^(-1/2)); finally U' <- U' R, V' <- V' R
    if (itq_iters > 0) {
      double* Ad = (double*)A.p;
      double* Bd = (double*)B.p;
      double* R = (double*)Rm.p;
      double* M = (double*)Mm.p;
      hipLaunchKernelGGL(identity_kernel, dim3(grid_for((int64_t)r * r)), dim3(kThreads), 0, stream, R, r);
      for (int it = 0; it < itq_iters; ++it) {
        rocblas_status s1 = rocblas_dgemm(hb, rocblas_operation_none, rocblas_operation_none, (rocblas_int)m, r, r, &one,
                                          Ub, (rocblas_int)m, R, r, &zero, Ad, (rocblas_int)m);
        rocblas_status s2 = rocblas_dgemm(hb, rocblas_operation_none, rocblas_operation_none, (rocblas_int)n, r, r, &one,
                                          Vb, (rocblas_int)n, R, r, &zero, Bd, (rocblas_int)n);
        hipLaunchKernelGGL(sign_kernel, dim3(grid_for(m * r)), dim3(kThreads), 0, stream, Ad, m * r);
        hipLaunchKernelGGL(sign_kernel, dim3(grid_for(n * r)), dim3(kThreads), 0, stream, Bd, n * r);
        rocblas_status s3 = rocblas_dgemm(hb, rocblas_operation_transpose, rocblas_operation_none, r, r, (rocblas_int)m,
                                          &one, Ub, (rocblas_int)m, Ad, (rocblas_int)m, &zero, M, r);
        rocblas_status s4 = rocblas_dgemm(hb, rocblas_operation_transpose, rocblas_operation_none, r, r, (rocblas_int)n,
                                          &one, Vb, (rocblas_int)n, Bd, (rocblas_int)n, &one, M, r);
        // R = polar factor of M = M (M^T M)^(-1/2) = P Q^T for M = P S Q^T:
        // N = M^T M = E diag(lambda) E^T (dsyevd), F = E diag(lambda^(-1/4)),
        // R = (M F) F^T
        double* N = (double*)Su.p;
        double* T1 = (double*)Svt.p;
        rocblas_status s5 = rocblas_dgemm(hb, rocblas_operation_transpose, rocblas_operation_none, r, r, r, &one, M, r,
                                          M, r, &zero, N, r);
        rocblas_status s6 = rocsolver_dsyevd(hb, rocblas_evect_original, rocblas_fill_upper, r, N, r, (double*)Sv.p,
                                             (double*)Ee.p, (rocblas_int*)info.p);
        rocblas_int sinfo = 0;
        if (s1 || s2 || s3 || s4 || s5 || s6 ||
            hipMemcpyAsync(&sinfo, info.p, sizeof sinfo, hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess || sinfo != 0) {
          err = "Joint-ITQ step failed (rocBLAS/rocSOLVER dsyevd, info " + std::to_string((int)sinfo) + ")";
          return LB_ERR_HIP;
        }
        hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for(r) < 64 ? grid_for(r) : 64, r), dim3(kThreads), 0, stream, N,
                           (int64_t)r, r, (const double*)Sv.p, -0.25);
        if (rocblas_dgemm(hb, rocblas_operation_none, rocblas_operation_none, r, r, r, &one, M, r, N, r, &zero, T1, r) !=
                rocblas_status_success ||
            rocblas_dgemm(hb, rocblas_operation_none, rocblas_operation_transpose, r, r, r, &one, T1, r, N, r, &zero, R,
                          r) != rocblas_status_success) {
          err = "rocBLAS dgemm (rotation) failed";
          return LB_ERR_HIP;
        }
      }
      if (rocblas_dgemm(hb, rocblas_operation_none, rocblas_operation_none, (rocblas_int)m, r, r, &one, Ub,
                        (rocblas_int)m, R, r, &zero, Ad, (rocblas_int)m) != rocblas_status_success ||
          rocblas_dgemm(hb, rocblas_operation_none, rocblas_operation_none, (rocblas_int)n, r, r, &one, Vb,
                        (rocblas_int)n, R, r, &zero, Bd, (rocblas_int)n) != rocblas_status_success ||
          hipMemcpyAsync(Ub, Ad, (size_t)(m * r) * dz, hipMemcpyDeviceToDevice, stream) != hipSuccess ||
          hipMemcpyAsync(Vb, Bd, (size_t)(n * r) * dz, hipMemcpyDeviceToDevice, stream) != hipSuccess) {
        err = "applying the Joint-ITQ rotation failed";
        return LB_ERR_HIP;
      }
    }
    // 3. sign-value split of both factors
    double sU = 0.0, sV = 0.0;
    hipLaunchKernelGGL(abs_kernel, dim3(grid_for(m * r)), dim3(kThreads), 0, stream, (const double*)Ub, m * r,
                       (double*)Mabs.p);
    int rc = power_rank1(hb, stream, (const double*)Mabs.p, m, r, (double*)p.p, (double*)qU.p, sU, err);
    if (rc) return rc;
    hipLaunchKernelGGL(scale_out_kernel, dim3(grid_for(m)), dim3(kThreads), 0, stream, (const double*)p.p, m, sU, out[b].h);
    hipLaunchKernelGGL(abs_kernel, dim3(grid_for(n * r)), dim3(kThreads), 0, stream, (const double*)Vb, n * r,
                       (double*)Mabs.p);
    rc = power_rank1(hb, stream, (const double*)Mabs.p, n, r, (double*)p.p, (double*)q.p, sV, err);
    if (rc) return rc;
    hipLaunchKernelGGL(scale_out_kernel, dim3(grid_for(n)), dim3(kThreads), 0, stream, (const double*)p.p, n, sV, out[b].g);
    hipLaunchKernelGGL(l_out_kernel, dim3(grid_for(r)), dim3(kThreads), 0, stream, (const double*)qU.p, sU,
                       (const double*)q.p, sV, r, out[b].l);
    hipLaunchKernelGGL(latent_out_kernel, dim3(grid_for(m * r)), dim3(kThreads), 0, stream, (const double*)Ub, m, r,
                       out[b].U);
    hipLaunchKernelGGL(latent_out_kernel, dim3(grid_for(n * r)), dim3(kThreads), 0, stream, (const double*)Vb, n, r,
                       out[b].V);
    // 4. residual for the next branch: X -= B A^T (R -= A B^T)
    if (b + 1 < nbranches) {
      hipLaunchKernelGGL(deployed_factors_kernel, dim3(grid_for((m + n) * r)), dim3(kThreads), 0, stream,
                         (const float*)out[b].U, (const uint16_t*)out[b].h, (const uint16_t*)out[b].l, m,
                         (const float*)out[b].V, (const uint16_t*)out[b].g, n, r, (double*)A.p, (double*)B.p);
      if (rocblas_dgemm(hb, rocblas_operation_none, rocblas_operation_transpose, (rocblas_int)n, (rocblas_int)m, r,
                        &minus_one, (const double*)B.p, (rocblas_int)n, (const double*)A.p, (rocblas_int)m, &one, Xd,
                        (rocblas_int)n) != rocblas_status_success) {
        err = "rocBLAS dgemm (residual) failed";
        return LB_ERR_HIP;
      }
    }
  }
  const hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    err = std::string("initialization: ") + hipGetErrorString(e);
    return LB_ERR_HIP;
  }
  return 0;
}

// ------------------------------------------------------------------ C ABI
namespace {

thread_local std::string g_init_error;

lb_status init_fail(lb_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_init_error = buf;
  return s;
}

constexpr int kInitMaxRank = 4096;
constexpr int kInitMaxDim = 32768;

}  // namespace

extern "C" {

lb_status littlebit_dual_svid_init(const float* W, int64_t m, int64_t n, int64_t ldw, int64_t r, int nbranches,
                                   int itq_iters, const lb_init_branch* out, void* stream) {
  if (!W || !out) return init_fail(LB_ERR_INVALID_ARG, "littlebit_dual_svid_init: NULL pointer");
  if (m < 1 || n < 1 || ldw < n)
    return init_fail(LB_ERR_INVALID_ARG, "littlebit_dual_svid_init: m=%lld n=%lld ldw=%lld", (long long)m,
                     (long long)n, (long long)ldw);
  if (nbranches < 1 || nbranches > 2)
    return init_fail(LB_ERR_INVALID_ARG, "littlebit_dual_svid_init: nbranches=%d (1 or 2)", nbranches);
  if (r < 1 || r > (m < n ? m : n) || r > kInitMaxRank)
    return init_fail(LB_ERR_INVALID_ARG, "littlebit_dual_svid_init: r=%lld outside 1..min(m, n, %d)", (long long)r,
                     kInitMaxRank);
  if (m > kInitMaxDim || n > kInitMaxDim)
    return init_fail(LB_ERR_UNSUPPORTED, "littlebit_dual_svid_init: m, n <= %d", kInitMaxDim);
  if (itq_iters < 0 || itq_iters > 1000)
    return init_fail(LB_ERR_INVALID_ARG, "littlebit_dual_svid_init: itq_iters=%d outside 0..1000", itq_iters);
  for (int b = 0; b < nbranches; ++b)
    if (!out[b].U || !out[b].V || !out[b].h || !out[b].l || !out[b].g)
      return init_fail(LB_ERR_INVALID_ARG, "littlebit_dual_svid_init: NULL output of branch %d", b);
  std::string err;
  const int rc = lb_run_dual_svid(W, m, n, ldw, (int)r, nbranches, itq_iters, out, (hipStream_t)stream, err);
  if (rc != 0) return init_fail((lb_status)rc, "littlebit_dual_svid_init: %s", err.c_str());
  return LB_OK;
}

const char* littlebit_init_last_error(void) { return g_init_error.c_str(); }

}  // extern "C"
