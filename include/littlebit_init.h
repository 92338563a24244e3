/*
 * littlebit_init.h -- offline initialization of LittleBit layer branches on
 * MI355X (gfx950): the step before the layer, which turns a dense weight
 * into the latent factors and fp16 scales that littlebit_pack and the layer
 * (littlebit.h) consume.
 *
 * A library of its own (liblittlebit_init.so), separate from the layer
 * library: it links rocBLAS and rocSOLVER, allocates device memory and
 * synchronises the stream, none of which the layer calls do.
 */
#ifndef LITTLEBIT_INIT_H
#define LITTLEBIT_INIT_H

#include "littlebit.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Dual-SVID initialization (explainx.ai explainer, "How it works" item 3:
 * training starts from a truncated SVD of the real weights whose signs and
 * magnitudes are mapped into the layer's parameters, and the second,
 * residual branch is fitted to the part of W the first leaves over).  It
 * turns a dense weight into branches for littlebit_pack and the layer.
 *
 * Per branch, from R (W for the first branch, then W minus the deployed
 * earlier branches): the rank-r truncated SVD R ~ P S Q^T gives the latent
 * factors U = P S^(1/2) (m x r) and V = Q S^(1/2) (n x r), each component
 * oriented so the largest-magnitude entry of its V column (first index on
 * ties) is positive; |U| and |V| are each approximated by the rank-1 product
 * a b^T of their leading singular triplet (a = sqrt(sigma) p, b =
 * sqrt(sigma) q, non-negative); h = a_U, g = a_V, l = b_U * b_V, rounded to
 * fp16 (nearest even).  The deployed branch diag(h) sign(U) diag(l)
 * sign(V)^T diag(g) (signs of the fp32 latents, -1 iff < 0) is subtracted
 * before the next branch.  Float64 throughout on the device (rocBLAS GEMMs,
 * rocSOLVER symmetric eigendecomposition of the smaller-side Gram matrix,
 * power iteration for the rank-1 fits).
 *
 *   W         device fp32, m x n row-major, row stride ldw >= n (elements).
 *   r         rank per branch, 1 <= r <= min(m, n), r <= 4096.
 *   nbranches 1 or 2; out[b] receives branch b:
 *             U device fp32 m x r row-major, V device fp32 n x r row-major
 *             (the latent factors; their signs are the binary factors),
 *             h (m), l (r), g (n) device fp16.
 *   itq_iters 0: no rotation.  > 0 (at most 1000): before the sign-value
 *             split, the latent factors of each branch are rotated by one
 *             orthogonal R (r x r), which leaves U V^T unchanged, chosen by
 *             that many Joint-ITQ iterations from R = I (explainx.ai
 *             explainer, LittleBit-2 paragraph: Internal Latent Rotation with
 *             Joint Iterative Quantization aligns the latent factors with the
 *             binary hypercube): B = sign([U; V] R), then R = P Q^T for the
 *             SVD P S Q^T of M = [U; V]^T B, computed as the polar factor
 *             M (M^T M)^(-1/2) (rocSOLVER dsyevd of M^T M).
 * Unlike the layer library this call allocates device memory (about
 * 8 (m n + k^2 + 4 max(m, n) r) bytes, k = min(m, n)), frees it before
 * returning, and returns after the work on `stream` has finished.
 * m, n <= 32768.  On failure the message is in littlebit_init_last_error.
 */
typedef struct lb_init_branch {
  float *U;
  float *V;
  uint16_t *h;
  uint16_t *l;
  uint16_t *g;
} lb_init_branch;

lb_status littlebit_dual_svid_init(const float *W, int64_t m, int64_t n,
                                   int64_t ldw, int64_t r, int nbranches,
                                   int itq_iters, const lb_init_branch *out,
                                   void *stream);

/* Thread-local message for the most recent failing initialization call. */
const char *littlebit_init_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LITTLEBIT_INIT_H */
