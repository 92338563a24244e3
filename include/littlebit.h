/*
 * littlebit.h -- C ABI of the MI355X (gfx950) LittleBit factored binary layer.
 *
 * The layer (explainx.ai explainer "Samsung LittleBit: A 13B LLM Under 1 GB,
 * and What the Paper Really Shows", section "How it works", items 1-3):
 * a dense m x n weight is replaced by one or two branches, each the product
 * of two thin sign matrices with FP16 scale vectors on the output rows (h),
 * the latent dimension (l) and the input columns (g); the second, residual
 * branch adds to the first.  For a token x (n values) the output is
 *
 *     y = sum_b  h_b * ( sign(U_b) . ( l_b * ( sign(V_b)^T . ( g_b * x ) ) ) )
 *
 * with U_b m x r_b, V_b n x r_b and sign(v) = -1 iff v < 0.
 *
 * Conventions for every entry point
 *   - Pointers named *_bits, h, l, g, x, y, dst, ws are DEVICE pointers
 *     (hipMalloc'd or torch CUDA tensors).  lb_layer / lb_branch structs and
 *     the y[] pointer array of littlebit_block_fwd live in HOST memory and are
 *     read only during the call.
 *   - The caller owns all memory.  No entry point allocates, frees or
 *     synchronises; work is enqueued on `stream` (a hipStream_t, NULL = the
 *     default stream) and the call returns once it is enqueued.  (The
 *     offline initialization, which does allocate and synchronise, is a
 *     separate library: littlebit_init.h.)
 *   - fp16 data is IEEE binary16, passed as uint16_t.
 *   - Arguments are validated before anything is enqueued; on failure nothing
 *     is launched and a negative lb_status is returned.  littlebit_last_error
 *     returns a thread-local message describing the last failure.  HIP
 *     failures map to LB_ERR_HIP.  Calls are thread-safe (no global mutable
 *     state besides the thread-local message and a per-device property
 *     cache).
 */
#ifndef LITTLEBIT_H
#define LITTLEBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lb_status {
  LB_OK = 0,
  LB_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, bad mask  */
  LB_ERR_UNSUPPORTED = -2, /* sizes beyond what the kernels support        */
  LB_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
  LB_ERR_HIP = -4          /* a HIP runtime call failed                    */
} lb_status;

typedef enum lb_dtype { LB_F32 = 0, LB_F16 = 1 } lb_dtype;

/* Path selection for littlebit_linear_fwd (flags argument). */
#define LB_PATH_AUTO 0u    /* decode kernels for batch <= 16, else prefill  */
#define LB_PATH_DECODE 1u  /* force the decode kernels (batch must be <= 16)*/
/* The decode kernels hold z of their tokens in LDS: when 16 tokens of a
 * layer's rank do not fit, a decode call runs as several launches of fewer
 * tokens each (LB_ERR_UNSUPPORTED, or prefill under LB_PATH_AUTO, only when
 * not even one token fits). */
#define LB_PATH_PREFILL 2u /* force the prefill (matrix-core GEMM) kernels  */
/* OR-able: run the decode path as two launches (V pass, then U pass) instead
 * of one launch whose workgroups exchange the rank-space intermediate through
 * the workspace.  Same results; for measurement. */
#define LB_DECODE_TWO_LAUNCHES 4u

/*
 * LB16 packed sign format.  A packed factor F has R rows and reduction
 * length K; F[a][k] = -1 is stored as bit 1 (+1 as bit 0).  The pages fix one
 * bit per sign entry (explainx.ai explainer, "How it works" item 1); the bit
 * order is this library's, chosen so that 64 lanes can turn a 32-bit word
 * into matrix-core operands with one shift and one mask per two values.
 *   - Rp = 16*ceil(R/16) rows and Kp = 64*ceil(K/64) columns are stored;
 *     padding bits are 0.  Total size: Rp*Kp/8 bytes.
 *   - Tile T = rows 16T..16T+15, 2*Kp bytes at byte offset T*2*Kp.
 *   - Lane L (0..63) of a tile covers row 16T + L%16 and column group
 *     c = L/16; in step s (columns 32s..32s+31) it owns k = 32s + 8c + e,
 *     e = 0..7.
 *   - 16-bit unit u (0 <= u < NU = Kp/64) of a lane holds steps 2u, 2u+1;
 *     element (step 2u+q, e) is bit 8*(e%2) + 7 - (4q + e/2).
 *   - Units are little-endian.  Units 2p and 2p+1 of lane L are the aligned
 *     32-bit word at tile byte 256p + 4L (unit 2p in the low half); when NU
 *     is odd the last unit sits alone at tile byte 256*(NU/2) + 2L.
 * sign(V_b)^T is packed with R = r_b, K = n; sign(U_b) with R = m, K = r_b.
 */

/* Bytes of a packed R x K factor (0 if R or K is not positive). */
size_t littlebit_packed_bytes(int64_t R, int64_t K);

/*
 * Pack the signs of a latent matrix into LB16 (explainx.ai explainer, "How
 * it works" item 1: only the signs of the thin factors are kept).
 *   latent    device, row-major `rows` x `cols` with leading dimension
 *             ld >= cols (elements).
 *   dtype     an lb_dtype value, LB_F32 or LB_F16 (passed as int so that any
 *             other value is rejected rather than being undefined).
 *   transpose 0: the factor is latent itself (R = rows, K = cols) -- use for
 *             U (m x r).  1: the factor is latent^T (R = cols, K = rows) -- use
 *             for V (n x r), giving sign(V)^T.
 *   dst       device, littlebit_packed_bytes(R, K) bytes, 4-byte aligned;
 *             every byte (padding included) is written.
 * Bit = 1 iff the latent value is < 0 (+0, -0 and NaN give +1).
 */
lb_status littlebit_pack(const void *latent, int dtype, int64_t rows,
                         int64_t cols, int64_t ld, int transpose, void *dst,
                         void *stream);

/*
 * The packing of the transpose of a packed factor: src holds an R x K factor
 * (littlebit_packed_bytes(R, K) bytes), dst receives the K x R factor with the
 * same bits (littlebit_packed_bytes(K, R) bytes, every byte written, pad bits
 * 0).  For the backward-input product of quantization-aware training
 * (explainx.ai explainer, "How it works" item 3: the model trains through
 * the binarized forward pass), dx = W^T dy, which is the layer with
 *   v_bits' = transpose(u_bits)  (R = r, K = m),
 *   u_bits' = transpose(v_bits)  (R = n, K = r),
 *   h' = g, l' = l, g' = h, m' = n, n' = m,
 * run through littlebit_linear_fwd.  src and dst: device, 4-byte aligned,
 * distinct.  Asynchronous on `stream`.
 */
lb_status littlebit_transpose_packed(const void *src, int64_t R, int64_t K,
                                     void *dst, void *stream);

typedef struct lb_branch {
  const void *v_bits; /* device, LB16 sign(V)^T: R = r, K = n               */
  const void *u_bits; /* device, LB16 sign(U):   R = m, K = r               */
  const uint16_t *h;  /* device fp16 [m]  row (output) scale, 16B aligned  */
  const uint16_t *l;  /* device fp16 [r]  latent scale, 16B aligned         */
  const uint16_t *g;  /* device fp16 [n]  column (input) scale, 16B aligned */
  int32_t r;          /* rank of this branch, 1 <= r <= 4096                */
} lb_branch;

typedef struct lb_layer {
  int32_t m;          /* outputs, 1 <= m                                    */
  int32_t n;          /* inputs, 1 <= n <= 32768                            */
  int32_t nbranches;  /* 1 or 2 (primary, residual)                         */
  lb_branch br[2];
} lb_layer;

/*
 * Workspace bytes littlebit_linear_fwd needs for this layer and batch
 * (0 on invalid arguments).  The workspace must be zero-filled once before
 * its first use; the library leaves it reusable after every call.  Its first
 * 4096 bytes are a header: one call counter per workgroup of the decode
 * kernel's single launch and a poll error word.  A header that was not
 * zero-filled (counters that differ between workgroups) is a precondition
 * violation: the call's z polls then wait in vain until their spin limit,
 * and the call reports it through littlebit_workspace_error.  Calls that run
 * concurrently must not share a workspace, and a workspace stays with the
 * device it was first used on.
 */
size_t littlebit_linear_workspace_bytes(const lb_layer *L, int64_t batch);

/*
 * y = layer(x) for `batch` tokens (explainx.ai explainer, "How it works"
 * items 1-3; the residual branch adds, item 3).
 *   branch_mask  bit b selects branch b (1 = primary only, 2 = residual
 *                only, 3 = both); selected branches must exist.
 *   x            device fp16, batch rows of n, row stride ldx >= n elements.
 *   y            device fp16, batch rows of m, row stride ldy >= m; the
 *                batch x m entries are overwritten (not accumulated), the
 *                rest of each row is untouched.
 *   ws, ws_bytes device workspace of at least
 *                littlebit_linear_workspace_bytes(L, batch) bytes, 256-byte
 *                aligned.
 *   flags        LB_PATH_* optionally OR-ed with LB_DECODE_TWO_LAUNCHES.
 * Intermediates: g*x and l*t are rounded to fp16 before the sign
 * contractions; accumulation is fp32; y is rounded to fp16 once.
 *
 * Decode (up to 16 tokens) runs, unless LB_DECODE_TWO_LAUNCHES is given, as
 * one launch of one workgroup per compute unit whose workgroups hand the
 * rank-space intermediate to each other through the workspace: every
 * workgroup of that launch must be resident at the same time.  The library
 * sizes the grid from the device's occupancy for this kernel, so the
 * precondition holds when no other kernel keeps compute units busy for
 * long while the call runs; if one does, a workgroup that waits more than
 * about 2^20 polls gives up, its outputs are wrong, and the workspace's
 * error word is set (littlebit_workspace_error reports it).
 */
lb_status littlebit_linear_fwd(const lb_layer *L, uint32_t branch_mask,
                               const uint16_t *x, int64_t batch, int64_t ldx,
                               uint16_t *y, int64_t ldy, void *ws,
                               size_t ws_bytes, uint32_t flags, void *stream);

/*
 * littlebit_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the intermediates live in a scratch
 * array that the library holds in device memory, 8 MiB per device, from the
 * first use of the library on the device until the process ends.  Same
 * arguments, results and residency precondition as littlebit_linear_fwd;
 * prefill runs in chunks of tokens whose intermediate fits the scratch.
 * Nothing is allocated or freed and nothing is synchronised.  Every call on
 * one device shares that device's scratch and leaves its contents for the
 * next: calls that may overlap on one device (different streams, or threads
 * without ordering) race and must not be issued.  LB_ERR_UNSUPPORTED if the
 * layer's decode intermediate exceeds the scratch (it cannot within the
 * rank and size limits above) or no 128-token prefill chunk fits.
 */
lb_status littlebit_linear_fwd_noalloc(const lb_layer *L, uint32_t branch_mask,
                                       const uint16_t *x, int64_t batch,
                                       int64_t ldx, uint16_t *y, int64_t ldy,
                                       uint32_t flags, void *stream);

/*
 * The seven projections of one decoder block in one call (q, k, v, o, gate,
 * up, down; all branches of each).  The pages compress the linear layers of
 * the Transformer blocks and keep the architecture (explainx.ai explainer,
 * "What LittleBit is"; trueseeker.com case, "The trace / claim to source":
 * only the Transformer blocks are quantized, embedding and head stay FP16),
 * so a block's seven projections are seven independent layers of the form
 * above.  q, k, v read x_qkv; o reads x_o; gate and up read x_gu; down reads
 * x_down.  Every x row stride equals that projection's n and every y row
 * stride its m (dense batch x n / batch x m arrays).  Attention, norms and
 * activations are not part of the layer and are left to the caller.  For
 * batch <= 16 all seven run in one launch (with the residency precondition
 * of littlebit_linear_fwd's decode); y[i] is written as by
 * littlebit_linear_fwd on layer i.  Workspace as for
 * littlebit_linear_workspace_bytes, with its own size.
 */
size_t littlebit_block_workspace_bytes(const lb_layer L[7], int64_t batch);

lb_status littlebit_block_fwd(const lb_layer L[7], const uint16_t *x_qkv,
                              const uint16_t *x_o, const uint16_t *x_gu,
                              const uint16_t *x_down, uint16_t *const y[7],
                              int64_t batch, void *ws, size_t ws_bytes,
                              void *stream);

/*
 * Failure report of the decode kernels' waits.  Enqueues, on `stream`, a
 * copy of the workspace's poll error word into *error (device, one uint32,
 * 4-byte aligned) and clears the word.  *error != 0 means that, in some
 * decode call on this workspace since the previous report, a workgroup gave
 * up waiting for the rank-space intermediate (see littlebit_linear_fwd):
 * that call's outputs are wrong.  ws_bytes >= 4096.
 */
lb_status littlebit_workspace_error(void *ws, size_t ws_bytes, uint32_t *error,
                                    void *stream);

/* Static description of a status code. */
const char *littlebit_status_string(lb_status s);

/* Thread-local message for the most recent failing call on this thread. */
const char *littlebit_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LITTLEBIT_H */
