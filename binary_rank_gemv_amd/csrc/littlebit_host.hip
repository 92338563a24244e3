// C ABI of the LittleBit gfx950 library: argument validation, workspace
// layout and kernel dispatch.  No allocation, no synchronisation.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "littlebit.h"
#include "lb_common.h"

hipError_t lb_launch_pack(const void* latent, int is_f16, long ld, int transpose, int R, int K,
                          void* dst, hipStream_t stream);
hipError_t lb_launch_prefill(const LbPrefillArgs& args, hipStream_t stream);
hipError_t lb_launch_transpose_packed(const void* src, int R, int K, void* dst, hipStream_t stream);
hipError_t lb_launch_decode(const LbDecodeArgs& args, void* sync, int allow_fused,
                            hipStream_t stream);
hipError_t lb_launch_take_error(void* sync, uint32_t* out, hipStream_t stream);

namespace {

thread_local std::string g_last_error;

lb_status fail(lb_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

lb_status hip_fail(hipError_t e, const char* what) {
  return fail(LB_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

constexpr int kMaxRank = 4096;
constexpr int kMaxN = 32768;
constexpr int kDecodeMaxBatch = 16;

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout: [header | decode z of every layer | prefill z].  Decode
// z: 16 rows of zs/2 tagged 64-bit words (two fp16 values each) per layer,
// reserved whatever the batch.  Prefill z: up to 8192 rows of zs fp16 values,
// in a region of its own, so a decode poll never meets plain prefill values.
struct LayerWs {
  int zs;             // halves per decode z row (branch regions of 64*ceil(r/64))
  int zoff[2];
  size_t z_bytes;     // decode region (16 rows)
  int zs_p;           // halves per prefill z row (branch regions of 128*ceil(r/128), zero-padded)
  int zoff_p[2];
};

// The decode kernels stage a token-major copy of z in LDS (zs + 8 halves per
// token); larger products of batch and rank go to the prefill kernels.
inline bool decode_fits(int zs, int64_t batch) {
  return (size_t)batch * (zs + 8) * sizeof(uint16_t) <= LB_DECODE_LDS_MAX;
}

// Tokens per decode launch: up to 16, fewer when z of 16 tokens exceeds the
// LDS (then a call of up to 16 tokens runs as several launches); 0 when not
// even one token fits.
inline int decode_chunk_tokens(int zs) {
  int t = 16;
  while (t > 0 && !decode_fits(zs, t)) --t;
  return t;
}

inline size_t prefill_z_bytes(int zs, int64_t tokens) {
  const int64_t t = tokens < LB_PREFILL_MAX_TOKENS ? tokens : LB_PREFILL_MAX_TOKENS;
  return round_up((size_t)t * zs * sizeof(uint16_t), 256);
}

LayerWs layer_ws(const lb_layer& L, const int* sel, int nsel, int64_t batch) {
  LayerWs w{};
  int zs = 0, zsp = 0;
  for (int i = 0; i < nsel; ++i) {
    w.zoff[i] = zs;
    zs += 64 * lb16_units(L.br[sel[i]].r);
    w.zoff_p[i] = zsp;
    zsp += 128 * ((L.br[sel[i]].r + 127) / 128);
  }
  w.zs = zs;
  w.zs_p = zsp;
  w.z_bytes = round_up((size_t)batch * zs * 4, 256);  // batch = 16: the reserved decode rows
  return w;
}

constexpr size_t kWsHeader = 4096;  // call counters and error word of the single-launch decode kernel

lb_status check_layer(const lb_layer* L, uint32_t mask, int* sel, int* nsel, const char* name) {
  if (!L) return fail(LB_ERR_INVALID_ARG, "%s: layer pointer is NULL", name);
  if (L->m < 1 || L->n < 1) return fail(LB_ERR_INVALID_ARG, "%s: m=%d n=%d must be >= 1", name, L->m, L->n);
  if (L->n > kMaxN) return fail(LB_ERR_UNSUPPORTED, "%s: n=%d exceeds %d", name, L->n, kMaxN);
  if (L->nbranches < 1 || L->nbranches > 2)
    return fail(LB_ERR_INVALID_ARG, "%s: nbranches=%d must be 1 or 2", name, L->nbranches);
  if (mask == 0 || (mask & ~3u)) return fail(LB_ERR_INVALID_ARG, "%s: branch_mask=%u must be 1, 2 or 3", name, mask);
  *nsel = 0;
  for (int b = 0; b < 2; ++b) {
    if (!(mask & (1u << b))) continue;
    if (b >= L->nbranches)
      return fail(LB_ERR_INVALID_ARG, "%s: branch_mask selects branch %d but nbranches=%d", name, b, L->nbranches);
    const lb_branch& B = L->br[b];
    if (B.r < 1) return fail(LB_ERR_INVALID_ARG, "%s: branch %d rank %d must be >= 1", name, b, B.r);
    if (B.r > kMaxRank) return fail(LB_ERR_UNSUPPORTED, "%s: branch %d rank %d exceeds %d", name, b, B.r, kMaxRank);
    if (!B.v_bits || !B.u_bits || !B.h || !B.l || !B.g)
      return fail(LB_ERR_INVALID_ARG, "%s: branch %d has a NULL pointer", name, b);
    if (!aligned(B.v_bits, 16) || !aligned(B.u_bits, 16))
      return fail(LB_ERR_INVALID_ARG, "%s: branch %d packed factors must be 16-byte aligned", name, b);
    if (!aligned(B.h, 16) || !aligned(B.l, 16) || !aligned(B.g, 16))
      return fail(LB_ERR_INVALID_ARG, "%s: branch %d scale vectors must be 16-byte aligned", name, b);
    sel[(*nsel)++] = b;
  }
  return LB_OK;
}

void fill_layer_args(LbLayerArgs& a, const lb_layer& L, const int* sel, int nsel, const LayerWs& w,
                     uint8_t* base, const uint16_t* x, long ldx, uint16_t* y, long ldy) {
  memset(&a, 0, sizeof a);
  a.nb = nsel;
  a.m = L.m;
  a.n = L.n;
  a.x = x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.z = reinterpret_cast<uint64_t*>(base);
  a.zs = w.zs;
  for (int i = 0; i < nsel; ++i) {
    const lb_branch& B = L.br[sel[i]];
    a.br[i].vbits = static_cast<const uint8_t*>(B.v_bits);
    a.br[i].ubits = static_cast<const uint8_t*>(B.u_bits);
    a.br[i].h = B.h;
    a.br[i].l = B.l;
    a.br[i].g = B.g;
    a.br[i].r = B.r;
    a.br[i].zoff = w.zoff[i];
  }
}

void fill_prefill_args(LbPrefillArgs& a, const lb_layer& L, const int* sel, int nsel, const LayerWs& w,
                       uint8_t* base, const uint16_t* x, long ldx, uint16_t* y, long ldy, int tokens) {
  memset(&a, 0, sizeof a);
  a.nb = nsel;
  a.m = L.m;
  a.n = L.n;
  a.M = tokens;
  a.x = x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.z = reinterpret_cast<uint16_t*>(base);
  a.zs = w.zs_p;
  for (int i = 0; i < nsel; ++i) {
    const lb_branch& B = L.br[sel[i]];
    a.br[i].vbits = static_cast<const uint8_t*>(B.v_bits);
    a.br[i].ubits = static_cast<const uint8_t*>(B.u_bits);
    a.br[i].h = B.h;
    a.br[i].l = B.l;
    a.br[i].g = B.g;
    a.br[i].r = B.r;
    a.br[i].zoff = w.zoff_p[i];
  }
}

// Launch the decode kernels for up to 16 tokens over `nl` prepared layers.
lb_status run_decode(LbLayerArgs* layers, int nl, int batch, void* sync, int allow_fused, hipStream_t stream) {
  LbDecodeArgs args;
  memset(&args, 0, sizeof args);
  args.nlayers = nl;
  args.batch = batch;
  int vt = 0, ut = 0;
  for (int i = 0; i < nl; ++i) {
    args.L[i] = layers[i];
    for (int b = 0; b < 2; ++b) {
      if (b < layers[i].nb) vt += (layers[i].br[b].r + 15) / 16;
      args.vt_end[2 * i + b] = vt;
    }
    ut += (layers[i].m + 15) / 16;
    args.ut_end[i] = ut;
  }
  args.nvt = vt;
  args.nut = ut;
  hipError_t e = lb_launch_decode(args, sync, allow_fused, stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return LB_OK;
}

}  // namespace

extern "C" {

size_t littlebit_packed_bytes(int64_t R, int64_t K) {
  if (R <= 0 || K <= 0) return 0;
  return (size_t)(16 * ((R + 15) / 16)) * (size_t)(64 * ((K + 63) / 64)) / 8;
}

lb_status littlebit_pack(const void* latent, int dtype, int64_t rows, int64_t cols, int64_t ld,
                         int transpose, void* dst, void* stream) {
  if (!latent || !dst) return fail(LB_ERR_INVALID_ARG, "littlebit_pack: NULL pointer");
  if (rows < 1 || cols < 1) return fail(LB_ERR_INVALID_ARG, "littlebit_pack: rows=%lld cols=%lld", (long long)rows, (long long)cols);
  if (ld < cols) return fail(LB_ERR_INVALID_ARG, "littlebit_pack: ld=%lld < cols=%lld", (long long)ld, (long long)cols);
  if (dtype != LB_F32 && dtype != LB_F16) return fail(LB_ERR_INVALID_ARG, "littlebit_pack: bad dtype %d", dtype);
  if (transpose != 0 && transpose != 1) return fail(LB_ERR_INVALID_ARG, "littlebit_pack: transpose must be 0 or 1");
  if (!aligned(dst, 4)) return fail(LB_ERR_INVALID_ARG, "littlebit_pack: dst must be 4-byte aligned");
  const int64_t R = transpose ? cols : rows, K = transpose ? rows : cols;
  if (R > (1LL << 30) || K > (1LL << 24)) return fail(LB_ERR_UNSUPPORTED, "littlebit_pack: factor too large");
  hipError_t e = lb_launch_pack(latent, dtype == LB_F16, (long)ld, transpose, (int)R, (int)K, dst,
                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "littlebit_pack launch");
  return LB_OK;
}

lb_status littlebit_transpose_packed(const void* src, int64_t R, int64_t K, void* dst, void* stream) {
  if (!src || !dst) return fail(LB_ERR_INVALID_ARG, "littlebit_transpose_packed: NULL pointer");
  if (R < 1 || K < 1) return fail(LB_ERR_INVALID_ARG, "littlebit_transpose_packed: R=%lld K=%lld", (long long)R, (long long)K);
  if (!aligned(src, 4) || !aligned(dst, 4))
    return fail(LB_ERR_INVALID_ARG, "littlebit_transpose_packed: src and dst must be 4-byte aligned");
  if (R > (1LL << 24) || K > (1LL << 24)) return fail(LB_ERR_UNSUPPORTED, "littlebit_transpose_packed: factor too large");
  if (src == dst) return fail(LB_ERR_INVALID_ARG, "littlebit_transpose_packed: src and dst must not be the same buffer");
  hipError_t e = lb_launch_transpose_packed(src, (int)R, (int)K, dst, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "littlebit_transpose_packed launch");
  return LB_OK;
}

size_t littlebit_linear_workspace_bytes(const lb_layer* L, int64_t batch) {
  int sel[2], nsel = 0;
  if (batch < 1 || !L || L->nbranches < 1 || L->nbranches > 2) return 0;
  if (check_layer(L, (1u << L->nbranches) - 1, sel, &nsel, "workspace") != LB_OK) return 0;
  const LayerWs w = layer_ws(*L, sel, nsel, kDecodeMaxBatch);
  return kWsHeader + w.z_bytes + prefill_z_bytes(w.zs_p, batch);
}

}  // extern "C"

namespace {

// Argument checks shared by littlebit_linear_fwd and its no-alloc variant
// (everything but the workspace).
lb_status check_linear_args(const char* name, const lb_layer* L, uint32_t branch_mask, const uint16_t* x,
                            int64_t batch, int64_t ldx, uint16_t* y, int64_t ldy, uint32_t flags, int* sel,
                            int* nsel) {
  lb_status st = check_layer(L, branch_mask, sel, nsel, name);
  if (st != LB_OK) return st;
  if (!x || !y) return fail(LB_ERR_INVALID_ARG, "%s: x or y is NULL", name);
  if (batch < 1) return fail(LB_ERR_INVALID_ARG, "%s: batch=%lld must be >= 1", name, (long long)batch);
  if (ldx < L->n || ldy < L->m) return fail(LB_ERR_INVALID_ARG, "%s: ldx/ldy smaller than n/m", name);
  if (ldx > INT32_MAX || ldy > INT32_MAX)
    return fail(LB_ERR_UNSUPPORTED, "%s: row strides above 2^31-1 elements", name);
  if (!aligned(x, 2) || !aligned(y, 2)) return fail(LB_ERR_INVALID_ARG, "%s: x and y must be 2-byte aligned", name);
  if ((flags & 3u) == 3u || (flags & ~(3u | LB_DECODE_TWO_LAUNCHES)))
    return fail(LB_ERR_INVALID_ARG, "%s: unknown flags %u", name, flags);
  if ((flags & 3u) == LB_PATH_DECODE && batch > kDecodeMaxBatch)
    return fail(LB_ERR_INVALID_ARG, "%s: decode path takes at most %d tokens", name, kDecodeMaxBatch);
  return LB_OK;
}

// The layer on a workspace whose size has been checked by the caller; prefill
// runs in chunks of at most max_prefill_tokens tokens.
lb_status linear_fwd_impl(const char* name, const lb_layer* L, const int* sel, int nsel, const uint16_t* x,
                          int64_t batch, int64_t ldx, uint16_t* y, int64_t ldy, void* ws, uint32_t flags,
                          int64_t max_prefill_tokens, hipStream_t stream) {
  const LayerWs w = layer_ws(*L, sel, nsel, kDecodeMaxBatch);
  const uint32_t path = flags & 3u;
  const int chunk = decode_chunk_tokens(w.zs);
  const bool prefill = path == LB_PATH_PREFILL || (path == LB_PATH_AUTO && (batch > kDecodeMaxBatch || chunk == 0));
  uint8_t* base = static_cast<uint8_t*>(ws) + kWsHeader;
  if (prefill) {
    for (int64_t t0 = 0; t0 < batch; t0 += max_prefill_tokens) {
      const int nt = (int)((batch - t0) < max_prefill_tokens ? (batch - t0) : max_prefill_tokens);
      LbPrefillArgs pa;
      fill_prefill_args(pa, *L, sel, nsel, w, base + w.z_bytes, x + t0 * ldx, (long)ldx, y + t0 * ldy,
                        (long)ldy, nt);
      hipError_t e = lb_launch_prefill(pa, stream);
      if (e != hipSuccess) return hip_fail(e, "prefill launch");
    }
    return LB_OK;
  }
  (void)name;
  for (int64_t t0 = 0; t0 < batch; t0 += chunk) {
    const int nb = (int)((batch - t0) < chunk ? (batch - t0) : chunk);
    LbLayerArgs la;
    fill_layer_args(la, *L, sel, nsel, w, base, x + t0 * ldx, (long)ldx, y + t0 * ldy, (long)ldy);
    lb_status st = run_decode(&la, 1, nb, ws, !(flags & LB_DECODE_TWO_LAUNCHES), stream);
    if (st != LB_OK) return st;
  }
  return LB_OK;
}

// ------------------------------------------------------- no-alloc variant
// The workspace of littlebit_linear_fwd_noalloc: one array per device,
// zero-filled when the code object is loaded onto the device (static storage
// without an initializer) and kept for the life of the process.  Host code
// never passes the array's name to a kernel: it is only a host-side stand-in
// for the symbol; its device address comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = 8u << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// This device's scratch address, looked up once per device (with that device
// current, as it is for the calling thread here).
lb_status scratch_for_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LB_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256)) return fail(LB_ERR_HIP, "scratch symbol address %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LB_OK;
}

}  // namespace

extern "C" {

lb_status littlebit_linear_fwd(const lb_layer* L, uint32_t branch_mask, const uint16_t* x, int64_t batch,
                               int64_t ldx, uint16_t* y, int64_t ldy, void* ws, size_t ws_bytes,
                               uint32_t flags, void* stream) {
  const char* name = "littlebit_linear_fwd";
  int sel[2], nsel = 0;
  lb_status st = check_linear_args(name, L, branch_mask, x, batch, ldx, y, ldy, flags, sel, &nsel);
  if (st != LB_OK) return st;
  if (!ws) return fail(LB_ERR_WORKSPACE, "%s: workspace is NULL", name);
  if (!aligned(ws, 256)) return fail(LB_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", name);
  const LayerWs w = layer_ws(*L, sel, nsel, kDecodeMaxBatch);
  const uint32_t path = flags & 3u;
  const int chunk = decode_chunk_tokens(w.zs);
  if (path == LB_PATH_DECODE && chunk == 0)
    return fail(LB_ERR_UNSUPPORTED, "%s: rank %d exceeds the decode kernels' LDS", name, w.zs);
  const bool prefill = path == LB_PATH_PREFILL || (path == LB_PATH_AUTO && (batch > kDecodeMaxBatch || chunk == 0));
  const size_t need = kWsHeader + w.z_bytes + (prefill ? prefill_z_bytes(w.zs_p, batch) : 0);
  if (ws_bytes < need)
    return fail(LB_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", name, ws_bytes, need);
  return linear_fwd_impl(name, L, sel, nsel, x, batch, ldx, y, ldy, ws, flags, LB_PREFILL_MAX_TOKENS,
                         (hipStream_t)stream);
}

lb_status littlebit_linear_fwd_noalloc(const lb_layer* L, uint32_t branch_mask, const uint16_t* x, int64_t batch,
                                       int64_t ldx, uint16_t* y, int64_t ldy, uint32_t flags, void* stream) {
  const char* name = "littlebit_linear_fwd_noalloc";
  int sel[2], nsel = 0;
  lb_status st = check_linear_args(name, L, branch_mask, x, batch, ldx, y, ldy, flags, sel, &nsel);
  if (st != LB_OK) return st;
  const LayerWs w = layer_ws(*L, sel, nsel, kDecodeMaxBatch);
  const uint32_t path = flags & 3u;
  const int chunk = decode_chunk_tokens(w.zs);
  if (path == LB_PATH_DECODE && chunk == 0)
    return fail(LB_ERR_UNSUPPORTED, "%s: rank %d exceeds the decode kernels' LDS", name, w.zs);
  const bool prefill = path == LB_PATH_PREFILL || (path == LB_PATH_AUTO && (batch > kDecodeMaxBatch || chunk == 0));
  const size_t fixed = kWsHeader + w.z_bytes;
  int64_t max_tokens = LB_PREFILL_MAX_TOKENS;
  if (prefill) {
    // prefill in chunks whose rank-space intermediate fits the scratch
    const size_t per_token = (size_t)w.zs_p * sizeof(uint16_t);
    const int64_t fit = fixed < kScratchBytes ? (int64_t)((kScratchBytes - fixed) / per_token) / 128 * 128 : 0;
    if (fit < 1)
      return fail(LB_ERR_UNSUPPORTED, "%s: %zu scratch bytes hold no 128-token prefill chunk of this layer", name,
                  kScratchBytes);
    max_tokens = fit < max_tokens ? fit : max_tokens;
  } else if (fixed > kScratchBytes) {
    return fail(LB_ERR_UNSUPPORTED, "%s: the layer needs %zu bytes of scratch, the limit is %zu", name, fixed,
                kScratchBytes);
  }
  void* ws = nullptr;
  st = scratch_for_device(&ws);
  if (st != LB_OK) return st;
  return linear_fwd_impl(name, L, sel, nsel, x, batch, ldx, y, ldy, ws, flags, max_tokens, (hipStream_t)stream);
}

size_t littlebit_block_workspace_bytes(const lb_layer L[7], int64_t batch) {
  if (!L || batch < 1) return 0;
  size_t total = 0, zp = 0;
  bool prefill = batch > kDecodeMaxBatch;
  for (int i = 0; i < 7; ++i) {
    int sel[2], nsel = 0;
    if (L[i].nbranches < 1 || L[i].nbranches > 2) return 0;
    if (check_layer(&L[i], (1u << L[i].nbranches) - 1, sel, &nsel, "workspace") != LB_OK) return 0;
    const LayerWs w = layer_ws(L[i], sel, nsel, kDecodeMaxBatch);
    total += w.z_bytes;
    const size_t p = prefill_z_bytes(w.zs_p, batch);
    if (p > zp) zp = p;
    prefill = prefill || decode_chunk_tokens(w.zs) == 0;
  }
  return kWsHeader + total + (prefill ? zp : 0);
}

lb_status littlebit_block_fwd(const lb_layer L[7], const uint16_t* x_qkv, const uint16_t* x_o,
                              const uint16_t* x_gu, const uint16_t* x_down, uint16_t* const y[7],
                              int64_t batch, void* ws, size_t ws_bytes, void* stream) {
  if (!L || !y) return fail(LB_ERR_INVALID_ARG, "littlebit_block_fwd: NULL layer or output array");
  if (!x_qkv || !x_o || !x_gu || !x_down) return fail(LB_ERR_INVALID_ARG, "littlebit_block_fwd: NULL input");
  if (batch < 1) return fail(LB_ERR_INVALID_ARG, "littlebit_block_fwd: batch must be >= 1");
  const uint16_t* xs[7] = {x_qkv, x_qkv, x_qkv, x_o, x_gu, x_gu, x_down};
  int sel[7][2], nsel[7];
  LayerWs w[7];
  size_t need = kWsHeader, zp = 0;
  for (int i = 0; i < 7; ++i) {
    if (L[i].nbranches < 1 || L[i].nbranches > 2)
      return fail(LB_ERR_INVALID_ARG, "littlebit_block_fwd: layer %d nbranches=%d", i, L[i].nbranches);
    lb_status st = check_layer(&L[i], (1u << L[i].nbranches) - 1, sel[i], &nsel[i], "littlebit_block_fwd");
    if (st != LB_OK) return st;
    if (!y[i]) return fail(LB_ERR_INVALID_ARG, "littlebit_block_fwd: y[%d] is NULL", i);
    if (!aligned(xs[i], 2) || !aligned(y[i], 2))
      return fail(LB_ERR_INVALID_ARG, "littlebit_block_fwd: inputs and outputs must be 2-byte aligned");
    w[i] = layer_ws(L[i], sel[i], nsel[i], kDecodeMaxBatch);
    need += w[i].z_bytes;
    const size_t p = prefill_z_bytes(w[i].zs_p, batch);
    if (p > zp) zp = p;
  }
  int chunk = kDecodeMaxBatch;
  for (int i = 0; i < 7; ++i) {
    const int c = decode_chunk_tokens(w[i].zs);
    chunk = c < chunk ? c : chunk;
  }
  const bool prefill = batch > kDecodeMaxBatch || chunk == 0;
  const size_t decode_bytes = need - kWsHeader;
  if (prefill) need += zp;
  if (L[0].n != L[1].n || L[0].n != L[2].n || L[4].n != L[5].n)
    return fail(LB_ERR_INVALID_ARG, "littlebit_block_fwd: q/k/v and gate/up must share their input size");
  if (!ws) return fail(LB_ERR_WORKSPACE, "littlebit_block_fwd: workspace is NULL");
  if (!aligned(ws, 256)) return fail(LB_ERR_WORKSPACE, "littlebit_block_fwd: workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(LB_ERR_WORKSPACE, "littlebit_block_fwd: workspace has %zu bytes, needs %zu", ws_bytes, need);

  if (prefill) {
    // the projections one after another, each as two matrix-core GEMMs
    uint8_t* base = static_cast<uint8_t*>(ws) + kWsHeader + decode_bytes;
    for (int i = 0; i < 7; ++i) {
      for (int64_t t0 = 0; t0 < batch; t0 += LB_PREFILL_MAX_TOKENS) {
        const int nt = (int)((batch - t0) < LB_PREFILL_MAX_TOKENS ? (batch - t0) : LB_PREFILL_MAX_TOKENS);
        LbPrefillArgs pa;
        fill_prefill_args(pa, L[i], sel[i], nsel[i], w[i], base, xs[i] + t0 * L[i].n, L[i].n,
                          y[i] + t0 * L[i].m, L[i].m, nt);
        hipError_t e = lb_launch_prefill(pa, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "prefill launch");
      }
    }
    return LB_OK;
  }
  for (int64_t t0 = 0; t0 < batch; t0 += chunk) {
    const int nb = (int)((batch - t0) < chunk ? (batch - t0) : chunk);
    LbLayerArgs la[7];
    uint8_t* base = static_cast<uint8_t*>(ws) + kWsHeader;
    for (int i = 0; i < 7; ++i) {
      fill_layer_args(la[i], L[i], sel[i], nsel[i], w[i], base, xs[i] + t0 * L[i].n, L[i].n,
                      y[i] + t0 * L[i].m, L[i].m);
      base += w[i].z_bytes;
    }
    lb_status st = run_decode(la, 7, nb, ws, 1, (hipStream_t)stream);
    if (st != LB_OK) return st;
  }
  return LB_OK;
}

lb_status littlebit_workspace_error(void* ws, size_t ws_bytes, uint32_t* error, void* stream) {
  if (!ws || !error) return fail(LB_ERR_INVALID_ARG, "littlebit_workspace_error: NULL pointer");
  if (!aligned(ws, 256)) return fail(LB_ERR_WORKSPACE, "littlebit_workspace_error: workspace must be 256-byte aligned");
  if (!aligned(error, 4)) return fail(LB_ERR_INVALID_ARG, "littlebit_workspace_error: error must be 4-byte aligned");
  if (ws_bytes < kWsHeader)
    return fail(LB_ERR_WORKSPACE, "littlebit_workspace_error: workspace has %zu bytes, needs %zu", ws_bytes, kWsHeader);
  hipError_t e = lb_launch_take_error(ws, error, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "littlebit_workspace_error launch");
  return LB_OK;
}

const char* littlebit_status_string(lb_status s) {
  switch (s) {
    case LB_OK: return "LB_OK";
    case LB_ERR_INVALID_ARG: return "LB_ERR_INVALID_ARG: invalid argument";
    case LB_ERR_UNSUPPORTED: return "LB_ERR_UNSUPPORTED: sizes beyond the supported range";
    case LB_ERR_WORKSPACE: return "LB_ERR_WORKSPACE: workspace missing or too small";
    case LB_ERR_HIP: return "LB_ERR_HIP: HIP runtime error";
  }
  return "unknown lb_status";
}

const char* littlebit_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
