"""ctypes binding of ``include/littlebit.h`` (argument marshalling only).

Every step of the layer runs in the HIP library ``_lib/liblittlebit.so``;
PyTorch provides device memory and the current stream.  Importing this module
raises if the library has not been built (``python -m
binary_rank_gemv_amd.build``) -- there is no fallback path.

The functions keep the C names:

* ``littlebit_pack(latent, transpose)`` -> packed uint8 tensor
* ``littlebit_transpose_packed(bits, R, K)`` -> packing of the K x R transpose
  (``LittleBitLayer.transposed()`` builds the layer of W^T from it)
* ``littlebit_linear_fwd(layer, x, branch_mask=3, path=LB_PATH_AUTO)`` -> y
* ``littlebit_linear_fwd_noalloc(layer, x, ...)`` -> y, on the library's
  per-device scratch instead of a workspace
* ``littlebit_block_fwd(layers, x_qkv, x_o, x_gu, x_down)`` -> list of 7 y
* ``littlebit_workspace_error(ws)`` -> device int32 tensor, non-zero if a
  decode call on ``ws`` gave up waiting since the previous report
* ``littlebit_packed_bytes``, ``littlebit_linear_workspace_bytes``,
  ``littlebit_block_workspace_bytes``, ``littlebit_status_string``,
  ``littlebit_last_error``
* ``littlebit_dual_svid_init(W, r, ...)`` -> branches; from the separate
  offline library ``_lib/liblittlebit_init.so`` (include/littlebit_init.h),
  loaded on first use
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

# LITTLEBIT_LIBRARY names another build of the same library (the host-side
# sanitizer build of the CPU tests); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("LITTLEBIT_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib",
                                                               "liblittlebit.so")
INIT_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "liblittlebit_init.so")

LB_OK, LB_ERR_INVALID_ARG, LB_ERR_UNSUPPORTED, LB_ERR_WORKSPACE, LB_ERR_HIP = 0, -1, -2, -3, -4
LB_F32, LB_F16 = 0, 1
LB_PATH_AUTO, LB_PATH_DECODE, LB_PATH_PREFILL = 0, 1, 2
LB_DECODE_TWO_LAUNCHES = 4

EXPORTED = (
    "littlebit_packed_bytes", "littlebit_pack", "littlebit_linear_workspace_bytes",
    "littlebit_linear_fwd", "littlebit_block_workspace_bytes", "littlebit_block_fwd",
    "littlebit_status_string", "littlebit_last_error", "littlebit_transpose_packed",
    "littlebit_workspace_error", "littlebit_linear_fwd_noalloc",
)
INIT_EXPORTED = ("littlebit_dual_svid_init", "littlebit_init_last_error")


class LittleBitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [status {status}]")
        self.status = status


class _Branch(ctypes.Structure):
    _fields_ = [("v_bits", ctypes.c_void_p), ("u_bits", ctypes.c_void_p),
                ("h", ctypes.c_void_p), ("l", ctypes.c_void_p), ("g", ctypes.c_void_p),
                ("r", ctypes.c_int32)]


class _InitBranch(ctypes.Structure):
    _fields_ = [("U", ctypes.c_void_p), ("V", ctypes.c_void_p), ("h", ctypes.c_void_p),
                ("l", ctypes.c_void_p), ("g", ctypes.c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("nbranches", ctypes.c_int32),
                ("br", _Branch * 2)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m binary_rank_gemv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, u32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int, ctypes.c_size_t
    lib.littlebit_packed_bytes.argtypes = [i64, i64]
    lib.littlebit_packed_bytes.restype = sz
    lib.littlebit_pack.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp]
    lib.littlebit_pack.restype = i32
    lib.littlebit_transpose_packed.argtypes = [vp, i64, i64, vp, vp]
    lib.littlebit_transpose_packed.restype = i32
    lib.littlebit_linear_workspace_bytes.argtypes = [ctypes.POINTER(_Layer), i64]
    lib.littlebit_linear_workspace_bytes.restype = sz
    lib.littlebit_linear_fwd.argtypes = [ctypes.POINTER(_Layer), u32, vp, i64, i64, vp, i64, vp, sz, u32, vp]
    lib.littlebit_linear_fwd.restype = i32
    lib.littlebit_block_workspace_bytes.argtypes = [ctypes.POINTER(_Layer), i64]
    lib.littlebit_block_workspace_bytes.restype = sz
    lib.littlebit_block_fwd.argtypes = [ctypes.POINTER(_Layer), vp, vp, vp, vp, ctypes.POINTER(vp), i64, vp, sz, vp]
    lib.littlebit_block_fwd.restype = i32
    lib.littlebit_linear_fwd_noalloc.argtypes = [ctypes.POINTER(_Layer), u32, vp, i64, i64, vp, i64, u32, vp]
    lib.littlebit_linear_fwd_noalloc.restype = i32
    lib.littlebit_workspace_error.argtypes = [vp, sz, vp, vp]
    lib.littlebit_workspace_error.restype = i32
    lib.littlebit_status_string.argtypes = [i32]
    lib.littlebit_status_string.restype = ctypes.c_char_p
    lib.littlebit_last_error.argtypes = []
    lib.littlebit_last_error.restype = ctypes.c_char_p
    return lib


LIB = _load()
_INIT_LIB = None


def _init_lib():
    """The offline initialization library, loaded on first use."""
    global _INIT_LIB
    if _INIT_LIB is None:
        if not os.path.exists(INIT_LIB_PATH):
            raise ImportError(f"{INIT_LIB_PATH} is missing: build it with `python -m binary_rank_gemv_amd.build`")
        lib = ctypes.CDLL(INIT_LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.littlebit_dual_svid_init.argtypes = [vp, i64, i64, i64, i64, i32, i32, ctypes.POINTER(_InitBranch), vp]
        lib.littlebit_dual_svid_init.restype = i32
        lib.littlebit_init_last_error.argtypes = []
        lib.littlebit_init_last_error.restype = ctypes.c_char_p
        _INIT_LIB = lib
    return _INIT_LIB


def _check(status: int):
    if status != LB_OK:
        raise LittleBitError(status, LIB.littlebit_last_error().decode())


def _stream_ptr(stream: Optional[torch.cuda.Stream] = None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t: torch.Tensor) -> int:
    return int(t.data_ptr())


# ------------------------------------------------------------------- wrappers

def littlebit_packed_bytes(R: int, K: int) -> int:
    return int(LIB.littlebit_packed_bytes(R, K))


def littlebit_status_string(status: int) -> str:
    return LIB.littlebit_status_string(status).decode()


def littlebit_last_error() -> str:
    return LIB.littlebit_last_error().decode()


def littlebit_pack(latent: torch.Tensor, transpose: bool, stream=None) -> torch.Tensor:
    """Pack sign(latent) (transpose=False) or sign(latent)^T (transpose=True)."""
    if latent.dim() != 2 or not latent.is_cuda or latent.stride(1) != 1:
        raise ValueError("latent must be a 2-D CUDA tensor with unit column stride")
    dtype = {torch.float32: LB_F32, torch.float16: LB_F16}.get(latent.dtype)
    if dtype is None:
        raise ValueError("latent must be float32 or float16")
    rows, cols = latent.shape
    R, K = (cols, rows) if transpose else (rows, cols)
    out = torch.empty(littlebit_packed_bytes(R, K), dtype=torch.uint8, device=latent.device)
    _check(LIB.littlebit_pack(_ptr(latent), dtype, rows, cols, latent.stride(0), int(transpose),
                              _ptr(out), _stream_ptr(stream)))
    return out


def littlebit_transpose_packed(bits: torch.Tensor, R: int, K: int, stream=None) -> torch.Tensor:
    """The packing of the K x R transpose of the packed R x K factor ``bits``."""
    if bits.dtype != torch.uint8 or not bits.is_cuda or bits.numel() != littlebit_packed_bytes(R, K):
        raise ValueError("bits must be the uint8 CUDA packing of an R x K factor")
    out = torch.empty(littlebit_packed_bytes(K, R), dtype=torch.uint8, device=bits.device)
    _check(LIB.littlebit_transpose_packed(_ptr(bits), R, K, _ptr(out), _stream_ptr(stream)))
    return out


def littlebit_dual_svid_init(W: torch.Tensor, r: int, nbranches: int = 2, itq_iters: int = 0,
                             stream=None) -> List[dict]:
    """Branches (dicts with U, V fp32 latents and fp16 h, l, g, all on W's
    device) of the Dual-SVID initialization of the dense weight W (m x n
    fp32 CUDA tensor, unit column stride), optionally with a Joint-ITQ
    rotation of the latent factors; ready for LittleBitLayer.from_latents."""
    if W.dtype != torch.float32 or not W.is_cuda or W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be a 2-D fp32 CUDA tensor with unit column stride")
    m, n = W.shape
    outs = []
    arr = (_InitBranch * nbranches)()
    for b in range(nbranches):
        br = {"U": torch.empty((m, r), dtype=torch.float32, device=W.device),
              "V": torch.empty((n, r), dtype=torch.float32, device=W.device),
              "h": torch.empty(m, dtype=torch.float16, device=W.device),
              "l": torch.empty(r, dtype=torch.float16, device=W.device),
              "g": torch.empty(n, dtype=torch.float16, device=W.device)}
        arr[b] = _InitBranch(_ptr(br["U"]), _ptr(br["V"]), _ptr(br["h"]), _ptr(br["l"]), _ptr(br["g"]))
        outs.append(br)
    lib = _init_lib()
    status = lib.littlebit_dual_svid_init(_ptr(W), m, n, W.stride(0), r, nbranches, itq_iters, arr,
                                          _stream_ptr(stream))
    if status != LB_OK:
        raise LittleBitError(status, lib.littlebit_init_last_error().decode())
    return outs


@dataclass
class LittleBitBranch:
    v_bits: torch.Tensor
    u_bits: torch.Tensor
    h: torch.Tensor
    l: torch.Tensor
    g: torch.Tensor
    r: int


@dataclass
class LittleBitLayer:
    """Device-resident packed layer (keeps the tensors the C struct points to)."""
    m: int
    n: int
    branches: List[LittleBitBranch] = field(default_factory=list)

    @staticmethod
    def from_latents(branches: Sequence[dict], device="cuda") -> "LittleBitLayer":
        """branches: dicts with U (m x r), V (n x r) latents and fp16 h, l, g (numpy or torch)."""
        out = []
        m = n = None
        for br in branches:
            U = torch.as_tensor(br["U"]).to(device).contiguous()
            V = torch.as_tensor(br["V"]).to(device).contiguous()
            m, r = U.shape
            n = V.shape[0]
            scales = {k: torch.as_tensor(br[k]).to(device=device, dtype=torch.float16).contiguous()
                      for k in ("h", "l", "g")}
            out.append(LittleBitBranch(v_bits=littlebit_pack(V, transpose=True),
                                       u_bits=littlebit_pack(U, transpose=False),
                                       r=int(r), **scales))
        return LittleBitLayer(m=int(m), n=int(n), branches=out)

    def transposed(self, stream=None) -> "LittleBitLayer":
        """The layer of W^T (m' = n, n' = m): sign(U) takes the V role and
        sign(V) the U role, h and g swap; littlebit_linear_fwd on it gives
        dx = W^T dy, the backward-input product of quantization-aware training."""
        out = []
        for b in self.branches:
            out.append(LittleBitBranch(v_bits=littlebit_transpose_packed(b.u_bits, self.m, b.r, stream),
                                       u_bits=littlebit_transpose_packed(b.v_bits, b.r, self.n, stream),
                                       h=b.g, l=b.l, g=b.h, r=b.r))
        return LittleBitLayer(m=self.n, n=self.m, branches=out)

    def c_struct(self) -> _Layer:
        s = _Layer()
        s.m, s.n, s.nbranches = self.m, self.n, len(self.branches)
        for i, b in enumerate(self.branches):
            s.br[i] = _Branch(_ptr(b.v_bits), _ptr(b.u_bits), _ptr(b.h), _ptr(b.l), _ptr(b.g), b.r)
        return s


class Workspace:
    """Zero-initialised device workspace, grown on demand (one per stream)."""

    def __init__(self):
        self._bufs = {}

    def get(self, nbytes: int, device: torch.device, stream_ptr: int) -> torch.Tensor:
        key = (str(device), stream_ptr)
        buf = self._bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._bufs[key] = buf
        return buf


_WS = Workspace()


def littlebit_workspace_error(workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """A one-element int32 device tensor receiving the workspace's poll error
    word (non-zero: a decode call on it since the previous report gave up
    waiting, and its outputs are wrong); the word is cleared.  Asynchronous
    on the stream: read the tensor after the stream has reached this point."""
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise ValueError("workspace must be a uint8 CUDA tensor")
    out = torch.empty(1, dtype=torch.int32, device=workspace.device)
    _check(LIB.littlebit_workspace_error(_ptr(workspace), workspace.numel(), _ptr(out), _stream_ptr(stream)))
    return out


def littlebit_linear_workspace_bytes(layer: LittleBitLayer, batch: int) -> int:
    return int(LIB.littlebit_linear_workspace_bytes(ctypes.byref(layer.c_struct()), batch))


def littlebit_block_workspace_bytes(layers: Sequence[LittleBitLayer], batch: int) -> int:
    arr = (_Layer * 7)(*[l.c_struct() for l in layers])
    return int(LIB.littlebit_block_workspace_bytes(arr, batch))


def littlebit_linear_fwd(layer: LittleBitLayer, x: torch.Tensor, branch_mask: int = 3,
                         path: int = LB_PATH_AUTO, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = layer(x) for x of shape (batch, n) fp16 on the GPU."""
    if x.dim() != 2 or x.dtype != torch.float16 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D CUDA float16 tensor with unit column stride")
    batch = x.shape[0]
    if branch_mask == 3 and len(layer.branches) == 1:
        branch_mask = 1
    y = out if out is not None else torch.empty((batch, layer.m), dtype=torch.float16, device=x.device)
    s = layer.c_struct()
    sp = _stream_ptr(stream)
    need = int(LIB.littlebit_linear_workspace_bytes(ctypes.byref(s), batch))
    ws = workspace if workspace is not None else _WS.get(need, x.device, sp)
    _check(LIB.littlebit_linear_fwd(ctypes.byref(s), branch_mask, _ptr(x), batch, x.stride(0),
                                    _ptr(y), y.stride(0), _ptr(ws), ws.numel(), path, sp))
    return y


def littlebit_linear_fwd_noalloc(layer: LittleBitLayer, x: torch.Tensor, branch_mask: int = 3,
                                 path: int = LB_PATH_AUTO, out: Optional[torch.Tensor] = None,
                                 stream=None) -> torch.Tensor:
    """littlebit_linear_fwd on the library's own per-device scratch (no
    workspace argument; the library allocates nothing).  `out` must be given
    where the caller cannot allocate either."""
    if x.dim() != 2 or x.dtype != torch.float16 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D CUDA float16 tensor with unit column stride")
    batch = x.shape[0]
    if branch_mask == 3 and len(layer.branches) == 1:
        branch_mask = 1
    y = out if out is not None else torch.empty((batch, layer.m), dtype=torch.float16, device=x.device)
    s = layer.c_struct()
    _check(LIB.littlebit_linear_fwd_noalloc(ctypes.byref(s), branch_mask, _ptr(x), batch, x.stride(0),
                                            _ptr(y), y.stride(0), path, _stream_ptr(stream)))
    return y


def littlebit_block_fwd(layers: Sequence[LittleBitLayer], x_qkv: torch.Tensor, x_o: torch.Tensor,
                        x_gu: torch.Tensor, x_down: torch.Tensor,
                        outs: Optional[Sequence[torch.Tensor]] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> List[torch.Tensor]:
    """The seven projections (q, k, v, o, gate, up, down) of one decoder block."""
    if len(layers) != 7:
        raise ValueError("a block has exactly 7 projections")
    xs = (x_qkv, x_qkv, x_qkv, x_o, x_gu, x_gu, x_down)
    batch = x_qkv.shape[0]
    for lay, xx in zip(layers, xs):
        if xx.shape != (batch, lay.n) or xx.dtype != torch.float16 or not xx.is_contiguous():
            raise ValueError("block inputs must be contiguous fp16 (batch, n) tensors")
    ys = list(outs) if outs is not None else [
        torch.empty((batch, lay.m), dtype=torch.float16, device=x_qkv.device) for lay in layers]
    arr = (_Layer * 7)(*[l.c_struct() for l in layers])
    yptrs = (ctypes.c_void_p * 7)(*[_ptr(y) for y in ys])
    sp = _stream_ptr(stream)
    need = int(LIB.littlebit_block_workspace_bytes(arr, batch))
    ws = workspace if workspace is not None else _WS.get(need, x_qkv.device, sp)
    _check(LIB.littlebit_block_fwd(arr, _ptr(x_qkv), _ptr(x_o), _ptr(x_gu), _ptr(x_down), yptrs,
                                   batch, _ptr(ws), ws.numel(), sp))
    return ys
