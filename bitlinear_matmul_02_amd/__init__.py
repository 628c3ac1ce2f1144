"""Python binding of libbitlinear: the BitNet b1.58 BitLinear forward on MI355X.

Argument marshalling only.  Every function here forwards torch tensors' device
pointers and the current HIP stream to the C ABI declared in
``include/bitlinear.h`` and raises ``BitLinearError`` on a non-zero status.
There is no fallback: if the HIP library is not built, every call raises.

Functions carry the C names:
    bitlinear_quant_act(x, x_q, x_ds, x_rowsum=None)
    bitlinear_pack_weights(w, packed, w_beta, workspace)
    bitlinear_gemv(x_q, x_ds, K, packed, w_beta, N, y, workspace=None)
    bitlinear_gemm(x_q, x_ds, K, packed, w_beta, N, y, workspace=None)
    bitlinear_forward_decode(x, packed, w_beta, N, y)
    bitlinear_relu2_mul(g, u, h)
    bitlinear_gemv_multi(x_q, x_ds, K, packed_list, beta_list, N_list, y_list)
    bitlinear_forward_decode_multi(x, packed_list, beta_list, N_list, y_list)
    bitlinear_gemv_glu(x_q, x_ds, K, packed_gate, beta_gate, packed_up, beta_up, N, h)
    bitlinear_forward_decode_glu(x, packed_gate, beta_gate, packed_up, beta_up, N, h)
    bitlinear_pack_weights_b1(w, packed, w_beta, workspace)      (binary weights)
    bitlinear_gemv_b1(x_q, x_ds, x_rowsum, K, packed, w_beta, N, y)
    bitlinear_gemm_b1(x_q, x_ds, x_rowsum, K, packed, w_beta, N, y)
    bitlinear_pack_weights_b3(w, packed, w_beta, workspace)      (base-3 ternary)
    bitlinear_gemv_b3(x_q, x_ds, x_rowsum, K, packed, w_beta, N, y)
    bitlinear_train_forward(x, packed, w_beta, N, y)            (training, straight-through)
    bitlinear_train_backward_input(dy, packed, w_beta, K, dx)
    bitlinear_train_backward_weight(dy, x, dw)
An fp32 output tensor can be passed with ``accumulate=True`` to the product
calls, which then add their result into it (``BITLINEAR_F32_ADD``); the calls
that quantize activations take ``rmsnorm=True`` to RMS-normalize each row
first (``BITLINEAR_X_RMSNORM``).
plus allocation helpers (``act_stride``, ``packed_bytes`` ...) and two
conveniences that allocate outputs (``quant_act``, ``pack_weights``,
``linear``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libbitlinear.so")

OK, ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_HIP = 0, -1, -2, -3, -4, -5
F32, BF16, I32, F32_ADD = 0, 1, 2, 3
X_RMSNORM = 16  # flag OR-ed into an activation dtype: RMS-normalize rows before quantizing
NOALLOC_SCRATCH_BYTES = 8 << 20  # device array behind bitlinear_gemv_noalloc
MAX_K, MAX_N, MAX_M, GEMV_MAX_M = 131072, 1 << 20, 1 << 20, 64

EXPORTS = (
    "bitlinear_version", "bitlinear_last_error", "bitlinear_act_stride", "bitlinear_packed_bytes",
    "bitlinear_pack_workspace_bytes", "bitlinear_gemv_workspace_bytes",
    "bitlinear_gemm_workspace_bytes", "bitlinear_quant_act", "bitlinear_pack_weights",
    "bitlinear_gemv", "bitlinear_gemm", "bitlinear_forward_decode", "bitlinear_relu2_mul",
    "bitlinear_gemv_multi", "bitlinear_forward_decode_multi", "bitlinear_gemv_glu",
    "bitlinear_forward_decode_glu", "bitlinear_packed_bytes_b1", "bitlinear_pack_weights_b1",
    "bitlinear_gemv_b1", "bitlinear_gemm_b1", "bitlinear_packed_bytes_b3", "bitlinear_pack_weights_b3",
    "bitlinear_gemv_b3", "bitlinear_train_forward", "bitlinear_train_backward_input",
    "bitlinear_train_backward_weight", "bitlinear_gemv_read_extent", "bitlinear_gemv_noalloc",
    "bitlinear_decode_rq",
)
MULTI_MAX = 4
DECODE_MAX_ACT_BYTES = 58368

_DTYPE = {torch.float32: F32, torch.bfloat16: BF16, torch.int32: I32}


class BitLinearError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("status %d: %s" % (status, message))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libbitlinear.so is not built (%s); run "
                          "`python -m bitlinear_matmul_02_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, p, i32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.bitlinear_version.restype = i32
    L.bitlinear_version.argtypes = []
    L.bitlinear_last_error.restype = ctypes.c_char_p
    L.bitlinear_last_error.argtypes = []
    for name in ("bitlinear_act_stride",):
        getattr(L, name).restype = i64
        getattr(L, name).argtypes = [i64]
    for name in ("bitlinear_packed_bytes", "bitlinear_pack_workspace_bytes"):
        getattr(L, name).restype = i64
        getattr(L, name).argtypes = [i64, i64]
    for name in ("bitlinear_gemv_workspace_bytes", "bitlinear_gemm_workspace_bytes"):
        getattr(L, name).restype = i64
        getattr(L, name).argtypes = [i64, i64, i64]
    L.bitlinear_quant_act.restype = i32
    L.bitlinear_quant_act.argtypes = [p, i32, i64, i64, p, p, p, p]
    L.bitlinear_pack_weights.restype = i32
    L.bitlinear_pack_weights.argtypes = [p, i64, i64, p, p, p, p]
    for name in ("bitlinear_gemv", "bitlinear_gemm"):
        getattr(L, name).restype = i32
        getattr(L, name).argtypes = [p, p, i64, i64, p, p, i64, p, i32, p, sz, p]
    L.bitlinear_forward_decode.restype = i32
    L.bitlinear_forward_decode.argtypes = [p, i32, i64, i64, p, p, i64, p, i32, p]
    L.bitlinear_packed_bytes_b1.restype = i64
    L.bitlinear_packed_bytes_b1.argtypes = [i64, i64]
    L.bitlinear_pack_weights_b1.restype = i32
    L.bitlinear_pack_weights_b1.argtypes = [p, i64, i64, p, p, p, p]
    L.bitlinear_gemv_b1.restype = i32
    L.bitlinear_gemv_b1.argtypes = [p, p, p, i64, i64, p, p, i64, p, i32, p]
    L.bitlinear_packed_bytes_b3.restype = i64
    L.bitlinear_packed_bytes_b3.argtypes = [i64, i64]
    L.bitlinear_pack_weights_b3.restype = i32
    L.bitlinear_pack_weights_b3.argtypes = [p, i64, i64, p, p, p, p]
    L.bitlinear_gemv_b3.restype = i32
    L.bitlinear_gemv_b3.argtypes = [p, p, p, i64, i64, p, p, i64, p, i32, p]
    L.bitlinear_train_forward.restype = i32
    L.bitlinear_train_forward.argtypes = [p, i64, i64, p, p, i64, p, p]
    L.bitlinear_train_backward_input.restype = i32
    L.bitlinear_train_backward_input.argtypes = [p, i64, i64, p, p, i64, p, p]
    L.bitlinear_train_backward_weight.restype = i32
    L.bitlinear_train_backward_weight.argtypes = [p, p, i64, i64, i64, p, p]
    L.bitlinear_gemm_b1.restype = i32
    L.bitlinear_gemm_b1.argtypes = [p, p, p, i64, i64, p, p, i64, p, i32, p]
    L.bitlinear_relu2_mul.restype = i32
    L.bitlinear_relu2_mul.argtypes = [p, p, i64, p, p]
    L.bitlinear_gemv_multi.restype = i32
    L.bitlinear_gemv_multi.argtypes = [p, p, i64, i64, i32, p, p, p, p, i32, p]
    L.bitlinear_forward_decode_multi.restype = i32
    L.bitlinear_forward_decode_multi.argtypes = [p, i32, i64, i64, i32, p, p, p, p, i32, p]
    L.bitlinear_gemv_glu.restype = i32
    L.bitlinear_gemv_glu.argtypes = [p, p, i64, i64, p, p, p, p, i64, p, p]
    L.bitlinear_forward_decode_glu.restype = i32
    L.bitlinear_forward_decode_glu.argtypes = [p, i32, i64, i64, p, p, p, p, i64, p, p]
    L.bitlinear_decode_rq.restype = i32
    L.bitlinear_decode_rq.argtypes = [p, p, i64, i64, i32, i32, p, p, p, p, i32, p, p, i32, p, sz, p]
    L.bitlinear_gemv_noalloc.restype = i32
    L.bitlinear_gemv_noalloc.argtypes = [p, p, i64, i64, p, p, i64, p, i32, p]
    L.bitlinear_gemv_read_extent.restype = i32
    L.bitlinear_gemv_read_extent.argtypes = [i64, i64, i64, i32, p, p]
    _lib = L
    return L


def last_error() -> str:
    return lib().bitlinear_last_error().decode()


def _check(status: int) -> None:
    if status != OK:
        raise BitLinearError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _record(stream, *tensors):
    """Tensors allocated on the current stream but used by work enqueued on
    ``stream``: mark them as used there, so that the caching allocator does
    not hand their memory out again before that stream's work is done."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


# --------------------------------------------------------------- size helpers
def act_stride(K: int) -> int:
    return int(lib().bitlinear_act_stride(K))


def packed_bytes(N: int, K: int) -> int:
    return int(lib().bitlinear_packed_bytes(N, K))


def packed_bytes_b1(N: int, K: int) -> int:
    return int(lib().bitlinear_packed_bytes_b1(N, K))


def packed_bytes_b3(N: int, K: int) -> int:
    return int(lib().bitlinear_packed_bytes_b3(N, K))


def pack_workspace_bytes(N: int, K: int) -> int:
    return int(lib().bitlinear_pack_workspace_bytes(N, K))


def gemv_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().bitlinear_gemv_workspace_bytes(M, N, K))


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().bitlinear_gemm_workspace_bytes(M, N, K))


def gemv_read_extent(M: int, N: int, K: int, fmt: int = 0) -> tuple[int, int]:
    """(activation, weight) read extents in bytes of the decode kernel's plan (host model)."""
    a, w = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().bitlinear_gemv_read_extent(M, N, K, fmt, ctypes.byref(a), ctypes.byref(w)))
    return a.value, w.value


# --------------------------------------------------------------- the C calls
def _xdtype(x, rmsnorm: bool) -> int:
    return _DTYPE[x.dtype] | (X_RMSNORM if rmsnorm else 0)


def bitlinear_quant_act(x, x_q, x_ds, x_rowsum=None, stream=None, rmsnorm: bool = False) -> None:
    """x [M][K] bf16/fp32 -> x_q [M][act_stride(K)] int8, x_ds [M] fp32, x_rowsum [M] int32."""
    M, K = x.shape
    _check(lib().bitlinear_quant_act(_ptr(x), _xdtype(x, rmsnorm), M, K, _ptr(x_q), _ptr(x_ds),
                                     _ptr(x_rowsum), _stream(stream)))


def bitlinear_pack_weights(w, packed, w_beta, workspace, stream=None) -> None:
    """w [N][K] fp32 latent weights -> packed 2-bit tiles + w_beta [1] fp32."""
    N, K = w.shape
    _check(lib().bitlinear_pack_weights(_ptr(w), N, K, _ptr(packed), _ptr(w_beta), _ptr(workspace),
                                        _stream(stream)))


def bitlinear_pack_weights_b1(w, packed, w_beta, workspace, stream=None) -> None:
    """w [N][K] fp32 latent weights -> 1-bit tiles (t = +1 where w >= 0, else -1) + w_beta."""
    N, K = w.shape
    _check(lib().bitlinear_pack_weights_b1(_ptr(w), N, K, _ptr(packed), _ptr(w_beta), _ptr(workspace),
                                           _stream(stream)))


def bitlinear_gemv_b1(x_q, x_ds, x_rowsum, K, packed, w_beta, N, y, stream=None, accumulate: bool = False) -> None:
    """y [M][N] = dequant(x_q . T^T) for binary weights, M <= 64 tokens."""
    _check(lib().bitlinear_gemv_b1(_ptr(x_q), _ptr(x_ds), _ptr(x_rowsum), x_ds.shape[0], K, _ptr(packed),
                                   _ptr(w_beta), N, _ptr(y), _ydtype(y, accumulate), _stream(stream)))


def bitlinear_gemm_b1(x_q, x_ds, x_rowsum, K, packed, w_beta, N, y, stream=None, accumulate: bool = False) -> None:
    """The binary-weight product for any number of tokens, on the int8 matrix cores."""
    _check(lib().bitlinear_gemm_b1(_ptr(x_q), _ptr(x_ds), _ptr(x_rowsum), x_ds.shape[0], K, _ptr(packed),
                                   _ptr(w_beta), N, _ptr(y), _ydtype(y, accumulate), _stream(stream)))


def bitlinear_pack_weights_b3(w, packed, w_beta, workspace, stream=None) -> None:
    """w [N][K] fp32 latent weights -> ternary codes five to a byte (base 3) + w_beta."""
    N, K = w.shape
    _check(lib().bitlinear_pack_weights_b3(_ptr(w), N, K, _ptr(packed), _ptr(w_beta), _ptr(workspace),
                                           _stream(stream)))


def bitlinear_gemv_b3(x_q, x_ds, x_rowsum, K, packed, w_beta, N, y, stream=None, accumulate: bool = False) -> None:
    """y [M][N] = dequant(x_q . T^T) from base-3 packed ternary weights, M <= 64 tokens."""
    _check(lib().bitlinear_gemv_b3(_ptr(x_q), _ptr(x_ds), _ptr(x_rowsum), x_ds.shape[0], K, _ptr(packed),
                                   _ptr(w_beta), N, _ptr(y), _ydtype(y, accumulate), _stream(stream)))


def _bf16_2d(t, name):
    if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous():
        raise BitLinearError(ERR_ARG, "%s must be a contiguous 2-D bf16 tensor" % name)


def bitlinear_train_forward(x, packed, w_beta, N, y, stream=None) -> None:
    """y [M][N] = beta * x . t^T (training forward, x bf16 unquantized, y fp32)."""
    _bf16_2d(x, "x")
    M, K = x.shape
    _check(lib().bitlinear_train_forward(_ptr(x), M, K, _ptr(packed), _ptr(w_beta), N, _ptr(y), _stream(stream)))


def bitlinear_train_backward_input(dy, packed, w_beta, K, dx, stream=None) -> None:
    """dx [M][K] = beta * dy . t (straight-through input gradient)."""
    _bf16_2d(dy, "dy")
    M, N = dy.shape
    _check(lib().bitlinear_train_backward_input(_ptr(dy), M, N, _ptr(packed), _ptr(w_beta), K, _ptr(dx),
                                                _stream(stream)))


def bitlinear_train_backward_weight(dy, x, dw, stream=None) -> None:
    """dw [N][K] = dy^T . x (straight-through gradient of the latent weights)."""
    _bf16_2d(dy, "dy")
    _bf16_2d(x, "x")
    M, N = dy.shape
    K = x.shape[1]
    _check(lib().bitlinear_train_backward_weight(_ptr(dy), _ptr(x), M, N, K, _ptr(dw), _stream(stream)))


def _ydtype(y, accumulate: bool) -> int:
    if accumulate:
        if y.dtype != torch.float32:
            raise BitLinearError(ERR_ARG, "accumulate needs an fp32 output")
        return F32_ADD
    return _DTYPE[y.dtype]


def _product(fn, x_q, x_ds, M, K, packed, w_beta, N, y, workspace, stream, accumulate):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(_ptr(x_q), _ptr(x_ds), M, K, _ptr(packed), _ptr(w_beta), N, _ptr(y), _ydtype(y, accumulate),
              _ptr(workspace), ws_bytes, _stream(stream)))


def bitlinear_gemv(x_q, x_ds, K, packed, w_beta, N, y, workspace=None, stream=None,
                   accumulate: bool = False) -> None:
    """y [M][N] = dequant(x_q . T^T) for M <= 64 tokens (y dtype fp32, bf16 or int32;
    with ``accumulate`` y += the fp32 result)."""
    _product(lib().bitlinear_gemv, x_q, x_ds, x_ds.shape[0], K, packed, w_beta, N, y, workspace,
             stream, accumulate)


def bitlinear_gemv_noalloc(x_q, x_ds, K, packed, w_beta, N, y, stream=None, accumulate: bool = False) -> None:
    """bitlinear_gemv without a workspace: split-k partial sums live in the library's
    device-resident scratch array (no allocation; calls on one GPU must not overlap)."""
    _check(lib().bitlinear_gemv_noalloc(_ptr(x_q), _ptr(x_ds), x_ds.shape[0], K, _ptr(packed), _ptr(w_beta), N,
                                        _ptr(y), _ydtype(y, accumulate), _stream(stream)))


def bitlinear_gemm(x_q, x_ds, K, packed, w_beta, N, y, workspace=None, stream=None,
                   accumulate: bool = False) -> None:
    """The same product for any number of tokens, on the int8 matrix cores."""
    _product(lib().bitlinear_gemm, x_q, x_ds, x_ds.shape[0], K, packed, w_beta, N, y, workspace,
             stream, accumulate)


def bitlinear_forward_decode(x, packed, w_beta, N, y, stream=None, accumulate: bool = False,
                             rmsnorm: bool = False) -> None:
    """y [M][N] = BitLinear(x) for M <= 64 tokens in one launch (quantization fused)."""
    M, K = x.shape
    _check(lib().bitlinear_forward_decode(_ptr(x), _xdtype(x, rmsnorm), M, K, _ptr(packed), _ptr(w_beta), N,
                                          _ptr(y), _ydtype(y, accumulate), _stream(stream)))


def _arrays(packed, w_beta, N, y, accumulate):
    count = len(packed)
    if not (count == len(w_beta) == len(N) == len(y)):
        raise BitLinearError(ERR_ARG, "multi: lists of different lengths")
    if len({t.dtype for t in y}) != 1:
        raise BitLinearError(ERR_ARG, "multi: outputs must share one dtype")
    vp = ctypes.c_void_p * count
    return (count, vp(*[t.data_ptr() for t in packed]), vp(*[t.data_ptr() for t in w_beta]),
            (ctypes.c_int64 * count)(*[int(n) for n in N]), vp(*[t.data_ptr() for t in y]),
            _ydtype(y[0], accumulate))


def bitlinear_gemv_multi(x_q, x_ds, K, packed, w_beta, N, y, stream=None, accumulate: bool = False) -> None:
    """y[i] (+)= dequant(x_q . T_i^T) for several BitLinears on one input, one launch."""
    count, pp, bp, nn, yp, ydt = _arrays(packed, w_beta, N, y, accumulate)
    _check(lib().bitlinear_gemv_multi(_ptr(x_q), _ptr(x_ds), x_ds.shape[0], K, count, pp, bp, nn, yp, ydt,
                                      _stream(stream)))


def bitlinear_forward_decode_multi(x, packed, w_beta, N, y, stream=None, accumulate: bool = False,
                                   rmsnorm: bool = False) -> None:
    """The same with the activation quantization fused (x bf16 / fp32)."""
    M, K = x.shape
    count, pp, bp, nn, yp, ydt = _arrays(packed, w_beta, N, y, accumulate)
    _check(lib().bitlinear_forward_decode_multi(_ptr(x), _xdtype(x, rmsnorm), M, K, count, pp, bp, nn, yp, ydt,
                                                _stream(stream)))


def _glu_out(h):
    if h.dtype != torch.float32:
        raise BitLinearError(ERR_ARG, "glu: h must be fp32")


def bitlinear_gemv_glu(x_q, x_ds, K, packed_gate, beta_gate, packed_up, beta_up, N, h, stream=None) -> None:
    """h = ReLU(BL_gate)^2 * BL_up on quantized activations, one launch."""
    _glu_out(h)
    _check(lib().bitlinear_gemv_glu(_ptr(x_q), _ptr(x_ds), x_ds.shape[0], K, _ptr(packed_gate), _ptr(beta_gate),
                                    _ptr(packed_up), _ptr(beta_up), N, _ptr(h), _stream(stream)))


def bitlinear_forward_decode_glu(x, packed_gate, beta_gate, packed_up, beta_up, N, h, stream=None,
                                 rmsnorm: bool = False) -> None:
    """The same with the activation quantization fused (x bf16 / fp32)."""
    _glu_out(h)
    M, K = x.shape
    _check(lib().bitlinear_forward_decode_glu(_ptr(x), _xdtype(x, rmsnorm), M, K, _ptr(packed_gate),
                                              _ptr(beta_gate), _ptr(packed_up), _ptr(beta_up), N, _ptr(h),
                                              _stream(stream)))


def bitlinear_decode_rq(x_q, x_ds, K, packed, w_beta, N, y, next_q, next_ds, workspace, stream=None,
                        accumulate: bool = False, glu: bool = False, next_rmsnorm: bool = False) -> None:
    """Products of bitlinear_gemv_multi (or the gated pair when ``glu``: packed = [gate, up],
    y = [h]) whose last workgroup quantizes y[0] (or h) into next_q / next_ds for the next
    BitLinear (RMS-normalized first with ``next_rmsnorm``)."""
    count = len(packed)
    P = ctypes.c_void_p * count
    Bp = ctypes.c_void_p * count
    Np = ctypes.c_int64 * count
    ys = list(y)
    if glu:
        assert count == 2 and len(ys) == 1
        Ns = [N, N] if isinstance(N, int) else list(N)
        ys = [ys[0], ys[0]]
    else:
        Ns = list(N)
    Y = ctypes.c_void_p * count
    ydt = _ydtype(ys[0], accumulate)
    _check(lib().bitlinear_decode_rq(_ptr(x_q), _ptr(x_ds), x_ds.shape[0], K, count, int(glu),
                                     P(*[t.data_ptr() for t in packed]), Bp(*[t.data_ptr() for t in w_beta]),
                                     Np(*Ns), Y(*[t.data_ptr() for t in ys]), ydt, _ptr(next_q), _ptr(next_ds),
                                     X_RMSNORM if next_rmsnorm else 0, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))


def bitlinear_relu2_mul(g, u, h, stream=None) -> None:
    """h = ReLU(g)^2 * u elementwise (fp32 tensors of one shape)."""
    if not (g.dtype == u.dtype == h.dtype == torch.float32) or not (g.shape == u.shape == h.shape):
        raise BitLinearError(ERR_ARG, "relu2_mul needs fp32 tensors of one shape")
    _check(lib().bitlinear_relu2_mul(_ptr(g), _ptr(u), g.numel(), _ptr(h), _stream(stream)))


def decode_fits(M: int, K: int) -> bool:
    return 1 <= M <= GEMV_MAX_M and M * ((K + 255) // 256 * 256 + 16) <= DECODE_MAX_ACT_BYTES


# ------------------------------------------------------------- conveniences
_ws_cache: dict = {}


def workspace(nbytes: int, device, stream=None) -> torch.Tensor | None:
    """A zero-filled workspace of at least nbytes, cached per device.  The
    products leave it zero again; calls on different streams must not overlap
    (they share it).  ``stream``: the stream the caller's kernels use it on."""
    if nbytes <= 0:
        return None
    key = torch.device(device)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=key)
        _ws_cache[key] = buf
    _record(stream, buf)
    return buf


def quant_act(x, with_rowsum: bool = False, stream=None, rmsnorm: bool = False):
    M, K = x.shape
    x_q = torch.empty((M, act_stride(K)), dtype=torch.int8, device=x.device)
    x_ds = torch.empty((M,), dtype=torch.float32, device=x.device)
    rs = torch.empty((M,), dtype=torch.int32, device=x.device) if with_rowsum else None
    bitlinear_quant_act(x, x_q, x_ds, rs, stream, rmsnorm=rmsnorm)
    _record(stream, x_q, x_ds, rs)
    return (x_q, x_ds, rs) if with_rowsum else (x_q, x_ds)


def pack_weights(w, stream=None):
    N, K = w.shape
    packed = torch.empty((packed_bytes(N, K),), dtype=torch.uint8, device=w.device)
    beta = torch.empty((1,), dtype=torch.float32, device=w.device)
    ws = torch.empty((pack_workspace_bytes(N, K),), dtype=torch.uint8, device=w.device)
    bitlinear_pack_weights(w, packed, beta, ws, stream)
    _record(stream, packed, beta, ws)
    return packed, beta


def pack_weights_b1(w, stream=None):
    N, K = w.shape
    packed = torch.empty((packed_bytes_b1(N, K),), dtype=torch.uint8, device=w.device)
    beta = torch.empty((1,), dtype=torch.float32, device=w.device)
    ws = torch.empty((pack_workspace_bytes(N, K),), dtype=torch.uint8, device=w.device)
    bitlinear_pack_weights_b1(w, packed, beta, ws, stream)
    _record(stream, packed, beta, ws)
    return packed, beta


def pack_weights_b3(w, stream=None):
    N, K = w.shape
    packed = torch.empty((packed_bytes_b3(N, K),), dtype=torch.uint8, device=w.device)
    beta = torch.empty((1,), dtype=torch.float32, device=w.device)
    ws = torch.empty((pack_workspace_bytes(N, K),), dtype=torch.uint8, device=w.device)
    bitlinear_pack_weights_b3(w, packed, beta, ws, stream)
    _record(stream, packed, beta, ws)
    return packed, beta


def linear(x, packed, w_beta, N: int, out_dtype=torch.float32, stream=None):
    """BitLinear forward: quantize x [M][K], then gemv (M <= 64) or gemm."""
    M, K = x.shape
    y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _record(stream, y)
    if M <= 4 and decode_fits(M, K):
        bitlinear_forward_decode(x, packed, w_beta, N, y, stream)
        return y
    x_q, x_ds = quant_act(x, stream=stream)
    if M <= GEMV_MAX_M:
        ws = workspace(gemv_workspace_bytes(M, N, K), x.device, stream)
        bitlinear_gemv(x_q, x_ds, K, packed, w_beta, N, y, ws, stream)
    else:
        ws = workspace(gemm_workspace_bytes(M, N, K), x.device, stream)
        bitlinear_gemm(x_q, x_ds, K, packed, w_beta, N, y, ws, stream)
    return y
