"""Plain CPU oracle for the BitNet b1.58 BitLinear forward (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.
The arithmetic lives in ``bitlinear_oracle.c`` (plain C, one IEEE operation
per line, built with ``-ffp-contract=off``); this module only marshals numpy
arrays.  Function-by-function citations of the pages are in that file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BETA_CHUNK = 4096

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_absmean.restype = ctypes.c_float
    lib.oracle_absmean.argtypes = [p, i64]
    lib.oracle_ternarize.restype = None
    lib.oracle_ternarize.argtypes = [p, i64, ctypes.c_float, p]
    lib.oracle_quant_act_f32.restype = None
    lib.oracle_quant_act_f32.argtypes = [p, i64, i64, p, p, p]
    lib.oracle_quant_act_bf16.restype = None
    lib.oracle_quant_act_bf16.argtypes = [p, i64, i64, p, p, p]
    lib.oracle_matmul_i32.restype = None
    lib.oracle_matmul_i32.argtypes = [p, p, i64, i64, i64, p, ctypes.c_int]
    lib.oracle_matmul_i32_pairs.restype = None
    lib.oracle_matmul_i32_pairs.argtypes = [p, p, i64, p, p, i64, p]
    lib.oracle_dequant_f32.restype = None
    lib.oracle_dequant_f32.argtypes = [p, p, ctypes.c_float, i64, i64, p]
    lib.oracle_f32_to_bf16.restype = None
    lib.oracle_f32_to_bf16.argtypes = [p, i64, p]
    lib.oracle_t2_bytes.restype = i64
    lib.oracle_t2_bytes.argtypes = [i64, i64]
    lib.oracle_pack_t2.restype = None
    lib.oracle_pack_t2.argtypes = [p, i64, i64, p]
    lib.oracle_unpack_t2.restype = i64
    lib.oracle_unpack_t2.argtypes = [p, i64, i64, p]
    lib.oracle_relu2_mul.restype = None
    lib.oracle_relu2_mul.argtypes = [p, p, i64, p]
    lib.oracle_add_f32.restype = None
    lib.oracle_add_f32.argtypes = [p, p, i64]
    lib.oracle_b1_bytes.restype = i64
    lib.oracle_b1_bytes.argtypes = [i64, i64]
    lib.oracle_binarize.restype = None
    lib.oracle_binarize.argtypes = [p, i64, p]
    lib.oracle_pack_b1.restype = None
    lib.oracle_pack_b1.argtypes = [p, i64, i64, p]
    lib.oracle_unpack_b1.restype = None
    lib.oracle_unpack_b1.argtypes = [p, i64, i64, p]
    lib.oracle_b3_bytes.restype = i64
    lib.oracle_b3_bytes.argtypes = [i64, i64]
    lib.oracle_pack_b3.restype = None
    lib.oracle_pack_b3.argtypes = [p, i64, i64, p]
    lib.oracle_unpack_b3.restype = None
    lib.oracle_unpack_b3.argtypes = [p, i64, i64, p]
    lib.oracle_train_forward.restype = None
    lib.oracle_train_forward.argtypes = [p, i64, i64, p, ctypes.c_float, i64, p, ctypes.c_int]
    lib.oracle_train_dx.restype = None
    lib.oracle_train_dx.argtypes = [p, i64, i64, p, ctypes.c_float, i64, p, ctypes.c_int]
    lib.oracle_train_dw.restype = None
    lib.oracle_train_dw.argtypes = [p, p, i64, i64, i64, p, ctypes.c_int]
    lib.oracle_rmsnorm_f32.restype = None
    lib.oracle_rmsnorm_f32.argtypes = [p, i64, i64, p]
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ weights
def absmean(w: np.ndarray) -> np.float32:
    """beta = mean |w| over the whole tensor (fp64, fixed order) -> fp32."""
    w = _c(w, np.float32)
    if w.size == 0:
        raise ValueError("absmean of an empty tensor is undefined")
    return np.float32(_load().oracle_absmean(_ptr(w), w.size))


def ternarize(w: np.ndarray, beta) -> np.ndarray:
    """t = clamp(round_half_even(w / (beta + 1e-8)), -1, 1) as int8."""
    w = _c(w, np.float32)
    t = np.empty(w.shape, dtype=np.int8)
    _load().oracle_ternarize(_ptr(w), w.size, ctypes.c_float(np.float32(beta)), _ptr(t))
    return t


# -------------------------------------------------------------- activations
def quant_act(x: np.ndarray, *, bf16_bits: bool = False):
    """Per-token absmax int8: returns (q [M][K] int8, ds [M] fp32, rowsum [M] int32).

    ``x`` is fp32 [M][K], or uint16 bf16 bit patterns when ``bf16_bits``.
    """
    if bf16_bits:
        x = _c(x, np.uint16)
    else:
        x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    ds = np.empty(M, dtype=np.float32)
    rs = np.empty(M, dtype=np.int32)
    fn = _load().oracle_quant_act_bf16 if bf16_bits else _load().oracle_quant_act_f32
    fn(_ptr(x), M, K, _ptr(q), _ptr(ds), _ptr(rs))
    return q, ds, rs


# ----------------------------------------------------------------- products
def matmul_i32(q: np.ndarray, t: np.ndarray, threads: int = 1) -> np.ndarray:
    """acc[m][n] = sum_k q[m][k] * t[n][k] (exact int32, naive loops)."""
    q = _c(q, np.int8)
    t = _c(t, np.int8)
    M, K = q.shape
    N, K2 = t.shape
    assert K == K2
    acc = np.empty((M, N), dtype=np.int32)
    _load().oracle_matmul_i32(_ptr(q), _ptr(t), M, N, K, _ptr(acc), int(threads))
    return acc


def matmul_i32_pairs(q: np.ndarray, t: np.ndarray, ms, ns) -> np.ndarray:
    """acc at the listed (m, n) pairs only."""
    q = _c(q, np.int8)
    t = _c(t, np.int8)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    assert ms.shape == ns.shape
    out = np.empty(ms.shape, dtype=np.int32)
    _load().oracle_matmul_i32_pairs(_ptr(q), _ptr(t), q.shape[1], _ptr(ms), _ptr(ns), ms.size,
                                    _ptr(out))
    return out


def dequant(acc: np.ndarray, ds: np.ndarray, beta) -> np.ndarray:
    """y[m][n] = (float)acc[m][n] * (ds[m] * beta) in fp32."""
    acc = _c(acc, np.int32)
    ds = _c(ds, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), dtype=np.float32)
    _load().oracle_dequant_f32(_ptr(acc), _ptr(ds), ctypes.c_float(np.float32(beta)), M, N,
                               _ptr(y))
    return y


def to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    y = _c(y, np.float32)
    out = np.empty(y.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16(_ptr(y), y.size, _ptr(out))
    return out


# ------------------------------------------------------------------ packing
def t2_bytes(N: int, K: int) -> int:
    return int(_load().oracle_t2_bytes(N, K))


def pack_t2(t: np.ndarray) -> np.ndarray:
    """Ternary codes [N][K] -> the 2-bit tiled format (uint8 buffer)."""
    t = _c(t, np.int8)
    N, K = t.shape
    out = np.empty(t2_bytes(N, K), dtype=np.uint8)
    _load().oracle_pack_t2(_ptr(t), N, K, _ptr(out))
    return out


def unpack_t2(packed: np.ndarray, N: int, K: int):
    """Inverse of pack_t2: returns (t [N][K] int8, count of invalid 10 codes)."""
    packed = _c(packed, np.uint8)
    assert packed.size >= t2_bytes(N, K)
    t = np.empty((N, K), dtype=np.int8)
    bad = _load().oracle_unpack_t2(_ptr(packed), N, K, _ptr(t))
    return t, int(bad)


# ------------------------------------------------------------ decoder glue
EPS_NORM = np.float32(1e-5)


def rmsnorm(x: np.ndarray) -> np.ndarray:
    """Row-wise RMS normalization (gain 1) of fp32 x [M][K]."""
    x = _c(x, np.float32)
    M, K = x.shape
    out = np.empty_like(x)
    _load().oracle_rmsnorm_f32(_ptr(x), M, K, _ptr(out))
    return out


def relu2_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = ReLU(g)^2 * u elementwise, fp32 (r = g if g > 0 else 0; (r*r)*u)."""
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    assert g.shape == u.shape
    h = np.empty_like(g)
    _load().oracle_relu2_mul(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def add_f32(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Residual sum x + r, fp32 (returns a new array)."""
    out = _c(x, np.float32).copy()
    r = _c(r, np.float32)
    assert out.shape == r.shape
    _load().oracle_add_f32(_ptr(out), _ptr(r), out.size)
    return out


# ------------------------------------------------------------ binary weights
def binarize(w: np.ndarray) -> np.ndarray:
    """int8 codes t = +1 where w >= 0, else -1."""
    w = _c(w, np.float32)
    t = np.empty(w.shape, dtype=np.int8)
    _load().oracle_binarize(_ptr(w), w.size, _ptr(t))
    return t


def b1_bytes(N: int, K: int) -> int:
    return int(_load().oracle_b1_bytes(N, K))


def pack_b1(t: np.ndarray) -> np.ndarray:
    t = _c(t, np.int8)
    N, K = t.shape
    out = np.empty(b1_bytes(N, K), dtype=np.uint8)
    _load().oracle_pack_b1(_ptr(t), N, K, _ptr(out))
    return out


def unpack_b1(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    assert packed.size >= b1_bytes(N, K)
    t = np.empty((N, K), dtype=np.int8)
    _load().oracle_unpack_b1(_ptr(packed), N, K, _ptr(t))
    return t


def b3_bytes(N: int, K: int) -> int:
    return int(_load().oracle_b3_bytes(N, K))


def pack_b3(t: np.ndarray) -> np.ndarray:
    """Ternary codes [N][K] -> base-3 tiles (five weights per byte)."""
    t = _c(t, np.int8)
    N, K = t.shape
    out = np.empty(b3_bytes(N, K), dtype=np.uint8)
    _load().oracle_pack_b3(_ptr(t), N, K, _ptr(out))
    return out


def unpack_b3(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    assert packed.size >= b3_bytes(N, K)
    t = np.empty((N, K), dtype=np.int8)
    _load().oracle_unpack_b3(_ptr(packed), N, K, _ptr(t))
    return t


def bitlinear_forward_b1(x_bf16_bits: np.ndarray, w: np.ndarray, threads: int = 1) -> dict:
    """BitLinear forward with binary weights; every intermediate as a dict."""
    beta = absmean(w)
    t = binarize(w)
    q, ds, rs = quant_act(x_bf16_bits, bf16_bits=True)
    acc = matmul_i32(q, t, threads=threads)
    y = dequant(acc, ds, beta)
    return {"beta": beta, "t": t, "q": q, "ds": ds, "rowsum": rs, "acc": acc, "y": y,
            "y_bf16": to_bf16_bits(y)}


# ------------------------------------------------------------ training step
def train_forward(x_bf16_bits: np.ndarray, t: np.ndarray, beta, threads: int = 1) -> np.ndarray:
    """y = x . (beta t)^T from bf16 x [M][K] and ternary codes t [N][K]."""
    xb = _c(x_bf16_bits, np.uint16)
    t = _c(t, np.int8)
    M, K = xb.shape
    N = t.shape[0]
    y = np.empty((M, N), dtype=np.float32)
    _load().oracle_train_forward(_ptr(xb), M, K, _ptr(t), float(beta), N, _ptr(y), threads)
    return y


def train_dx(dy_bf16_bits: np.ndarray, t: np.ndarray, beta, threads: int = 1) -> np.ndarray:
    """dx = dy . (beta t) from bf16 dy [M][N] and ternary codes t [N][K]."""
    dyb = _c(dy_bf16_bits, np.uint16)
    t = _c(t, np.int8)
    M, N = dyb.shape
    K = t.shape[1]
    dx = np.empty((M, K), dtype=np.float32)
    _load().oracle_train_dx(_ptr(dyb), M, N, _ptr(t), float(beta), K, _ptr(dx), threads)
    return dx


def train_dw(dy_bf16_bits: np.ndarray, x_bf16_bits: np.ndarray, threads: int = 1) -> np.ndarray:
    """dw = dy^T . x (the straight-through gradient of the latent weights)."""
    dyb = _c(dy_bf16_bits, np.uint16)
    xb = _c(x_bf16_bits, np.uint16)
    M, N = dyb.shape
    K = xb.shape[1]
    dw = np.empty((N, K), dtype=np.float32)
    _load().oracle_train_dw(_ptr(dyb), _ptr(xb), M, N, K, _ptr(dw), threads)
    return dw


# ------------------------------------------------------------ whole forward
def bitlinear_forward(x_bf16_bits: np.ndarray, w: np.ndarray, threads: int = 1) -> dict:
    """Whole BitLinear forward; returns every intermediate as a dict."""
    beta = absmean(w)
    t = ternarize(w, beta)
    q, ds, rs = quant_act(x_bf16_bits, bf16_bits=True)
    acc = matmul_i32(q, t, threads=threads)
    y = dequant(acc, ds, beta)
    return {"beta": beta, "t": t, "q": q, "ds": ds, "rowsum": rs, "acc": acc, "y": y,
            "y_bf16": to_bf16_bits(y)}
