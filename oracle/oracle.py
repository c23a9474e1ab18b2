"""numpy front end of the C oracle in ``zq_oracle.c`` (test infrastructure only).

Every function takes and returns host numpy arrays.  fp16 data travels as
``numpy.float16`` arrays (the bytes are handed to the C code unchanged, the C
code decodes binary16 itself).  Sources are cited in ``zq_oracle.c``:
ZeroQuant summary page, Sec. 3.4 "Group-wise Weight Quantization" (paper
Sec. 4.1, Eq. (2)), "Token-wise Activation Quantization" (paper Sec. 4.1) and
"Quantization-Optimized Transformer Kernels" (paper Sec. 4.3, App. D, Fig. 2).
"""
import ctypes
import os

import numpy as np

from . import build as _build

__all__ = [
    "lib", "half_to_double", "double_to_half", "quantize_weights", "pack_w4",
    "unpack_w4", "layernorm", "quant_tokens", "gemm_i32", "epilogue",
    "linear", "gemm_w8a16", "calibrate_minmax", "quant_static", "threads",
    "set_threads",
]

_lib = None


def lib():
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is None:
        # ZQ_ORACLE_LIB lets the mutation tests point the pins at a variant
        # of the oracle with a planted mistake.
        path = os.environ.get("ZQ_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.zqo_half_to_double_array.argtypes = [P, ctypes.c_size_t, P]
        L.zqo_double_to_half_array.argtypes = [P, ctypes.c_size_t, P]
        L.zqo_quantize_weights.argtypes = [P, I, I, I, I, P, P]
        L.zqo_quantize_weights.restype = I
        L.zqo_pack_w4.argtypes = [P, I, I, P]
        L.zqo_unpack_w4.argtypes = [P, I, I, P]
        L.zqo_layernorm.argtypes = [P, P, P, ctypes.c_float, I, I, P]
        L.zqo_quant_tokens.argtypes = [P, I, I, P, P]
        L.zqo_gemm_i32.argtypes = [P, P, I, I, I, P]
        L.zqo_gemm_i32.restype = ctypes.c_long
        L.zqo_epilogue.argtypes = [P, P, P, I, P, I, I, I, P, P]
        L.zqo_gemm_w8a16.argtypes = [P, P, P, I, P, I, I, I, I, P, P]
        L.zqo_calibrate_minmax.argtypes = [P, ctypes.c_size_t, ctypes.c_float,
                                           I, P]
        L.zqo_quant_static.argtypes = [P, ctypes.c_size_t, P, P]
        L.zqo_quant_static.restype = ctypes.c_float
        L.zqo_threads.argtypes = []
        L.zqo_threads.restype = I
        L.zqo_set_threads.argtypes = [I]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _h(a):
    """fp16 array viewed as raw uint16 bits (contiguous)."""
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


def half_to_double(h):
    h = _h(h)
    out = np.empty(h.shape, np.float64)
    lib().zqo_half_to_double_array(_ptr(h), h.size, _ptr(out))
    return out


def double_to_half(v):
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().zqo_double_to_half_array(_ptr(v), v.size, _ptr(out))
    return out.view(np.float16)


def quantize_weights(w, G, bits):
    """Group-wise quantization of fp16 W[N,K] -> (codes int8 [N,K], sw fp32 [N/G])."""
    w = _h(w)
    N, K = w.shape
    q = np.empty((N, K), np.int8)
    sw = np.empty(N // G if G > 0 else 0, np.float32)
    rc = lib().zqo_quantize_weights(_ptr(w), N, K, G, bits, _ptr(q), _ptr(sw))
    if rc != 0:
        raise ValueError(f"bad arguments N={N} K={K} G={G} bits={bits}")
    return q, sw


def pack_w4(q):
    q = _c(q, np.int8)
    N, K = q.shape
    assert K % 2 == 0
    p = np.empty((N, K // 2), np.uint8)
    lib().zqo_pack_w4(_ptr(q), N, K, _ptr(p))
    return p


def unpack_w4(p, K=None):
    p = _c(p, np.uint8)
    N = p.shape[0]
    K = 2 * p.shape[1] if K is None else K
    q = np.empty((N, K), np.int8)
    lib().zqo_unpack_w4(_ptr(p), N, K, _ptr(q))
    return q


def layernorm(x, gamma=None, beta=None, eps=1e-5):
    x = _h(x)
    M, K = x.shape
    g = None if gamma is None else _h(gamma)
    b = None if beta is None else _h(beta)
    h = np.empty((M, K), np.uint16)
    lib().zqo_layernorm(_ptr(x), _ptr(g), _ptr(b), ctypes.c_float(eps), M, K,
                        _ptr(h))
    return h.view(np.float16)


def quant_tokens(h):
    """Token-wise quantization of fp16 [M,K] -> (qx int8 [M,K], sx fp32 [M])."""
    h = _h(h)
    M, K = h.shape
    q = np.empty((M, K), np.int8)
    sx = np.empty(M, np.float32)
    lib().zqo_quant_tokens(_ptr(h), M, K, _ptr(q), _ptr(sx))
    return q, sx


def gemm_i32(qx, qw, check_overflow=True):
    """acc[t,n] = sum_k qx[t,k]*qw[n,k] in int64, returned as int32."""
    qx = _c(qx, np.int8)
    qw = _c(qw, np.int8)
    M, K = qx.shape
    N, K2 = qw.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    over = lib().zqo_gemm_i32(_ptr(qx), _ptr(qw), M, N, K, _ptr(acc))
    if check_overflow and over:
        raise OverflowError(f"{over} accumulators exceed int32")
    return acc


def epilogue(acc, sx, sw, G, bias=None, act=0):
    """fp64 dequant (+bias, +GeLU) -> (z float64 [M,N], y fp16 [M,N])."""
    acc = _c(acc, np.int32)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    M, N = acc.shape
    b = None if bias is None else _h(bias)
    z = np.empty((M, N), np.float64)
    y = np.empty((M, N), np.uint16)
    lib().zqo_epilogue(_ptr(acc), _ptr(sx), _ptr(sw), G, _ptr(b), act, M, N,
                       _ptr(z), _ptr(y))
    return z, y.view(np.float16)


def linear(x, qw, sw, G, bias=None, act=0, ln=False, gamma=None, beta=None,
           eps=1e-5):
    """One quantized linear, step by step: [LN] -> token quant -> int GEMM ->
    epilogue.  ``qw`` holds unpacked int8 codes [N,K].  Returns a dict of
    every intermediate."""
    h = layernorm(x, gamma, beta, eps) if ln else np.ascontiguousarray(
        x, dtype=np.float16)
    qx, sx = quant_tokens(h)
    acc = gemm_i32(qx, qw)
    z, y = epilogue(acc, sx, sw, G, bias, act)
    return {"h": h, "qx": qx, "sx": sx, "acc": acc, "z": z, "y": y}


def gemm_w8a16(x, q, sw, G, bias=None, act=0):
    """W8A16 linear (fp16 activations x [M,K], int8 codes q [N,K], group
    scales sw [N/G]): fp64 (z [M,N]) and its fp16 rounding (y)."""
    x = _h(x)
    q = _c(q, np.int8)
    sw = _c(sw, np.float32)
    M, K = x.shape
    N, K2 = q.shape
    assert K == K2 and N % G == 0
    b = None if bias is None else _h(bias)
    z = np.empty((M, N), np.float64)
    y = np.empty((M, N), np.uint16)
    lib().zqo_gemm_w8a16(_ptr(x), _ptr(q), _ptr(sw), G, _ptr(b), act, M, N, K,
                         _ptr(z), _ptr(y))
    return z, y.view(np.float16)


def calibrate_minmax(x, state=None, momentum=0.95):
    """One calibration step of the static per-tensor range (moving average
    of batch min/max; the first call, state None, initializes).  Returns the
    new state float32 [2] = (x_min, x_max)."""
    x = _h(x)
    first = state is None
    st = np.zeros(2, np.float32) if first else np.array(state, np.float32)
    lib().zqo_calibrate_minmax(_ptr(x), x.size, ctypes.c_float(momentum),
                               int(first), _ptr(st))
    return st


def quant_static(x, state):
    """Eq. (2) over the whole tensor with S = max(|x_min|, |x_max|) / 127:
    (codes int8 of x's shape, S)."""
    x = _h(x)
    st = np.ascontiguousarray(state, np.float32)
    q = np.empty(x.shape, np.int8)
    s = lib().zqo_quant_static(_ptr(x), x.size, _ptr(st), _ptr(q))
    return q, np.float32(s)


def threads():
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().zqo_threads())


def set_threads(n):
    """Thread count of the oracle's later parallel loops (timing only)."""
    lib().zqo_set_threads(int(n))
