"""ctypes binding of libzq (include/zq.h): argument marshalling only.

Each function checks dtypes/devices/shapes of the torch tensors it is given,
allocates outputs with torch when the caller passes none (PyTorch is the
device-memory and stream plumbing), and calls the C entry point of the same
name on the current HIP stream.  Every computation happens in libzq's
kernels; there is no fallback: if the library is missing or a call fails,
an exception is raised.
"""
import ctypes
import os

import torch

__all__ = ["ZQError", "library_path", "lib", "quantize_weights",
           "ln_quant_act", "quant_act", "gemm_w8a8", "gemm_w4a8",
           "gemm_w8a8_i32", "gemm_w4a8_i32", "gemm_w8a8_quant",
           "gemm_w4a8_quant", "gemm_quant_workspace_bytes", "gemm_plan",
           "gemm_w8a16", "gemm_w8a16_plan", "calibrate_minmax",
           "quant_act_static", "gemm_tune", "sched_export", "sched_import",
           "sched_clear", "sched_entries", "Chain", "gemm_w8a8_ws",
           "gemm_w4a8_ws", "gemm_workspace_bytes", "gemm_ws_plan",
           "gemm_noalloc", "NOALLOC_SCRATCH_BYTES", "chunked_layout",
           "pack_chunked", "gemm_w8a8_chunked", "gemm_w4a8_chunked",
           "gemm_chunked_i32", "gemm_chunked_plan",
           "ACT_NONE", "ACT_GELU"]

ACT_NONE = 0
ACT_GELU = 1
NOALLOC_SCRATCH_BYTES = 4 << 20   # ZQ_NOALLOC_SCRATCH_BYTES
_STATUS = {0: "ZQ_OK", 1: "ZQ_EINVAL", 2: "ZQ_ESHAPE", 3: "ZQ_EHIP",
           4: "ZQ_EUNSUPPORTED"}


class ZQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def library_path() -> str:
    return os.environ.get(
        "ZQ_LIBRARY",
        os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzq.so"))


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built; run "
                "`python -m int4_quantized_transformer_amd.build` first")
        L = ctypes.CDLL(path)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        sigs = {
            "zq_quantize_weights": [P, I, I, I, I, P, P, P],
            "zq_ln_quant_act": [P, P, P, F, I, I, P, P, P, P],
            "zq_quant_act": [P, I, I, P, P, P],
            "zq_gemm_w8a8": [P, P, P, P, I, P, I, I, I, I, P, P],
            "zq_gemm_w4a8": [P, P, P, P, I, P, I, I, I, I, P, P],
            "zq_gemm_w8a8_i32": [P, P, I, I, I, P, P],
            "zq_gemm_w4a8_i32": [P, P, I, I, I, P, P],
            "zq_gemm_w8a8_quant": [P, P, P, P, I, P, I, I, I, I, P, P, P,
                                   ctypes.c_size_t, P],
            "zq_gemm_w4a8_quant": [P, P, P, P, I, P, I, I, I, I, P, P, P,
                                   ctypes.c_size_t, P],
            "zq_gemm_plan": [I, I, I, I, ctypes.c_char_p, I],
            "zq_gemm_w8a16": [P, P, P, I, P, I, I, I, I, P, P],
            "zq_gemm_w8a8_xq": [P, P, P, I, P, I, I, I, I, P, P, P, P],
            "zq_gemm_w4a8_xq": [P, P, P, I, P, I, I, I, I, P, P, P, P],
            "zq_gemm_xq_plan": [I, I, I, I, ctypes.c_char_p, I],
            "zq_gemm_w8a16_plan": [I, I, I, ctypes.c_char_p, I],
            "zq_calibrate_minmax": [P, I, I, F, I, P, P],
            "zq_quant_act_static": [P, I, I, P, P, P, P],
            "zq_gemm_tune": [I, P, P, P, P, I, P, I, P, I, I, I, P, I, P, P, P],
            "zq_sched_export": [P, ctypes.c_size_t, P],
            "zq_sched_import": [ctypes.c_char_p],
            "zq_chain_create": [I, P],
            "zq_chain_add_ln_quant": [P, P, P, P, F, I, P, P, P],
            "zq_chain_add_quant": [P, P, I, P, P],
            "zq_chain_add_gemm": [P, I, P, P, P, P, I, P, I, I, I, P],
            "zq_chain_add_gemm_quant": [P, I, P, P, P, P, I, P, I, I, I, P, P,
                                        P, ctypes.c_size_t],
            "zq_chain_add_gemm_w8a16": [P, P, P, P, I, P, I, I, I, P],
            "zq_chain_add_gemm_xq": [P, I, P, P, P, I, P, I, I, I, P, P, P],
            "zq_chain_add_gemm_ws": [P, I, P, P, P, P, I, P, I, I, I, P, P,
                                     ctypes.c_size_t],
            "zq_chain_run": [P, I, P],
            "zq_gemm_w8a8_ws": [P, P, P, P, I, P, I, I, I, I, P, P,
                                ctypes.c_size_t, P],
            "zq_gemm_w4a8_ws": [P, P, P, P, I, P, I, I, I, I, P, P,
                                ctypes.c_size_t, P],
            "zq_gemm_ws_plan": [I, I, I, I, ctypes.c_char_p, I],
            "zq_gemm_noalloc": [I, P, P, P, P, I, P, I, I, I, I, P, P],
            "zq_chain_run_eager": [P, I, P],
            "zq_chain_add_gemm_chunked": [P, I, P, P, P, P, I, P, I, I, I, P],
            "zq_chunked_layout": [I, I, I, P, P],
            "zq_pack_chunked": [P, I, I, I, P, P],
            "zq_gemm_w8a8_chunked": [P, P, P, P, I, P, I, I, I, I, P, P],
            "zq_gemm_w4a8_chunked": [P, P, P, P, I, P, I, I, I, I, P, P],
            "zq_gemm_chunked_i32": [I, P, P, I, I, I, P, P],
            "zq_gemm_chunked_plan": [I, I, I, I, ctypes.c_char_p, I],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = I
        L.zq_gemm_workspace_bytes.argtypes = [I, I, I, I]
        L.zq_gemm_workspace_bytes.restype = ctypes.c_size_t
        L.zq_gemm_quant_workspace_bytes.argtypes = [I, I]
        L.zq_gemm_quant_workspace_bytes.restype = ctypes.c_size_t
        for name in ("zq_chain_graphs", "zq_chain_length"):
            getattr(L, name).argtypes = [P]
            getattr(L, name).restype = I
        L.zq_chain_destroy.argtypes = [P]
        L.zq_chain_destroy.restype = None
        L.zq_sched_clear.argtypes = []
        L.zq_sched_clear.restype = None
        L.zq_sched_entries.argtypes = []
        L.zq_sched_entries.restype = I
        L.zq_last_error.argtypes = []
        L.zq_last_error.restype = ctypes.c_char_p
        L.zq_version.argtypes = []
        L.zq_version.restype = I
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise ZQError(status, lib().zq_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype, dev=None, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize_weights(w, G, bits, qw=None, sw=None, stream=None):
    """Group-wise W8 (int8 [N,K]) or nibble-packed W4 (uint8 [N,K/2]) codes
    and fp32 scales [N/G] of fp16 weights W[N,K]."""
    _need(w, "w", torch.float16, dim=2)
    N, K = w.shape
    if qw is None:
        qw = (torch.empty(N, K, dtype=torch.int8, device=w.device) if bits == 8
              else torch.empty(N, K // 2, dtype=torch.uint8, device=w.device))
    if sw is None:
        sw = torch.empty(max(N // G, 1) if G > 0 else 1, dtype=torch.float32,
                         device=w.device)
    _need(qw, "qw", torch.int8 if bits == 8 else torch.uint8, w.device)
    _need(sw, "sw", torch.float32, w.device)
    _check(lib().zq_quantize_weights(_p(w), N, K, G, bits, _p(qw), _p(sw),
                                     _stream(w, stream)))
    return qw, sw


def ln_quant_act(x, gamma=None, beta=None, eps=1e-5, qx=None, sx=None,
                 ln_out=None, stream=None):
    """LayerNorm + token-wise INT8 quantization: returns (qx, sx), or
    (qx, sx, ln_out) when ``ln_out`` is True or a tensor."""
    _need(x, "x", torch.float16, dim=2)
    M, K = x.shape
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, torch.float16, x.device)
            if t.numel() != K:
                raise ValueError(f"{name} must have K={K} elements")
    qx = torch.empty(M, K, dtype=torch.int8, device=x.device) if qx is None else qx
    sx = torch.empty(M, dtype=torch.float32, device=x.device) if sx is None else sx
    _need(qx, "qx", torch.int8, x.device)
    _need(sx, "sx", torch.float32, x.device)
    want_ln = ln_out is not None and ln_out is not False
    if ln_out is True:
        ln_out = torch.empty_like(x)
    if want_ln:
        _need(ln_out, "ln_out", torch.float16, x.device)
    _check(lib().zq_ln_quant_act(_p(x), _p(gamma), _p(beta),
                                 ctypes.c_float(eps), M, K, _p(qx), _p(sx),
                                 _p(ln_out) if want_ln else None,
                                 _stream(x, stream)))
    return (qx, sx, ln_out) if want_ln else (qx, sx)


def quant_act(x, qx=None, sx=None, stream=None):
    """Token-wise INT8 quantization of fp16 x[M,K] -> (qx, sx)."""
    _need(x, "x", torch.float16, dim=2)
    M, K = x.shape
    qx = torch.empty(M, K, dtype=torch.int8, device=x.device) if qx is None else qx
    sx = torch.empty(M, dtype=torch.float32, device=x.device) if sx is None else sx
    _need(qx, "qx", torch.int8, x.device)
    _need(sx, "sx", torch.float32, x.device)
    _check(lib().zq_quant_act(_p(x), M, K, _p(qx), _p(sx), _stream(x, stream)))
    return qx, sx


def _gemm(fn, bits, qx, sx, qw, sw, G, bias, act, y, stream):
    _need(qx, "qx", torch.int8, dim=2)
    M, K = qx.shape
    _need(qw, "qw", torch.int8 if bits == 8 else torch.uint8, qx.device, 2)
    N = qw.shape[0]
    if qw.shape[1] != (K if bits == 8 else K // 2):
        raise ValueError(f"qw shape {tuple(qw.shape)} does not match K={K}")
    _need(sx, "sx", torch.float32, qx.device)
    _need(sw, "sw", torch.float32, qx.device)
    if bias is not None:
        _need(bias, "bias", torch.float16, qx.device)
    y = torch.empty(M, N, dtype=torch.float16, device=qx.device) if y is None else y
    _need(y, "y", torch.float16, qx.device)
    _check(fn(_p(qx), _p(sx), _p(qw), _p(sw), G, _p(bias), int(act), M, N, K,
              _p(y), _stream(qx, stream)))
    return y


def gemm_w8a8(qx, sx, qw, sw, G, bias=None, act=ACT_NONE, y=None, stream=None):
    """y[M,N] fp16 = act(sx[t]*sw[n//G]*sum_k qx*qw + bias)."""
    return _gemm(lib().zq_gemm_w8a8, 8, qx, sx, qw, sw, G, bias, act, y, stream)


def gemm_w4a8(qx, sx, qw4, sw, G, bias=None, act=ACT_NONE, y=None, stream=None):
    """As gemm_w8a8 with nibble-packed W4 weights uint8 [N, K/2]."""
    return _gemm(lib().zq_gemm_w4a8, 4, qx, sx, qw4, sw, G, bias, act, y, stream)


def gemm_quant_workspace_bytes(M, N):
    """Device workspace bytes that the _quant GEMMs need for an M x N output."""
    return int(lib().zq_gemm_quant_workspace_bytes(M, N))


def _gemm_quant(fn, bits, qx, sx, qw, sw, G, bias, act, qy, sy, ws, stream):
    _need(qx, "qx", torch.int8, dim=2)
    M, K = qx.shape
    _need(qw, "qw", torch.int8 if bits == 8 else torch.uint8, qx.device, 2)
    N = qw.shape[0]
    if qw.shape[1] != (K if bits == 8 else K // 2):
        raise ValueError(f"qw shape {tuple(qw.shape)} does not match K={K}")
    _need(sx, "sx", torch.float32, qx.device)
    _need(sw, "sw", torch.float32, qx.device)
    if bias is not None:
        _need(bias, "bias", torch.float16, qx.device)
    qy = torch.empty(M, N, dtype=torch.int8, device=qx.device) if qy is None else qy
    sy = torch.empty(M, dtype=torch.float32, device=qx.device) if sy is None else sy
    if ws is None:
        ws = torch.empty(max(gemm_quant_workspace_bytes(M, N), 16),
                         dtype=torch.uint8, device=qx.device)
    _need(qy, "qy", torch.int8, qx.device)
    _need(sy, "sy", torch.float32, qx.device)
    _need(ws, "ws", torch.uint8, qx.device)
    _check(fn(_p(qx), _p(sx), _p(qw), _p(sw), G, _p(bias), int(act), M, N, K,
              _p(qy), _p(sy), _p(ws), ws.numel(), _stream(qx, stream)))
    return qy, sy


def gemm_w8a8_quant(qx, sx, qw, sw, G, bias=None, act=ACT_NONE, qy=None,
                    sy=None, ws=None, stream=None):
    """The fp16 output of gemm_w8a8 quantized token-wise for the next linear:
    (qy int8 [M,N], sy fp32 [M]), equal to quant_act(gemm_w8a8(...))."""
    return _gemm_quant(lib().zq_gemm_w8a8_quant, 8, qx, sx, qw, sw, G, bias,
                       act, qy, sy, ws, stream)


def gemm_w4a8_quant(qx, sx, qw4, sw, G, bias=None, act=ACT_NONE, qy=None,
                    sy=None, ws=None, stream=None):
    """As gemm_w8a8_quant with nibble-packed W4 weights uint8 [N, K/2]."""
    return _gemm_quant(lib().zq_gemm_w4a8_quant, 4, qx, sx, qw4, sw, G, bias,
                       act, qy, sy, ws, stream)


def _gemm_i32(fn, bits, qx, qw, acc, stream):
    _need(qx, "qx", torch.int8, dim=2)
    M, K = qx.shape
    _need(qw, "qw", torch.int8 if bits == 8 else torch.uint8, qx.device, 2)
    N = qw.shape[0]
    if qw.shape[1] != (K if bits == 8 else K // 2):
        raise ValueError(f"qw shape {tuple(qw.shape)} does not match K={K}")
    acc = torch.empty(M, N, dtype=torch.int32, device=qx.device) if acc is None else acc
    _need(acc, "acc", torch.int32, qx.device)
    _check(fn(_p(qx), _p(qw), M, N, K, _p(acc), _stream(qx, stream)))
    return acc


def gemm_w8a8_i32(qx, qw, acc=None, stream=None):
    """Raw int32 accumulator acc[M,N] = sum_k qx[t,k]*qw[n,k]."""
    return _gemm_i32(lib().zq_gemm_w8a8_i32, 8, qx, qw, acc, stream)


def gemm_w4a8_i32(qx, qw4, acc=None, stream=None):
    return _gemm_i32(lib().zq_gemm_w4a8_i32, 4, qx, qw4, acc, stream)


def chunked_layout(N, K, bits):
    """(rows per block, chunk bytes) of the chunk-contiguous decode layout
    for the shape."""
    r, c = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().zq_chunked_layout(N, K, bits, ctypes.byref(r),
                                   ctypes.byref(c)))
    return r.value, c.value


def pack_chunked(qw, bits, qd=None, stream=None):
    """Row-major codes (int8 [N,K] for W8, packed uint8 [N,K/2] for W4) in
    the chunk-contiguous decode layout (same dtype and shape)."""
    _need(qw, "qw", torch.int8 if bits == 8 else torch.uint8, dim=2)
    N, kb = qw.shape
    K = kb if bits == 8 else 2 * kb
    qd = torch.empty_like(qw) if qd is None else qd
    _need(qd, "qd", qw.dtype, qw.device, 2)
    if qd.shape != qw.shape:
        raise ValueError(f"qd shape {tuple(qd.shape)} != {tuple(qw.shape)}")
    _check(lib().zq_pack_chunked(_p(qw), N, K, bits, _p(qd),
                                 _stream(qw, stream)))
    return qd


def gemm_w8a8_chunked(qx, sx, qd, sw, G, bias=None, act=ACT_NONE, y=None,
                      stream=None):
    """gemm_w8a8 over weights in the chunk-contiguous layout (pack_chunked),
    1..16 tokens; y is bit-identical to gemm_w8a8 on the row-major codes."""
    return _gemm(lib().zq_gemm_w8a8_chunked, 8, qx, sx, qd, sw, G, bias, act,
                 y, stream)


def gemm_w4a8_chunked(qx, sx, qd4, sw, G, bias=None, act=ACT_NONE, y=None,
                      stream=None):
    """As gemm_w8a8_chunked with packed W4 codes."""
    return _gemm(lib().zq_gemm_w4a8_chunked, 4, qx, sx, qd4, sw, G, bias, act,
                 y, stream)


def gemm_chunked_i32(bits, qx, qd, acc=None, stream=None):
    """Raw int32 accumulator of the chunk-layout GEMM."""
    fn = lib().zq_gemm_chunked_i32
    return _gemm_i32(lambda *a: fn(bits, *a), bits, qx, qd, acc, stream)


def gemm_chunked_plan(M, N, K, bits):
    """The kernel configuration of the chunk-layout GEMM for the shape."""
    buf = ctypes.create_string_buffer(160)
    _check(lib().zq_gemm_chunked_plan(M, N, K, bits, buf, 160))
    return buf.value.decode()


def _gemm_xq(fn, bits, x, qw, sw, G, bias, act, y, qx, sx, stream):
    _need(x, "x", torch.float16, dim=2)
    M, K = x.shape
    _need(qw, "qw", torch.int8 if bits == 8 else torch.uint8, x.device, 2)
    N = qw.shape[0]
    if qw.shape[1] != (K if bits == 8 else K // 2):
        raise ValueError(f"qw shape {tuple(qw.shape)} does not match K={K}")
    _need(sw, "sw", torch.float32, x.device)
    if bias is not None:
        _need(bias, "bias", torch.float16, x.device)
    y = torch.empty(M, N, dtype=torch.float16, device=x.device) if y is None else y
    qx = torch.empty(M, K, dtype=torch.int8, device=x.device) if qx is None else qx
    sx = torch.empty(M, dtype=torch.float32, device=x.device) if sx is None else sx
    _need(y, "y", torch.float16, x.device)
    _need(qx, "qx", torch.int8, x.device)
    _need(sx, "sx", torch.float32, x.device)
    _check(fn(_p(x), _p(qw), _p(sw), G, _p(bias), int(act), M, N, K, _p(y),
              _p(qx), _p(sx), _stream(x, stream)))
    return y, qx, sx


def gemm_w8a8_xq(x, qw, sw, G, bias=None, act=ACT_NONE, y=None, qx=None,
                 sx=None, stream=None):
    """The linear of an fp16 activation x [M,K]: token-wise codes and scales
    (returned, equal to quant_act(x)) and y = gemm_w8a8 of them, with the
    quantization done inside the GEMV for one token.  Returns (y, qx, sx)."""
    return _gemm_xq(lib().zq_gemm_w8a8_xq, 8, x, qw, sw, G, bias, act, y, qx,
                    sx, stream)


def gemm_w4a8_xq(x, qw4, sw, G, bias=None, act=ACT_NONE, y=None, qx=None,
                 sx=None, stream=None):
    """As gemm_w8a8_xq with packed INT4 weights qw4 [N,K/2]."""
    return _gemm_xq(lib().zq_gemm_w4a8_xq, 4, x, qw4, sw, G, bias, act, y, qx,
                    sx, stream)


def gemm_xq_plan(M, N, K, bits) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().zq_gemm_xq_plan(M, N, K, bits, buf, 256))
    return buf.value.decode()


def gemm_w8a16(x, qw, sw, G, bias=None, act=ACT_NONE, y=None, stream=None):
    """y[M,N] fp16 = act(sw[n//G] * sum_k x[t,k]*qw[n,k] + bias) with fp16
    activations x [M,K] and INT8 weights qw [N,K]."""
    _need(x, "x", torch.float16, dim=2)
    M, K = x.shape
    _need(qw, "qw", torch.int8, x.device, 2)
    N = qw.shape[0]
    if qw.shape[1] != K:
        raise ValueError(f"qw shape {tuple(qw.shape)} does not match K={K}")
    _need(sw, "sw", torch.float32, x.device)
    if bias is not None:
        _need(bias, "bias", torch.float16, x.device)
    y = torch.empty(M, N, dtype=torch.float16, device=x.device) if y is None else y
    _need(y, "y", torch.float16, x.device)
    _check(lib().zq_gemm_w8a16(_p(x), _p(qw), _p(sw), G, _p(bias), int(act), M,
                               N, K, _p(y), _stream(x, stream)))
    return y


def gemm_w8a16_plan(M, N, K) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().zq_gemm_w8a16_plan(M, N, K, buf, 256))
    return buf.value.decode()


def calibrate_minmax(x, state=None, momentum=0.95, stream=None):
    """One calibration batch of the static per-tensor range: state (device
    fp32 [2] = x_min, x_max) is created from x when None, else moved by the
    moving average.  Returns the state tensor."""
    _need(x, "x", torch.float16, dim=2)
    M, K = x.shape
    first = state is None
    if first:
        state = torch.zeros(2, dtype=torch.float32, device=x.device)
    _need(state, "state", torch.float32, x.device)
    _check(lib().zq_calibrate_minmax(_p(x), M, K, ctypes.c_float(momentum),
                                     int(first), _p(state), _stream(x, stream)))
    return state


def quant_act_static(x, state, qx=None, s_out=None, stream=None):
    """Eq. (2) over the whole of x with the frozen scale of ``state``:
    (qx int8 [M,K], S fp32 [1])."""
    _need(x, "x", torch.float16, dim=2)
    M, K = x.shape
    _need(state, "state", torch.float32, x.device)
    qx = torch.empty(M, K, dtype=torch.int8, device=x.device) if qx is None else qx
    s_out = torch.empty(1, dtype=torch.float32, device=x.device) if s_out is None else s_out
    _need(qx, "qx", torch.int8, x.device)
    _need(s_out, "s_out", torch.float32, x.device)
    _check(lib().zq_quant_act_static(_p(x), M, K, _p(state), _p(qx), _p(s_out),
                                     _stream(x, stream)))
    return qx, s_out


def gemm_plan(M, N, K, bits) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().zq_gemm_plan(M, N, K, bits, buf, 256))
    return buf.value.decode()


PLAN_KINDS = {0: "skinny", 1: "tiled", 2: "stream", 3: "gemv"}


def gemm_tune(qx, sx, qw, sw, G, ms, bias=None, act=ACT_NONE, y=None, reps=10,
              stream=None):
    """Times every GEMM kernel and tile that applies at each token count of
    ``ms`` (ascending) on these buffers (qx/sx/y sized for the largest) and
    stores the fastest in the schedule table for (previous count, count].
    Returns [(kind, tile or -1, microseconds)] per count.  Synchronizes."""
    _need(qx, "qx", torch.int8, dim=2)
    bits = 8 if qw.dtype == torch.int8 else 4
    _need(qw, "qw", torch.int8 if bits == 8 else torch.uint8, qx.device, 2)
    _need(sx, "sx", torch.float32, qx.device)
    _need(sw, "sw", torch.float32, qx.device)
    if bias is not None:
        _need(bias, "bias", torch.float16, qx.device)
    ms = [int(m) for m in ms]
    M, K = qx.shape
    N = qw.shape[0]
    if not ms or ms[-1] > M or sx.numel() < ms[-1]:
        raise ValueError(f"token counts {ms} exceed the buffers' {M} rows")
    if y is None:
        y = torch.empty(ms[-1], N, dtype=torch.float16, device=qx.device)
    _need(y, "y", torch.float16, qx.device)
    if y.numel() < ms[-1] * N:
        raise ValueError("y is smaller than the largest token count needs")
    n = len(ms)
    arr = (ctypes.c_int * n)(*ms)
    chosen = (ctypes.c_int * (2 * n))()
    us = (ctypes.c_float * n)()
    _check(lib().zq_gemm_tune(bits, _p(qx), _p(sx), _p(qw), _p(sw), G, _p(bias),
                              int(act), arr, n, N, K, _p(y), int(reps), chosen,
                              us, _stream(qx, stream)))
    return [(PLAN_KINDS[chosen[2 * i]], chosen[2 * i + 1], us[i])
            for i in range(n)]


def sched_export() -> str:
    """The schedule table as text, one entry per line."""
    need = ctypes.c_size_t(0)
    _check(lib().zq_sched_export(None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(need.value)
    _check(lib().zq_sched_export(buf, need.value, None))
    return buf.value.decode()


def sched_import(text: str):
    _check(lib().zq_sched_import(text.encode()))


def sched_clear():
    lib().zq_sched_clear()


def sched_entries() -> int:
    return lib().zq_sched_entries()


class Chain:
    """A recorded sequence of libzq calls over buffers of ``max_m`` token
    rows, replayed as one HIP graph per token count (zq_chain_*).  The
    chain keeps a reference to every tensor it was given, so they stay
    allocated while it lives."""

    def __init__(self, max_m):
        h = ctypes.c_void_p()
        _check(lib().zq_chain_create(int(max_m), ctypes.byref(h)))
        self._h = h
        self.max_m = int(max_m)
        self._keep = []
        self.device = None

    def _rows(self, t, name, dtype, width=None):
        _need(t, name, dtype, self.device)
        if self.device is None:
            self.device = t.device
        if t.shape[0] < self.max_m or (width is not None and t.dim() == 2
                                       and t.shape[1] != width):
            raise ValueError(f"{name} {tuple(t.shape)} must hold {self.max_m} "
                             f"rows" + (f" of {width}" if width else ""))
        self._keep.append(t)

    def _dev(self, t, name, dtype):
        if t is None:
            return
        _need(t, name, dtype, self.device)
        if self.device is None:
            self.device = t.device
        self._keep.append(t)

    def ln_quant(self, x, qx, sx, gamma=None, beta=None, eps=1e-5, ln_out=None):
        K = x.shape[1]
        self._rows(x, "x", torch.float16, K)
        self._rows(qx, "qx", torch.int8, K)
        self._rows(sx, "sx", torch.float32)
        self._dev(gamma, "gamma", torch.float16)
        self._dev(beta, "beta", torch.float16)
        if ln_out is not None:
            self._rows(ln_out, "ln_out", torch.float16, K)
        _check(lib().zq_chain_add_ln_quant(self._h, _p(x), _p(gamma), _p(beta),
                                           ctypes.c_float(eps), K, _p(qx),
                                           _p(sx), _p(ln_out)))

    def quant(self, x, qx, sx):
        K = x.shape[1]
        self._rows(x, "x", torch.float16, K)
        self._rows(qx, "qx", torch.int8, K)
        self._rows(sx, "sx", torch.float32)
        _check(lib().zq_chain_add_quant(self._h, _p(x), K, _p(qx), _p(sx)))

    def _gemm_common(self, qx, sx, qw, sw, bias):
        K = qx.shape[1]
        bits = 8 if qw.dtype == torch.int8 else 4
        self._rows(qx, "qx", torch.int8, K)
        self._rows(sx, "sx", torch.float32)
        self._dev(qw, "qw", torch.int8 if bits == 8 else torch.uint8)
        self._dev(sw, "sw", torch.float32)
        self._dev(bias, "bias", torch.float16)
        if qw.shape[1] != (K if bits == 8 else K // 2):
            raise ValueError(f"qw shape {tuple(qw.shape)} does not match K={K}")
        return bits, qw.shape[0], K

    def gemm(self, qx, sx, qw, sw, G, y, bias=None, act=ACT_NONE):
        bits, N, K = self._gemm_common(qx, sx, qw, sw, bias)
        self._rows(y, "y", torch.float16, N)
        _check(lib().zq_chain_add_gemm(self._h, bits, _p(qx), _p(sx), _p(qw),
                                       _p(sw), G, _p(bias), int(act), N, K,
                                       _p(y)))

    def gemm_quant(self, qx, sx, qw, sw, G, qy, sy, ws, bias=None,
                   act=ACT_NONE):
        bits, N, K = self._gemm_common(qx, sx, qw, sw, bias)
        self._rows(qy, "qy", torch.int8, N)
        self._rows(sy, "sy", torch.float32)
        self._dev(ws, "ws", torch.uint8)
        _check(lib().zq_chain_add_gemm_quant(self._h, bits, _p(qx), _p(sx),
                                             _p(qw), _p(sw), G, _p(bias),
                                             int(act), N, K, _p(qy), _p(sy),
                                             _p(ws), ws.numel()))

    def gemm_ws(self, qx, sx, qw, sw, G, y, ws, bias=None, act=ACT_NONE):
        """gemm_w8a8_ws / gemm_w4a8_ws (ws: uint8 workspace, or None when no
        token count up to max_m needs one)."""
        bits, N, K = self._gemm_common(qx, sx, qw, sw, bias)
        self._rows(y, "y", torch.float16, N)
        self._dev(ws, "ws", torch.uint8)
        _check(lib().zq_chain_add_gemm_ws(self._h, bits, _p(qx), _p(sx), _p(qw),
                                          _p(sw), G, _p(bias), int(act), N, K,
                                          _p(y), _p(ws),
                                          0 if ws is None else ws.numel()))

    def gemm_chunked(self, qx, sx, qd, sw, G, y, bias=None, act=ACT_NONE):
        """gemm_w8a8_chunked / gemm_w4a8_chunked (weights from pack_chunked;
        the chain's max_m must be at most 16)."""
        bits, N, K = self._gemm_common(qx, sx, qd, sw, bias)
        self._rows(y, "y", torch.float16, N)
        _check(lib().zq_chain_add_gemm_chunked(self._h, bits, _p(qx), _p(sx),
                                               _p(qd), _p(sw), G, _p(bias),
                                               int(act), N, K, _p(y)))

    def gemm_w8a16(self, x, qw, sw, G, y, bias=None, act=ACT_NONE):
        K = x.shape[1]
        self._rows(x, "x", torch.float16, K)
        self._dev(qw, "qw", torch.int8)
        self._dev(sw, "sw", torch.float32)
        self._dev(bias, "bias", torch.float16)
        N = qw.shape[0]
        self._rows(y, "y", torch.float16, N)
        _check(lib().zq_chain_add_gemm_w8a16(self._h, _p(x), _p(qw), _p(sw), G,
                                             _p(bias), int(act), N, K, _p(y)))

    def gemm_xq(self, x, qw, sw, G, y, qx, sx, bias=None, act=ACT_NONE):
        """gemm_w8a8_xq / gemm_w4a8_xq: the fp16 activation x quantized by
        the GEMM (codes and scales into qx, sx)."""
        K = x.shape[1]
        bits = 8 if qw.dtype == torch.int8 else 4
        self._rows(x, "x", torch.float16, K)
        self._rows(qx, "qx", torch.int8, K)
        self._rows(sx, "sx", torch.float32)
        self._dev(qw, "qw", torch.int8 if bits == 8 else torch.uint8)
        self._dev(sw, "sw", torch.float32)
        self._dev(bias, "bias", torch.float16)
        if qw.shape[1] != (K if bits == 8 else K // 2):
            raise ValueError(f"qw shape {tuple(qw.shape)} does not match K={K}")
        N = qw.shape[0]
        self._rows(y, "y", torch.float16, N)
        _check(lib().zq_chain_add_gemm_xq(self._h, bits, _p(x), _p(qw), _p(sw),
                                          G, _p(bias), int(act), N, K, _p(y),
                                          _p(qx), _p(sx)))

    def _stream(self, stream):
        if stream is not None:
            return ctypes.c_void_p(int(stream))
        if self.device is None:
            return None
        return ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    def run(self, M, stream=None):
        """Launches the graph for M rows (captured on first use)."""
        _check(lib().zq_chain_run(self._h, int(M), self._stream(stream)))

    def run_eager(self, M, stream=None):
        """Launches the recorded calls one by one."""
        _check(lib().zq_chain_run_eager(self._h, int(M), self._stream(stream)))

    @property
    def graphs(self) -> int:
        return lib().zq_chain_graphs(self._h)

    def __len__(self):
        return lib().zq_chain_length(self._h)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().zq_chain_destroy(self._h)
            self._h = ctypes.c_void_p()
            self._keep = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gemm_workspace_bytes(M, N, K, bits) -> int:
    """Workspace bytes gemm_w8a8_ws / gemm_w4a8_ws use for this shape (0:
    they run without one)."""
    return int(lib().zq_gemm_workspace_bytes(int(M), int(N), int(K), int(bits)))


def gemm_ws_plan(M, N, K, bits) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().zq_gemm_ws_plan(M, N, K, bits, buf, 256))
    return buf.value.decode()


def _gemm_ws(fn, bits, qx, sx, qw, sw, G, bias, act, y, ws, stream):
    _need(qx, "qx", torch.int8, dim=2)
    M, K = qx.shape
    N = qw.shape[0]
    need = gemm_workspace_bytes(M, N, K, bits)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=qx.device)
    if ws is not None:
        _need(ws, "ws", torch.uint8, qx.device)
    y = torch.empty(M, N, dtype=torch.float16, device=qx.device) if y is None else y
    _need(qw, "qw", torch.int8 if bits == 8 else torch.uint8, qx.device, 2)
    if qw.shape[1] != (K if bits == 8 else K // 2):
        raise ValueError(f"qw shape {tuple(qw.shape)} does not match K={K}")
    _need(sx, "sx", torch.float32, qx.device)
    _need(sw, "sw", torch.float32, qx.device)
    if bias is not None:
        _need(bias, "bias", torch.float16, qx.device)
    _need(y, "y", torch.float16, qx.device)
    _check(fn(_p(qx), _p(sx), _p(qw), _p(sw), G, _p(bias), int(act), M, N, K,
              _p(y), _p(ws), 0 if ws is None else ws.numel(),
              _stream(qx, stream)))
    return y


def gemm_w8a8_ws(qx, sx, qw, sw, G, bias=None, act=ACT_NONE, y=None, ws=None,
                 stream=None):
    """gemm_w8a8 with a workspace (allocated here when not given): decode-
    sized M over few weight tiles splits K; y is bit-identical."""
    return _gemm_ws(lib().zq_gemm_w8a8_ws, 8, qx, sx, qw, sw, G, bias, act, y,
                    ws, stream)


def gemm_w4a8_ws(qx, sx, qw, sw, G, bias=None, act=ACT_NONE, y=None, ws=None,
                 stream=None):
    return _gemm_ws(lib().zq_gemm_w4a8_ws, 4, qx, sx, qw, sw, G, bias, act, y,
                    ws, stream)


def gemm_noalloc(bits, qx, sx, qw, sw, G, bias=None, act=ACT_NONE, y=None,
                 stream=None):
    """zq_gemm_noalloc: gemm_w8a8_ws / gemm_w4a8_ws with the library's own
    per-device scratch array instead of a workspace (the call allocates
    nothing on the device; y is allocated here when not given)."""
    _need(qx, "qx", torch.int8, dim=2)
    M, K = qx.shape
    N = qw.shape[0]
    y = torch.empty(M, N, dtype=torch.float16, device=qx.device) if y is None else y
    _need(qw, "qw", torch.int8 if bits == 8 else torch.uint8, qx.device, 2)
    _need(sx, "sx", torch.float32, qx.device)
    _need(sw, "sw", torch.float32, qx.device)
    if bias is not None:
        _need(bias, "bias", torch.float16, qx.device)
    _need(y, "y", torch.float16, qx.device)
    _check(lib().zq_gemm_noalloc(int(bits), _p(qx), _p(sx), _p(qw), _p(sw), G,
                                 _p(bias), int(act), M, N, K, _p(y),
                                 _stream(qx, stream)))
    return y
