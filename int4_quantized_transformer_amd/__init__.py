"""zq: the fused quantized linear layer of ZeroQuant, native on MI355X.

The compute lives in ``libzq.so`` (hand-written HIP kernels for gfx950 behind a
C ABI declared in ``include/zq.h``).  This package is a thin ctypes binding
over it plus the seeded synthetic workloads.  Nothing here falls back to a CPU
or PyTorch implementation: if the library is missing, every call raises.
"""
__all__ = ["quantize_weights", "ln_quant_act", "quant_act", "gemm_w8a8",
           "gemm_w4a8", "gemm_w8a8_i32", "gemm_w4a8_i32", "gemm_w8a8_quant",
           "gemm_w4a8_quant", "gemm_quant_workspace_bytes", "gemm_plan",
           "gemm_w8a16", "gemm_w8a16_plan", "gemm_w8a8_xq", "gemm_w4a8_xq",
           "gemm_xq_plan", "calibrate_minmax",
           "quant_act_static", "gemm_tune", "sched_export", "sched_import",
           "sched_clear", "sched_entries", "Chain", "gemm_w8a8_ws",
           "gemm_w4a8_ws", "gemm_workspace_bytes", "gemm_ws_plan",
           "gemm_noalloc", "NOALLOC_SCRATCH_BYTES", "chunked_layout",
           "pack_chunked", "gemm_w8a8_chunked", "gemm_w4a8_chunked",
           "gemm_chunked_i32", "gemm_chunked_plan", "lib",
           "ZQError", "library_path", "ACT_NONE", "ACT_GELU"]


def __getattr__(name):
    # The binding is imported on first use so that importing the workloads
    # module alone never needs the shared library.
    if name in __all__:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
