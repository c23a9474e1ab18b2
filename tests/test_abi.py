"""CPU checks of the C ABI: the library loads, exports every function that
include/zq.h declares, and its host-side argument checks return the
documented statuses before anything is launched (no GPU is touched)."""
import ctypes
import os
import re

import pytest

from int4_quantized_transformer_amd import _lib as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zq.h")

OK, EINVAL, ESHAPE, EHIP, EUNSUP = 0, 1, 2, 3, 4
# Fake, 256-byte aligned "device" addresses: every call below fails its
# argument check before any pointer is used.
A, B, C, D, E = (ctypes.c_void_p(0x10000 * i) for i in range(1, 6))


def declared_functions():
    with open(HEADER) as f:
        src = f.read()
    return sorted(set(re.findall(r"\b(zq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = Z.lib()
    names = declared_functions()
    assert "zq_gemm_w8a8" in names and "zq_ln_quant_act" in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in zq.h but not exported"
    assert L.zq_version() == 106


def test_last_error_starts_empty_and_is_set_on_failure():
    L = Z.lib()
    assert L.zq_quant_act(None, 4, 64, B, C, None) == EINVAL
    assert b"null" in L.zq_last_error()
    assert L.zq_quant_act(A, 0, 64, B, C, None) == OK   # M = 0: empty call
    assert L.zq_last_error() == b""


def test_quant_argument_checks():
    L = Z.lib()
    assert L.zq_quant_act(A, -1, 64, B, C, None) == ESHAPE
    assert L.zq_quant_act(A, 4, 0, B, C, None) == ESHAPE
    assert L.zq_quant_act(A, 4, 65537, B, C, None) == EUNSUP
    assert L.zq_ln_quant_act(A, None, None, ctypes.c_float(-1.0), 4, 64, B, C,
                             None, None) == EINVAL
    assert L.zq_ln_quant_act(A, None, None, ctypes.c_float(1e-5), 4, 64, None,
                             C, None, None) == EINVAL
    assert L.zq_ln_quant_act(A, None, None, ctypes.c_float(1e-5), 0, 64, B, C,
                             None, None) == OK


def test_quantize_weights_argument_checks():
    L = Z.lib()
    assert L.zq_quantize_weights(A, 96, 64, 64, 8, B, C, None) == ESHAPE  # N % G
    assert L.zq_quantize_weights(A, 128, 63, 64, 4, B, C, None) == ESHAPE  # odd K, W4
    assert L.zq_quantize_weights(A, 128, 64, 64, 5, B, C, None) == EINVAL  # bits
    assert L.zq_quantize_weights(A, 128, 64, 0, 8, B, C, None) == ESHAPE
    assert L.zq_quantize_weights(None, 128, 64, 64, 8, B, C, None) == EINVAL


@pytest.mark.parametrize("fn", ["zq_gemm_w8a8", "zq_gemm_w4a8"])
def test_gemm_argument_checks(fn):
    f = getattr(Z.lib(), fn)
    # (qx, sx, qw, sw, G, bias, act, M, N, K, y, stream)
    assert f(A, B, C, D, 64, None, 0, 16, 256, 100, E, None) == EUNSUP  # K % 64
    assert f(A, B, C, D, 64, None, 0, 16, 96, 256, E, None) == ESHAPE   # N % G
    assert f(A, B, C, D, 0, None, 0, 16, 256, 256, E, None) == ESHAPE   # G
    assert f(A, B, C, D, 64, None, 2, 16, 256, 256, E, None) == EINVAL  # act
    assert f(A, B, C, D, 64, None, 0, -1, 256, 256, E, None) == ESHAPE
    assert f(A, B, C, D, 64, None, 0, 16, 0, 256, E, None) == ESHAPE
    assert f(None, B, C, D, 64, None, 0, 16, 256, 256, E, None) == EINVAL
    assert f(A, None, C, D, 64, None, 0, 16, 256, 256, E, None) == EINVAL
    assert f(ctypes.c_void_p(0x10008), B, C, D, 64, None, 0, 16, 256, 256, E,
             None) == EINVAL                                            # align
    big = 131_072                                   # K > ZQ_MAX_GEMM_K_*
    assert f(A, B, C, D, 64, None, 0, 16, 256, big, E, None) == EUNSUP   # int32 bound
    assert f(A, B, C, D, 64, None, 0, 0, 256, 256, E, None) == OK       # empty


def test_gemm_i32_argument_checks():
    L = Z.lib()
    assert L.zq_gemm_w8a8_i32(A, B, 4, 64, 96, C, None) == EUNSUP
    assert L.zq_gemm_w4a8_i32(A, B, 4, 64, 128, None, None) == EINVAL
    assert L.zq_gemm_w8a8_i32(A, B, 0, 64, 128, C, None) == OK
    # M == 0: the M-sized buffers may be NULL (an empty torch tensor's pointer)
    assert L.zq_gemm_w8a8_i32(None, B, 0, 64, 128, None, None) == OK
    assert L.zq_gemm_w8a8(None, None, B, C, 64, None, 0, 0, 64, 128, None,
                          None) == OK
    assert L.zq_quant_act(None, 0, 64, None, None, None) == OK
    assert L.zq_gemm_w8a8_i32(None, B, 1, 64, 128, C, None) == EINVAL


def _header_define(name):
    import re
    hdr = os.path.join(os.path.dirname(__file__), "..", "include", "zq.h")
    with open(hdr) as f:
        m = re.search(rf"#define {name} (\d+)", f.read())
    return int(m.group(1))


def test_header_limits_match_int32_bound():
    # The calls take any two's-complement code: -128 * -128 for W8, and
    # 16 * (-8) * (-128) on the W4 path (which accumulates 16 * acc).  The
    # bound is the largest multiple of 64 with K * 16384 <= 2^31 - 1.
    worst = max(128 * 128, 16 * 8 * 128)
    for name in ("ZQ_MAX_GEMM_K_W8", "ZQ_MAX_GEMM_K_W4"):
        k = _header_define(name)
        assert k % 64 == 0
        assert k * worst <= 2 ** 31 - 1 < (k + 64) * worst


@pytest.mark.parametrize("fn,bits", [("zq_gemm_w8a8", 8), ("zq_gemm_w4a8", 4)])
def test_gemm_k_limit_is_enforced(fn, bits):
    # the largest K passes the checks (M == 0: nothing is launched), the next
    # multiple of 64 is refused before any launch
    L = Z.lib()
    f = getattr(L, fn)
    k = _header_define("ZQ_MAX_GEMM_K_W8" if bits == 8 else "ZQ_MAX_GEMM_K_W4")
    assert f(None, None, B, C, 64, None, 0, 0, 64, k, None, None) == OK
    assert f(A, B, B, C, 64, None, 0, 16, 64, k + 64, E, None) == EUNSUP
    assert "int32" in Z.lib().zq_last_error().decode()


def test_gemm_plan_covers_every_regime():
    # one token with whole 1 KB weight-row pieces: GEMV; other problems of
    # up to 64 tokens with even N: streaming rings of 1, 16, 32 or 64 token
    # rows, except W8 over N >= 8192 with more than 32 tokens (64x64
    # tiles); odd N: the skinny kernel (64x64 tiles when N gives at least
    # 128 of them); above 64 tokens: tiled
    assert Z.gemm_plan(1, 4096, 4096, 8).startswith("gemv")
    assert Z.gemm_plan(1, 4096, 4096, 4).startswith("gemv")
    assert Z.gemm_plan(1, 4096, 1024, 4).startswith("stream")
    assert Z.gemm_plan(1, 77, 192, 8).startswith("skinny")
    assert Z.gemm_plan(16, 4096, 4096, 8).startswith("stream BN=16 MX=16")
    assert Z.gemm_plan(17, 4096, 4096, 8).startswith("stream BN=16 MX=32")
    assert Z.gemm_plan(33, 4096, 4096, 8).startswith("stream BN=16 MX=64")
    assert Z.gemm_plan(64, 4096, 4096, 4).startswith("stream BN=16 MX=64")
    assert Z.gemm_plan(64, 6144, 6144, 8).startswith("stream BN=32 MX=64")
    assert Z.gemm_plan(17, 8192, 4096, 8).startswith("stream BN=32 MX=32")
    assert Z.gemm_plan(33, 8192, 4096, 8).startswith("tiled cfg=22")
    assert Z.gemm_plan(64, 16384, 4096, 4).startswith("stream BN=32 MX=64")
    assert Z.gemm_plan(40, 77, 4096, 8).startswith("skinny")
    assert Z.gemm_plan(40, 8191, 4096, 8).startswith("tiled cfg=22")
    assert Z.gemm_plan(65, 4096, 4096, 8).startswith("tiled")
    assert Z.gemm_plan(2048, 4096, 4096, 8).startswith("tiled")
    with pytest.raises(Z.ZQError):
        Z.gemm_plan(16, 256, 256, 3)


def test_gemm_w8a16_argument_checks():
    f = Z.lib().zq_gemm_w8a16
    # (x, qw, sw, G, bias, act, M, N, K, y, stream)
    assert f(A, B, C, 64, None, 0, 16, 256, 100, D, None) == EUNSUP  # K % 64
    assert f(A, B, C, 64, None, 0, 16, 96, 256, D, None) == ESHAPE        # N % G
    assert f(A, B, C, 0, None, 0, 16, 256, 256, D, None) == ESHAPE        # G
    assert f(A, B, C, 64, None, 3, 16, 256, 256, D, None) == EINVAL       # act
    assert f(A, B, C, 64, None, 0, -1, 256, 256, D, None) == ESHAPE
    assert f(None, B, C, 64, None, 0, 16, 256, 256, D, None) == EINVAL
    assert f(A, None, C, 64, None, 0, 16, 256, 256, D, None) == EINVAL
    assert f(ctypes.c_void_p(0x10008), B, C, 64, None, 0, 16, 256, 256, D,
             None) == EINVAL                                            # align
    assert f(A, B, C, 64, None, 0, 16, 256, 1048640, D, None) == EUNSUP
    assert f(None, B, C, 64, None, 0, 0, 256, 256, None, None) == OK      # empty
    assert Z.gemm_w8a16_plan(1, 18432, 6144).startswith("gemv-a16")
    assert Z.gemm_w8a16_plan(1, 18432, 6000 + 64).startswith("stream-a16 MX=1")
    assert Z.gemm_w8a16_plan(2, 18432, 6144).startswith("stream-a16 MX=16")
    assert Z.gemm_w8a16_plan(2, 18431, 6144).startswith("tiled-a16 cfg=4")
    assert Z.gemm_w8a16_plan(17, 18432, 6144).startswith("stream-a16 MX=32 NW=4 cfg=0 BN=32")
    assert Z.gemm_w8a16_plan(17, 4096, 6144).startswith("stream-a16 MX=32 NW=4 cfg=0 BN=16")
    assert Z.gemm_w8a16_plan(33, 6144, 6144).startswith("stream-a16 MX=64 NW=4 cfg=0 BN=16")
    assert Z.gemm_w8a16_plan(33, 18432, 6144).startswith("tiled-a16 cfg=4")
    assert Z.gemm_w8a16_plan(40, 999, 256).startswith("tiled-a16 cfg=4")
    assert Z.gemm_w8a16_plan(2048, 18432, 6144).startswith("tiled-a16 cfg=3")
    assert Z.gemm_w8a16_plan(100, 256, 512).startswith("tiled-a16 cfg=1")


def test_static_range_argument_checks():
    L = Z.lib()
    F = ctypes.c_float
    assert L.zq_calibrate_minmax(A, 4, 64, F(0.95), 0, None, None) == EINVAL
    assert L.zq_calibrate_minmax(A, 0, 64, F(0.95), 0, B, None) == ESHAPE
    assert L.zq_calibrate_minmax(A, 4, 64, F(1.5), 0, B, None) == EINVAL
    assert L.zq_quant_act_static(A, 4, 64, None, C, D, None) == EINVAL
    assert L.zq_quant_act_static(A, -1, 64, B, C, D, None) == ESHAPE
    assert L.zq_quant_act_static(None, 0, 64, B, None, D, None) == OK


@pytest.fixture
def empty_table():
    Z.sched_clear()
    yield
    Z.sched_clear()


def test_sched_table_import_export(empty_table):
    assert Z.sched_entries() == 0 and Z.sched_export() == ""
    assert Z.gemm_plan(128, 3072, 1024, 8).startswith("tiled")
    assert "[table]" not in Z.gemm_plan(128, 3072, 1024, 8)
    text = ("# bits N K lo hi kind tile\n"
            "8 3072 1024 65 256 tiled 22\n"
            "\n"
            "8 3072 1024 1 1 gemv 0\n"
            "8 3072 1024 2 16 stream 0\n"
            "4 3072 1024 17 64 skinny 0\n")
    Z.sched_import(text)
    assert Z.sched_entries() == 4
    assert Z.gemm_plan(128, 3072, 1024, 8).startswith("tiled cfg=22")
    assert Z.gemm_plan(128, 3072, 1024, 8).endswith("[table]")
    assert Z.gemm_plan(1, 3072, 1024, 8).startswith("gemv")
    assert Z.gemm_plan(9, 3072, 1024, 8).startswith("stream")
    assert Z.gemm_plan(40, 3072, 1024, 4).startswith("skinny BN=16 MF=3")
    # outside every range, or another shape: the built-in rules
    assert "[table]" not in Z.gemm_plan(257, 3072, 1024, 8)
    assert "[table]" not in Z.gemm_plan(128, 3072, 768, 8)
    assert "[table]" not in Z.gemm_plan(40, 3072, 1024, 8)
    # export is sorted by (bits, N, K, lo) and reads back the same
    out = Z.sched_export()
    assert out.splitlines() == ["4 3072 1024 17 64 skinny 0",
                                "8 3072 1024 1 1 gemv 0",
                                "8 3072 1024 2 16 stream 0",
                                "8 3072 1024 65 256 tiled 22"]
    Z.sched_clear()
    Z.sched_import(out)
    assert Z.sched_export() == out


def test_sched_import_overlap_splits_ranges(empty_table):
    Z.sched_import("8 1024 512 1 1000 tiled 0\n")
    Z.sched_import("8 1024 512 100 199 tiled 4\n")
    assert Z.sched_export().splitlines() == ["8 1024 512 1 99 tiled 0",
                                             "8 1024 512 100 199 tiled 4",
                                             "8 1024 512 200 1000 tiled 0"]
    assert Z.gemm_plan(150, 1024, 512, 8).startswith("tiled cfg=4")
    assert Z.gemm_plan(250, 1024, 512, 8).startswith("tiled cfg=0")


@pytest.mark.parametrize("line", [
    "8 3072 768 1 2 gemv 0",        # gemv is for one token only
    "8 3072 768 1 65 stream 0",     # stream: at most 64 tokens
    "8 3073 768 1 16 stream 0",     # stream: even N
    "8 3072 768 1 65 skinny 0",     # skinny: at most 64 tokens
    "4 3072 768 1 64 tiled 16",     # W8-only tile for W4
    "8 3072 768 1 64 tiled 29",     # no such tile
    "8 3072 768 1 64 tiled 28",     # W4-only tile for W8
    "8 3072 768 0 64 tiled 0",      # M from 1
    "8 3072 768 9 8 tiled 0",       # empty range
    "8 3072 700 1 8 tiled 0",       # K % 64
    "5 3072 768 1 8 tiled 0",       # bits
    "8 3072 768 1 8 huge 0",        # kind
    "8 3072 768 1 8 tiled 0 extra",
    "8 3072 768 1 8 tiled",
])
def test_sched_import_rejects_bad_lines(empty_table, line):
    L = Z.lib()
    good = b"8 1024 512 1 8 tiled 0\n"
    assert L.zq_sched_import(good + line.encode() + b"\n") == EINVAL
    assert b"line 2" in L.zq_last_error()
    assert Z.sched_entries() == 0       # all or nothing


def test_sched_export_buffer_handling(empty_table):
    L = Z.lib()
    Z.sched_import("8 1024 512 1 8 tiled 0\n")
    need = ctypes.c_size_t(0)
    assert L.zq_sched_export(None, 0, ctypes.byref(need)) == OK
    assert need.value == len("8 1024 512 1 8 tiled 0\n") + 1
    small = ctypes.create_string_buffer(5)
    assert L.zq_sched_export(small, 5, None) == OK
    assert small.value == b"8 10"                   # truncated, NUL-terminated
    assert L.zq_sched_export(None, 4, None) == EINVAL
    assert L.zq_sched_import(None) == EINVAL


def test_gemm_tune_argument_checks():
    f = Z.lib().zq_gemm_tune
    ms = (ctypes.c_int * 3)(16, 64, 128)
    bad = (ctypes.c_int * 3)(16, 16, 128)
    zero = (ctypes.c_int * 1)(0)
    # (bits, qx, sx, qw, sw, G, bias, act, ms, nm, N, K, y, reps, chosen, us, stream)
    assert f(5, A, B, C, D, 64, None, 0, ms, 3, 256, 256, E, 5, None, None, None) == EINVAL
    assert f(8, A, B, C, D, 64, None, 0, bad, 3, 256, 256, E, 5, None, None, None) == EINVAL
    assert f(8, A, B, C, D, 64, None, 0, zero, 1, 256, 256, E, 5, None, None, None) == EINVAL
    assert f(8, A, B, C, D, 64, None, 0, ms, 0, 256, 256, E, 5, None, None, None) == EINVAL
    assert f(8, A, B, C, D, 64, None, 0, ms, 3, 256, 256, E, 0, None, None, None) == EINVAL
    assert f(8, A, B, C, D, 64, None, 0, ms, 3, 256, 256, None, 5, None, None, None) == EINVAL
    assert f(8, A, B, C, D, 64, None, 0, ms, 3, 96, 256, E, 5, None, None, None) == ESHAPE
    assert f(8, A, B, C, D, 64, None, 0, ms, 3, 256, 100, E, 5, None, None, None) == EUNSUP
    assert Z.sched_entries() == 0


def test_chain_host_side():
    L = Z.lib()
    h = ctypes.c_void_p()
    assert L.zq_chain_create(0, ctypes.byref(h)) == EINVAL
    assert L.zq_chain_create(128, None) == EINVAL
    assert L.zq_chain_create(128, ctypes.byref(h)) == OK
    try:
        assert L.zq_chain_length(h) == 0 and L.zq_chain_graphs(h) == 0
        F = ctypes.c_float
        assert L.zq_chain_add_ln_quant(h, A, None, None, F(1e-5), 768, B, C,
                                       None) == OK
        assert L.zq_chain_add_ln_quant(h, A, None, None, F(-1.0), 768, B, C,
                                       None) == EINVAL
        assert L.zq_chain_add_quant(h, A, 70000, B, C) == EUNSUP
        assert L.zq_chain_add_quant(h, None, 768, B, C) == EINVAL
        # (c, bits, qx, sx, qw, sw, G, bias, act, N, K, y)
        assert L.zq_chain_add_gemm(h, 8, B, C, D, E, 64, None, 1, 3072, 768,
                                   A) == OK
        assert L.zq_chain_add_gemm(h, 8, B, C, D, E, 64, None, 1, 3000, 768,
                                   A) == ESHAPE
        assert L.zq_chain_add_gemm(h, 3, B, C, D, E, 64, None, 1, 3072, 768,
                                   A) == EINVAL
        assert L.zq_chain_add_gemm(h, 8, B, C, D, E, 64, None, 1, 3072, 768,
                                   None) == EINVAL
        ws_need = Z.lib().zq_gemm_quant_workspace_bytes(128, 3072)
        assert ws_need == 128 * 3072 * 2
        # (c, bits, qx, sx, qw, sw, G, bias, act, N, K, qy, sy, ws, ws_bytes)
        assert L.zq_chain_add_gemm_quant(h, 4, B, C, D, E, 64, None, 1, 3072,
                                         768, A, B, C, ws_need - 1) == EINVAL
        assert b"workspace" in L.zq_last_error()
        assert L.zq_chain_add_gemm_quant(h, 4, B, C, D, E, 64, None, 1, 3072,
                                         768, A, B, C, ws_need) == OK
        # (c, x, qw, sw, G, bias, act, N, K, y)
        assert L.zq_chain_add_gemm_w8a16(h, A, B, C, 64, None, 0, 768, 3072,
                                         D) == OK
        assert L.zq_chain_add_gemm_w8a16(h, A, B, C, 64, None, 0, 768, 3000,
                                         D) == EUNSUP
        # (c, bits, x, qw, sw, G, bias, act, N, K, y, qx, sx)
        assert L.zq_chain_add_gemm_xq(h, 8, A, B, C, 64, None, 0, 768, 3072,
                                      D, E, A) == OK
        assert L.zq_chain_add_gemm_xq(h, 4, A, B, C, 64, None, 0, 768, 3000,
                                      D, E, A) == EUNSUP
        assert L.zq_chain_add_gemm_xq(h, 8, A, B, C, 64, None, 0, 768, 3072,
                                      D, None, A) == EINVAL
        assert L.zq_chain_add_gemm_xq(h, 6, A, B, C, 64, None, 0, 768, 3072,
                                      D, E, A) == EINVAL
        assert L.zq_chain_length(h) == 5
        assert L.zq_chain_run(h, 129, None) == EINVAL
        assert L.zq_chain_run(h, -1, None) == EINVAL
        assert L.zq_chain_run_eager(h, 129, None) == EINVAL
        assert L.zq_chain_run(h, 0, None) == OK          # empty: no launch
        assert L.zq_chain_run_eager(h, 0, None) == OK
        assert L.zq_chain_graphs(h) == 0
        assert L.zq_chain_run(None, 1, None) == EINVAL
        assert L.zq_chain_add_quant(None, A, 768, B, C) == EINVAL
    finally:
        L.zq_chain_destroy(h)
    L.zq_chain_destroy(None)


def test_gemm_ws_plans_and_checks(empty_table):
    L = Z.lib()
    # 33 .. 64 tokens over few 64 x 64 tiles: K split, workspace sk * M * N * 4
    assert Z.gemm_workspace_bytes(64, 6144, 6144, 8) == 2 * 64 * 6144 * 4
    assert Z.gemm_ws_plan(64, 6144, 6144, 8).startswith("splitk SK=2 tiled cfg=22")
    assert Z.gemm_workspace_bytes(64, 4096, 16384, 4) == 4 * 64 * 4096 * 4
    assert Z.gemm_workspace_bytes(64, 1024, 24576, 8) == 8 * 64 * 1024 * 4
    # no split: too few or too many tokens, enough tiles, K not in whole
    # slices, slices shorter than 3072 k, fewer than 128 workgroups
    # (and at most 32 tokens, or packed W4 in two slices: the plain call's
    # streaming rings are as fast)
    for shape in [(16, 4096, 16384, 8), (65, 4096, 16384, 8), (64, 8192, 16384, 8),
                  (64, 4096, 16448, 8), (64, 4096, 4096, 8), (64, 4096, 768, 8),
                  (33, 1024, 16384, 8), (32, 6144, 6144, 8), (48, 6144, 6144, 4)]:
        assert Z.gemm_workspace_bytes(*shape) == 0, shape
        assert not Z.gemm_ws_plan(*shape).startswith("splitk")
    assert Z.gemm_workspace_bytes(0, 4096, 4096, 8) == 0
    assert Z.gemm_workspace_bytes(64, 4096, 4096, 5) == 0
    # a table entry for the shape wins
    Z.sched_import("8 6144 6144 17 64 skinny 0\n")
    assert Z.gemm_workspace_bytes(64, 6144, 6144, 8) == 0
    assert Z.gemm_ws_plan(64, 6144, 6144, 8).startswith("skinny")
    Z.sched_clear()
    f = L.zq_gemm_w8a8_ws
    # (qx, sx, qw, sw, G, bias, act, M, N, K, y, ws, ws_bytes, stream)
    need = Z.gemm_workspace_bytes(64, 6144, 6144, 8)
    assert f(A, B, C, D, 128, None, 0, 64, 6144, 6144, E, None, 0, None) == EINVAL
    assert f(A, B, C, D, 128, None, 0, 64, 6144, 6144, E, A, need - 1, None) == EINVAL
    assert b"workspace" in L.zq_last_error()
    assert f(A, B, C, D, 128, None, 0, 64, 6144, 6144, E,
             ctypes.c_void_p(0x10008), need, None) == EINVAL     # misaligned
    assert f(A, B, C, D, 128, None, 0, 64, 6144, 6000, E, A, need, None) == EUNSUP
    assert f(A, B, C, D, 100, None, 0, 64, 6144, 6144, E, A, need, None) == ESHAPE
    # a shape that does not split needs no workspace
    assert f(None, B, C, D, 128, None, 0, 0, 4096, 4096, E, None, 0, None) == OK
    assert f(None, None, C, D, 128, None, 0, 0, 4096, 4096, None, None, 0, None) == OK
    assert L.zq_gemm_ws_plan(64, 4096, 4096, 3, ctypes.create_string_buffer(8), 8) == EINVAL


def test_chain_ws_gemm_host_side():
    L = Z.lib()
    h = ctypes.c_void_p()
    assert L.zq_chain_create(128, ctypes.byref(h)) == OK
    try:
        need = max(Z.gemm_workspace_bytes(m, 6144, 6144, 8) for m in range(1, 65))
        assert need == Z.gemm_workspace_bytes(64, 6144, 6144, 8) > 0
        # (c, bits, qx, sx, qw, sw, G, bias, act, N, K, y, ws, ws_bytes)
        assert L.zq_chain_add_gemm_ws(h, 8, A, B, C, D, 128, None, 0, 6144, 6144,
                                      E, A, need - 1) == EINVAL
        assert L.zq_chain_add_gemm_ws(h, 8, A, B, C, D, 128, None, 0, 6144, 6144,
                                      E, None, 0) == EINVAL
        assert L.zq_chain_add_gemm_ws(h, 8, A, B, C, D, 128, None, 0, 6144, 6144,
                                      E, A, need) == OK
        # a shape no token count splits needs no workspace
        assert L.zq_chain_add_gemm_ws(h, 4, A, B, C, D, 128, None, 0, 4096, 4096,
                                      E, None, 0) == OK
        assert L.zq_chain_add_gemm_ws(h, 5, A, B, C, D, 128, None, 0, 4096, 4096,
                                      E, None, 0) == EINVAL
        assert L.zq_chain_length(h) == 2
    finally:
        L.zq_chain_destroy(h)


@pytest.mark.parametrize("shape,plan", [
    # one round of tiles: the smallest tile that fits the 256 compute units
    ((128, 768, 3072, 8), "tiled cfg=22 "),
    ((2048, 768, 3072, 8), "tiled cfg=21 "),
    ((4096, 768, 3072, 8), "tiled cfg=15 "),      # BERT-base FFN2
    ((128, 18432, 6144, 8), "tiled cfg=15 "),
    # larger problems: fill x quality among the big tiles
    ((4096, 3072, 768, 8), "tiled cfg=13 "),      # BERT-base FFN1
    ((4096, 2304, 768, 8), "tiled cfg=14 "),      # BERT-base QKV
    # W4: two-block 128x128 below K = 4096; the persistent ping-pong kernel
    # over N >= 16384 (NeoX FFN1); otherwise the W8 picker (NeoX FFN2)
    ((8192, 4096, 1024, 4), "tiled cfg=0 "),
    ((2048, 24576, 6144, 4), "tiled cfg=28 "),
    ((2048, 6144, 24576, 4), "tiled cfg=13 "),
    # decode-sized token counts
    ((64, 16384, 4096, 8), "tiled cfg=22 "),
    ((64, 4096, 4096, 8), "stream BN=16 MX=64 "),
    ((32, 12288, 4096, 8), "stream BN=32 MX=32 "),
    ((64, 6144, 24576, 4), "stream BN=32 MX=64 "),
    ((16, 24576, 6144, 4), "stream BN=32 MX=16 "),
    ((16, 12288, 4096, 8), "stream BN=16 MX=16 "),
    ((16, 6144, 6144, 8), "stream BN=32 MX=16 "),
])
def test_tile_rule_regression(empty_table, shape, plan):
    # the plans the schedule tuner measured best for these shapes
    assert Z.gemm_plan(*shape).startswith(plan), Z.gemm_plan(*shape)


@pytest.mark.parametrize("fn", ["zq_gemm_w8a8_xq", "zq_gemm_w4a8_xq"])
def test_gemm_xq_argument_checks(fn):
    f = getattr(Z.lib(), fn)
    # (x, qw, sw, G, bias, act, M, N, K, y, qx, sx, stream)
    assert f(A, B, C, 64, None, 0, 1, 256, 100, D, E, A, None) == EUNSUP  # K % 64
    assert f(A, B, C, 64, None, 0, 1, 96, 256, D, E, A, None) == ESHAPE   # N % G
    assert f(A, B, C, 64, None, 2, 1, 256, 256, D, E, A, None) == EINVAL  # act
    assert f(None, B, C, 64, None, 0, 1, 256, 256, D, E, A, None) == EINVAL
    assert f(A, B, C, 64, None, 0, 1, 256, 256, D, None, A, None) == EINVAL  # qx
    assert f(A, B, C, 64, None, 0, 1, 256, 256, D, E, None, None) == EINVAL  # sx
    assert f(A, B, C, 64, None, 0, 1, 256, 256, None, E, A, None) == EINVAL  # y
    assert f(ctypes.c_void_p(0x10008), B, C, 64, None, 0, 1, 256, 256, D, E, A,
             None) == EINVAL                                              # x align
    assert f(A, B, C, 64, None, 0, 1, 256, 65600, D, E, A, None) == EUNSUP  # row K
    assert f(None, B, C, 64, None, 0, 0, 256, 256, None, None, None,
             None) == OK                                                  # empty


def test_gemm_xq_plan_names_the_form():
    assert Z.gemm_xq_plan(1, 4096, 16384, 8).startswith("quantize-on-load gemv")
    assert Z.gemm_xq_plan(1, 6144, 24576, 4).startswith("quantize-on-load gemv")
    # past 32768 k the GEMV re-reads the row from the caches: two launches
    assert Z.gemm_xq_plan(1, 4096, 65536, 8).startswith("row-quant + gemv")
    assert Z.gemm_xq_plan(16, 4096, 16384, 8).startswith("row-quant + stream")
    assert Z.gemm_xq_plan(2048, 6144, 24576, 4).startswith("row-quant + tiled")


@pytest.mark.parametrize("N,K,bits,rows,chunk", [
    (12288, 4096, 8, 16, 512), (4096, 4096, 8, 16, 256),
    (16384, 4096, 8, 16, 512), (4096, 16384, 8, 16, 256),
    (18432, 6144, 8, 16, 256), (6144, 6144, 8, 32, 256),
    (24576, 6144, 4, 32, 128), (6144, 24576, 4, 32, 128),
    (16384, 1024, 4, 32, 256)])
def test_chunked_layout_of_the_decode_shapes(N, K, bits, rows, chunk):
    # the 16-token ring each decode linear of GPT-J-6B / GPT-NeoX-20B runs
    L = Z.lib()
    r, c = ctypes.c_int(0), ctypes.c_int(0)
    assert L.zq_chunked_layout(N, K, bits, ctypes.byref(r), ctypes.byref(c)) == OK
    assert (r.value, c.value) == (rows, chunk)


def test_chunked_argument_checks():
    L = Z.lib()
    r, c = ctypes.c_int(0), ctypes.c_int(0)
    assert L.zq_chunked_layout(40, 256, 8, ctypes.byref(r), ctypes.byref(c)) == EUNSUP
    assert L.zq_chunked_layout(256, 320, 8, ctypes.byref(r), ctypes.byref(c)) == EUNSUP
    assert L.zq_chunked_layout(256, 256, 5, ctypes.byref(r), ctypes.byref(c)) == EINVAL
    # pack: null / overlapping buffers
    assert L.zq_pack_chunked(None, 256, 256, 8, B, None) == EINVAL
    assert L.zq_pack_chunked(A, 256, 256, 8, ctypes.c_void_p(0x10000 + 4096),
                             None) == EINVAL
    # (qx, sx, qd, sw, G, bias, act, M, N, K, y, stream)
    f = L.zq_gemm_w8a8_chunked
    assert f(A, B, C, D, 64, None, 0, 17, 256, 256, E, None) == EUNSUP   # M > 16
    assert f(A, B, C, D, 64, None, 0, 4, 40, 256, E, None) == EUNSUP     # N % BN
    assert f(A, B, C, D, 64, ctypes.c_void_p(0x60002), 0, 4, 256, 256, E,
             None) == EINVAL                                             # bias
    assert f(A, B, C, D, 64, None, 0, 0, 256, 256, E, None) == OK        # empty
    assert f(A, B, C, D, 64, None, 2, 4, 256, 256, E, None) == EINVAL    # act
    assert f(A, B, C, D, 48, None, 0, 4, 256, 256, E, None) == ESHAPE    # N % G
    assert L.zq_gemm_chunked_i32(5, A, B, 4, 256, 256, C, None) == EINVAL
    buf = ctypes.create_string_buffer(160)
    assert L.zq_gemm_chunked_plan(16, 6144, 24576, 4, buf, 160) == OK
    assert buf.value.startswith(b"chunked stream BN=32 CK=128")


def test_chain_chunked_gemm_host_side():
    L = Z.lib()
    for max_m, want in ((16, OK), (17, EUNSUP)):
        h = ctypes.c_void_p()
        assert L.zq_chain_create(max_m, ctypes.byref(h)) == OK
        # (chain, bits, qx, sx, qd, sw, G, bias, act, N, K, y)
        assert L.zq_chain_add_gemm_chunked(h, 8, A, B, C, D, 128, None, 0,
                                           8192, 1024, E) == want
        assert L.zq_chain_add_gemm_chunked(h, 8, A, B, C, D, 128, None, 0,
                                           40, 1024, E) == EUNSUP  # N % BN
        assert L.zq_chain_add_gemm_chunked(h, 5, A, B, C, D, 128, None, 0,
                                           8192, 1024, E) == EINVAL
        assert L.zq_chain_length(h) == (1 if want == OK else 0)
        L.zq_chain_destroy(h)
