"""GPU test of zq_gemm_noalloc, the entry point for callers that cannot
allocate: the split-K GEMM with the library's per-device scratch array,
called through the C ABI, against zq_gemm_w8a8_ws / zq_gemm_w4a8_ws (bit-
identical) and the oracle (1 fp16 ulp + 1e-3), on two calls in a row with
the second on a smaller problem, plus a shape that does not split (no
scratch used) and an empty call."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import int4_quantized_transformer_amd as zq
from int4_quantized_transformer_amd import workloads as W

from _util import assert_fp16_close_to_oracle, dev, needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]

P = ctypes.c_void_p


def _inputs(M, N, K, G, bits, seed):
    x = W.randn_fp16((M, K), seed=seed, std=1.0)
    w = W.randn_fp16((N, K), seed=seed + 1, std=0.02)
    b = W.randn_fp16((N,), seed=seed + 2, std=0.5)
    qx, sx = oracle.quant_tokens(x.numpy())
    q, sw = oracle.quantize_weights(w.numpy(), G, bits)
    qw = q if bits == 8 else oracle.pack_w4(q)
    z, _ = oracle.epilogue(oracle.gemm_i32(qx, q), sx, sw, G, b.numpy(), 1)
    d = dev()
    return (torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
            torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), b.to(d), z)


def _call_c(bits, qx, sx, qw, sw, G, b, act):
    M, K = qx.shape
    N = qw.shape[0]
    y = torch.empty(M, N, dtype=torch.float16, device=qx.device)
    st = zq.lib().zq_gemm_noalloc(bits, P(qx.data_ptr()), P(sx.data_ptr()),
                                  P(qw.data_ptr()), P(sw.data_ptr()), G,
                                  P(b.data_ptr()), act, M, N, K,
                                  P(y.data_ptr()),
                                  P(torch.cuda.current_stream().cuda_stream))
    assert st == 0, zq.lib().zq_last_error()
    return y


@pytest.mark.parametrize("bits", [8, 4])
def test_noalloc_matches_workspace_call_twice_second_smaller(bits):
    zq.sched_clear()
    G = 128
    # first: 64 x 4096 x 16384 splits K in 4 (the 4 MiB maximum);
    # second: 40 x 2048 x 12288, a smaller split
    first, second = (64, 4096, 16384), (40, 2048, 12288)
    for (M, N, K), seed in ((first, 7), (second, 11)):
        need = zq.gemm_workspace_bytes(M, N, K, bits)
        assert 0 < need <= zq.NOALLOC_SCRATCH_BYTES, need
        qx, sx, qw, sw, b, z = _inputs(M, N, K, G, bits, seed + bits)
        y = to_np(_call_c(bits, qx, sx, qw, sw, G, b, 1))
        ws_fn = zq.gemm_w8a8_ws if bits == 8 else zq.gemm_w4a8_ws
        y_ws = to_np(ws_fn(qx, sx, qw, sw, G, b, 1))
        assert np.array_equal(y.view(np.uint16), y_ws.view(np.uint16)), (M, N, K)
        assert_fp16_close_to_oracle(y, z, zq.gemm_ws_plan(M, N, K, bits))
    assert zq.gemm_workspace_bytes(*first, 8) == zq.NOALLOC_SCRATCH_BYTES


def test_noalloc_without_a_split_and_empty():
    # a shape that does not split runs the plain plan (scratch unused)
    M, N, K, G = 16, 1024, 1024, 64
    assert zq.gemm_workspace_bytes(M, N, K, 8) == 0
    qx, sx, qw, sw, b, z = _inputs(M, N, K, G, 8, 3)
    y = to_np(_call_c(8, qx, sx, qw, sw, G, b, 1))
    assert_fp16_close_to_oracle(y, z, zq.gemm_plan(M, N, K, 8))
    L = zq.lib()
    assert L.zq_gemm_noalloc(8, None, None, P(qw.data_ptr()), P(sw.data_ptr()),
                             G, None, 0, 0, N, K, None, None) == 0
    assert L.zq_gemm_noalloc(5, None, None, P(qw.data_ptr()), P(sw.data_ptr()),
                             G, None, 0, 0, N, K, None, None) == 1
