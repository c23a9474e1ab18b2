"""GPU parity of the GEMMs with token-quantized output (zq_gemm_*_quant):
the quantization of the next linear's input at the producing linear.

* Exact: (qy, sy) equal, bit for bit, zq_gemm_* (fp16 y) followed by
  zq_quant_act(y) on the same inputs, over every GEMM plan (tiled with
  several tile shapes, GEMV, streaming, skinny), ragged M and N, G not a
  multiple of 32 and odd N with a bias.
* Oracle: against the oracle's fp64 epilogue rounded to fp16 and its token
  quantizer.  The GPU fp16 y is within 1 fp16 ulp + 1e-3 of the oracle
  epilogue; with S = amax/127 a difference dy moves a code by dy/S, so codes
  agree within 1 and scales within 2e-3 (relative) unless amax itself is
  below about 0.1 (not the case for these inputs).
"""
import numpy as np
import pytest
import torch

import oracle
import int4_quantized_transformer_amd as zq
from int4_quantized_transformer_amd import workloads as W

from _util import dev, needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [  # (M, N, K, G, bits, bias, act)
    (4096, 3072, 768, 64, 8, True, 1),     # BERT-base FFN1: 192x256 tiles
    (4096, 2304, 768, 64, 8, True, 0),     # 288x128 tiles
    (4096, 768, 3072, 64, 8, False, 0),    # 96x128 tiles
    (2048, 4096, 1024, 128, 8, True, 1),   # 128x128 tiles
    (300, 1024, 640, 64, 4, True, 1),      # W4, ragged M
    (130, 320, 192, 32, 8, True, 1),       # ragged N tile
    (8192, 4096, 1024, 64, 4, True, 1),    # BERT-large FFN1, W4
    (257, 1000, 320, 8, 8, True, 1),       # G % 32 != 0
    (200, 999, 256, 3, 8, True, 0),        # odd N with bias
    (1, 4096, 4096, 128, 8, True, 1),      # decode GEMV
    (16, 2048, 1024, 64, 4, False, 1),     # decode streaming kernel
    (64, 512, 512, 64, 8, True, 0),        # decode skinny kernel
]


def _inputs(M, N, K, G, bits, bias, seed):
    x = W.randn_fp16((M, K), seed=seed, std=1.0)
    w = W.randn_fp16((N, K), seed=seed + 1, std=0.02)
    b = W.randn_fp16((N,), seed=seed + 2, std=0.5) if bias else None
    qx, sx = oracle.quant_tokens(x.numpy())
    q, sw = oracle.quantize_weights(w.numpy(), G, bits)
    qw = q if bits == 8 else oracle.pack_w4(q)
    return qx, sx, q, qw, sw, b


@pytest.mark.parametrize("M,N,K,G,bits,bias,act", CASES)
def test_quantized_output(M, N, K, G, bits, bias, act):
    d = dev()
    qx, sx, q, qw, sw, b = _inputs(M, N, K, G, bits, bias, M + N + K + G)
    tqx, tsx = torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d)
    tqw, tsw = torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d)
    tb = None if b is None else b.to(d)
    fused = zq.gemm_w8a8_quant if bits == 8 else zq.gemm_w4a8_quant
    plain = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    qy, sy = fused(tqx, tsx, tqw, tsw, G, tb, act)
    y = plain(tqx, tsx, tqw, tsw, G, tb, act)
    qy2, sy2 = zq.quant_act(y)
    torch.cuda.synchronize()
    qy_np, sy_np = to_np(qy), to_np(sy)
    assert np.array_equal(sy_np, to_np(sy2))
    assert np.array_equal(qy_np, to_np(qy2))

    # against the oracle, on sampled rows
    g = np.random.default_rng(M * 7 + N)
    rows = np.unique(np.concatenate([[0, M - 1], g.choice(M, size=min(M, 24),
                                                         replace=False)]))
    acc = oracle.gemm_i32(qx[rows], q)
    z, _ = oracle.epilogue(acc, sx[rows], sw, G, None if b is None else b.numpy(),
                           act)
    y16 = oracle.double_to_half(z)
    q_ref, s_ref = oracle.quant_tokens(y16)
    assert np.allclose(sy_np[rows], s_ref, rtol=2e-3, atol=0)
    dq = np.abs(qy_np[rows].astype(np.int32) - q_ref.astype(np.int32))
    assert dq.max() <= 1


def test_workspace_is_checked():
    d = dev()
    M, N, K, G = 64, 256, 128, 64
    qx = torch.zeros(M, K, dtype=torch.int8, device=d)
    sx = torch.ones(M, dtype=torch.float32, device=d)
    qw = torch.zeros(N, K, dtype=torch.int8, device=d)
    sw = torch.ones(N // G, dtype=torch.float32, device=d)
    small = torch.empty(16, dtype=torch.uint8, device=d)
    with pytest.raises(zq.ZQError):
        zq.gemm_w8a8_quant(qx, sx, qw, sw, G, ws=small)


def test_repeated_calls_reuse_workspace():
    # one workspace through consecutive calls of different shapes (stale
    # contents from a larger call must never be read), the last ones smaller
    d = dev()
    ws = torch.empty(zq.gemm_quant_workspace_bytes(4096, 3072), dtype=torch.uint8,
                     device=d)
    for (M, N, K) in [(4096, 3072, 768), (4096, 2304, 768), (4096, 3072, 768),
                      (4096, 768, 3072), (1024, 1024, 512)]:
        qx, sx, q, qw, sw, b = _inputs(M, N, K, 64, 8, True, 5 + M)
        args = (torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
                torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), 64,
                b.to(d), 1)
        qy, sy = zq.gemm_w8a8_quant(*args, ws=ws)
        qy2, sy2 = zq.quant_act(zq.gemm_w8a8(*args))
        torch.cuda.synchronize()
        assert np.array_equal(to_np(qy), to_np(qy2))
        assert np.array_equal(to_np(sy), to_np(sy2))
