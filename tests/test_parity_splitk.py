"""GPU parity of the GEMM calls with a workspace (zq_gemm_w8a8_ws /
zq_gemm_w4a8_ws): for 33 .. 64 tokens over few weight tiles the K range is
split over several workgroups whose exact int32 partial sums a second
kernel adds before the shared epilogue.

* Exact: y equals the call without a workspace bit for bit (integer partial
  sums are order-free and the epilogue is the same code).
* Oracle: y within 1 fp16 ulp + 1e-3 of the oracle's fp64 epilogue on every
  row, and the split's int32 sums equal the oracle's GEMM.
* A workspace reused across calls of different shapes (its contents never
  need clearing), and shapes that do not split run unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
import int4_quantized_transformer_amd as zq
from int4_quantized_transformer_amd import workloads as W

from _util import assert_fp16_close_to_oracle, dev, needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def _inputs(M, N, K, G, bits, seed):
    x = W.randn_fp16((M, K), seed=seed, std=1.0)
    w = W.randn_fp16((N, K), seed=seed + 1, std=0.02)
    b = W.randn_fp16((N,), seed=seed + 2, std=0.5)
    qx, sx = oracle.quant_tokens(x.numpy())
    q, sw = oracle.quantize_weights(w.numpy(), G, bits)
    qw = q if bits == 8 else oracle.pack_w4(q)
    return qx, sx, q, qw, sw, b


CASES = [  # (M, N, K, G, bits, act)
    (64, 4096, 16384, 128, 8, 0),    # GPT-J FFN2, 64 tokens: 4 slices
    (64, 6144, 6144, 128, 8, 0),     # NeoX attention output: 2 slices
    (33, 4096, 12288, 128, 8, 1),
    (48, 4096, 16384, 128, 4, 1),    # W4 in 4 slices
    (64, 1024, 24576, 128, 4, 0),    # 8 slices
    (40, 2046, 12288, 2, 8, 1),      # N % 4 != 0: scalar reduction path
    (64, 4104, 6144, 8, 8, 0),       # ragged N tile
]


@pytest.mark.parametrize("M,N,K,G,bits,act", CASES)
def test_ws_gemm_splits_and_matches(M, N, K, G, bits, act):
    assert zq.gemm_workspace_bytes(M, N, K, bits) > 0
    assert zq.gemm_ws_plan(M, N, K, bits).startswith("splitk")
    d = dev()
    qx, sx, q, qw, sw, b = _inputs(M, N, K, G, bits, M + N + K + bits)
    args = (torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
            torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), G, b.to(d),
            act)
    plain = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    wsfn = zq.gemm_w8a8_ws if bits == 8 else zq.gemm_w4a8_ws
    y0 = to_np(plain(*args))
    y1 = to_np(wsfn(*args))
    assert np.array_equal(y1.view(np.uint16), y0.view(np.uint16))
    acc = oracle.gemm_i32(qx, q)
    z, _ = oracle.epilogue(acc, sx, sw, G, b.numpy(), act)
    assert_fp16_close_to_oracle(y1, z, zq.gemm_ws_plan(M, N, K, bits))


def test_ws_partials_are_the_exact_sums():
    # the split's workspace planes add up to the oracle's int32 GEMM
    M, N, K, G = 64, 4096, 16384, 128
    qx, sx, q, qw, sw, b = _inputs(M, N, K, G, 8, 77)
    d = dev()
    need = zq.gemm_workspace_bytes(M, N, K, 8)
    sk = need // (M * N * 4)
    ws = torch.empty(need, dtype=torch.uint8, device=d)
    zq.gemm_w8a8_ws(torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
                    torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), G,
                    b.to(d), 0, ws=ws)
    planes = to_np(ws.view(torch.int32)).reshape(sk, M, N).astype(np.int64)
    assert np.array_equal(planes.sum(axis=0), oracle.gemm_i32(qx, q))


def test_ws_reused_across_shapes_and_unsplit_shapes():
    d = dev()
    ws = torch.full((zq.gemm_workspace_bytes(64, 4096, 16384, 8),), 0x5A,
                    dtype=torch.uint8, device=d)
    for (M, N, K, bits) in [(64, 4096, 16384, 8), (64, 1024, 24576, 4),
                            (16, 4096, 4096, 8), (64, 8192, 1024, 8),
                            (64, 6144, 6144, 8), (64, 4096, 4096, 8),
                            (300, 1024, 512, 4)]:
        qx, sx, q, qw, sw, b = _inputs(M, N, K, 64, bits, 5 + M + K)
        args = (torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
                torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), 64,
                b.to(d), 1)
        plain = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
        wsfn = zq.gemm_w8a8_ws if bits == 8 else zq.gemm_w4a8_ws
        y1 = to_np(wsfn(*args, ws=ws))
        y0 = to_np(plain(*args))
        assert np.array_equal(y1.view(np.uint16), y0.view(np.uint16)), (M, N, K)


def test_ws_small_workspace_is_refused():
    d = dev()
    M, N, K = 64, 4096, 16384
    qx = torch.zeros(M, K, dtype=torch.int8, device=d)
    sx = torch.ones(M, dtype=torch.float32, device=d)
    qw = torch.zeros(N, K, dtype=torch.int8, device=d)
    sw = torch.ones(N // 128, dtype=torch.float32, device=d)
    small = torch.empty(1024, dtype=torch.uint8, device=d)
    with pytest.raises(zq.ZQError):
        zq.gemm_w8a8_ws(qx, sx, qw, sw, 128, ws=small)
