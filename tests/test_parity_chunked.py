"""GPU parity of the chunk-contiguous decode layout.

* zq_pack_chunked: byte-exact against the layout written out in numpy
  (a permutation of the row-major bytes: qd[((rb*NC + c)*BN + r)*CK + b] =
  qw[(rb*BN + r)*R + c*CK + b]).
* zq_gemm_chunked_i32 on the packed oracle codes: int32 accumulators
  bit-exact against oracle.gemm_i32 on the row-major codes, 1..16 tokens
  (one token: the chunked GEMV, or the ring for K > 32768),
  every ring the layout selects (W8 16- and 32-row blocks, W4, resident
  activations with 512- / 256-byte and 256- / 128-byte chunks), the full
  code range.
* zq_gemm_{w8a8,w4a8}_chunked: fp16 y within 1 fp16 ulp + 1e-3 of the
  oracle's fp64 epilogue, with and without bias / GeLU, and bit-identical
  to zq_gemm_{w8a8,w4a8} on the row-major codes.
* The GPT-J-6B and GPT-NeoX-20B decode linears at 1 and 16 tokens, full
  size: y bit-identical to the row-major call, sampled columns against the
  oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import int4_quantized_transformer_amd as zq
from int4_quantized_transformer_amd import workloads as W

from _util import assert_fp16_close_to_oracle, dev, needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def chunked_bytes(qw_bytes, bn, ck):
    """Row-major byte matrix [N, R] -> the chunked layout's bytes."""
    N, R = qw_bytes.shape
    nc = R // ck
    return (qw_bytes.reshape(N // bn, bn, nc, ck).transpose(0, 2, 1, 3)
            .reshape(-1))


def _codes(shape, lo, hi, seed):
    g = np.random.default_rng(seed)
    return g.integers(lo, hi + 1, size=shape).astype(np.int8)


def _to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def _rowmajor(q, bits):
    return q if bits == 8 else oracle.pack_w4(q)


def _pack(q, bits):
    return zq.pack_chunked(_to_dev(_rowmajor(q, bits)), bits)


# (N, K) per bits covering every ring the layout picks (see
# zq_chunked_layout): W8 resident K <= 4096 (N/16 >= 512), resident K <= 6144,
# 32-row blocks (256 < N/16, N/32 <= 256), 16-row blocks; W4 resident
# K <= 4096 / 6144 (N/32 >= 512) and plain
LAYOUT_SHAPES = [
    (8, 8192, 1024), (8, 8192, 4608), (8, 6144, 768), (8, 256, 512),
    (8, 1024, 8192), (4, 16384, 1024), (4, 16384, 5120), (4, 64, 256),
    (4, 2048, 9216),
    # K > 32768: one token runs the ring (the activation row exceeds the
    # one-token kernel's LDS image)
    (8, 64, 33024), (4, 64, 33024),
]


@pytest.mark.parametrize("bits,N,K", LAYOUT_SHAPES)
def test_pack_matches_layout(bits, N, K):
    bn, ck = zq.chunked_layout(N, K, bits)
    q = _codes((N, K), -127 if bits == 8 else -8, 127 if bits == 8 else 7,
               N + K + bits)
    rm = _rowmajor(q, bits)
    qd = zq.pack_chunked(_to_dev(rm), bits)
    torch.cuda.synchronize()
    got = to_np(qd).reshape(-1).view(np.uint8)
    assert np.array_equal(got, chunked_bytes(rm.view(np.uint8), bn, ck))


@pytest.mark.parametrize("bits,N,K", LAYOUT_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_chunked_i32_bit_exact(bits, N, K, M):
    qmax = 127 if bits == 8 else 7
    qx = _codes((M, K), -127, 127, M * 7 + K + bits)
    q = _codes((N, K), -qmax - 1, qmax, N * 11 + K + bits)  # incl. -128 / -8
    acc = zq.gemm_chunked_i32(bits, _to_dev(qx), _pack(q, bits))
    ref = oracle.gemm_i32(qx, q)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(acc), ref), zq.gemm_chunked_plan(M, N, K, bits)


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("bits", [8, 4])
def test_chunked_i32_extreme_codes(M, bits):
    K, N = 24576, 64
    qmax = 127 if bits == 8 else 7
    qx = np.full((M, K), 127, np.int8)
    qx[::2] = -127
    q = np.full((N, K), qmax, np.int8)
    q[1::2] = -qmax if bits == 8 else -8
    acc = zq.gemm_chunked_i32(bits, _to_dev(qx), _pack(q, bits))
    ref = oracle.gemm_i32(qx, q)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(acc), ref)


@pytest.mark.parametrize("M,N,K,G", [
    (1, 256, 512, 64), (16, 8192, 1024, 128), (5, 6144, 768, 128),
    (16, 1024, 8192, 128), (3, 64, 256, 4), (9, 16384, 1024, 128)])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("bias,act", [(True, 0), (True, 1), (False, 0)])
def test_chunked_fused_vs_oracle(M, N, K, G, bits, bias, act):
    seed = M + 3 * N + 7 * K + G + bits
    x = W.randn_fp16((M, K), seed=seed, std=1.0)
    w = W.randn_fp16((N, K), seed=seed + 1, std=0.02)
    b = W.randn_fp16((N,), seed=seed + 2, std=0.5) if bias else None
    qx, sx = oracle.quant_tokens(x.numpy())
    q, sw = oracle.quantize_weights(w.numpy(), G, bits)
    d = dev()
    tq, tsx, tsw = _to_dev(qx), _to_dev(sx), _to_dev(sw)
    tb = None if b is None else b.to(d)
    fc = zq.gemm_w8a8_chunked if bits == 8 else zq.gemm_w4a8_chunked
    fr = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    y = fc(tq, tsx, _pack(q, bits), tsw, G, tb, act)
    y_rm = fr(tq, tsx, _to_dev(_rowmajor(q, bits)), tsw, G, tb, act)
    acc = oracle.gemm_i32(qx, q)
    z, _ = oracle.epilogue(acc, sx, sw, G, None if b is None else b.numpy(),
                           act)
    torch.cuda.synchronize()
    what = zq.gemm_chunked_plan(M, N, K, bits)
    assert_fp16_close_to_oracle(to_np(y), z, what)
    assert np.array_equal(to_np(y).view(np.uint16),
                          to_np(y_rm).view(np.uint16)), what


def test_chunked_rejects_what_it_cannot_run():
    d = dev()
    qx = torch.zeros(17, 1024, dtype=torch.int8, device=d)
    sx = torch.ones(17, device=d)
    qd = torch.zeros(256, 1024, dtype=torch.int8, device=d)
    sw = torch.ones(2, device=d)
    with pytest.raises(zq.ZQError, match="EUNSUPPORTED"):   # M > 16
        zq.gemm_w8a8_chunked(qx, sx, qd, sw, 128)
    b = torch.zeros(257, dtype=torch.float16, device=d)[1:]  # 2-byte aligned
    with pytest.raises(zq.ZQError, match="EINVAL"):
        zq.gemm_w8a8_chunked(qx[:4], sx[:4], qd, sw, 128, bias=b)
    with pytest.raises(zq.ZQError, match="EUNSUPPORTED"):   # N % 16 != 0
        zq.pack_chunked(torch.zeros(40, 256, dtype=torch.int8, device=d), 8)


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("wl,li", [("gptj-6b", 0), ("gptj-6b", 1),
                                   ("gptj-6b", 2), ("gptj-6b", 3),
                                   ("neox-20b", 0), ("neox-20b", 1),
                                   ("neox-20b", 2), ("neox-20b", 3)])
def test_chunked_decode_linears_full_size(wl, li, M):
    cfg = W.workload(wl)
    lin = cfg.linears[li]
    N, K, bits, G = lin.N, lin.K, lin.bits, cfg.G
    seed = 5000 + 10 * li + bits + M
    qx = _codes((M, K), -127, 127, seed)
    sx = (np.random.default_rng(seed + 1).random(M).astype(np.float32)
          * 0.05 + 1e-3)
    w = W.randn_fp16((N, K), seed=seed + 2, std=0.02)
    q, sw = oracle.quantize_weights(w.numpy(), G, bits)
    b = W.randn_fp16((N,), seed=seed + 3, std=0.01)
    act = 1 if lin.gelu else 0
    d = dev()
    tq, tsx, tsw, tb = _to_dev(qx), _to_dev(sx), _to_dev(sw), b.to(d)
    fc = zq.gemm_w8a8_chunked if bits == 8 else zq.gemm_w4a8_chunked
    fr = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    y = fc(tq, tsx, _pack(q, bits), tsw, G, tb, act)
    y_rm = fr(tq, tsx, _to_dev(_rowmajor(q, bits)), tsw, G, tb, act)
    cols = np.sort(np.random.default_rng(seed + 4).choice(N, 256,
                                                          replace=False))
    acc = oracle.gemm_i32(qx, np.ascontiguousarray(q[cols]))
    z = np.empty((M, cols.size), np.float64)
    for j, n in enumerate(cols):
        zz, _ = oracle.epilogue(acc[:, j:j + 1], sx, sw[n // G:n // G + 1], 1,
                                b.numpy()[n:n + 1], act)
        z[:, j] = zz[:, 0]
    torch.cuda.synchronize()
    yn = to_np(y)
    what = f"{wl} linear {li} " + zq.gemm_chunked_plan(M, N, K, bits)
    assert np.array_equal(yn.view(np.uint16), to_np(y_rm).view(np.uint16)), what
    assert_fp16_close_to_oracle(yn[:, cols], z, what)


@pytest.mark.parametrize("M", [1, 5, 16])
def test_chunked_chain_graph_and_eager_vs_oracle(M):
    """Two chunked-layout GEMMs (W8 with resident activations, then W4)
    recorded in a chain of 16 rows: the HIP graph and the native eager run
    over the first M rows give the same bits, within the oracle tolerance,
    and leave the rows past M untouched."""
    d = dev()
    G = 128
    lins = [(8, 8192, 1024, 0), (4, 2048, 2048, 1)]
    ch = zq.Chain(16)
    ref, outs = [], []
    for li, (bits, N, K, act) in enumerate(lins):
        x = W.randn_fp16((16, K), seed=70 + li, std=1.0)
        w = W.randn_fp16((N, K), seed=80 + li, std=0.02)
        b = W.randn_fp16((N,), seed=90 + li, std=0.5)
        qx, sx = oracle.quant_tokens(x.numpy())
        q, sw = oracle.quantize_weights(w.numpy(), G, bits)
        y = torch.full((16, N), 7.0, dtype=torch.float16, device=d)
        ch.gemm_chunked(_to_dev(qx), _to_dev(sx), _pack(q, bits), _to_dev(sw),
                        G, y, b.to(d), act)
        acc = oracle.gemm_i32(qx[:M], q)
        z, _ = oracle.epilogue(acc, sx[:M], sw, G, b.numpy(), act)
        ref.append(z)
        outs.append(y)
    ch.run(M)
    torch.cuda.synchronize()
    graph = [to_np(y).copy() for y in outs]
    for y in outs:
        y.fill_(7.0)
    ch.run_eager(M)
    torch.cuda.synchronize()
    for li, (y, g, z) in enumerate(zip(outs, graph, ref)):
        e = to_np(y)
        assert np.array_equal(e.view(np.uint16), g.view(np.uint16)), li
        assert_fp16_close_to_oracle(g[:M], z, f"chain linear {li}")
        assert (g[M:] == 7.0).all(), li


@pytest.mark.parametrize("bits", [8, 4])
def test_chunked_empty_m_is_a_no_op(bits):
    """No tokens: the calls succeed and write nothing."""
    d = dev()
    N, K, G = 256, 512, 64
    qd = _pack(np.zeros((N, K), np.int8), bits)
    qx = torch.empty(0, K, dtype=torch.int8, device=d)
    sx = torch.empty(0, dtype=torch.float32, device=d)
    sw = torch.ones(N // G, dtype=torch.float32, device=d)
    y = torch.full((1, N), 7.0, dtype=torch.float16, device=d)
    fc = zq.gemm_w8a8_chunked if bits == 8 else zq.gemm_w4a8_chunked
    fc(qx, sx, qd, sw, G, None, 0, y[:0])
    acc = zq.gemm_chunked_i32(bits, qx, qd)
    torch.cuda.synchronize()
    assert acc.shape == (0, N)
    assert (to_np(y) == 7.0).all()


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("bits", [8, 4])
def test_chunked_at_the_int32_bound(bits, M):
    """The largest K below the accumulator bound that the layout tiles
    (130816 = 511 chunks of 256 bytes; W4: 1022 chunks of 128), every code at
    its two's-complement extreme: |acc| reaches 128 * 128 * K, within 0.2%
    of 2^31 - 1, and must be exact."""
    K, N, G = 130816, 64, 32
    assert K <= 131008 and 128 * 128 * K <= 2 ** 31 - 1
    lo, hi = (-128, 127) if bits == 8 else (-8, 7)
    ts = np.where(np.arange(M) % 2 == 0, -128, 127).astype(np.int8)
    rs = np.where((np.arange(N) // 3) % 2 == 0, lo, hi).astype(np.int8)
    qx = np.repeat(ts[:, None], K, axis=1).astype(np.int8)
    q = np.repeat(rs[:, None], K, axis=1).astype(np.int8)
    sx = np.full(M, 1e-5, np.float32)
    sw = np.full(N // G, 1e-4 if bits == 8 else 1e-3, np.float32)
    tq, tsx, tsw = _to_dev(qx), _to_dev(sx), _to_dev(sw)
    qd = _pack(q, bits)
    acc = zq.gemm_chunked_i32(bits, tq, qd)
    fc = zq.gemm_w8a8_chunked if bits == 8 else zq.gemm_w4a8_chunked
    fr = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    y = fc(tq, tsx, qd, tsw, G, None, 0)
    y_rm = fr(tq, tsx, _to_dev(_rowmajor(q, bits)), tsw, G, None, 0)
    ref = oracle.gemm_i32(qx, q)
    torch.cuda.synchronize()
    what = zq.gemm_chunked_plan(M, N, K, bits)
    assert np.abs(ref.astype(np.int64)).max() == 128 * (-lo) * K
    assert np.array_equal(to_np(acc), ref), what
    assert np.array_equal(to_np(y).view(np.uint16),
                          to_np(y_rm).view(np.uint16)), what
