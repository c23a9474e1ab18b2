"""GPU parity of the INT8 GEMMs against the CPU oracle.

* zq_gemm_{w8a8,w4a8}_i32 on the oracle's codes: int32 accumulators
  bit-exact, over shapes that cover every kernel (GEMV, streaming rings of
  1 / 16 / 32 / 64 token rows with 16- and 32-row blocks, skinny for odd N,
  tiled), ragged M/N tails, several k-tiles, K % 128 == 64, and extreme
  codes.
* zq_gemm_{w8a8,w4a8}: fp16 outputs within 1 fp16 ulp + 1e-3 of the
  oracle's fp64 epilogue, with and without bias and GeLU.
* The same fp16 bits from every kernel (GEMV, streaming, skinny, tiled) for
  a token, and the linear epilogue correctly rounded (acc * fl32(sx * sw)
  + b, one rounding to fp16).
"""
import numpy as np
import pytest
import torch

import oracle
import int4_quantized_transformer_amd as zq
from int4_quantized_transformer_amd import workloads as W

from _util import assert_fp16_close_to_oracle, dev, needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]

SHAPES = [  # (M, N, K)
    (1, 16, 64), (1, 200, 192), (16, 256, 256), (17, 320, 192),
    (33, 48, 640), (63, 64, 64), (64, 4096, 128), (64, 100, 1024),
    (65, 320, 576), (128, 128, 128), (200, 384, 1024), (257, 200, 64),
    (300, 1000, 640), (512, 768, 3072), (1, 4096, 4096), (7, 64, 24576),
    (1, 1000, 1024), (1, 77, 2048), (1, 3000, 8192), (16, 24, 2048),
    (40, 8200, 384), (64, 12288, 256),
    # 17 .. 64 tokens: rings of 32 / 64 token rows, 16-row blocks (N <= 4096)
    # and 32-row blocks with a ragged last block, K tails; odd N: skinny
    (64, 4098, 640), (20, 6144, 1088), (48, 200, 4160), (33, 4096, 2048),
    (40, 77, 1024),
    # up to 16 tokens, 4096 < N <= 8192: W8 rings of 32-row blocks
    (16, 6144, 512), (9, 8190, 1088),
]


def _codes(shape, lo, hi, seed):
    g = np.random.default_rng(seed)
    return g.integers(lo, hi + 1, size=shape).astype(np.int8)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_i32_w8a8_bit_exact(M, N, K):
    qx = _codes((M, K), -127, 127, M * 7 + K)
    qw = _codes((N, K), -127, 127, N * 11 + K)
    acc = zq.gemm_w8a8_i32(torch.from_numpy(qx).to(dev()),
                           torch.from_numpy(qw).to(dev()))
    ref = oracle.gemm_i32(qx, qw)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(acc), ref), zq.gemm_plan(M, N, K, 8)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_i32_w4a8_bit_exact(M, N, K):
    qx = _codes((M, K), -127, 127, M * 5 + K)
    q4 = _codes((N, K), -8, 7, N * 13 + K)     # full nibble range incl. -8
    packed = oracle.pack_w4(q4)
    acc = zq.gemm_w4a8_i32(torch.from_numpy(qx).to(dev()),
                           torch.from_numpy(packed).to(dev()))
    ref = oracle.gemm_i32(qx, q4)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(acc), ref), zq.gemm_plan(M, N, K, 4)


@pytest.mark.parametrize("M", [1, 16, 64, 130])
@pytest.mark.parametrize("bits", [8, 4])
def test_i32_extreme_codes(M, bits):
    # every product at its maximum magnitude: |acc| = K*127*qmax
    K, N = 24576, 64
    qmax = 127 if bits == 8 else 7
    qx = np.full((M, K), 127, np.int8)
    qx[::2] = -127
    q = np.full((N, K), qmax, np.int8)
    q[1::2] = -qmax if bits == 8 else -8
    qw = q if bits == 8 else oracle.pack_w4(q)
    fn = zq.gemm_w8a8_i32 if bits == 8 else zq.gemm_w4a8_i32
    acc = fn(torch.from_numpy(qx).to(dev()), torch.from_numpy(qw).to(dev()))
    ref = oracle.gemm_i32(qx, q)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(acc), ref)


@pytest.mark.parametrize("M,N,K,G", [
    (16, 256, 256, 64), (1, 4096, 1024, 128), (5, 384, 768, 128),
    (64, 512, 512, 64), (100, 320, 192, 64), (300, 768, 768, 64),
    (257, 1000, 320, 8), (2048, 256, 512, 128), (3, 20, 64, 4),
    (1, 2048, 4096, 64), (1, 72, 2048, 8), (48, 8192, 512, 128)])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("bias,act", [(True, 0), (True, 1), (False, 1),
                                      (False, 0)])
def test_fused_epilogue_vs_oracle(M, N, K, G, bits, bias, act):
    seed = M + 3 * N + 7 * K + G + bits
    x = W.randn_fp16((M, K), seed=seed, std=1.0)
    w = W.randn_fp16((N, K), seed=seed + 1, std=0.02)
    b = W.randn_fp16((N,), seed=seed + 2, std=0.5) if bias else None
    qx, sx = oracle.quant_tokens(x.numpy())
    q, sw = oracle.quantize_weights(w.numpy(), G, bits)
    qw = q if bits == 8 else oracle.pack_w4(q)
    d = dev()
    fn = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    y = fn(torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
           torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), G,
           None if b is None else b.to(d), act)
    acc = oracle.gemm_i32(qx, q)
    z, _ = oracle.epilogue(acc, sx, sw, G, None if b is None else b.numpy(),
                           act)
    torch.cuda.synchronize()
    assert_fp16_close_to_oracle(to_np(y), z, zq.gemm_plan(M, N, K, bits))


def test_empty_m_is_a_no_op():
    d = dev()
    qx = torch.empty(0, 128, dtype=torch.int8, device=d)
    qw = torch.zeros(64, 128, dtype=torch.int8, device=d)
    acc = zq.gemm_w8a8_i32(qx, qw)
    assert acc.shape == (0, 64)


def test_plans_used_by_tests_cover_every_kernel():
    for bits in (8, 4):
        plans = {zq.gemm_plan(M, N, K, bits).split()[0] for M, N, K in SHAPES}
        assert plans == {"gemv", "stream", "skinny", "tiled"}, bits


@pytest.mark.parametrize("M", [40, 256])
@pytest.mark.parametrize("bits", [8, 4])
def test_gelu_epilogue_dense_range(M, bits):
    # acc[t,n] = 127 * qw[n,0] (one-hot tokens); with sw = 1/127 and
    # sx[t] = 0.002 (t+1) the epilogue input z covers about [-8, 8] densely
    K, N, G = 128, 256, 64
    qmax = 127 if bits == 8 else 7
    qx = np.zeros((M, K), np.int8)
    qx[:, 0] = 127
    q = np.zeros((N, K), np.int8)
    q[:, 0] = np.clip(np.round(np.linspace(-qmax, qmax, N)), -qmax, qmax)
    qw = q if bits == 8 else oracle.pack_w4(q)
    sx = (0.002 * (np.arange(M) + 1) * (127 / qmax) * (64 / M)).astype(np.float32)
    sw = np.full(N // G, 1 / 127, np.float32)
    d = dev()
    fn = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    y = fn(torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
           torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), G, None, 1)
    z, _ = oracle.epilogue(oracle.gemm_i32(qx, q), sx, sw, G, None, 1)
    torch.cuda.synchronize()
    assert np.abs(z).max() > 7.5
    assert_fp16_close_to_oracle(to_np(y), z, zq.gemm_plan(M, N, K, bits))


def _epilogue_inputs(M, N, K, G, bits, seed):
    x = W.randn_fp16((M, K), seed=seed, std=1.0)
    w = W.randn_fp16((N, K), seed=seed + 1, std=0.02)
    b = W.randn_fp16((N,), seed=seed + 2, std=0.5)
    qx, sx = oracle.quant_tokens(x.numpy())
    q, sw = oracle.quantize_weights(w.numpy(), G, bits)
    qw = q if bits == 8 else oracle.pack_w4(q)
    return qx, sx, q, qw, sw, b


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("act", [0, 1])
def test_output_bits_do_not_depend_on_plan(bits, act):
    # a row of y depends only on that token's codes and scale, so rows
    # computed by the one-token GEMV, the streaming rings (16, 20 and 40
    # tokens), the skinny kernel (40 tokens, forced through the schedule
    # table) and the tiled (256 tokens) kernels must be the same bits
    N, K, G = 512, 2048, 64
    qx, sx, q, qw, sw, b = _epilogue_inputs(256, N, K, G, bits, 97 + bits + act)
    d = dev()
    fn = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    tqw, tsw, tb = torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), b.to(d)

    def run(r0, r1):
        return fn(torch.from_numpy(qx[r0:r1]).to(d),
                  torch.from_numpy(sx[r0:r1]).to(d), tqw, tsw, G, tb, act)

    assert zq.gemm_plan(256, N, K, bits).startswith("tiled")
    full = to_np(run(0, 256))
    for (r0, r1, plan) in [(5, 6, "gemv"), (200, 201, "gemv"), (16, 32, "stream"),
                           (100, 120, "stream BN=16 MX=32"),
                           (100, 140, "stream BN=16 MX=64"), (100, 140, "skinny")]:
        if plan == "skinny":
            zq.sched_import(f"{bits} {N} {K} 17 64 skinny 0\n")
        try:
            assert zq.gemm_plan(r1 - r0, N, K, bits).startswith(plan)
            part = to_np(run(r0, r1))
        finally:
            zq.sched_clear()
        assert np.array_equal(part.view(np.uint16), full[r0:r1].view(np.uint16)), plan


@pytest.mark.parametrize("M", [1, 16, 40, 300])
@pytest.mark.parametrize("bits", [8, 4])
def test_linear_epilogue_is_correctly_rounded(M, bits):
    # without an activation each output is acc * fl32(sx * sw) + b rounded
    # once to the nearest fp16 (ties to even).  In fp64 the product is exact
    # (|acc| < 2^25, 24-bit scale) and the sum is within 2^-53 relative of
    # the exact value, which moves the fp16 rounding only for a value that
    # close to an fp16 tie; numpy's fp64 -> fp16 conversion rounds
    # correctly (once, not through fp32)
    N, K, G = 384, 2048, 64
    qx, sx, q, qw, sw, b = _epilogue_inputs(M, N, K, G, bits, 31 * M + bits)
    d = dev()
    fn = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    y = fn(torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
           torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), G, b.to(d), 0)
    acc = oracle.gemm_i32(qx, q).astype(np.float64)
    sc = (sx[:, None] * np.repeat(sw, G)[None, :]).astype(np.float32)
    assert sc.dtype == np.float32 and sx.dtype == np.float32
    ref = (acc * sc.astype(np.float64) + b.numpy().astype(np.float64)).astype(np.float16)
    torch.cuda.synchronize()
    got = to_np(y)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), \
        (zq.gemm_plan(M, N, K, bits), int((got != ref).sum()))


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M", [1, 16, 40, 100])
def test_gemm_at_the_int32_bound(bits, M):
    # K = ZQ_MAX_GEMM_K_W8/W4 = 131008 with every code at its two's-complement
    # extreme (-128 for int8 activations and W8 weights, -8 for nibbles):
    # the W8 sum reaches 128 * 128 * K and the W4 path's 16 * acc reaches
    # 16 * 8 * 128 * K, both within 2^31 - 1 by 0.05%.  Token signs and
    # weight-row signs vary so both the largest positive and the largest
    # negative sums occur.
    K = 131008
    assert K * 16384 <= 2 ** 31 - 1 < (K + 64) * 16384
    lo, hi = (-128, 127) if bits == 8 else (-8, 7)
    N, G = 64, 32
    ts = np.where(np.arange(M) % 2 == 0, -128, 127).astype(np.int8)
    rs = np.where((np.arange(N) // 3) % 2 == 0, lo, hi).astype(np.int8)
    qx = np.repeat(ts[:, None], K, axis=1).astype(np.int8)
    q = np.repeat(rs[:, None], K, axis=1).astype(np.int8)
    qw = q if bits == 8 else oracle.pack_w4(q)
    sx = np.full(M, 1e-5, np.float32)
    sw = np.full(N // G, 1e-4 if bits == 8 else 1e-3, np.float32)
    d = dev()
    tqx, tqw = torch.from_numpy(qx).to(d), torch.from_numpy(qw).to(d)
    tsx, tsw = torch.from_numpy(sx).to(d), torch.from_numpy(sw).to(d)
    hook = zq.gemm_w8a8_i32 if bits == 8 else zq.gemm_w4a8_i32
    fn = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    fws = zq.gemm_w8a8_ws if bits == 8 else zq.gemm_w4a8_ws
    acc = to_np(hook(tqx, tqw))
    y = to_np(fn(tqx, tsx, tqw, tsw, G, None, 0))
    y_ws = to_np(fws(tqx, tsx, tqw, tsw, G, None, 0))
    ref = oracle.gemm_i32(qx, q)
    assert np.abs(ref.astype(np.int64)).max() == 128 * (-lo) * K
    assert np.array_equal(acc, ref), zq.gemm_plan(M, N, K, bits)
    z, _ = oracle.epilogue(ref, sx, sw, G, None, 0)
    assert_fp16_close_to_oracle(y, z, zq.gemm_plan(M, N, K, bits))
    assert np.array_equal(y_ws.view(np.uint16), y.view(np.uint16))


def _fused_inputs(M, N, K, G, bits, seed):
    x = W.randn_fp16((M, K), seed=seed, std=1.0)
    w = W.randn_fp16((N, K), seed=seed + 1, std=0.02)
    b = W.randn_fp16((N + 1,), seed=seed + 2, std=0.5)
    qx, sx = oracle.quant_tokens(x.numpy())
    q, sw = oracle.quantize_weights(w.numpy(), G, bits)
    qw = q if bits == 8 else oracle.pack_w4(q)
    return qx, sx, q, qw, sw, b


@pytest.mark.parametrize("act", [0, 1])
def test_w8_ring_with_32_row_blocks_fused_vs_oracle_and_tiles(act, empty_table):
    # 16 tokens over 4096 < N <= 8192: the W8 ring of 32-row blocks (two row
    # fragments per block share the gathered group scales and bias pairs).
    # Its fp16 output against the oracle, and bit-identical to the same rows
    # from the tiled kernel (forced through the schedule table).
    M, N, K, G = 16, 6144, 512, 128
    qx, sx, q, qw, sw, b = _fused_inputs(M, N, K, G, 8, 4242 + act)
    assert zq.gemm_plan(M, N, K, 8).startswith("stream BN=32 MX=16")
    d = dev()
    args = (torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
            torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), G,
            b[:N].to(d), act)
    y = to_np(zq.gemm_w8a8(*args))
    z, _ = oracle.epilogue(oracle.gemm_i32(qx, q), sx, sw, G, b[:N].numpy(), act)
    assert_fp16_close_to_oracle(y, z, zq.gemm_plan(M, N, K, 8))
    zq.sched_import(f"8 {N} {K} 1 64 tiled 22\n")
    assert zq.gemm_plan(M, N, K, 8).startswith("tiled cfg=22")
    y_t = to_np(zq.gemm_w8a8(*args))
    assert np.array_equal(y.view(np.uint16), y_t.view(np.uint16))


@pytest.mark.parametrize("M,N,K,bits", [(16, 6144, 512, 8), (16, 4096, 1024, 8),
                                        (9, 2048, 1024, 4), (1, 1000, 1024, 8),
                                        (40, 4098, 640, 8), (300, 1000, 640, 8)])
def test_bias_only_2_byte_aligned(M, N, K, bits):
    # a bias view that starts 2 bytes into its allocation (b[1:]); the ring
    # kernels read bias pairs as 4-byte words when they can and per element
    # otherwise
    G = 8 if N % 8 == 0 else 2
    qx, sx, q, qw, sw, b = _fused_inputs(M, N, K, G, bits, 77 * M + N)
    d = dev()
    bd = b.to(d)[1:]
    assert bd.data_ptr() % 4 == 2
    fn = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    y = to_np(fn(torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
                 torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), G,
                 bd, 1))
    z, _ = oracle.epilogue(oracle.gemm_i32(qx, q), sx, sw, G, b[1:].numpy(), 1)
    assert_fp16_close_to_oracle(y, z, zq.gemm_plan(M, N, K, bits))


@pytest.fixture
def empty_table():
    zq.sched_clear()
    yield
    zq.sched_clear()


# Rings of 2 .. 16 token rows with resident activations: every workgroup
# takes at least two row blocks, so each wave copies the activations of its
# K-chunks once.  Shapes: both resident variants (2 chunks of 512 weight
# bytes per wave, 6 of 256), a partial last chunk (K % 512 or K % 256 != 0
# for W8, half chunks for W4), waves without chunks (K of one or two
# chunks), ragged last row block, M < 16.
RESIDENT = [  # (M, N, K, bits, chunks per wave held)
    (16, 8192, 4096, 8, 2), (9, 8200, 4160, 8, 6), (2, 12288, 6144, 8, 6),
    (16, 8192, 512, 8, 2), (5, 8194, 64, 8, 2), (3, 8192, 1600, 8, 2),
    (16, 16384, 6144, 4, 6), (7, 16400, 1088, 4, 2), (16, 16384, 256, 4, 2),
    (12, 16416, 4096, 4, 2), (8, 16384, 4224, 4, 6)]


@pytest.mark.parametrize("M,N,K,bits,xr", RESIDENT)
def test_resident_ring_i32_bit_exact(M, N, K, bits, xr):
    plan = zq.gemm_plan(M, N, K, bits)
    assert plan.startswith("stream") and f"xres={xr}" in plan, plan
    qx = _codes((M, K), -127, 127, M * 3 + K + bits)
    if bits == 8:
        q = _codes((N, K), -127, 127, N + 5 * K)
        qw = q
        fn = zq.gemm_w8a8_i32
    else:
        q = _codes((N, K), -8, 7, N + 9 * K)
        qw = oracle.pack_w4(q)
        fn = zq.gemm_w4a8_i32
    acc = fn(torch.from_numpy(qx).to(dev()), torch.from_numpy(qw).to(dev()))
    ref = oracle.gemm_i32(qx, q)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(acc), ref), plan


@pytest.mark.parametrize("M,N,K,bits", [(16, 8192, 4160, 8), (11, 16384, 2048, 4)])
@pytest.mark.parametrize("act", [0, 1])
def test_resident_ring_fused_vs_oracle_and_tiles(M, N, K, bits, act, empty_table):
    # the fused epilogue of the resident ring against the oracle, and bit
    # for bit the rows the tiled kernel gives (forced through the table)
    G = 128
    qx, sx, q, qw, sw, b = _fused_inputs(M, N, K, G, bits, 31 * M + K + act)
    assert "xres=" in zq.gemm_plan(M, N, K, bits)
    d = dev()
    fn = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    args = (torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
            torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), G,
            b[:N].to(d), act)
    y = to_np(fn(*args))
    z, _ = oracle.epilogue(oracle.gemm_i32(qx, q), sx, sw, G, b[:N].numpy(), act)
    assert_fp16_close_to_oracle(y, z, zq.gemm_plan(M, N, K, bits))
    zq.sched_import(f"{bits} {N} {K} 1 64 tiled 22\n")
    assert zq.gemm_plan(M, N, K, bits).startswith("tiled cfg=22")
    y_t = to_np(fn(*args))
    assert np.array_equal(y.view(np.uint16), y_t.view(np.uint16))
