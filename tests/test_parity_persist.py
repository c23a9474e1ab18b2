"""GPU parity of the persistent ping-pong kernel (one workgroup per compute
unit looping over 256 x 256 tiles, the copy ring running across tile
boundaries, two wave groups alternating between LDS reads and MFMAs; packed
W4 weights), forced through the schedule table:

* int32 accumulators bit-exact against the oracle's integer GEMM, with more
  tiles than compute units (workgroups that run several tiles), a ragged
  last token tile, and single-round problems;
* the fused epilogue (bias, GeLU) within 1 fp16 ulp + 1e-3 of the oracle's
  fp64 epilogue, and bit-identical to the plan the built-in rules pick;
* problems the kernel does not take whole (N not a multiple of 256, K with
  a half stage, groups smaller than a 32-column fragment, a 2-byte-aligned
  bias) run the same tile shape in the ordinary tiled kernel: same checks.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import int4_quantized_transformer_amd as zq
from int4_quantized_transformer_amd import workloads as W

from _util import assert_fp16_close_to_oracle, dev, needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]

CFGS = {4: (28,)}
STAGES = {28: (3, 128)}  # ring depth, k per stage
SHAPES = [  # (M, N, K, G)
    (300, 33280, 384, 128),    # 2 x 130 = 260 tiles: some workgroups run 2
    (2048, 10240, 512, 64),    # 8 x 40 = 320 tiles
    (256, 1024, 1024, 128),    # one round of 4 tiles
    (1000, 4096, 768, 64),     # ragged token tail, 64 tiles
]
ODD = [  # shapes the persistent kernel hands to the ordinary tiled kernel
    (300, 1000, 384, 8),       # N % 256 != 0, groups of 8
    (512, 2048, 576, 128),     # K % 128 == 64
    (512, 2048, 1024, 16),     # G < 32
]


@functools.lru_cache(maxsize=None)
def _case(M, N, K, G, bits):
    seed = M + 3 * N + 7 * K + bits
    x = W.randn_fp16((M, K), seed=seed, std=1.0)
    w = W.randn_fp16((N, K), seed=seed + 1, std=0.02)
    b = W.randn_fp16((N,), seed=seed + 2, std=0.5)
    qx, sx = oracle.quant_tokens(x.numpy())
    q, sw = oracle.quantize_weights(w.numpy(), G, bits)
    acc = oracle.gemm_i32(qx, q)
    z, _ = oracle.epilogue(acc, sx, sw, G, b.numpy(), 1)
    return qx, sx, q, sw, b, acc, z


def _force(bits, N, K, cfg):
    zq.sched_clear()
    zq.sched_import(f"{bits} {N} {K} 1 100000 tiled {cfg}\n")


@pytest.fixture(autouse=True)
def empty_table():
    zq.sched_clear()
    yield
    zq.sched_clear()


@pytest.mark.parametrize("M,N,K,G", SHAPES + ODD)
@pytest.mark.parametrize("bits", [4])
def test_persistent_configs_vs_oracle(M, N, K, G, bits):
    qx, sx, q, sw, b, acc_ref, z = _case(M, N, K, G, bits)
    qw = q if bits == 8 else oracle.pack_w4(q)
    d = dev()
    tqx, tsx = torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d)
    tqw, tsw, tb = torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), b.to(d)
    hook = zq.gemm_w8a8_i32 if bits == 8 else zq.gemm_w4a8_i32
    fn = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    y_default = to_np(fn(tqx, tsx, tqw, tsw, G, tb, 1))
    for cfg in CFGS[bits]:
        _force(bits, N, K, cfg)
        plan = zq.gemm_plan(M, N, K, bits)
        assert plan.startswith(f"tiled cfg={cfg} "), plan
        S, kps = STAGES[cfg]
        whole = N % 256 == 0 and K % kps == 0 and K // kps >= S
        assert ("persistent" in plan) == whole, plan
        acc = to_np(hook(tqx, tqw))
        assert np.array_equal(acc, acc_ref), plan
        y = to_np(fn(tqx, tsx, tqw, tsw, G, tb, 1))
        assert_fp16_close_to_oracle(y, z, plan)
        assert np.array_equal(y.view(np.uint16), y_default.view(np.uint16)), plan


@pytest.mark.parametrize("bits", [4])
@pytest.mark.parametrize("bias,act", [(False, 0), (True, 0), (False, 1)])
def test_persistent_epilogue_variants(bits, bias, act):
    M, N, K, G = 600, 2560, 512, 128
    qx, sx, q, sw, b, acc_ref, _ = _case(M, N, K, G, bits)
    z, _ = oracle.epilogue(acc_ref, sx, sw, G, b.numpy() if bias else None, act)
    qw = q if bits == 8 else oracle.pack_w4(q)
    d = dev()
    fn = zq.gemm_w8a8 if bits == 8 else zq.gemm_w4a8
    for cfg in CFGS[bits]:
        _force(bits, N, K, cfg)
        plan = zq.gemm_plan(M, N, K, bits)
        assert "persistent ping-pong" in plan, plan
        y = to_np(fn(torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
                     torch.from_numpy(qw).to(d), torch.from_numpy(sw).to(d), G,
                     b.to(d) if bias else None, act))
        assert_fp16_close_to_oracle(y, z, plan)


def test_persistent_with_2_byte_aligned_bias():
    # the kernel gathers bias pairs as words: a b[1:] view runs the ordinary
    # tiled kernel with the same tile shape
    M, N, K, G, bits = 512, 2048, 512, 128, 4
    qx, sx, q, sw, _, acc_ref, _ = _case(M, N, K, G, bits)
    b = W.randn_fp16((N + 1,), seed=99, std=0.5)
    z, _ = oracle.epilogue(acc_ref, sx, sw, G, b[1:].numpy(), 1)
    d = dev()
    bd = b.to(d)[1:]
    assert bd.data_ptr() % 4 == 2
    _force(bits, N, K, 28)
    y = to_np(zq.gemm_w4a8(torch.from_numpy(qx).to(d), torch.from_numpy(sx).to(d),
                           torch.from_numpy(oracle.pack_w4(q)).to(d),
                           torch.from_numpy(sw).to(d), G, bd, 1))
    assert_fp16_close_to_oracle(y, z, zq.gemm_plan(M, N, K, bits))


def test_wide_w4_prefill_takes_the_ping_pong_kernel():
    # the built-in rule: packed W4 over N >= 16384 with K >= 4096 (the
    # GPT-NeoX-20B FFN1 shape); N = 6144 (FFN2) keeps the 192 x 256 tiles
    assert "ping-pong" in zq.gemm_plan(2048, 24576, 6144, 4)
    assert zq.gemm_plan(2048, 6144, 24576, 4).startswith("tiled cfg=13 ")
    assert "ping-pong" not in zq.gemm_plan(2048, 24576, 6144, 8)
