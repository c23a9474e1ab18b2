"""Parity at the full sizes of the five synthetic workloads, through the
same C-ABI calls (and therefore the same kernels and launch configurations)
that bench.py times.

For every linear of every workload and every token count M:
  * weights: zq_quantize_weights codes / packed bytes / scales bit-exact
    against the oracle on the whole matrix;
  * activations: LayerNorm + token quantization (QKV, FFN1 inputs) or plain
    token quantization (attn-out, FFN2 inputs) on the whole [M, K] input,
    checked as in test_parity_quant (bit-exact codes on the oracle's own
    fp16 values; +-1 code in <= 0.1% after the fused LayerNorm);
  * GEMM: the fused call over the whole problem, with sampled token rows
    (all rows when M <= 64) compared with the oracle's int32 GEMM and fp64
    epilogue computed on the same quantized inputs (1 fp16 ulp + 1e-3), and
    the raw int32 hook bit-exact on the same rows;
  * the linears without LayerNorm (attn-out, FFN2) also through the
    quantize-on-load call on the fp16 input: codes, scales and y
    bit-identical to the quantizer followed by the fused GEMM (one kernel
    at one token).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import int4_quantized_transformer_amd as zq
from int4_quantized_transformer_amd import workloads as W

from _util import (assert_codes_within_one, assert_fp16_close_to_oracle, dev,
                   needs_gpu, to_np)

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [(wl.index, li, mi) for wl in W.WORKLOADS
         for li in range(len(wl.linears)) for mi in range(len(wl.M))]


@functools.lru_cache(maxsize=1)
def _weights(wi, li):
    wl = W.workload(wi)
    L = wl.linears[li]
    w, b = W.gen_weights(wl, li)
    q_ref, sw_ref = oracle.quantize_weights(w.numpy(), wl.G, L.bits)
    qw, sw = zq.quantize_weights(w.to(dev()), wl.G, L.bits)
    return w, b, q_ref, sw_ref, qw, sw


def _rows(M, seed):
    if M <= 64:
        return np.arange(M)
    g = np.random.default_rng(seed)
    pick = g.choice(M, size=30, replace=False)
    return np.unique(np.concatenate([[0, 1, M - 1], pick]))


@pytest.mark.parametrize("wi,li,mi", CASES,
                         ids=[f"{W.workload(a).name}-{W.workload(a).linears[b].name}"
                              f"-M{W.workload(a).M[c]}" for a, b, c in CASES])
def test_workload_linear(wi, li, mi):
    wl = W.workload(wi)
    L = wl.linears[li]
    M = wl.M[mi]
    d = dev()
    w, b, q_ref, sw_ref, qw, sw = _weights(wi, li)

    # ---- weights (checked once per linear, at the first token count)
    if mi == 0:
        torch.cuda.synchronize()
        assert np.array_equal(to_np(sw), sw_ref)
        got = to_np(qw)
        exp = q_ref if L.bits == 8 else oracle.pack_w4(q_ref)
        assert np.array_equal(got, exp)

    # ---- activations
    x = W.gen_activations(wl, li, m_index=mi)
    xd = x.to(d)
    if L.ln:
        qx, sx = zq.ln_quant_act(xd, None, None, wl.ln_eps)
        h_ref = oracle.layernorm(x.numpy(), None, None, wl.ln_eps)
    else:
        qx, sx = zq.quant_act(xd)
        h_ref = x.numpy()
    qx_ref, sx_ref = oracle.quant_tokens(h_ref)
    torch.cuda.synchronize()
    qx_np, sx_np = to_np(qx), to_np(sx)
    if L.ln:
        assert_codes_within_one(qx_np, qx_ref, 1e-3, "ln_quant qx")
        assert np.allclose(sx_np, sx_ref, rtol=2e-3, atol=0)
        # the same quantizer on the oracle's LayerNorm output: bit-exact
        qx2, sx2 = zq.quant_act(torch.from_numpy(h_ref).to(d))
        torch.cuda.synchronize()
        assert np.array_equal(to_np(qx2), qx_ref)
        assert np.array_equal(to_np(sx2), sx_ref)
    else:
        assert np.array_equal(qx_np, qx_ref)
        assert np.array_equal(sx_np, sx_ref)

    # ---- GEMM over the whole problem, compared on sampled rows
    fused = zq.gemm_w8a8 if L.bits == 8 else zq.gemm_w4a8
    raw = zq.gemm_w8a8_i32 if L.bits == 8 else zq.gemm_w4a8_i32
    y = fused(qx, sx, qw, sw, wl.G, b.to(d), int(L.gelu))
    acc = raw(qx, qw)
    torch.cuda.synchronize()
    rows = _rows(M, 1000 * wi + 10 * li + mi)
    ridx = torch.from_numpy(rows).to(d)
    acc_ref = oracle.gemm_i32(qx_np[rows], q_ref)
    assert np.array_equal(to_np(acc[ridx]), acc_ref), zq.gemm_plan(M, L.N, L.K, L.bits)
    z, _ = oracle.epilogue(acc_ref, sx_np[rows], sw_ref, wl.G, b.numpy(),
                           int(L.gelu))
    assert_fp16_close_to_oracle(to_np(y[ridx]), z,
                                f"{wl.name}.{L.name} M={M} "
                                f"{zq.gemm_plan(M, L.N, L.K, L.bits)}")

    # ---- the quantize-on-load call on the fp16 input (linears without
    # LayerNorm): codes, scales and y bit-identical to the two calls above
    if not L.ln:
        xq = zq.gemm_w8a8_xq if L.bits == 8 else zq.gemm_w4a8_xq
        yq, qxq, sxq = xq(xd, qw, sw, wl.G, b.to(d), int(L.gelu))
        torch.cuda.synchronize()
        plan = zq.gemm_xq_plan(M, L.N, L.K, L.bits)
        assert np.array_equal(to_np(sxq), sx_np), plan
        assert np.array_equal(to_np(qxq), qx_np), plan
        assert np.array_equal(to_np(yq).view(np.uint16),
                              to_np(y).view(np.uint16)), plan
