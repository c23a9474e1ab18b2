"""GPU end to end against the oracle end to end: the fused LayerNorm +
token quantization on the GPU feeding the GPU GEMM, against the oracle's
LayerNorm, quantizer, integer GEMM and fp64 epilogue.

The fused LN+quant may move a code by one where the fp16 LayerNorm output
sits at a rounding boundary (at most 0.1% of codes, checked elsewhere), and
its scale may differ from the oracle's within 2e-3.  With qx' - qx in
{-1, 0, 1} at the flipped positions F of token t, the accumulators differ by
at most D[t, n] = sum over k in F of |qw[n, k]|, so for the linear epilogue

    |y_gpu - z_oracle| <= sw * (sx_gpu * D + |sx_gpu - sx_oracle| * |acc|)
                          + 1 fp16 ulp + 1e-3

and with GeLU the same bound times GeLU's Lipschitz constant (under 1.13).
Every output must lie within that bound, which the test computes exactly
from the two sides' codes."""
import numpy as np
import pytest
import torch

import oracle
import int4_quantized_transformer_amd as zq
from int4_quantized_transformer_amd import workloads as W

from _util import dev, fp16_ulp, needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]

GELU_LIP = 1.13


@pytest.mark.parametrize("name,li,rows", [
    ("single", 0, None),           # the whole of the one-linear workload
    ("bert-base", 0, 48),          # QKV, sampled token rows
    ("bert-base", 2, 48),          # FFN1 with GeLU
    ("bert-large", 2, 32),         # FFN1, W4 weights
    ("neox-20b", 2, 8),            # FFN1 W4, 2048 tokens
])
def test_end_to_end_within_derived_bound(name, li, rows):
    wl = W.workload(name)
    L = wl.linears[li]
    assert L.ln
    M = wl.M[-1]
    w, b = W.gen_weights(wl, li)
    x = W.gen_activations(wl, li, M=M, m_index=len(wl.M) - 1)
    d = dev()
    qw, sw = zq.quantize_weights(w.to(d), wl.G, L.bits)
    qx_g, sx_g = zq.ln_quant_act(x.to(d), eps=wl.ln_eps)
    g8 = zq.gemm_w8a8 if L.bits == 8 else zq.gemm_w4a8
    act = zq.ACT_GELU if L.gelu else zq.ACT_NONE
    y_g = g8(qx_g, sx_g, qw, sw, wl.G, b.to(d), act)
    torch.cuda.synchronize()

    if rows is None:
        sel = np.arange(M)
    else:
        g = np.random.default_rng(M + li)
        sel = np.unique(np.concatenate([[0, M - 1], g.choice(M, rows, replace=False)]))
    xs = x.numpy()[sel]
    q, sw_o = oracle.quantize_weights(w.numpy(), wl.G, L.bits)
    h = oracle.layernorm(xs, None, None, wl.ln_eps)
    qx_o, sx_o = oracle.quant_tokens(h)
    acc_o = oracle.gemm_i32(qx_o, q).astype(np.float64)
    z, _ = oracle.epilogue(acc_o.astype(np.int32), sx_o, sw_o, wl.G, b.numpy(), act)

    qg = to_np(qx_g)[sel].astype(np.int32)
    sxg = to_np(sx_g)[sel].astype(np.float64)
    flips = np.abs(qg - qx_o.astype(np.int32))
    assert flips.max() <= 1
    D = flips.astype(np.float64) @ np.abs(q.astype(np.float64)).T
    swn = np.repeat(sw_o.astype(np.float64), wl.G)[None, :]
    bound = swn * (sxg[:, None] * D
                   + np.abs(sxg - sx_o.astype(np.float64))[:, None] * np.abs(acc_o))
    if act == zq.ACT_GELU:
        bound *= GELU_LIP
    bound += fp16_ulp(z) + 1e-3
    err = np.abs(to_np(y_g)[sel].astype(np.float64) - z)
    bad = err > bound
    assert not bad.any(), (
        f"{bad.sum()} of {bad.size} outside the derived bound; worst excess "
        f"{(err - bound).max():.3g}; {int((flips != 0).sum())} flipped codes")
