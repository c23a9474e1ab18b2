"""Seeded synthetic workloads for the fused quantized linear layer.

This module holds shapes and random inputs only -- none of the method's
arithmetic.  Both the HIP path's tests/benchmarks and the CPU oracle draw
their inputs from here, so both see identical bytes.

Five workloads (shapes from the ZeroQuant summary page, Sec. 5
"Experimental Analysis": BERT-base/large encoders, GPT-J-6B and GPT-NeoX-20B decoders;
W4/8 puts INT4 on the feed-forward weights and INT8 on attention weights,
Sec. 3.4 "Group-wise Weight Quantization"):

  0 ``single``      one linear, T=16, K=N=256, 64-row groups, W8
  1 ``bert-base``   4096 tokens, hidden 768, 64-row groups, all W8
  2 ``bert-large``  8192 tokens, hidden 1024, 64-row groups, FFN at W4
  3 ``gptj-6b``     M in {1,16,64,2048}, hidden 4096, 128-row groups, all W8
  4 ``neox-20b``    M in {1,16,2048}, hidden 6144, 128-row groups, FFN at W4

Value recipe (the pages' benchmarks use real data and trained weights, which
are stood in for by these draws):
  * weights ~ N(0, 0.02), bias ~ N(0, 0.01), drawn in fp32, cast to fp16;
  * activations ~ N(0, 1) with a fixed random subset of "outlier" feature
    channels multiplied by a factor (2 channels x20 for ``single``, 1% of K
    x20 for the BERT shapes, 0.5% of K x30 for the GPT shapes; at least 1);
  * LayerNorm gamma = 1, beta = 0, eps = 1e-5.
Seeds: weights and bias of linear l of workload c come from
``torch.Generator().manual_seed(100*c + l)`` (W first, then bias); the outlier
channels from seed ``100*c + l + 50_000``; the activations for the i-th M
value from seed ``100*c + l + 10_000*(i+1)``.
"""
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

__all__ = ["Linear", "Workload", "WORKLOADS", "workload", "gen_weights",
           "gen_activations", "outlier_channels", "randn_fp16", "layer_chain"]


@dataclass(frozen=True)
class Linear:
    name: str
    N: int          # output features (weight rows)
    K: int          # input features
    bits: int       # 8 or 4
    ln: bool        # input goes through LayerNorm + quantization
    gelu: bool      # GeLU in the epilogue


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    M: Tuple[int, ...]          # token counts (batch * seqlen)
    G: int                      # weight rows per quantization group
    linears: Tuple[Linear, ...]
    outlier_frac: Optional[float]
    outlier_count: Optional[int]
    outlier_factor: float
    ln_eps: float = 1e-5
    note: str = ""

    def n_outliers(self, K: int) -> int:
        if self.outlier_count is not None:
            return self.outlier_count
        return max(1, int(round(self.outlier_frac * K)))

    def seed(self, lin: int) -> int:
        return 100 * self.index + lin


def _encoder(h, ffn_bits):
    return (
        Linear("qkv", 3 * h, h, 8, True, False),
        Linear("attn_out", h, h, 8, False, False),
        Linear("ffn1", 4 * h, h, ffn_bits, True, True),
        Linear("ffn2", h, 4 * h, ffn_bits, False, False),
    )


WORKLOADS: Tuple[Workload, ...] = (
    Workload(0, "single", (16,), 64,
             (Linear("single", 256, 256, 8, True, False),),
             None, 2, 20.0),
    Workload(1, "bert-base", (4096,), 64, _encoder(768, 8), 0.01, None, 20.0,
             note="batch 32 x seq 128"),
    Workload(2, "bert-large", (8192,), 64, _encoder(1024, 4), 0.01, None, 20.0,
             note="batch 64 x seq 128; FFN weights INT4"),
    Workload(3, "gptj-6b", (1, 16, 64, 2048), 128, _encoder(4096, 8), 0.005,
             None, 30.0, note="decode M in {1,16,64}, prefill 2048"),
    Workload(4, "neox-20b", (1, 16, 2048), 128, _encoder(6144, 4), 0.005, None,
             30.0, note="decode M in {1,16}, prefill 2048; FFN weights INT4"),
)


def workload(key) -> Workload:
    if isinstance(key, int):
        return WORKLOADS[key]
    for w in WORKLOADS:
        if w.name == key:
            return w
    raise KeyError(key)


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(int(seed))


def gen_weights(wl: Workload, lin: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """fp16 W[N,K] ~ N(0, 0.02) and fp16 bias[N] ~ N(0, 0.01), on the CPU."""
    L = wl.linears[lin]
    g = _gen(wl.seed(lin))
    w = (torch.randn(L.N, L.K, generator=g) * 0.02).to(torch.float16)
    b = (torch.randn(L.N, generator=g) * 0.01).to(torch.float16)
    return w, b


def outlier_channels(wl: Workload, lin: int) -> torch.Tensor:
    L = wl.linears[lin]
    g = _gen(wl.seed(lin) + 50_000)
    return torch.randperm(L.K, generator=g)[: wl.n_outliers(L.K)]


def gen_activations(wl: Workload, lin: int, m_index: int = 0,
                    M: Optional[int] = None) -> torch.Tensor:
    """fp16 X[M,K] ~ N(0,1) with the workload's outlier channels scaled."""
    L = wl.linears[lin]
    M = wl.M[m_index] if M is None else M
    g = _gen(wl.seed(lin) + 10_000 * (m_index + 1))
    x = torch.randn(M, L.K, generator=g)
    x[:, outlier_channels(wl, lin)] *= wl.outlier_factor
    return x.to(torch.float16)


def randn_fp16(shape, seed: int, std: float = 1.0, mean: float = 0.0):
    """Generic seeded fp16 draw for edge-case tests."""
    g = _gen(seed)
    return (torch.randn(*shape, generator=g) * std + mean).to(torch.float16)


def layer_chain(wl: Workload, max_m: int, device, seed: int = 0,
                layers: int = 1, quant_on_load: bool = False):
    """The four linears of one encoder layer of ``wl`` over ``max_m`` tokens,
    recorded as a zq Chain: LN + token quantization -> QKV; token
    quantization -> attention output; LN + token quantization -> FFN1 (GeLU,
    output quantized for FFN2) -> FFN2.  The attention core and the residual
    adds lie outside the quantized linear path, so the attention context and
    the FFN block's input are seeded inputs of their own (N(0,1) with the
    workload's outlier channels, like the layer input).  Weights are the
    workload's, quantized on the device.  ``layers`` > 1 records the layer's
    calls that many times over the same weights and buffers (a stand-in for
    a model's stack of layers when timing launches).  ``quant_on_load``
    records attn-out and FFN2 as quantize-on-load calls instead (FFN1 writes
    its fp16 output to the start of ``ws``, where the quantized-output call
    keeps it, and FFN2 quantizes it; the codes and scales land in the same
    buffers): six calls per layer, the same results.  Returns (chain,
    buffers)."""
    from . import _lib as zq
    qkv, ao, f1, f2 = wl.linears
    h = qkv.K
    g = _gen(seed)

    def act(K):
        x = torch.randn(max_m, K, generator=g)
        x[:, torch.randperm(K, generator=g)[: wl.n_outliers(K)]] *= wl.outlier_factor
        return x.to(torch.float16).to(device)

    def lin(i):
        w, b = gen_weights(wl, i)
        qw, sw = zq.quantize_weights(w.to(device), wl.G, wl.linears[i].bits)
        return qw, sw, b.to(device)

    def empty(*shape, dtype=torch.float16):
        return torch.empty(*shape, dtype=dtype, device=device)

    B = {"x": act(h), "ctx": act(h), "h1": act(h),
         "gamma": (1.0 + 0.1 * torch.randn(h, generator=g)).half().to(device),
         "beta": (0.1 * torch.randn(h, generator=g)).half().to(device)}
    for i, L in enumerate(wl.linears):
        B[f"qw{i}"], B[f"sw{i}"], B[f"b{i}"] = lin(i)
    for i, K in enumerate((h, h, h, f2.K)):
        B[f"qx{i}"] = empty(max_m, K, dtype=torch.int8)
        B[f"sx{i}"] = empty(max_m, dtype=torch.float32)
    B["y_qkv"] = empty(max_m, qkv.N)
    B["y_ao"] = empty(max_m, ao.N)
    B["y_out"] = empty(max_m, f2.N)
    B["ws"] = empty(zq.gemm_quant_workspace_bytes(max_m, f1.N), dtype=torch.uint8)
    h2 = B["ws"].view(torch.float16)[: max_m * f1.N].view(max_m, f1.N)
    act1 = zq.ACT_GELU if f1.gelu else zq.ACT_NONE
    c = zq.Chain(max_m)
    for _ in range(layers):
        c.ln_quant(B["x"], B["qx0"], B["sx0"], B["gamma"], B["beta"], wl.ln_eps)
        c.gemm(B["qx0"], B["sx0"], B["qw0"], B["sw0"], wl.G, B["y_qkv"], B["b0"])
        if quant_on_load:
            c.gemm_xq(B["ctx"], B["qw1"], B["sw1"], wl.G, B["y_ao"], B["qx1"],
                      B["sx1"], B["b1"])
        else:
            c.quant(B["ctx"], B["qx1"], B["sx1"])
            c.gemm(B["qx1"], B["sx1"], B["qw1"], B["sw1"], wl.G, B["y_ao"],
                   B["b1"])
        c.ln_quant(B["h1"], B["qx2"], B["sx2"], B["gamma"], B["beta"], wl.ln_eps)
        if quant_on_load:
            c.gemm(B["qx2"], B["sx2"], B["qw2"], B["sw2"], wl.G, h2, B["b2"],
                   act1)
            c.gemm_xq(h2, B["qw3"], B["sw3"], wl.G, B["y_out"], B["qx3"],
                      B["sx3"], B["b3"])
        else:
            c.gemm_quant(B["qx2"], B["sx2"], B["qw2"], B["sw2"], wl.G, B["qx3"],
                         B["sx3"], B["ws"], B["b2"], act1)
            c.gemm(B["qx3"], B["sx3"], B["qw3"], B["sw3"], wl.G, B["y_out"],
                   B["b3"])
    return c, B
