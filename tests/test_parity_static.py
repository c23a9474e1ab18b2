"""GPU parity of the static per-tensor activation quantizer (the prior-PTQ
comparator: a moving-average calibrated range, one frozen scale).

* Calibration: after each of several seeded batches the device state
  {x_min, x_max} equals the oracle's bit for bit (min/max are exact; the
  moving average uses the same fp32 operations).
* Quantization: codes and S equal the oracle's for the same state, including
  a batch that exceeds the calibrated range (codes clamp to +-127), a ragged
  K and a misaligned tensor (the scalar path).
* Reduction: with the range (-a, a) of a single token the codes equal the
  token-wise quantizer's.
"""
import numpy as np
import pytest
import torch

import oracle
import int4_quantized_transformer_amd as zq
from int4_quantized_transformer_amd import workloads as W

from _util import dev, needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def _batch(M, K, seed, scale=1.0):
    x = W.randn_fp16((M, K), seed=seed).float() * scale
    g = torch.Generator().manual_seed(seed + 1)
    ch = torch.randperm(K, generator=g)[: max(1, K // 100)]
    x[:, ch] *= 20.0
    return x.half()


@pytest.mark.parametrize("M,K", [(512, 768), (33, 1000), (7, 13)])
def test_calibration_and_quantization_match_oracle(M, K):
    d = dev()
    st_ref = None
    st = None
    for i in range(5):
        x = _batch(M, K, 100 * M + i)
        st_ref = oracle.calibrate_minmax(x.numpy(), st_ref)
        st = zq.calibrate_minmax(x.to(d), st)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(st), st_ref), i
    for scale in (1.0, 3.0):            # 3.0: beyond the calibrated range
        x = _batch(M, K, 7 * M + K, scale)
        q, s = zq.quant_act_static(x.to(d), st)
        q_ref, s_ref = oracle.quant_static(x.numpy(), st_ref)
        torch.cuda.synchronize()
        assert to_np(s)[0] == s_ref
        assert np.array_equal(to_np(q), q_ref)
        if scale > 1.0:
            assert np.abs(q_ref).max() == 127


def test_static_quantizer_misaligned_tensor():
    d = dev()
    x = _batch(64, 257, 3)
    st = zq.calibrate_minmax(x.to(d))
    base = torch.empty(64 * 257 + 1, dtype=torch.float16, device=d)
    base[1:] = x.to(d).flatten()
    xm = base[1:].view(64, 257)             # 2-byte aligned, not 16
    q, s = zq.quant_act_static(xm, st)
    q_ref, s_ref = oracle.quant_static(x.numpy(), to_np(st))
    torch.cuda.synchronize()
    assert to_np(s)[0] == s_ref
    assert np.array_equal(to_np(q), q_ref)


def test_static_reduces_to_token_wise_for_one_token():
    d = dev()
    x = _batch(1, 1024, 9)
    a = float(np.abs(x.numpy().astype(np.float32)).max())
    st = torch.tensor([-a, a], dtype=torch.float32, device=d)
    q, s = zq.quant_act_static(x.to(d), st)
    qt, st_ = zq.quant_act(x.to(d))
    torch.cuda.synchronize()
    assert to_np(s)[0] == to_np(st_)[0]
    assert torch.equal(q, qt)
