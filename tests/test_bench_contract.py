"""CPU checks of bench.py's contract: it refuses more than one GPU before
touching any device, and its algorithmic byte counts (the numerators of the
roofline's achieved rate) follow the per-launch formulas of the design:
GEMM  MK + NK*bits/8 + 4N/G + 4M + 2N + 2MN,  quantizer  2MK + MK + 4M
(+ 4K of gamma and beta for a LayerNorm row)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _run([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_gemm_bytes_formula():
    # BERT-base FFN1: 4096 tokens, 3072 x 768, W8, 64-row groups
    M, N, K, G = 4096, 3072, 768, 64
    want = M * K + N * K + 4 * (N // G) + 4 * M + 2 * N + 2 * M * N
    assert bench.gemm_bytes(M, N, K, 8, G) == want == 30693568
    # W4 weights are half the bytes
    assert bench.gemm_bytes(M, N, K, 8, G) - bench.gemm_bytes(M, N, K, 4, G) == N * K // 2
    # one token: the weights are nearly all of it
    b1 = bench.gemm_bytes(1, 16384, 4096, 8, 128)
    assert 16384 * 4096 <= b1 < 16384 * 4096 * 1.01


def test_quant_bytes_formula():
    assert bench.quant_bytes(4096, 768) == 2 * 4096 * 768 + 4096 * 768 + 4 * 4096
    assert bench.quant_bytes(2048, 6144, ln=True) == (2 * 2048 * 6144 + 2048 * 6144
                                                      + 4 * 2048 + 4 * 6144)


def test_default_workload_is_the_largest_single_gpu_config():
    # the headline step is GPT-NeoX-20B at 2048 tokens: four linears, INT4
    # feed-forward weights, and the largest integer work of the five
    from int4_quantized_transformer_amd import workloads as W
    wl = W.workload("neox-20b")
    ops = {w.name: sum(2 * max(w.M) * L.N * L.K for L in w.linears)
           for w in W.WORKLOADS}
    assert max(ops, key=ops.get) == "neox-20b"
    assert max(wl.M) == 2048
    import inspect
    assert 'default="neox-20b"' in inspect.getsource(bench.parse)
