"""Host replay of the GEMM kernels' copy addresses under AddressSanitizer and
UBSan (CPU only).  The configuration list is generated from the kernel
source (every Tile<...> / Stream<...> that zq_gemm.hip launches, the W4
parameter expanded both ways and invalid instances skipped by the replay),
so no configuration the kernels use escapes it; the shapes are every
linear of the five workloads at each of their token counts plus ragged and
odd shapes of the parity tests.  tests/index_replay.cpp states the checks."""
import os
import re
import shutil
import subprocess

import pytest

from int4_quantized_transformer_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int4_quantized_transformer_amd", "csrc")


def _configs():
    with open(os.path.join(CSRC, "zq_gemm.hip")) as f:
        src = f.read()
    out = []
    for kind, pat in (("ZQ_TILE", r"run_tiled<Tile<([^<>]*)>"),
                      ("ZQ_PINGPONG", r"run_pingpong<Tile<([^<>]*)>"),
                      ("ZQ_STREAM", r"run_stream<Stream<([^<>]*)>"),
                      ("ZQ_TILE", r"using C[48] = Tile<([^<>]*)>")):
        for args in re.findall(pat, src):
            args = " ".join(args.split())
            for w4 in ("false", "true"):
                expanded = re.sub(r"\bW4\b", w4, args)
                line = f"{kind}({expanded})"
                if line not in out:
                    out.append(line)
    return out


def _shapes():
    shapes = set()
    for wl in W.WORKLOADS:
        for M in wl.M:
            for L in wl.linears:
                shapes.add((M, L.N, L.K, L.bits))
    for M, N, K in [(300, 1000, 384), (512, 2048, 576), (17, 320, 192),
                    (65, 320, 576), (9, 8190, 1088), (64, 4098, 640),
                    (20, 6144, 1088), (48, 200, 4160), (1, 3000, 8192),
                    (33, 4096, 2048), (257, 200, 64), (1000, 4096, 768),
                    (300, 33280, 384), (7, 64, 24576), (16, 24, 2048),
                    (9, 8200, 4160), (5, 8194, 64), (7, 16400, 1088),
                    (12, 16416, 4096), (16, 16384, 256)]:
        for bits in (8, 4):
            shapes.add((M, N, K, bits))
    return sorted(shapes)


def test_configs_cover_the_tables():
    cfgs = _configs()
    assert sum(c.startswith("ZQ_TILE") for c in cfgs) >= 40
    assert any(c.startswith("ZQ_PINGPONG") for c in cfgs)
    assert sum(c.startswith("ZQ_STREAM") for c in cfgs) >= 20


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_copy_addresses_in_bounds_under_sanitizers(tmp_path):
    cfg = tmp_path / "index_configs.h"
    cfg.write_text("#define ZQ_CONFIGS \\\n" +
                   " \\\n".join("  " + c for c in _configs()) + "\n")
    exe = tmp_path / "index_replay"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           f"-I{CSRC}", f"-I{tmp_path}",
           os.path.join(ROOT, "tests", "index_replay.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    inp = "".join(f"{M} {N} {K} {b}\n" for M, N, K, b in _shapes())
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True,
                       timeout=900, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.strip().splitlines()[-1].startswith("OK ")
