"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer (the
GPU code cannot be built with them on this platform).

* The C ABI's host validation (csrc/abi.cpp) is built with g++ and the
  sanitizers, linked with stand-in launchers (tests/san/abi_stubs.cpp), and
  driven through every entry point's rejection and accepted paths
  (tests/san/abi_driver.c); any report aborts the run.
* The fp64 oracle (oracle/gdn_oracle.c) is built with gcc and the
  sanitizers and run, in a child process with the sanitizer runtime
  preloaded, over small dense and packed inputs (an empty sequence
  included) for the forward, the decode step, the backward and the
  channel-wise decay and Gated DeltaNet-2 forwards; its results must equal
  the regular build's.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                               reason="gcc/g++ not available")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@needs_gcc
@pytest.mark.skipif(not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"),
                    reason="HIP headers not installed")
def test_abi_validation_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src, comp in (("gated_delta_rule_58_amd/csrc/abi.cpp", ["g++", "-std=c++17"]),
                      ("tests/san/abi_stubs.cpp", ["g++", "-std=c++17"]),
                      ("tests/san/abi_driver.c", ["gcc", "-std=c99"])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(comp + SAN + inc + ["-c", os.path.join(ROOT, src), "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_san")
    _run(["g++"] + SAN + objs + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                                 "-o", exe])
    r = _run([exe], env=ENV, timeout=120)
    assert "0 failures" in r.stdout, r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


CHILD = r'''
import sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import gdn_inputs as gi
import oracle

san = oracle.load(sys.argv[2])
ref = oracle.load(oracle.LIB_PATH)

def same(a, b):
    for x, y in zip(a if isinstance(a, tuple) else (a,), b if isinstance(b, tuple) else (b,)):
        if x is None and y is None:
            continue
        assert np.array_equal(np.asarray(x), np.asarray(y)), "sanitized build differs"

cu = [0, 37, 37, 101, 102, 170]
dense = gi.chunk_inputs(2, 70, 2, 16, 12, "f32", s0_std=0.1, seed=1)
packed = gi.chunk_inputs(1, cu[-1], 2, 16, 16, "f32", s0_std=0.1, seed=2, cu_seqlens=cu)
for inp in (dense, packed):
    a = [inp[x] for x in ("q", "k", "v", "log_alpha", "beta", "S0", "cu_seqlens")]
    same(oracle.fwd(*a, lib=san), oracle.fwd(*a, lib=ref))
    rng = np.random.default_rng(3)
    dO = rng.standard_normal(inp["v"].shape)
    same(oracle.bwd(*a[:6], a[6], dO, None, lib=san), oracle.bwd(*a[:6], a[6], dO, None, lib=ref))
d = gi.decode_inputs(2, 3, 16, 12, steps=1, dtype="f32", seed=4)
s = [d[x][0] for x in ("q", "k", "v", "log_alpha", "beta")]
same(oracle.step(*s, d["S0"], lib=san), oracle.step(*s, d["S0"], lib=ref))
kd = gi.kda_inputs(1, cu[-1], 2, 16, 16, "f32", s0_std=0.1, seed=5, cu_seqlens=cu)
ka = [kd[x] for x in ("q", "k", "v", "log_alpha", "beta", "S0", "cu_seqlens")]
same(oracle.kda_fwd(*ka, lib=san), oracle.kda_fwd(*ka, lib=ref))
g2 = gi.gdn2_inputs(2, 50, 2, 16, 16, "f32", s0_std=0.1, seed=6)
ga = [g2[x] for x in ("q", "k", "v", "log_alpha", "erase", "write", "S0")]
same(oracle.gdn2_fwd(*ga, lib=san), oracle.gdn2_fwd(*ga, lib=ref))
print("sanitized oracle ok")
'''


@needs_gcc
def test_oracle_under_sanitizers(tmp_path):
    import oracle
    oracle.load()   # make sure the regular build exists
    so = str(tmp_path / "liboracle_san.so")
    _run(["gcc", "-fopenmp", "-fPIC", "-shared", "-std=c99"] + SAN +
         ["-o", so, os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True,
                           text=True).stdout.strip()
    env = dict(ENV, LD_PRELOAD=f"{asan} {ubsan}", OMP_NUM_THREADS="2")
    r = _run([sys.executable, "-c", CHILD, ROOT, so], env=env, timeout=600, cwd=ROOT)
    assert "sanitized oracle ok" in r.stdout
