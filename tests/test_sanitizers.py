"""The oracle and the library's host-side argument handling under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU (no GPU needed): each is rebuilt with the sanitizers into
a temporary directory and exercised in a child process that preloads the sanitizer runtime (the
Python interpreter itself is not instrumented); any report fails the run.

- `oracle/oracle.c` (gcc): the forward recurrence, its reverse-mode gradients and the KDA
  recurrence on small ragged shapes, with and without S0 and gates (a -inf reset included),
  n_h = 1..3, and an empty sequence.
- `delta_abi.cpp` (clang, host code only), linked with the kernels' objects as built: the whole
  host-side ABI suite (`tests/test_abi_host.py`: exports, shape and argument errors, aliasing,
  workspace sizes, fault injection), which returns before any kernel launch.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _child(code, preload, timeout=600):
    env = dict(ENV, LD_PRELOAD=preload, PYTHONPATH=os.pathsep.join([ROOT, HERE]))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


ORACLE_RUN = r"""
import numpy as np
import oracle
oracle._LIB_PATH = %r
rng = np.random.default_rng(1)
def run(B, L, H, dk, dv, nh, gated, s0):
    q = rng.standard_normal((B, L, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, L * nh, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, L * nh, H, dv)).astype(np.float32)
    beta = rng.random((B, L * nh, H)).astype(np.float32)
    g = (-rng.random((B, L, H))).astype(np.float32) if gated else None
    if gated and L > 0:
        g[0, L // 2, 0] = -np.inf
    S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32) if s0 else None
    O, S = oracle.fwd(q, k, v, beta, g, S0, n_h=nh)
    dO = rng.standard_normal(O.shape).astype(np.float32)
    oracle.bwd(q, k, v, beta, g, S0, dO, rng.standard_normal(S.shape).astype(np.float32), n_h=nh)
    if nh == 1:
        a = (-rng.random((B, L, H, dk))).astype(np.float32)
        oracle.fwd_kda(q, k, v, beta, a, S0)
for case in [(1, 7, 2, 16, 24, 1, True, True), (2, 33, 3, 32, 16, 2, False, False),
             (1, 5, 1, 16, 16, 3, True, False), (1, 0, 2, 16, 16, 1, True, True)]:
    run(*case)
print("oracle ran under the sanitizers")
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared"] + SAN +
                   ["-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    rt = [subprocess.run(["gcc", "-print-file-name=" + n], capture_output=True, text=True).stdout.strip()
          for n in ("libasan.so", "libubsan.so")]
    assert _child(ORACLE_RUN % lib, ":".join(rt)).strip().endswith("oracle ran under the sanitizers")


ABI_RUN = r"""
import sys
import chunkwise_delta_rule_chunked_amd as D
D._LIB = %r
import pytest
sys.exit(pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", "tests/test_abi_host.py"]))
"""


def test_abi_host_checks_under_asan_ubsan(tmp_path):
    clang = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
    rt = sorted(glob.glob(os.path.join(ROCM, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                       "libclang_rt.asan-x86_64.so")))
    objs = sorted(glob.glob(os.path.join(ROOT, "chunkwise_delta_rule_chunked_amd", "_build", "*.o")))
    objs = [o for o in objs if os.path.basename(o) != "delta_abi.o"]
    if not os.path.exists(clang) or not rt or len(objs) < 5:
        pytest.skip("needs ROCm's clang, its sanitizer runtime and the library's built objects")
    abi = str(tmp_path / "delta_abi_san.o")
    subprocess.run([clang, "-x", "c++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                    "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include")] + SAN +
                   ["-c", os.path.join(ROOT, "chunkwise_delta_rule_chunked_amd", "csrc", "delta_abi.cpp"), "-o", abi],
                   check=True)
    lib = str(tmp_path / "libdelta_san.so")
    subprocess.run([os.path.join(ROCM, "bin", "hipcc"), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, abi] + objs,
                   check=True, capture_output=True)
    undef = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in undef and "__ubsan_" in undef  # the host code really is instrumented
    out = _child(ABI_RUN % lib, rt[-1])
    assert " passed" in out and " failed" not in out
