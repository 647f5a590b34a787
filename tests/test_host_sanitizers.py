"""The library's host logic under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

``skg_api.cpp`` (argument checks, geometry, dispatch, warm-up keys,
crossover) is rebuilt with the host-side sanitizers and linked with the
normally built kernel objects and ``tests/host_asan/driver.cpp``, which
calls every host-only entry point over a grid of shapes, 200,000 random (also
absurd) configurations and every argument check.  No GPU call is reached.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "host_asan")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
# host-only sanitizers: each -fsanitize= follows -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _objects():
    objs = [os.path.join(BUILD, f) for f in sorted(os.listdir(BUILD))
            if f.endswith(".o") and f != "skg_api.o"] if os.path.isdir(BUILD) else []
    return objs


def test_host_logic_under_sanitizers():
    objs = _objects()
    if not os.path.exists(HIPCC) or len(objs) < 5:
        pytest.skip("needs hipcc and the built kernel objects (_build/*.o)")
    os.makedirs(OUT, exist_ok=True)
    api = os.path.join(OUT, "skg_api_san.o")
    drv = os.path.join(OUT, "driver.o")
    exe = os.path.join(OUT, "driver")
    csrc = os.path.join(ROOT, "latency_decode_gemm_amd", "csrc")
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC"] + SAN +
                   ["-c", os.path.join(csrc, "skg_api.cpp"), "-o", api], check=True,
                   capture_output=True)
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17"] + SAN +
                   ["-c", os.path.join(ROOT, "tests", "host_asan", "driver.cpp"), "-o", drv],
                   check=True, capture_output=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950"] + SAN + [drv, api] + objs + ["-o", exe],
                   check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr, r.stderr
    assert "host driver: 0 failures" in r.stdout
