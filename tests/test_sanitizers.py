"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only).

* The fp64 oracle (oracle/oracle.c), built with gcc and both sanitizers (leak checking on),
  driven through every entry point on small random inputs with edge cases
  (tests/sanitize/oracle_driver.c).
* The C ABI's validation layer (csrc/la_abi.hip, host code instrumented; device code as
  usual), linked with the library's other objects and driven through every rejection path
  with fake device addresses and through the host-only workspace and segment queries over
  shapes up to 2^40 tokens (tests/sanitize/abi_driver.cpp).  No device is touched.

Each driver exits non-zero if a call returns other than expected; a sanitizer finding
aborts it.  Built under _build/sanitize (not committed)."""

import os
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
OUT = ROOT / "_build" / "sanitize"
SAN = Path(__file__).resolve().parent / "sanitize"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizers on host code only: each -fsanitize= applies to the host pass
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_asan_ubsan():
    OUT.mkdir(parents=True, exist_ok=True)
    exe = OUT / "oracle_san"
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", str(ROOT / "oracle" / "oracle.c"),
          str(SAN / "oracle_driver.c"), "-o", str(exe), "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    r = _run([str(exe)], env=env)
    assert "all calls as expected" in r.stdout


def test_abi_validation_under_asan_ubsan():
    from gated_delta_rule_chunkwise_amd import build as hip_build

    objs = sorted((ROOT / "_build").glob("*.o"))
    if not any(o.name == "chunk.o" for o in objs):
        hip_build.build()
        objs = sorted((ROOT / "_build").glob("*.o"))
    OUT.mkdir(parents=True, exist_ok=True)
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", f"-I{ROOT / 'include'}",
             f"-I{ROOT / 'gated_delta_rule_chunkwise_amd' / 'csrc'}"] + HOST_SAN
    abi_o, drv_o, exe = OUT / "la_abi.o", OUT / "abi_driver.o", OUT / "abi_san"
    _run([HIPCC, *flags, "-c", str(ROOT / "gated_delta_rule_chunkwise_amd" / "csrc" / "la_abi.hip"), "-o", str(abi_o)])
    _run([HIPCC, *flags, "-c", "-x", "hip", str(SAN / "abi_driver.cpp"), "-o", str(drv_o)])
    others = [str(o) for o in objs if o.name != "la_abi.o"]
    _run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, str(drv_o), str(abi_o), *others, "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    r = _run([str(exe)], env=env)
    assert "all calls as expected" in r.stdout
