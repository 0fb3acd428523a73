"""The executor's host paths under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): executor.cpp is rebuilt with both sanitizers on its host side
and linked with the library's other objects into tests/host_sanitize's
driver, which exercises configuration, workspace and buffer validation, the
op lists of every schedule, call-order checks and the context-free entry
points' argument checks, none of which touches a GPU."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
CSRC = os.path.join(ROOT, "tensor_model_transformer_tmp_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OTHER_OBJS = ("gemm_bf16.hip.o", "gemm_f32.hip.o", "elementwise.hip.o", "attention.hip.o", "probe.hip.o")
# host-side instrumentation only: every -fsanitize= follows -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.timeout(600)
def test_executor_host_paths_clean_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC) or not all(os.path.exists(os.path.join(BUILD, o)) for o in OTHER_OBJS):
        pytest.skip("needs hipcc and the library's objects (python -m tensor_model_transformer_tmp_amd.build)")
    exe_o = str(tmp_path / "executor_san.o")
    drv_o = str(tmp_path / "host_paths.o")
    exe = str(tmp_path / "host_paths")
    common = ["-O1", "-g", "-std=c++17", "-I" + os.path.join(ROOT, "include"), *SAN]
    _run([HIPCC, *common, "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-Wno-inline-asm", "-x", "hip", "-c",
          os.path.join(CSRC, "executor.cpp"), "-o", exe_o])
    _run([HIPCC, *common, "-x", "c++", "-c", os.path.join(ROOT, "tests", "host_sanitize", "host_paths.cpp"),
          "-o", drv_o])
    _run([HIPCC, "--offload-arch=gfx950", *SAN, "-o", exe, drv_o, exe_o,
          *[os.path.join(BUILD, o) for o in OTHER_OBJS]])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env, timeout=300)
    assert "host paths OK" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
