"""The C ABI's host code under AddressSanitizer.

A copy of the library is built with the host code of api.hip (argument
validation, status codes, the codebook), gemm.hip and prefill.hip (the
planners and the plan-name writer) instrumented (hipcc's -Xarch_host, so the
device code is unchanged), linked with the other objects of the regular
build, and driven by tests/host_asan_driver.c: every host-only query and every
entry point whose arguments fail validation before a launch, with host buffers
of exactly the sizes passed.  Any out-of-bounds access, use after free or
similar error in that code aborts the driver with the sanitizer's report.

Runs on the CPU only (no device call is made), and is skipped where a GPU is
present, where hipcc is missing or where the regular build's objects are not
there yet (build() makes them)."""

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_only_gemm_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "asan")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
INSTRUMENTED = ["api.hip", "gemm.hip", "prefill.hip"]
PLAIN = ["quant.o", "gemm_b3.o", "gemm_b8.o", "prefill_b3.o", "prefill_b8.o", "measure.o"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-ffp-contract=off",
         "-fno-gpu-rdc", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"),
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
# the decode kernels keep their accumulators in ordinary VGPRs, as in the
# regular build
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

pytestmark = [
    pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host-only check: run without a GPU"),
    pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                       reason="hipcc / clang not installed"),
    pytest.mark.skipif(not all(os.path.exists(os.path.join(BUILD, o)) for o in PLAIN),
                       reason="the regular build's objects are missing (run build())"),
]


def _newer(target, sources):
    return os.path.exists(target) and all(os.path.getmtime(target) >= os.path.getmtime(s)
                                          for s in sources)


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), r.stderr[-4000:])


def _compile(src):
    obj = os.path.join(OUT, src.replace(".hip", ".o"))
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [
        os.path.join(ROOT, "include", "w4a16.h")]
    if not _newer(obj, deps):
        _run([HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj])
    return obj


@pytest.fixture(scope="module")
def driver():
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(INSTRUMENTED)) as ex:
        objs = list(ex.map(_compile, INSTRUMENTED))
    plain = [os.path.join(BUILD, o) for o in PLAIN]
    lib = os.path.join(OUT, "libw4a16_asan.so")
    if not _newer(lib, objs + plain):
        _run([CLANG + "++", "-shared", "-fsanitize=address", "-o", lib] + objs + plain +
             ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    exe = os.path.join(OUT, "host_asan_driver")
    src = os.path.join(ROOT, "tests", "host_asan_driver.c")
    _run([CLANG, "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
          "-I" + os.path.join(ROOT, "include"), src, "-o", exe, "-L" + OUT, "-lw4a16_asan",
          "-Wl,-rpath," + OUT])
    return exe


def test_host_code_clean_under_address_sanitizer(driver):
    # leak checking off: the HIP runtime keeps allocations until exit
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=120)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host asan ok" in r.stdout
