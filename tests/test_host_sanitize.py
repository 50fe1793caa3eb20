"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every HIP source is compiled with the sanitizers on its host side (device code is built as usual
and never runs here) and linked into ``host_fuzz/host_fuzz.cpp``, which drives every entry point of
the C ABI with random and extreme arguments: the descriptor builders, the workspace planners and
the argument checks of every launching call. Where no GPU is visible an accepted call ends at a
launch the HIP runtime refuses, so the fuzzer's fake device pointers are never used. A sanitizer
report, a crash or a status that breaks the header's rules fails the test; two planted mistakes
show that the sanitizers are really on.
"""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "block_diffusion_drafting_draft_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = ["attn.hip", "verify.hip", "match.hip", "select.hip", "commit.hip", "awl.hip", "train_attn.hip"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
HOST_SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="the ROCm compilers are needed for the sanitizer build")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{res.stderr[-4000:]}")


@pytest.fixture(scope="module")
def fuzz_exe(tmp_path_factory):
    out = tmp_path_factory.mktemp("host_sanitize")
    # sanitizers on the host side of each HIP source only: each flag goes after -Xarch_host
    host_flags = [x for f in HOST_SAN for x in ("-Xarch_host", f)]

    def compile_hip(src):
        obj = str(out / (os.path.splitext(src)[0] + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_flags,
              "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_hip, SOURCES))
    drv = str(out / "host_fuzz.o")
    _run([CLANG, "-O1", "-g", "-std=c++17", *HOST_SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          "-I", INCLUDE, "-c", os.path.join(HERE, "host_fuzz", "host_fuzz.cpp"), "-o", drv])
    exe = str(out / "host_fuzz")
    _run([CLANG, *HOST_SAN, drv, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    return exe


def _exec(exe, *args, timeout=240):
    return subprocess.run([exe, *args], capture_output=True, text=True, env=ENV, timeout=timeout)


def test_sanitizers_catch_planted_mistakes(fuzz_exe):
    res = _exec(fuzz_exe, "--plant-overflow")
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr, res.stderr[-2000:]
    res = _exec(fuzz_exe, "--plant-signed-overflow")
    assert res.returncode != 0 and "signed integer overflow" in res.stderr, res.stderr[-2000:]


@pytest.mark.parametrize("seed", [1, 0x5EED, 0xD3D0])
def test_host_code_is_clean_under_fuzz(fuzz_exe, seed):
    res = _exec(fuzz_exe, "20000", str(seed))
    assert res.returncode == 0, (res.stdout[-1000:], res.stderr[-4000:])
    assert "accepted calls" in res.stdout
