"""Host code under the sanitizers (CPU only, no GPU calls).

Three programs are built in a temporary directory and run, each with AddressSanitizer and
UndefinedBehaviorSanitizer on its host code (errors abort):
  - the CPU oracle (oracle/moe_oracle.c, gcc) driven through every entry point on small inputs;
  - the library's host side (all of csrc/, device code compiled as usual, host code sanitized)
    driven through workspace planning over many shapes and the argument checks of every entry
    point -- no call reaches a kernel launch;
  - the FP8 quantiser's scalar helpers (csrc/fp8_codec.h) against searches written from the
    format's definition, including NaN, infinities and FLT_MAX.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "sparse_mixture_experts_softmax_amd", "csrc")

# sanitizer options for the host half of a HIP compile: each flag behind -Xarch_host so that the
# device half is built as usual
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
]
HIP_FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="4")


def _run(cmd, cwd, timeout=600):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=timeout, env=ENV)
    assert r.returncode == 0, "%s\n--- stdout\n%s\n--- stderr\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-8000:])
    return r.stdout


needs_hipcc = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "moe_oracle.c"),
          os.path.join(NATIVE, "oracle_check.c"), "-lm", "-o", exe], str(tmp_path))
    assert _run([exe], str(tmp_path)).strip().endswith("oracle_check ok")


@needs_hipcc
def test_fp8_codec_helpers_under_sanitizers(tmp_path):
    exe = str(tmp_path / "fp8_codec_check")
    _run(["hipcc"] + HIP_FLAGS + HOST_SANITIZE + [os.path.join(NATIVE, "fp8_codec_check.hip"), "-o", exe],
         str(tmp_path))
    assert _run([exe], str(tmp_path)).strip().endswith("fp8_codec_check ok")


@needs_hipcc
def test_library_host_validation_under_sanitizers(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs, objs = [], []
    for src in srcs + [os.path.join(NATIVE, "abi_host_check.cpp")]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        procs.append(subprocess.Popen(["hipcc"] + HIP_FLAGS + HOST_SANITIZE + lang + ["-c", src, "-o", obj],
                                      cwd=str(tmp_path), stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
    for p in procs:
        out, _ = p.communicate(timeout=900)
        assert p.returncode == 0, out[-4000:]
    exe = str(tmp_path / "abi_host_check")
    _run(["hipcc", "--offload-arch=gfx950"] + HOST_SANITIZE + objs + ["-o", exe], str(tmp_path))
    assert _run([exe], str(tmp_path)).strip().endswith("abi_host_check ok")
