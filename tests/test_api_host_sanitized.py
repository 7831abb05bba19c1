"""The host side of libjas.so (argument validation, geometry, dispatch in
jas_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.

jas_api.cpp is rebuilt with host-only sanitizers, linked with the kernel
objects of the normal build, and tests/test_api_host.py runs against that
library in a child process with the sanitizer runtime preloaded.  Every
call there fails validation before any HIP call, so no GPU is needed.
Skipped when the normal build's objects or the runtime are missing.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "deterministic_attention_softmax_amd")
OBJS = ["jas_attn.hip.o", "jas_kernels_bf16.hip.o", "jas_kernels_f16.hip.o",
        "jas_kernels_f32.hip.o", "jas_launch.hip.o"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_host_api_under_sanitizers(tmp_path):
    objs = [os.path.join(PKG, "_build", o) for o in OBJS]
    rt = runtime()
    if not all(os.path.exists(o) for o in objs) or rt is None or not os.path.exists(HIPCC):
        pytest.skip("needs the library's build objects, hipcc and the sanitizer runtime")
    api_o = str(tmp_path / "jas_api.o")
    lib = str(tmp_path / "libjas_sanitized.so")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(PKG, 'csrc')}"]
    subprocess.run([HIPCC, *flags, *SAN, "-Xarch_host", "-fno-sanitize-recover=all", "-c",
                    os.path.join(PKG, "csrc", "jas_api.cpp"), "-o", api_o],
                   check=True, capture_output=True, text=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, api_o, *objs, "-o", lib],
                   check=True, capture_output=True, text=True)
    code = ("import sys\n"
            "import deterministic_attention_softmax_amd as j\n"
            "j.LIB_PATH = sys.argv[1]\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-s', '-p', 'no:cacheprovider', '-m', 'not gpu',\n"
            "                      'tests/test_api_host.py']))\n")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([sys.executable, "-c", code, lib], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
