"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host side (cpk_api.cpp: argument validation, the chunk and
ladder arithmetic, the step planner, workspace sizing) is rebuilt with ASan
and UBSan and linked with the already compiled device objects; the oracle
(orc.c) is rebuilt with the same sanitizers.  The host ABI tests and the
oracle pins then run against both in a child process with the sanitizer
runtime preloaded; any report aborts the child and fails this test.  No GPU
is touched: without one, the host ABI tests stop at validation."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "chunked_prefill_causal_kv_amd")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
DEVICE_SOURCES = ["k_copy.hip", "k_attn.hip", "k_decode.hip", "cpk_noalloc.hip"]


def _device_objects():
    sys.path.insert(0, PKG)
    import build as libbuild   # the library's own build script
    sys.path.pop(0)
    os.makedirs(libbuild.BUILD_DIR, exist_ok=True)
    objs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(libbuild.BUILD_DIR, src + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(
                os.path.join(libbuild.CSRC, src)):
            obj = libbuild._compile(src)
        objs.append(obj)
    return objs


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and RUNTIME),
                    reason="ROCm clang with its sanitizer runtime is not installed")
def test_host_code_clean_under_asan_and_ubsan(tmp_path):
    pkg = tmp_path / "pkg"
    lib_dir = pkg / "chunked_prefill_causal_kv_amd"
    orc_dir = pkg / "oracle"
    lib_dir.mkdir(parents=True)
    orc_dir.mkdir(parents=True)
    shutil.copy(os.path.join(PKG, "__init__.py"), lib_dir)
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), orc_dir)
    shutil.copy(os.path.join(ROOT, "oracle", "orc.c"), orc_dir)
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    # host-only instrumentation of the HIP compile: every sanitizer flag is
    # scoped to the host pass, and the device pass is told not to sanitize
    host = []
    for f in san:
        host += ["-Xarch_host", f]
    api_obj = str(tmp_path / "cpk_api.o")
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-fno-gpu-sanitize"] + host +
         ["-I", os.path.join(ROOT, "include"), "-c", os.path.join(PKG, "csrc", "cpk_api.cpp"),
          "-o", api_obj])
    # the sanitizer runtime is preloaded in the child, so the shared library
    # links without it
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", api_obj] + _device_objects() +
         ["-o", str(lib_dir / "libcpk.so")])
    _run([CLANG, "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
          "-fPIC"] + san + [str(orc_dir / "orc.c"), "-o", str(orc_dir / "liborc.so"), "-lm"])
    env = dict(os.environ)
    env.update({
        "PYTHONPATH": os.pathsep.join([str(pkg), ROOT]),
        "LD_PRELOAD": RUNTIME[-1],
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    probe = ("import chunked_prefill_causal_kv_amd as c, oracle as o; "
             "o._load(); print(c.LIB_PATH); print(o._LIB_PATH)")
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True,
                       cwd=str(tmp_path))
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.split() == [str(lib_dir / "libcpk.so"), str(orc_dir / "liborc.so")], r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_abi.py"),
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, cwd=str(tmp_path), timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout and "failed" not in r.stdout
