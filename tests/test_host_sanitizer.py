"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The host sources of libbsattn (argument checks and workspace layout in
``api.cpp``, the block-index builder, the calibration search) do index
arithmetic on caller buffers.  This test builds them with g++
``-fsanitize=address,undefined`` into a library whose kernel launchers are
the no-device stand-ins of ``host_sanitize/no_device_stubs.cpp``.  It then
runs the CPU tests that call the library (block index, ABI, calibration)
against that library in a child Python that has the ASan runtime preloaded.
Any sanitizer report ends that child with an error.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_flash_amd", "csrc")
STUBS = os.path.join(ROOT, "tests", "host_sanitize", "no_device_stubs.cpp")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("api.cpp", "block_index.cpp", "calibrate.cpp")] + [STUBS]
HOST_TESTS = ["tests/test_block_index.py", "tests/test_abi.py", "tests/test_calibration.py"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _libasan():
    if shutil.which("g++") is None:
        return None
    p = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    asan = _libasan()
    if asan is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("g++ with libasan and the HIP runtime library are needed")
    out = tmp_path_factory.mktemp("host_sanitize")
    flags = ["-std=c++17", "-fPIC", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include")]
    procs, objs = [], []
    for src in HOST_SOURCES:
        obj = str(out / (os.path.basename(src) + ".o"))
        procs.append((src, subprocess.Popen(["g++", *flags, "-c", src, "-o", obj],
                                            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    for src, pr in procs:
        log = pr.communicate()[0]
        assert pr.returncode == 0, f"compiling {src} failed:\n{log}"
    lib = str(out / "libbsattn_host_asan.so")
    r = subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", *objs, "-L", os.path.join(ROCM, "lib"),
                        f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lamdhip64", "-Wl,--no-undefined", "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return lib, asan


def _env(lib, asan):
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
        "BSATTN_LIB": lib,
        "PYTHONPATH": ROOT + os.pathsep + env.get("PYTHONPATH", ""),
    })
    return env


def test_library_is_instrumented(sanitized_lib):
    lib, asan = sanitized_lib
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms or "__asan_loadN" in syms
    assert "__ubsan_handle_" in syms
    # the child process loads this library, not the in-tree one
    code = "from block_sparse_attention_flash_amd import _abi; print(_abi.load()._name)"
    r = subprocess.run([sys.executable, "-c", code], env=_env(lib, asan), cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().splitlines()[-1] == lib


def test_host_tests_clean_under_sanitizers(sanitized_lib):
    lib, asan = sanitized_lib
    cmd = [sys.executable, "-m", "pytest", *HOST_TESTS, "-m", "not gpu", "-q", "-x", "-p", "no:cacheprovider"]
    r = subprocess.run(cmd, env=_env(lib, asan), cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
