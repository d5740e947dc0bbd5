"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the host code, without a GPU.

Builds (under _build/san) the C oracle with gcc's -fsanitize=address,undefined and the
HIP library with the same sanitizers on its host code only (hipcc's -Xarch_host: the
device code is built as usual and never runs here), then runs the oracle's pins and the
C ABI's argument checks against them, each in a process that preloads the matching
sanitizer runtime (gcc's for the oracle, clang's for the library). Any report aborts that
process (-fno-sanitize-recover), which fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "_build", "san")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "router.hip", "align.hip", "elementwise.hip", "w4a16_stream.hip",
           "w4a16_tiled.hip", "fp8_stream.hip", "fp8_tiled.hip"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout[-4000:]}\n{p.stderr[-4000:]}"
    return p


def _build_oracle():
    out = os.path.join(SAN, "liboracle.so")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-o", out, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    return out


def _build_library():
    csrc = os.path.join(ROOT, "quantized_mixture_experts_amd", "csrc")
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(SAN, src.replace(".hip", ".o"))
        extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if src == "fp8_tiled.hip" else []
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN, *extra,
               "-I", os.path.join(ROOT, "include"), "-c", os.path.join(csrc, src), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out.decode(errors="replace")[-4000:]
    lib = os.path.join(SAN, "libqmoe.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, "-o", lib, *objs])
    return lib


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _gcc_asan_runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _env(env_extra):
    return dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", **env_extra)


def _check_loaded(env_extra, module, lib):
    """The instrumented build is the one a process with these settings maps."""
    code = ("import sys; sys.path[:0] = [%r, %r]; import conftest, os\n"
            "class S: pass\n"
            "conftest.pytest_sessionstart(S())\n"
            "%s\n"
            "print(open('/proc/self/maps').read())" % (ROOT, os.path.join(ROOT, "tests"), module))
    p = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(env_extra),
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr[-4000:]
    assert lib in p.stdout
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms


def _pytest(files, env_extra):
    env = _env(env_extra)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                           "-p", "no:cacheprovider", *files],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)


@pytest.mark.slow
def test_oracle_under_asan_and_ubsan():
    rt = _gcc_asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    os.makedirs(SAN, exist_ok=True)
    lib = _build_oracle()
    extra = {"LD_PRELOAD": rt, "QMOE_TEST_ORACLE_LIBRARY": lib}
    _check_loaded(extra, "import oracle; oracle._load()", lib)
    files = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    p = _pytest(files, extra)
    assert p.returncode == 0, p.stdout[-6000:] + p.stderr[-6000:]
    assert " passed" in p.stdout


@pytest.mark.slow
def test_library_host_code_under_asan_and_ubsan():
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    os.makedirs(SAN, exist_ok=True)
    lib = _build_library()
    extra = {"LD_PRELOAD": rt, "QMOE_TEST_LIBRARY": lib}
    _check_loaded(extra, "from quantized_mixture_experts_amd import binding; binding.load()", lib)
    p = _pytest([os.path.join(ROOT, "tests", "test_abi_cpu.py")], extra)
    assert p.returncode == 0, p.stdout[-6000:] + p.stderr[-6000:]
    assert " passed" in p.stdout
