"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer, each
exercised in a child process with the sanitizer runtime preloaded and every
report fatal:

* the oracle (gcc, -fsanitize=address,undefined) running its own pins, the
  fp32 mode's among them;
* the library's host layer -- argument validation and dispatch in
  kda_api.hip -- (hipcc, with the sanitizers on the host pass only: the GPU
  code is built as usual) running the C-ABI tests, which reach every
  validation branch without a device.
The builds go to a temporary directory; nothing in the tree is replaced."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, env, cwd=ROOT, timeout=900):
    return subprocess.run(cmd, cwd=cwd, env=env, capture_output=True, text=True, timeout=timeout)


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="kda_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_oracle_under_asan_and_ubsan(tmp):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    lib = os.path.join(tmp, "libkda_oracle_san.so")
    r = _run([gcc, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
              "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
              os.path.join(ROOT, "oracle", "kda_oracle.c"), "-o", lib, "-lm"], os.environ.copy())
    assert r.returncode == 0, r.stderr[-2000:]
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run([gcc, "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, KDA_ORACLE_LIB=lib, LD_PRELOAD="%s:%s" % (asan, ubsan), OMP_NUM_THREADS="4", **SAN_ENV)
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"], env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_host_layer_under_asan_and_ubsan(tmp):
    from linear_attention_recurrence_token_amd import _build
    try:
        hipcc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    lib = os.path.join(tmp, "libkda_san.so")
    # sanitizers on the host pass only (the kernels are built as usual)
    cmd = [hipcc, "--offload-arch=" + _build.ARCH, "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-I", os.path.join(ROOT, "include"), "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xarch_host", "-fno-omit-frame-pointer"] + _build.DEVICE_FLAGS
    cmd += [os.path.join(_build.CSRC, s) for s in _build.SOURCES] + ["-o", lib]
    r = _run(cmd, os.environ.copy())
    assert r.returncode == 0, r.stderr[-3000:]
    rt = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "llvm", "lib", "clang")
    found = []
    for root, _dirs, files in os.walk(rt if os.path.isdir(rt) else "/opt/rocm/llvm/lib/clang"):
        if "libclang_rt.asan-x86_64.so" in files:
            found.append(os.path.join(root, "libclang_rt.asan-x86_64.so"))
    if not found:
        pytest.skip("clang AddressSanitizer runtime not found")
    env = dict(os.environ, LD_PRELOAD=found[0], **SAN_ENV)
    script = ("import sys; sys.path.insert(0, %r); from linear_attention_recurrence_token_amd import kda; "
              "kda.LIB_PATH = %r; import pytest; "
              "sys.exit(pytest.main(['-q', '-x', '-s', '-p', 'no:cacheprovider', 'tests/test_abi.py']))" % (ROOT, lib))
    r = _run([sys.executable, "-c", script], env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
