"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the CPU-side code
(no GPU needed).

* The oracle (oracle/msa_oracle.c) with a driver that calls every entry point
  on small ragged inputs and every argument check (tests/sanitize/oracle_driver.c).
* libmsa's host code (argument checks, workspace layout and window search in
  msa_api.hip; the device code is built without sanitizers) with a driver that
  sweeps the size queries, calls every entry point with arguments its host
  checks reject, and passes enum values outside the enumerators the way a C
  caller may (tests/sanitize/abi_driver.cpp, abi_enum.c).

Any sanitizer report aborts the driver, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), res.stdout[-4000:], res.stderr[-4000:])
    return res


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "msa_oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    res = _run([exe], env=SAN_ENV, timeout=300)
    assert "oracle driver ok" in res.stdout


def test_host_code_under_asan_ubsan(tmp_path):
    from block_sparse_attention_qk_amd import build as b
    hipcc = b.hipcc()
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    csrc, inc = b.CSRC, b.INCLUDE
    objs = []
    # device kernels: the normal flags; host code of msa_api.hip: sanitized host pass only
    for src in b.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        flags = list(b.HIPCC_FLAGS)
        if src == "msa_api.hip":
            flags = [x for x in flags if x != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                         "-Xarch_host", "-fsanitize=address",
                                                         "-Xarch_host", "-fsanitize=undefined",
                                                         "-Xarch_host", "-fno-sanitize-recover=all"]
        _run([hipcc] + flags + ["-I", inc, "-I", csrc, "-c", os.path.join(csrc, src), "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_driver.o")
    _run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", inc, "-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    enum = str(tmp_path / "abi_enum.o")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", inc, "-c", os.path.join(HERE, "abi_enum.c"), "-o", enum])
    exe = str(tmp_path / "abi_asan")
    libdir = os.path.join(rocm, "lib")
    _run(["g++", "-fsanitize=address,undefined", drv, enum] + objs +
         ["-L", libdir, "-Wl,-rpath," + libdir, "-lamdhip64", "-o", exe])
    # the HIP runtime's own allocations are not this code's: leak checking off here
    env = dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = _run([exe], env=env, timeout=300)
    assert "abi driver ok" in res.stdout
