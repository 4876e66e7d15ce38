"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The oracle (oracle/oracle.c) is compiled by gcc with -fsanitize=address,undefined
  and every pin of tests/oracle_pins.py runs against it in a child process with the
  sanitizer runtimes preloaded.
* The HIP library is compiled by hipcc with the sanitizers on its host code only
  (each -fsanitize after -Xarch_host; the gfx950 device code is built as usual), and
  tests/test_abi.py -- every entry point's host-side validation and the exported
  symbols -- runs against it in a child process under the clang runtime.

A sanitizer report makes the child fail (halt_on_error), so the test fails with it.
The builds land in a temporary directory keyed by the sources' hash."""
import glob
import hashlib
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "online_softmax_04_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _hash(files):
    h = hashlib.sha256()
    for f in sorted(files):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def _run(cmd, env, timeout):
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    print(out[-4000:])
    assert "AddressSanitizer" not in out and "runtime error:" not in out, "sanitizer report"
    assert r.returncode == 0, f"exit status {r.returncode}"


def test_oracle_pins_under_asan_ubsan():
    src = os.path.join(ROOT, "oracle", "oracle.c")
    out_dir = os.path.join(tempfile.gettempdir(), f"osm_oracle_san_{_hash([src])}")
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "liboracle_san.so")
    if not os.path.exists(lib):
        subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-shared", "-fPIC", src, "-o", lib + ".tmp", "-lm", "-lpthread"],
                       check=True)
        os.replace(lib + ".tmp", lib)
    pre = ":".join(subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True,
                                  check=True).stdout.strip() for n in ("libasan.so", "libubsan.so"))
    env = dict(os.environ, LD_PRELOAD=pre, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    script = ("import sys; sys.path[:0] = ['.', 'tests']\n"
              "import oracle\n"
              "from oracle_pins import ALL_PINS\n"
              f"orc = oracle.load({lib!r})\n"
              "for pin in ALL_PINS:\n"
              "    pin(orc)\n"
              "print('pins passed:', len(ALL_PINS))\n")
    _run([sys.executable, "-c", script], env, timeout=900)


def test_abi_under_asan_ubsan():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))
                  + [os.path.join(ROOT, "include", "fa.h")])
    out_dir = os.path.join(tempfile.gettempdir(), f"osm_fa_san_{_hash(srcs)}")
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libfa_san.so")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
             "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-I",
             os.path.join(ROOT, "include"), "-I", CSRC]
    if not os.path.exists(lib):
        procs, objs = [], []
        for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
            obj = os.path.join(out_dir, os.path.basename(src) + ".o")
            objs.append(obj)
            procs.append(subprocess.Popen([HIPCC, *flags, "-c", src, "-o", obj],
                                          stdout=subprocess.DEVNULL, stderr=subprocess.PIPE))
        for p in procs:
            _, err = p.communicate(timeout=900)
            assert p.returncode == 0, err.decode()[-3000:]
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
                        "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs, "-o",
                        lib + ".tmp"], check=True, capture_output=True)
        os.replace(lib + ".tmp", lib)
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("clang sanitizer runtime not installed")
    env = dict(os.environ, LD_PRELOAD=rt[0], ONLINE_SOFTMAX_04_AMD_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
          "tests/test_abi.py"], env, timeout=900)
