"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. The oracle (plain C) built with gcc -fsanitize=address,undefined runs the
   oracle pin tests.
2. The library's host layer (argument validation, workspace layout, dispatch
   in abi.cpp and static_ws.hip) is recompiled with host-only sanitizers and
   linked with the kernels' objects from the regular build; the C-ABI
   validation tests run against it.  No GPU work happens: every call there is
   rejected on the host or is a size query.

Each run is a child process with the sanitizer runtime preloaded; any report
aborts it (no recovery), which fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_moe_expert_router_amd", "csrc")
ROCM = "/opt/rocm"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd[:3], r.stdout[-3000:], r.stderr[-3000:])
    return r


def _child(script, lib, preload, tmp_path):
    path = tmp_path / "child.py"
    path.write_text(script)
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, str(path), lib], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
          os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", lib, "-lm"])
    preload = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    script = (
        "import sys\n"
        "sys.path[:0] = [%r, %r]\n"
        "import oracle\n"
        "oracle._LIB = sys.argv[1]\n"
        "import pytest\n"
        "rc = pytest.main(['-q', '-p', 'no:cacheprovider', %r])\n"
        "assert oracle.lib()._name == sys.argv[1]\n"
        "sys.exit(rc)\n" % (ROOT, os.path.join(ROOT, "tests"), os.path.join(ROOT, "tests", "test_oracle_pins.py")))
    r = _child(script, lib, preload, tmp_path)
    assert " passed" in r.stdout and " failed" not in r.stdout, r.stdout[-2000:]


def test_abi_validation_under_asan_ubsan(tmp_path):
    from quantized_moe_expert_router_amd import build as b
    host = ("abi.cpp", "static_ws.hip")   # rebuilt below with host sanitizers; the kernels link as built
    objs = {s: os.path.join(ROOT, "_build", s + ".o") for s in b.SOURCES if s not in host}
    if not all(os.path.exists(o) for o in objs.values()):
        for s in objs:
            b._compile(s)
    san_objs = []
    for src in host:
        out = str(tmp_path / (src + ".o"))
        _run([os.path.join(ROCM, "bin", "hipcc"), "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"),
              *HOST_SAN, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out])
        san_objs.append(out)
    lib = str(tmp_path / "libmoeq_san.so")
    link = [os.path.join(ROCM, "lib", "llvm", "bin", "clang++"), "-shared", "-fPIC", "-shared-libsan"]
    link += ["-fsanitize=address,undefined", *objs.values(), *san_objs]
    link += ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", lib]
    _run(link)
    rts = glob.glob(os.path.join(ROCM, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                 "libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    script = (
        "import sys\n"
        "sys.path[:0] = [%r, %r]\n"
        "from quantized_moe_expert_router_amd import moeq\n"
        "moeq.LIB_PATH = sys.argv[1]\n"
        "import pytest\n"
        "rc = pytest.main(['-q', '-p', 'no:cacheprovider', %r])\n"
        "assert moeq.lib()._name == sys.argv[1]\n"
        "sys.exit(rc)\n" % (ROOT, os.path.join(ROOT, "tests"), os.path.join(ROOT, "tests", "test_abi_cpu.py")))
    r = _child(script, lib, rts[0], tmp_path)
    assert " passed" in r.stdout and " failed" not in r.stdout, r.stdout[-2000:]
