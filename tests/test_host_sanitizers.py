"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libmla is compiled (the kernels for gfx950 as usual, never
run here) with both sanitizers on the host side only (the kernels' host-side
launchers and helpers, the argument validation, the workspace arithmetic)
into a separate library; the host ABI tests (tests/test_abi_host.py: exports,
argument errors, workspace sizes) then run against it in a child process with
the sanitizer runtime preloaded, and any sanitizer report fails the test. No
GPU is used (the argument checks return before anything would be launched).
"""

import os
import shlex
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_kv_28_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"

# the sanitizers apply to host code only
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all"
FLAGS = ("-O1 -g -std=c++17 -fPIC --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops "
         "-Wno-unused-command-line-argument -Werror=unused-value")

pytestmark = [
    pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists(CLANG), reason="ROCm compilers absent"),
    pytest.mark.timeout(600),
]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError("%s failed:\n%s%s" % (cmd[:3], r.stdout[-3000:], r.stderr[-3000:]))
    return r


def _build(out_dir):
    objs = []
    for src in sorted(os.listdir(CSRC)):
        if not (src.endswith(".hip") or src.endswith(".cpp")):
            continue
        obj = os.path.join(out_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([HIPCC] + shlex.split(FLAGS) + shlex.split(SAN) + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    lib = os.path.join(out_dir, "libmla_host_san.so")
    _run([HIPCC, "-shared", "-fPIC", "-shared-libsan"] + shlex.split(SAN) + ["-o", lib] + objs)
    return lib


def test_host_abi_under_asan_and_ubsan(tmp_path):
    lib = _build(str(tmp_path))
    syms = _run(["nm", "-D", lib]).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms   # the host code is instrumented
    runtime = _run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    assert os.path.exists(runtime), runtime
    driver = (
        "import sys, pytest\n"
        "sys.path.insert(0, %r)\n"
        "import mla_latent_kv_28_amd as mla\n"
        "mla.LIB_PATH = %r\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
        % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi_host.py")))
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", driver], capture_output=True, text=True, env=env, cwd=ROOT)
    out = r.stdout + r.stderr
    print(out[-2000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out
    assert r.returncode == 0
    assert " passed" in r.stdout
