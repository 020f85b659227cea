"""Host AddressSanitizer / UndefinedBehaviorSanitizer run of the CPU tests.

The host runtime behind the C ABI (api.cpp: validation, planning with maps
and per-call coverage vectors, workspace layout; schedule.cpp: the schedule
builder and balance accounting) and the C oracle are rebuilt with
-fsanitize=address,undefined (gcc, host code only; the HIP kernel objects
are linked unchanged), and the CPU test modules that drive them run against
those builds in a copy of the tree, with the ASan runtime preloaded into the
Python process.  Any invalid access, use after free, overflow or undefined
operation aborts the run (leak checking is off: the interpreter itself keeps
memory until exit).  CPU only; no GPU call is made.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_sequence_dfa_amd")
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
# CPU test modules that exercise the sanitized code (the schedule builder,
# validation and planning through the ABI, the oracle and its pins)
MODULES = ["test_abi.py", "test_schedule.py", "test_golden.py", "test_tolerance.py",
           "test_oracle.py", "test_timeline.py", "test_bench_cpu.py"]


def _libasan():
    path = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _copy_tree(dst):
    os.makedirs(os.path.join(dst, "long_context_sequence_dfa_amd"))
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            shutil.copy(os.path.join(PKG, f), os.path.join(dst, "long_context_sequence_dfa_amd", f))
    os.makedirs(os.path.join(dst, "oracle"))
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c")):
            shutil.copy(os.path.join(ROOT, "oracle", f), os.path.join(dst, "oracle", f))
    shutil.copytree(os.path.join(ROOT, "include"), os.path.join(dst, "include"))
    os.makedirs(os.path.join(dst, "tests"))
    for f in os.listdir(os.path.join(ROOT, "tests")):
        if f.endswith(".py") and (not f.startswith("test_") or f in MODULES):
            shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    for f in ("bench.py", "__graft_entry__.py"):
        shutil.copy(os.path.join(ROOT, f), os.path.join(dst, f))


def _build_sanitized(dst, tmp):
    from long_context_sequence_dfa_amd import _build
    kernels = sorted(os.path.join(_build.BUILD, f) for f in os.listdir(_build.BUILD)
                     if f.endswith(".hip.o")) if os.path.isdir(_build.BUILD) else []
    if not kernels:
        _build.build()
        kernels = sorted(os.path.join(_build.BUILD, f) for f in os.listdir(_build.BUILD)
                         if f.endswith(".hip.o"))
    objs = []
    for src in ("api.cpp", "schedule.cpp"):
        obj = os.path.join(tmp, src + ".o")
        subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
                               "-I", f"{ROCM}/include", "-I", os.path.join(ROOT, "include"),
                               "-I", os.path.join(PKG, "csrc"), "-c", os.path.join(PKG, "csrc", src),
                               "-o", obj])
        objs.append(obj)
    subprocess.check_call(["g++", "-shared", *SAN, "-o",
                           os.path.join(dst, "long_context_sequence_dfa_amd", "libdfa.so"), *objs,
                           *kernels, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    subprocess.check_call(["gcc", "-O1", "-g", "-fopenmp", "-shared", "-fPIC", *SAN, "-o",
                           os.path.join(dst, "oracle", "liboracle.so"),
                           os.path.join(dst, "oracle", "oracle.c"), "-lm"])


@pytest.mark.skipif(_libasan() is None or not os.path.exists(f"{ROCM}/lib/libamdhip64.so"),
                    reason="needs gcc's ASan runtime and the HIP runtime library")
def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    dst = str(tmp_path / "tree")
    _copy_tree(dst)
    _build_sanitized(dst, str(tmp_path))
    env = dict(os.environ)
    env.update(LD_PRELOAD=_libasan(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="4", PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *[os.path.join("tests", m) for m in MODULES]],
                       cwd=dst, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    m = re.search(r"(\d+) passed", r.stdout)
    assert m and int(m.group(1)) >= 100, tail
    print(r.stdout.strip().splitlines()[-1])
