"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The CPU oracle, built with gcc's -fsanitize=address,undefined, runs the
  whole oracle pin suite (tests/test_oracle_pins.py) in a child process that
  preloads gcc's ASan runtime.
- The host side of libepl.so (argument validation, workspace carving: every
  path that runs without a GPU), built with hipcc -Xarch_host
  -fsanitize=address / undefined (the device code is not instrumented), runs
  the C-ABI suite (tests/test_abi.py) in a child process that preloads
  clang's ASan runtime.
- A canary: a copy of the oracle with one planted out-of-bounds store must
  be stopped by ASan, so a silently inactive sanitizer cannot pass.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import build as oracle_build  # noqa: E402
from permute_ep_layout_amd import build as hip_build  # noqa: E402

GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g"]
HIP_SAN = []
for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"):
    HIP_SAN += ["-Xarch_host", flag]      # host pass only


def _gcc_asan_runtime():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run(args, preload, extra_env, timeout=600):
    env = dict(os.environ)
    env.update({"LD_PRELOAD": preload, "ASAN_OPTIONS": "detect_leaks=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
                "PYTHONDONTWRITEBYTECODE": "1"})
    env.update(extra_env)
    return subprocess.run([sys.executable, *args], capture_output=True, text=True, cwd=ROOT,
                          env=env, timeout=timeout)


def _clean(proc):
    text = proc.stdout + proc.stderr
    return "AddressSanitizer" not in text and "runtime error:" not in text


@pytest.fixture(scope="module")
def gcc_asan():
    rt = _gcc_asan_runtime()
    if rt is None:
        pytest.skip("gcc's ASan runtime is not available")
    return rt


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path, gcc_asan):
    lib = str(tmp_path / "libepl_oracle_san.so")
    oracle_build.build(extra_flags=GCC_SAN, out=lib)
    env = {"EPL_ORACLE_LIB": lib}
    active = _run(["-c", "import ctypes; ctypes.CDLL(None)['__asan_init']"], gcc_asan, env)
    assert active.returncode == 0, active.stderr[-2000:]
    proc = _run(["-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x", "-p",
                 "no:cacheprovider"], gcc_asan, env)
    assert proc.returncode == 0 and _clean(proc), (proc.stdout[-3000:], proc.stderr[-3000:])


def test_planted_overflow_is_caught(tmp_path, gcc_asan):
    """The canary: the oracle's scan with one store moved one element on
    writes past the end of expert_start_loc; ASan must abort the child."""
    src = open(oracle_build.SRC).read()
    line = "expert_start_loc[e] = (int32_t)running;"
    assert src.count(line) == 1
    bad = tmp_path / "epl_oracle.c"
    bad.write_text(src.replace(line, "expert_start_loc[e + 1] = (int32_t)running;"))
    lib = str(tmp_path / "libepl_oracle_bad.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-fPIC", "-shared", *GCC_SAN, str(bad), "-o", lib,
                    "-lm"], check=True)
    code = ("import numpy as np, oracle; "
            "oracle.default().scan(np.ones(1024, np.int32))")
    proc = _run(["-c", code], gcc_asan, {"EPL_ORACLE_LIB": lib})
    assert proc.returncode != 0
    assert "AddressSanitizer" in proc.stderr and "heap-buffer-overflow" in proc.stderr


def test_host_library_abi_suite_under_asan_and_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None or shutil.which(hip_build.hipcc()) is None:
        pytest.skip("hipcc or clang's ASan runtime is not available")
    lib = str(tmp_path / "libepl_san.so")
    hip_build.build(out=lib, extra_flags=HIP_SAN)
    env = {"EPL_LIB": lib}
    check = ("import permute_ep_layout_amd as epl, ctypes; "
             "assert epl.load()._name == " + repr(lib) + "; "
             "ctypes.CDLL(None)['__asan_init']")
    active = _run(["-c", check], rt, env)
    assert active.returncode == 0, active.stderr[-2000:]
    proc = _run(["-m", "pytest", "tests/test_abi.py", "-q", "-x", "-p", "no:cacheprovider"],
                rt, env)
    assert proc.returncode == 0 and _clean(proc), (proc.stdout[-3000:], proc.stderr[-3000:])
