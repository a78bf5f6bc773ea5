"""The oracle and the library's host layer under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

* The oracle's C source is built with gcc ``-fsanitize=address,undefined
  -fno-sanitize-recover=all`` and every pin of ``oracle_pins.py`` runs against
  it: an out-of-bounds access, use after free or undefined operation anywhere
  the pins reach aborts the run.
* The host layer (``mha_api.cpp``: argument validation, workspace layouts,
  plan choice, error messages) is built the same way with g++ against
  launchers that report "no device" (``sanitize_stubs.cpp``), and the
  validation tests of ``test_abi_cpu.py`` run against that build.

Both run in child processes with the sanitizer runtime preloaded (the Python
interpreter itself is not instrumented); leak checking is off, since the
interpreter keeps its allocations until exit.
"""
import os
import pathlib
import subprocess
import sys

import pytest

import oracle

ROOT = pathlib.Path(__file__).resolve().parent.parent
CSRC = ROOT / "transformer_head_scaled_softmax_amd" / "csrc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _asan_runtime() -> str:
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    path = p.stdout.strip()
    if not os.path.isabs(path):
        pytest.skip("gcc has no AddressSanitizer runtime")
    return path


def _env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = os.pathsep.join([str(ROOT), str(ROOT / "tests")])
    return env


_PINS = """
import sys
import oracle, oracle_pins
res = oracle_pins.run_all(oracle.Oracle(sys.argv[1]))
bad = {k: v for k, v in res.items() if v}
print(len(res), "pins run;", len(bad), "failed")
for k, v in bad.items():
    print(k, v[:3])
sys.exit(1 if bad else 0)
"""


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    str(oracle.SOURCE), "-o", str(lib), "-lm"], check=True)
    res = subprocess.run([sys.executable, "-c", _PINS, str(lib)], capture_output=True, text=True, env=_env(),
                         timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "0 failed" in res.stdout


def test_host_layer_under_sanitizers(tmp_path):
    lib = tmp_path / "libmha_host_san.so"
    subprocess.run(["g++", "-std=c++17", *SAN, "-w", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", f"-I{CSRC}", str(CSRC / "mha_api.cpp"),
                    str(ROOT / "tests" / "sanitize_stubs.cpp"), "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", str(lib)], check=True)
    env = _env()
    env["MHA_TEST_LIB"] = str(lib)
    # Tests that inspect or launch the real libmha.so in a process of their
    # own are left to the ordinary run.
    skip = ("exports_every_declared_symbol or without_a_device or one_sided or bench_refuses "
            "or python_binding")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          str(ROOT / "tests" / "test_abi_cpu.py"), "-k", f"not ({skip})"],
                         capture_output=True, text=True, env=env, cwd=str(ROOT), timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-3000:]
    assert " passed" in res.stdout
