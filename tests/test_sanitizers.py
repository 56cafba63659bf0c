"""CPU sanitizer runs: the host code of the library (argument checks, workspace carve-up,
launch set-up) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven by the
host ABI tests, and the fp64 oracle built the same way and driven by its pins.  Each runs in a
child process that preloads the matching ASan runtime; any sanitizer report fails the run
(errors are not recoverable and halt the child)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:detect_odr_violation=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(env_extra, tests):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + tests, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=900)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-3000:]
    assert "AddressSanitizer" not in r.stdout and "runtime error:" not in r.stdout


def test_host_api_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    from gated_delta_rule_39_amd._build import asan_runtime, build_library
    lib = build_library(out=str(tmp_path / "libkda_asan.so"),
                        extra_flags=["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                                     "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                                     "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libasan"])
    _run({"LD_PRELOAD": asan_runtime(), "KDA_LIBRARY": lib}, ["tests/test_abi_host.py"])


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    from oracle import build_oracle
    lib = build_oracle(out=str(tmp_path / "libkda_oracle_asan.so"),
                       extra_flags=["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                    "-fno-omit-frame-pointer"])
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.fail("gcc's libasan.so not found")
    _run({"LD_PRELOAD": rt, "KDA_ORACLE_LIBRARY": lib},
         ["tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py"])
