"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The pin suites (tests/test_oracle_pins*.py, without the planted-mistake tests, which load
mutants of their own) run in a child process against a build of oracle/tt_oracle.c with
-fsanitize=address,undefined and no recovery, loaded through TT_ORACLE_LIB with the ASan
runtime preloaded: any out-of-bounds access, use after free or undefined operation in the
oracle ends that run with an error.  A second test plants a one-past-the-end read into a
copy of the source and checks that such a run does fail, so a silently inactive sanitizer
cannot pass for a clean oracle."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tt_oracle.c")
SAN = ["-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
       "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime():
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    lib = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                         text=True).stdout.strip()
    if not lib or not os.path.isabs(lib) or not os.path.exists(lib):
        pytest.skip("the ASan runtime is not installed")
    return lib


def _build(src_text, out):
    c = out.with_suffix(".c")
    c.write_text(src_text)
    subprocess.check_call(["gcc"] + SAN + [str(c), "-o", str(out), "-lm"])
    return str(out)


def _env(lib, asan_rt):
    env = dict(os.environ)
    env.update(TT_ORACLE_LIB=lib, LD_PRELOAD=asan_rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
    return env


def test_oracle_pins_pass_under_address_and_undefined_behavior_sanitizers(tmp_path):
    rt = _runtime()
    lib = _build(open(SRC).read(), tmp_path / "libtt_oracle_san.so")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-k", "not planted", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_pins_d.py")],
                       cwd=ROOT, env=_env(lib, rt), capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout


def test_sanitized_run_catches_a_planted_out_of_bounds_read(tmp_path):
    rt = _runtime()
    src = open(SRC).read()
    old = "for (int64_t j = 0; j < D; ++j) Y[b * D + j] += w * row[j];"
    assert old in src
    bad = src.replace(old, "for (int64_t j = 0; j <= D; ++j) Y[b * D + j] += w * row[j];", 1)
    lib = _build(bad, tmp_path / "libtt_oracle_oob.so")
    probe = ("import numpy as np, oracle\n"
             "from tensor_train_compressed_ttembeddingbag_amd import workloads as W\n"
             "wl = W.WORKLOADS['tiny']\n"
             "b = W.make_batch(wl, 0)\n"
             "oracle.forward(wl.p, wl.q, wl.ranks, wl.E, W.make_cores(wl), b['indices'],\n"
             "               b['offsets'], 8)\n")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=_env(lib, rt),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr
