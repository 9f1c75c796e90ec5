"""The C oracle under AddressSanitizer + UndefinedBehaviorSanitizer and under
ThreadSanitizer (CPU only).  Each sanitized build runs every oracle entry
point over the cases of oracle_sanitize_driver.py in a child process with the
sanitizer runtime preloaded; the run must finish without a report, and its
outputs must equal, bit for bit, those of the plain build (the sanitizers
change no arithmetic)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "oracle_sanitize_driver.py")

BUILDS = {
    "plain": ([], None, {}),
    "asan_ubsan": (["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"],
                   "libasan.so", {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                                  "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}),
    "tsan": (["-fsanitize=thread", "-g"], "libtsan.so", {"TSAN_OPTIONS": "halt_on_error=1:report_signal_unsafe=0"}),
}


def _run(tmp_path, name):
    flags, runtime, env_extra = BUILDS[name]
    lib = oracle.build(out=str(tmp_path / ("liboracle_%s.so" % name)), extra_flags=flags)
    out = tmp_path / ("out_%s.npz" % name)
    env = dict(os.environ, **env_extra)
    if runtime:
        env["LD_PRELOAD"] = subprocess.run(["gcc", "-print-file-name=" + runtime], capture_output=True, text=True,
                                           check=True).stdout.strip()
    r = subprocess.run([sys.executable, DRIVER, lib, str(out)], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, "%s run failed (%d):\n%s" % (name, r.returncode, report[-4000:])
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer", "ERROR: LeakSanitizer"):
        assert marker not in report, "%s reported:\n%s" % (name, report[-4000:])
    return dict(np.load(out))


@pytest.mark.parametrize("name", ["asan_ubsan", "tsan"])
def test_oracle_under_sanitizers(tmp_path, name):
    plain = _run(tmp_path, "plain")
    san = _run(tmp_path, name)
    assert sorted(plain) == sorted(san)
    for key in plain:
        a, b = plain[key], san[key]
        assert a.dtype == b.dtype and a.shape == b.shape, key
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), "%s: %s differs from the plain build" % (name, key)


def test_sanitizer_harness_catches_a_planted_overread(tmp_path):
    """The harness can fail: a copy of the oracle whose mean-pool reads one
    group member too many (past the end of the last row for the last group)
    must be reported by AddressSanitizer."""
    src = open(oracle._SRC).read()
    good = "for (int i = g * r + 1; i < g * r + r; ++i)"
    assert src.count(good) == 1
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(good, "for (int i = g * r + 1; i <= g * r + r; ++i)"))
    flags, runtime, env_extra = BUILDS["asan_ubsan"]
    lib = oracle.build(src=str(mutant), out=str(tmp_path / "libmutant.so"), extra_flags=flags)
    env = dict(os.environ, **env_extra)
    env["LD_PRELOAD"] = subprocess.run(["gcc", "-print-file-name=" + runtime], capture_output=True, text=True,
                                       check=True).stdout.strip()
    r = subprocess.run([sys.executable, DRIVER, lib, str(tmp_path / "o.npz")], capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode != 0 and "ERROR: AddressSanitizer" in r.stderr
