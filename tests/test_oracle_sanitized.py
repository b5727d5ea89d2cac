"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer, run against every
pin (CPU only).

The oracle indexes caller-sized buffers with int64 arithmetic and every GPU verdict rests on
it, so its pins also run on a sanitized build: gcc -fsanitize=address,undefined with
recovery off (the first report aborts the process).  The pins run in a child process that
has the sanitizer runtimes preloaded from its start, because an instrumented library cannot
be loaded into an interpreter that started without them.  The HIP library is never loaded.
"""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {here!r}]
import oracle, oracle_pins
o = oracle.Oracle({lib!r})
for pin in oracle_pins.ALL_PINS:
    pin(o)
    print("ok", pin.__name__, flush=True)
print("ALL_PINS_OK", len(oracle_pins.ALL_PINS), flush=True)
"""


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc has no {name}")
    return path


def test_oracle_pins_under_asan_ubsan():
    preload = ":".join(_runtime(n) for n in ("libasan.so", "libubsan.so"))
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.build(os.path.join(tmp, "liboracle_san.so"), extra_cflags=SAN_FLAGS)
        env = dict(os.environ)
        env["LD_PRELOAD"] = preload
        # the interpreter itself is not instrumented: its allocations at exit are not the
        # oracle's, so leak checking is off; every other ASan/UBSan report aborts
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
        env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
        env["OMP_NUM_THREADS"] = "4"
        res = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, here=HERE, lib=lib)],
                             capture_output=True, text=True, env=env, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, f"sanitized oracle run failed (rc={res.returncode}):\n{out[-4000:]}"
    assert "ALL_PINS_OK" in res.stdout, out[-4000:]
    for word in ("AddressSanitizer", "runtime error:"):
        assert word not in out, out[-4000:]


def test_sanitizer_catches_a_planted_overread():
    # the same harness on a copy of the oracle with one planted out-of-bounds read (the code
    # word one packed row past the column's own, which leaves the buffer at the last row):
    # the child must stop with an AddressSanitizer report, so the test above is not vacuous
    preload = ":".join(_runtime(n) for n in ("libasan.so", "libubsan.so"))
    anchor = "uint32_t w = Wq[(k / 8) * N + n];"
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert anchor in src
    with tempfile.TemporaryDirectory() as tmp:
        bad = os.path.join(tmp, "oracle_overread.c")
        with open(bad, "w") as f:
            f.write(src.replace(anchor, "uint32_t w = Wq[(k / 8 + 1) * N + n];"))
        lib = oracle.build(os.path.join(tmp, "liboracle_bad.so"), source=bad, extra_cflags=SAN_FLAGS)
        env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   OMP_NUM_THREADS="2")
        res = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, here=HERE, lib=lib)],
                             capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode != 0 and "AddressSanitizer" in res.stderr, (res.returncode, res.stderr[-2000:])
