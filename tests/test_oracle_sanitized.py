"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, gcc) runs every pin without a report: no out-of-bounds
access, use after free, or undefined arithmetic on the paths the pins
exercise (including the breakdown, zero-diagonal, pattern-error and
non-finite cases).  The pins run in a child process with the sanitizer
runtime preloaded (the Python interpreter itself is not instrumented)."""
import os
import subprocess
import sys

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


SAN = ("-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g")


def _run_pins(lib):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    code = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle as O, test_oracle_pins as P\n"
        "with O.using_library(%r):\n"
        "    for pin in P.ALL_PINS:\n"
        "        pin()\n"
        "print('all pins ran')\n" % (HERE, os.path.dirname(HERE), lib))
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                          timeout=900)


def test_pins_under_asan_and_ubsan(tmp_path):
    lib = O.compile_source(os.path.join(os.path.dirname(O.__file__), "oracle.c"),
                           str(tmp_path / "liboracle_san.so"), extra=SAN)
    r = _run_pins(lib)
    report = r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "all pins ran" in r.stdout
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report


def test_harness_reports_a_planted_overread(tmp_path):
    """A copy of the oracle whose dot product reads one element past the end
    must make the sanitized pin run fail with an AddressSanitizer report."""
    src = open(os.path.join(os.path.dirname(O.__file__), "oracle.c")).read()
    old = "for (int64_t i = 0; i < n; ++i)\n        s += a[i] * b[i];"
    assert src.count(old) == 1
    path = tmp_path / "oracle_overread.c"
    path.write_text(src.replace(old, old.replace("i < n", "i <= n")))
    lib = O.compile_source(str(path), str(tmp_path / "liboracle_overread.so"), extra=SAN)
    r = _run_pins(lib)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr
