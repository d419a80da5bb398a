"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle is the checker of every parity claim, so a read past an array, an
uninitialised accumulator or a signed overflow in it would be a wrong
reference.  This builds oracle/moe_oracle.c with gcc's ASan and UBSan
(aborting at the first report) and runs all of the oracle's pins
(tests/test_oracle.py) against that build in a child process, with the
sanitizer runtime preloaded (the interpreter itself is not instrumented; the
arrays the pins pass come from numpy's malloc, so ASan guards their ends).
"""

import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
# the oracle's own flags (oracle/build.py) plus the sanitizers
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fPIC", "-shared"]


def _runtime(name: str) -> str:
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


@pytest.fixture(scope="module")
def sanitized_lib():
    d = tempfile.mkdtemp(prefix="oracle_san_")
    lib = os.path.join(d, "liboracle_san.so")
    r = subprocess.run(["gcc", *SAN_FLAGS, "-o", lib, SRC, "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(f"sanitized oracle build failed:\n{r.stderr[-3000:]}")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (os.path.isabs(asan) and os.path.exists(asan) and os.path.isabs(ubsan) and os.path.exists(ubsan)):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    yield lib, asan, ubsan


def test_oracle_pins_under_asan_ubsan(sanitized_lib):
    lib, asan, ubsan = sanitized_lib
    env = dict(os.environ)
    env.update(
        MOE_ORACLE_LIB=lib,
        LD_PRELOAD=":".join(p for p in (asan, ubsan, env.get("LD_PRELOAD", "")) if p),
        # the interpreter's own allocations are never freed at exit: no leak report
        ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
    )
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, f"pins failed or a sanitizer reported under ASan/UBSan:\n{tail}"
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail


def test_sanitizer_catches_a_planted_overflow(sanitized_lib, tmp_path):
    """The set-up itself: a planted out-of-bounds read in a copy of the oracle
    (the layout counter indexed one past the expert range) must abort."""
    lib, asan, ubsan = sanitized_lib
    text = open(SRC).read()
    # plant: the layout's slot read at token_per_expert[e + E] instead of [e]
    needle = "send_token_idx[t * k + j] = token_per_expert[e];"
    assert needle in text, "the layout's slot assignment changed; update the planted mistake"
    bad = text.replace(needle, "send_token_idx[t * k + j] = token_per_expert[e + num_experts];", 1)
    src = tmp_path / "bad.c"
    src.write_text(bad)
    out = tmp_path / "libbad.so"
    subprocess.run(["gcc", *SAN_FLAGS, "-o", str(out), str(src), "-lm"], check=True, capture_output=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=":".join(p for p in (asan, ubsan, env.get("LD_PRELOAD", "")) if p),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0")
    code = ("import sys; sys.path.insert(0, %r); import numpy as np, oracle; "
            "o = oracle.Oracle(%r); o.layout(np.array([[0, 1], [1, 0]], np.int32), 2, 1)" % (ROOT, str(out)))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]
