"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

kv_oracle.c is built with gcc's address and undefined-behaviour sanitizers
(host code; nothing here touches a GPU) and the oracle pin suite
(test_oracle_pins.py) runs against that build through KVO_ORACLE_LIB: every
store, retrieve, encoder and decoder path the pins drive must run without an
out-of-bounds access, a use of freed memory or undefined behaviour.  A
planted heap overflow in a separate probe library checks first that the
sanitizer runtime is live in this setup (the Python interpreter is not
instrumented, so the runtime is preloaded)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
GCC = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _env(oracle_lib=None):
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    if oracle_lib is not None:
        env["KVO_ORACLE_LIB"] = oracle_lib
    return env


@pytest.mark.parametrize("sanitizer,body,report", [
    ("address", "int* p = malloc(4 * sizeof(int)); p[0] = i; int v = p[i]; free(p); return v;",
     "heap-buffer-overflow"),
    ("undefined", "int big = 2147483647 - 2; return big + i;", "signed integer overflow"),
], ids=["address", "undefined"])
def test_sanitizer_runtime_is_live(tmp_path, sanitizer, body, report):
    src = tmp_path / "probe.c"
    src.write_text("#include <stdlib.h>\nint probe(int i) { " + body + " }\n")
    so = tmp_path / "probe.so"
    subprocess.run(GCC + ["-fsanitize=" + sanitizer, "-fno-sanitize-recover=undefined", "-o", str(so), str(src)],
                   check=True)
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).probe(4)"
    r = subprocess.run([sys.executable, "-c", code], env=_env(), capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and report in r.stderr, r.stderr[-2000:]


def test_oracle_pins_pass_under_sanitizers(tmp_path):
    so = tmp_path / "kvo_sanitized.so"
    subprocess.run(GCC + SANITIZE + ["-I", ORACLE, "-o", str(so), os.path.join(ORACLE, "kv_oracle.c"), "-lm"],
                   check=True)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=_env(str(so)),
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0 and " passed" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
