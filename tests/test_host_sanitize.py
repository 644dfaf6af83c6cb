"""Host code under the address and undefined-behaviour sanitizers (no GPU).

* The C ABI's argument checks (sparse_moe_expert_sigmoid_amd/csrc/checks.cc):
  every entry point of include/moe.h runs its check before it touches the
  device, so these cases are exactly what a call with such arguments returns:
  misaligned and NULL pointers, negative T, k above 16 or above E, unknown
  router, format, layout or activation, widths past the limits, workspaces
  that are NULL, misaligned or one byte short, overlapping buffers, and the
  small-batch split plan of moe_forward (tests/native/abi_checks.cc).
* The CPU oracle (oracle/oracle.c) on small inputs in every format, router
  and activation (tests/native/oracle_sanitize.c).
Both build with the host compiler alone (no HIP headers) and fail on the
first sanitizer report."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
# (verify_asan_link_order=0: the environment may preload a library ahead of
# the sanitizer runtime; the checks themselves are unaffected)
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    print(r.stdout)
    print(r.stderr[-4000:])
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    return r.stdout


def test_abi_argument_checks_sanitized(tmp_path):
    exe = str(tmp_path / "abi_checks")
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-Wextra", *SAN, "-o", exe,
                    os.path.join(HERE, "native", "abi_checks.cc"),
                    os.path.join(ROOT, "sparse_moe_expert_sigmoid_amd", "csrc", "checks.cc")],
                   check=True)
    out = _run(exe)
    assert "argument checks: 0 failures" in out


def test_oracle_sanitized(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-O1", "-std=c11", "-Wall", "-ffp-contract=off", *SAN, "-o", exe,
                    os.path.join(HERE, "native", "oracle_sanitize.c"),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    out = _run(exe)
    assert "oracle under sanitizers: 0 failures" in out
