"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers in tests/sanitize/ are built with gcc/g++ and -fsanitize=address,undefined
(every report fatal) and run here:
- oracle_driver.c with oracle/oracle.c: every oracle routine on exactly-sized heap blocks
  over edge-case shapes, with LeakSanitizer on;
- abi_driver.cpp with the library's host code (csrc/api.cpp) and stub launchers in place of
  the device code: every entry point on valid, invalid and swept edge-case arguments, with
  the workspace-query/call contract checked; it also sweeps the one-launch drafter's
  geometry (draft_geo) over head shapes against what that kernel assumes of it (grid,
  row splits, piece coverage, LDS sizes, hand-off word regions).
A planted overrun in the oracle and a workspace check off by one byte in api.cpp are each
caught by these drivers (the second through the stub launchers' layout check), and so is
a drafter geometry that admits one piece too many per lane."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _have_asan(compiler):
    if not shutil.which(compiler):
        return False
    out = subprocess.run([compiler, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return os.path.isabs(out) and os.path.exists(out)


def _run(exe, leaks):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=%d:abort_on_error=0:halt_on_error=1" % leaks,
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


@pytest.mark.skipif(not _have_asan("gcc"), reason="gcc without AddressSanitizer runtime")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", *SAN, "-std=gnu11", "-fopenmp", os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"], check=True)
    r = _run(exe, 1)
    if r.returncode != 0 and "LeakSanitizer has encountered a fatal error" in r.stderr:
        r = _run(exe, 0)   # leak checking is unavailable under some process tracers
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitizer driver: ok" in r.stdout


@pytest.mark.skipif(not _have_asan("g++"), reason="g++ without AddressSanitizer runtime")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    csrc = os.path.join(ROOT, "fine_grained_moe_router_amd", "csrc")
    subprocess.run(["g++", *SAN, "-std=c++17", "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
                    os.path.join(csrc, "api.cpp"), os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
                    "-o", exe], check=True)
    r = _run(exe, 1)
    if r.returncode != 0 and "LeakSanitizer has encountered a fatal error" in r.stderr:
        r = _run(exe, 0)
    assert r.returncode == 0, r.stdout + r.stderr
    line = [l for l in r.stdout.splitlines() if l.startswith("ABI sanitizer driver: ok")]
    assert line, r.stdout
    accepted, rejected = [int(t) for t in line[0].replace("(", " ").split() if t.isdigit()]
    assert accepted > 1000 and rejected > 1000, line[0]
