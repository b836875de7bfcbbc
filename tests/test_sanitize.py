"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

* ``mamba_ssd_scan_forward_amd/_build/host_check``: ssd_api.hip's host side (problem
  checks, the planner, workspace sizing, the plan description and the validation of every
  entry point) over about 1.5 million problems, edge and overflow values included, linked
  with csrc/host_check.cpp.
* ``oracle/_build/sanitize_check``: the float64 oracle (oracle/ssd_oracle.c) on small
  plain and packed problems, forward and backward, plus two facts any correct recurrence
  meets (zero decay gives y_t = x_t (B_t . C_t); a packed split restarts the state).

Both programs are built by ``__graft_entry__.build()``; a test rebuilds its program when a
source is newer than it.  Any sanitizer report ends the program with a non-zero status.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

ENV = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _stale(binary, sources):
    if not os.path.exists(binary):
        return True
    t = os.path.getmtime(binary)
    return any(os.path.getmtime(s) > t for s in sources)


def _run(binary):
    res = subprocess.run([binary], capture_output=True, text=True, env=ENV, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_host_code_under_sanitizers():
    from mamba_ssd_scan_forward_amd import build as b
    csrc = os.path.join(ROOT, "mamba_ssd_scan_forward_amd", "csrc")
    sources = glob.glob(os.path.join(csrc, "*.h")) + glob.glob(os.path.join(csrc, "*.hip")) + \
        [b.HOST_CHECK_SRC, os.path.join(ROOT, "include", "ssd.h")]
    if _stale(b.HOST_CHECK, sources):
        b.build_host_check()
    out = _run(b.HOST_CHECK)
    assert " 0 failures" in out, out[-2000:]


def test_oracle_under_sanitizers():
    from oracle import build as ob
    if _stale(ob.CHECK, [ob.SRC, ob.CHECK_SRC]):
        ob.build_sanitize_check()
    out = _run(ob.CHECK)
    assert "0 failures" in out, out[-2000:]
