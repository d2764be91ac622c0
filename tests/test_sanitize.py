"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

- the fp64 oracle (oracle/flare_oracle.c): every entry point on small and
  degenerate shapes in exactly sized heap buffers (oracle_sanitize_main.c);
- the piece arithmetic the planner and the kernels share
  (rank_latent_attention_amd/csrc/pieces.h), through pieces_check.cpp.

Any report aborts the program (-fno-sanitize-recover=all), so a clean exit
with "ok" is the pass condition.  CPU only.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, exe):
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-4000:] + r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c99", *SAN, os.path.join(HERE, "oracle_sanitize_main.c"), "-o", exe, "-lm"], exe)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_pieces_under_sanitizers(tmp_path):
    exe = str(tmp_path / "pieces_san")
    _run(["g++", "-std=c++17", *SAN, os.path.join(HERE, "pieces_check.cpp"), "-o", exe], exe)
