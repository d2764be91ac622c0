"""Host check of the piece arithmetic shared by the planner and the kernels
(rank_latent_attention_amd/csrc/pieces.h): exact against 64-bit integer
division on every piece boundary of many (total, nwg) pairs."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_pieces_exact(tmp_path):
    exe = str(tmp_path / "pieces_check")
    subprocess.run(["g++", "-O2", "-std=c++17", os.path.join(HERE, "pieces_check.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
