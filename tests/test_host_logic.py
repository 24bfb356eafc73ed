"""Host-side checks of helpers the kernels share with nothing else: built
with hipcc and run on the CPU (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _build_and_run(src, tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "check")
    cmd = [HIPCC, "-O2", "-std=c++17", "--offload-arch=gfx950",
           f"-I{os.path.join(ROOT, 'include')}",
           f"-I{os.path.join(ROOT, 'paged_mqa_logits_indexer_amd', 'csrc')}",
           os.path.join(ROOT, "tests", "host", src), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return subprocess.run([exe], capture_output=True, text=True, timeout=120)


def test_bin_key_ranges_match_the_bins_of_every_half(tmp_path):
    # The selector classifies scores against the threshold bin by FP16-key
    # ranges instead of computing each score's bin: the ranges must give the
    # same answer for all 65536 encodings and all 1025 thresholds.
    res = _build_and_run("bin_ranges_check.hip", tmp_path)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "mismatches 0" in res.stdout
