"""Device-code resource checks of the hot kernels (CPU only: hipcc cross-compiles).

A kernel that indexes a by-value argument array with a runtime index makes
the compiler copy the whole argument struct to per-lane scratch memory, a
silent several-fold slowdown of the launch.  The hot kernels must use no
scratch at all and stay within the register budget their launch bounds give.
"""
import os
import re
import subprocess

import pytest

from transformer_latent_pixel_amd import build as B



def _kernels(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [B.hipcc(), *[f for f in B.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    names = re.findall(r"^\s+\.name:\s+(\S+)", text, re.M)
    scratch = re.findall(r"^\s+\.private_segment_fixed_size:\s+(\d+)", text, re.M)
    spills = re.findall(r"^\s+\.vgpr_spill_count:\s+(\d+)", text, re.M)
    assert len(names) == len(scratch) == len(spills) > 0
    return list(zip(names, map(int, scratch), map(int, spills)))


@pytest.mark.parametrize("src", ["gemm.hip", "attention.hip", "misc.hip"])
def test_hot_kernels_use_no_scratch(src, tmp_path):
    for name, scratch, spills in _kernels(src, tmp_path):
        assert scratch == 0 and spills == 0, (name, scratch, spills)
