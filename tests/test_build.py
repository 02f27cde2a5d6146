"""Build checks that need no GPU: every kernel of the library compiles for
gfx950 without register spills (scratch memory per lane), which would put
per-lane memory traffic into the hot loops, and within the 160 KB of LDS a
workgroup may use (a larger one would fail only at launch)."""
import os
import re
import shutil
import subprocess

import pytest

from linear_attention_rnn_gdn_amd import build as hip_build


def test_no_kernel_uses_scratch(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc) and not shutil.which(hipcc):
        pytest.skip("hipcc not available")
    cmd = [hipcc] + hip_build.HIPCC_FLAGS + hip_build.SOURCES + ["-o", str(tmp_path / "x.so"),
                                                                 "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", out.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", out.stderr)]
    assert names and len(names) == len(scratch)
    spilled = [(n, b) for n, b in zip(names, scratch) if b]
    assert not spilled, f"kernels using scratch: {spilled}"
    lds = [int(x) for x in re.findall(r"LDS Size \[bytes/block\]: (\d+)", out.stderr)]
    assert len(lds) == len(names)
    big = [(n, b) for n, b in zip(names, lds) if b > 160 * 1024]
    assert not big, f"kernels over 160 KB of LDS: {big}"
