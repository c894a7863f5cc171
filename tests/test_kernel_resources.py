"""CPU test of the compiled gfx950 kernels' resources: no kernel may use
scratch (stack) memory.  A kernel that keeps per-thread arrays or call
frames in scratch pays a memory round trip for them on every step; the
LL hand-off measured twice as slow with 424 bytes of scratch per lane.
The compiler's resource report is read for every kernel of the library."""
import os
import re
import subprocess

import pytest

from recv_fifo_plane_amd import build as B


def _report(src: str) -> str:
    cmd = [B.HIPCC] + B.COMMON + B.DEVICE + ["-Rpass-analysis=kernel-resource-usage",
                                            "--offload-device-only", "-c", src, "-o", os.devnull]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=900)
    assert r.returncode == 0, r.stdout[-3000:]
    return r.stdout


@pytest.mark.parametrize("name", ["kernels.hip", "noalloc.hip"])
def test_no_kernel_uses_scratch(name):
    text = _report(os.path.join(B.CSRC, name))
    blocks = text.split("Function Name: ")[1:]
    assert blocks, "no resource report"
    bad = []
    for blk in blocks:
        kernel = blk.split()[0]
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", blk)
        assert m, kernel
        if int(m.group(1)):
            bad.append((kernel[:90], int(m.group(1))))
    assert not bad, bad
