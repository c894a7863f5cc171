"""The paired launch shape places workgroups by the XCD id they read when
the device deals blocks to 8 XCDs in strict rotation, and by block index
otherwise (XFER_XCD_BY_ID=0 forces the latter).  Both placements are
permutations of the grid: every transfer must match the oracle either way.
The forced run is a child process, since the choice is made once per
device."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys
sys.path.insert(0, %(root)r)
sys.path.insert(0, %(tests)r)
import torch
from gpu_cases import run_transfers
for proto, nch, nslots, slot, lanes in (("simple", 4, 4, 4096, 2), ("ll", 3, 8, 4096, 1),
                                        ("zc", 4, 1, 4096, 2), ("zcd", 3, 1, 4096, 1)):
    run_transfers(proto, nch, nslots, slot, [1, 4097, 100_003], lanes=lanes, block=128,
                  xcd_pairing=1, label="by block index")
print("child ok", flush=True)
'''


def test_paired_placement_by_block_index_matches_oracle():
    env = dict(os.environ, XFER_XCD_BY_ID="0")
    code = CHILD % {"root": ROOT, "tests": os.path.join(ROOT, "tests")}
    r = subprocess.run([sys.executable, "-u", "-c", code], env=env, cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=150)
    print(r.stdout[-3000:])
    assert r.returncode == 0 and "child ok" in r.stdout
