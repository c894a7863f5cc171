"""GPU parity of SIMPLE waits on control words in host memory.  There one
wave per workgroup polls the counter and hands its value to the other waves
through LDS, so workgroups of one, two and sixteen waves must give the same
destination, counters and FIFO bytes as the oracle, in plain transfers and in
the ping-pong kernel (send then receive in one workgroup)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import compare_state, log, run_transfers, to_dev, to_host

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 4097, 100_003, 1 << 20]


@pytest.mark.parametrize("block", [64, 128, 1024])
@pytest.mark.parametrize("fifo_loc", ["device", "host"])
def test_host_counters_any_workgroup_size(block, fifo_loc):
    run_transfers("simple", 3, 2, 8192, SIZES, fifo_loc=fifo_loc, lanes=2, block=block,
                  ctrl_loc=2)


@pytest.mark.parametrize("fifo_loc,ctrl_loc", [("device", 1), ("device", 2), ("host", 2)])
@pytest.mark.parametrize("size", [8, 4097, 300_001])
def test_simple_pingpong(fifo_loc, ctrl_loc, size):
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    nch, nslots, slot, lanes, iters = 2, 4, 16 << 10, 2, 40
    log("case: SIMPLE ping-pong %s ctrl=%d size=%d" % (fifo_loc, ctrl_loc, size))
    A = synth.uint8_uniform(size, 900 + size)
    conns = [xf.Conn("simple", nch, nslots, slot, fifo_loc, wgs_per_channel=lanes,
                     block_threads=256, ctrl_loc=ctrl_loc) for _ in range(2)]
    ocs = [oracle.Conn("simple", nch, nslots, slot) for _ in range(2)]
    a = to_dev(A)
    b = torch.zeros_like(a)
    c = torch.zeros_like(a)
    X.run_pingpong(conns[0], conns[1], a, b, c, size, iters)
    torch.cuda.synchronize()
    ob, oc = np.zeros_like(A), np.zeros_like(A)
    oracle.run_pingpong(ocs[0], ocs[1], A, ob, oc, size, iters)
    assert np.array_equal(to_host(b), ob) and np.array_equal(to_host(c), oc)
    compare_state(conns[0], ocs[0], nch, "fwd")
    compare_state(conns[1], ocs[1], nch, "rev")
    for x in conns + ocs:
        x.close()
