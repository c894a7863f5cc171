"""GPU parity of LL connections in the striped line layout: where a whole
step fits the lanes at one line per thread, lane w owns a stripe of every
slot's lines and its waves cover several steps at once (groups of up to
nslots steps, one head store per group).  Destination (with guards),
counters and FIFO bytes must equal the oracle's for every shape: groups of
1 to 4 steps, stripes rounded up past the step's lines (lanes that own no
line), one slot, host-memory FIFOs, message lists, the ping-pong and
jitter."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import compare_state, log, run_message_list, run_transfers, to_dev, to_host

pytestmark = pytest.mark.gpu

# (nch, nslots, slot_bytes, lanes, block, fifo_loc): stripe q and group m
SHAPES = [
    (1, 8, 32768, 16, 1024, "device"),  # the ping-pong workload: q 256, m 4
    (2, 3, 8192, 2, 1024, "device"),    # q 512, m 2
    (3, 2, 4096, 3, 512, "device"),     # 512 lines over 3 lanes: q 256, lane 2 owns none
    (2, 1, 4096, 2, 1024, "device"),    # one slot: groups of one step
    (1, 8, 1024, 1, 256, "device"),     # q 128, m 2
    (2, 4, 8192, 2, 1024, "host"),      # q 512, m 2, FIFO in pinned host memory
]


def _sizes(slot, nch):
    S = slot // 2
    return [1, 7, 4099, nch * S * 5 + 5, 100_001, nch * S * 2]


@pytest.mark.parametrize("shape", SHAPES, ids=["-".join(map(str, s)) for s in SHAPES])
def test_striped_transfers_match_oracle(shape):
    nch, nslots, slot, lanes, block, loc = shape
    run_transfers("ll", nch, nslots, slot, _sizes(slot, nch), fifo_loc=loc, lanes=lanes,
                  block=block, kind="int32", label="striped")


@pytest.mark.parametrize("shape", SHAPES[:3], ids=["-".join(map(str, s)) for s in SHAPES[:3]])
@pytest.mark.parametrize("seed", [3, 0xC0FFEE])
def test_striped_under_jitter(shape, seed):
    nch, nslots, slot, lanes, block, loc = shape
    run_transfers("ll", nch, nslots, slot, _sizes(slot, nch)[:5], fifo_loc=loc, lanes=lanes,
                  block=block, jitter=seed, label="striped jitter")


def test_striped_message_list():
    sizes = [5, 40000, 1, 16384, 65536, 3, 99_999]
    run_message_list("ll", 2, 3, 8192, sizes, lanes=2, block=1024, repeat=2)


# 100 003 bytes: seven steps, so a round is two groups of the four steps a
# lane's waves cover (endpoint X loads the first group's source words ahead)
@pytest.mark.parametrize("size", [8, 16384, 16385, 65536, 100_003])
@pytest.mark.parametrize("jitter", [0, 0x7A11])
def test_striped_pingpong_matches_oracle(size, jitter):
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    iters = 40
    log("case: striped ping-pong %d jitter=%#x" % (size, jitter))
    A = synth.int32_uniform_bytes(size, 11 + size)
    conns = [xf.Conn("ll", 1, 8, 32768, wgs_per_channel=16, block_threads=1024)
             for _ in range(2)]
    if jitter:
        for i, c in enumerate(conns):
            c.set_jitter(jitter + i)
    ocs = [oracle.Conn("ll", 1, 8, 32768) for _ in range(2)]
    a = to_dev(A)
    b = torch.zeros_like(a)
    c = torch.zeros_like(a)
    X.run_pingpong(conns[0], conns[1], a, b, c, size, iters)
    torch.cuda.synchronize()
    ob, oc = np.zeros_like(A), np.zeros_like(A)
    oracle.run_pingpong(ocs[0], ocs[1], A, ob, oc, size, iters)
    assert np.array_equal(to_host(b), ob) and np.array_equal(to_host(c), oc)
    compare_state(conns[0], ocs[0], 1, "striped fwd")
    compare_state(conns[1], ocs[1], 1, "striped rev")
    for x in conns + ocs:
        x.close()
