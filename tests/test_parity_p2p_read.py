"""GPU parity of P2P read: the SIMPLE FIFO lives in the send side's memory,
after its head/ptrExchange blocks, and tail in the receive side's own blocks
("transport建立", p2pSendSetup and p2pRecvConnect listings).  The protocol
is unchanged, so destination (with guards), counters and FIFO bytes must
equal the oracle's SIMPLE mode exactly, alone, in a batch with write-mode
connections and in the ping-pong kernel."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import compare_state, log, run_transfers, to_dev, to_host

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 15, 16, 17, 4095, 4096, 4097, 65536 + 13, 300_001]


@pytest.mark.parametrize("nch,nslots,lanes", [(1, 1, 1), (1, 3, 2), (3, 2, 1), (4, 8, 3)])
def test_p2p_read(nch, nslots, lanes):
    run_transfers("simple", nch, nslots, 4096, SIZES, lanes=lanes, p2p_read=1)


@pytest.mark.parametrize("src_off,dst_off", [(1, 0), (5, 11), (15, 1)])
def test_p2p_read_misaligned(src_off, dst_off):
    run_transfers("simple", 2, 3, 512, [1, 100, 5000, 33333], lanes=2, src_off=src_off,
                  dst_off=dst_off, p2p_read=1)


@pytest.mark.parametrize("block,ordering", [(64, 0), (1024, 0), (256, 1)])
def test_p2p_read_shapes_and_ordering(block, ordering):
    run_transfers("simple", 2, 4, 8192, [100_000, 7], block=block, lanes=2, ordering=ordering,
                  p2p_read=1)


def test_p2p_read_in_a_batch_with_write_mode():
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    n = 3 << 20
    log("case: P2P read + write in one batch")
    A = synth.uint8_uniform(2 * n, 41)
    a = to_dev(A)
    b = torch.zeros_like(a)
    rd = xf.Conn("simple", 4, 4, 64 << 10, "device", wgs_per_channel=2, p2p_read=1)
    wr = xf.Conn("simple", 4, 4, 64 << 10, "device", wgs_per_channel=2)
    for _ in range(2):
        X.run_batch([rd, wr], [a.data_ptr(), a.data_ptr() + n], [b.data_ptr(), b.data_ptr() + n],
                    [n, n])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(b), A)
    for conn, half in ((rd, A[:n]), (wr, A[n:])):
        o = oracle.Conn("simple", 4, 4, 64 << 10)
        B = np.zeros(n, dtype=np.uint8)
        for _ in range(2):
            o.run(np.ascontiguousarray(half), B)
        compare_state(conn, o, 4, "batch")
        o.close()
    rd.close()
    wr.close()


@pytest.mark.parametrize("size", [8, 300_001])
def test_p2p_read_pingpong(size):
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    log("case: P2P read ping-pong size=%d" % size)
    A = synth.uint8_uniform(size, 1300 + size)
    conns = [xf.Conn("simple", 2, 4, 16 << 10, "device", wgs_per_channel=2, block_threads=256,
                     p2p_read=1) for _ in range(2)]
    ocs = [oracle.Conn("simple", 2, 4, 16 << 10) for _ in range(2)]
    a = to_dev(A)
    b = torch.zeros_like(a)
    c = torch.zeros_like(a)
    X.run_pingpong(conns[0], conns[1], a, b, c, size, 30)
    torch.cuda.synchronize()
    ob, oc = np.zeros_like(A), np.zeros_like(A)
    oracle.run_pingpong(ocs[0], ocs[1], A, ob, oc, size, 30)
    assert np.array_equal(to_host(b), ob) and np.array_equal(to_host(c), oc)
    compare_state(conns[0], ocs[0], 2, "fwd")
    compare_state(conns[1], ocs[1], 2, "rev")
    for x in conns + ocs:
        x.close()
