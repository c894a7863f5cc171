"""GPU parity under jitter (xfer_conn_set_jitter): every wave sleeps a
pseudo-random time where a step is acquired and where it is published, so
producer and consumer, and the waves of one side, reach the shared words in
orders that undisturbed runs rarely take.  The destination (with guards),
counters and FIFO bytes must still equal the oracle's exactly, for every
protocol and FIFO placement, for several seeds; so must the ping-pong and
the zero-copy ring batch."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import compare_state, log, run_transfers, to_dev, to_host

pytestmark = pytest.mark.gpu

SIZES = [1, 17, 4097, 65536 + 13, 200_001]
SEEDS = [1, 0xBEEF, 0x9E3779B9]


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("proto,fifo_loc", [("simple", "device"), ("simple", "host"),
                                            ("simple", "relay"), ("ll", "device"),
                                            ("ll", "host"), ("zc", "device"), ("zcd", "device")])
def test_parity_under_jitter(proto, fifo_loc, seed):
    slot = 2048 if proto == "ll" else 4096
    run_transfers(proto, 3, 2, slot, SIZES, fifo_loc=fifo_loc, lanes=2, jitter=seed,
                  kind="int32" if proto == "ll" else "uint8")


@pytest.mark.parametrize("seed", SEEDS)
def test_one_slot_under_jitter(seed):
    # a single slot: every step waits on the previous one's head
    for proto in ("simple", "ll"):
        run_transfers(proto, 2, 1, 1024, [50_000], lanes=3, block=128, jitter=seed)


@pytest.mark.parametrize("proto", ["simple", "ll"])
def test_pingpong_under_jitter(proto):
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    size, iters = 10_001, 25
    log("case: %s ping-pong under jitter" % proto)
    A = synth.uint8_uniform(size, 77)
    conns = [xf.Conn(proto, 2, 4, 8192, wgs_per_channel=2) for _ in range(2)]
    for i, c in enumerate(conns):
        c.set_jitter(0x51ED + i)
    ocs = [oracle.Conn(proto, 2, 4, 8192) for _ in range(2)]
    a = to_dev(A)
    b = torch.zeros_like(a)
    c = torch.zeros_like(a)
    X.run_pingpong(conns[0], conns[1], a, b, c, size, iters)
    torch.cuda.synchronize()
    ob, oc = np.zeros_like(A), np.zeros_like(A)
    oracle.run_pingpong(ocs[0], ocs[1], A, ob, oc, size, iters)
    assert np.array_equal(to_host(b), ob) and np.array_equal(to_host(c), oc)
    compare_state(conns[0], ocs[0], 2, "fwd")
    compare_state(conns[1], ocs[1], 2, "rev")
    for x in conns + ocs:
        x.close()


@pytest.mark.parametrize("proto", ["zc", "zcd"])
def test_zero_copy_ring_batch_under_jitter(proto):
    # every edge of the ring, after two batches under jitter, must hold the
    # oracle's counters (and B the oracle's bytes)
    import torch

    from recv_fifo_plane_amd import workloads as W
    cfg = dict(W.W4_RING if proto == "zc" else W.W4D_RING, slice_bytes=3 << 20)
    log("case: %s ring under jitter" % proto)
    ring = W.make_ring(cfg)
    for i, e in enumerate(ring.edges.values()):
        e.set_jitter(0xA11CE + i)
    S = cfg["slice_bytes"]
    nch = cfg["channels_per_edge"]
    A = synth.uint8_uniform(8 * S, 5)
    a = to_dev(A)
    b = torch.zeros_like(a)
    ocns = {k: oracle.Conn(proto, nch, 1, cfg["slot_bytes"]) for k in ring.edges}
    B = np.zeros_like(A)
    for _ in range(2):
        ring.run(a, b)
        for (r, d), o in ocns.items():
            o.run(np.ascontiguousarray(A[r * S:(r + 1) * S]), B[d * S:(d + 1) * S])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(b), B)
    for k, e in ring.edges.items():
        compare_state(e, ocns[k], nch, "%s ring under jitter, edge %s" % (proto, k))
        ocns[k].close()
    ring.close()
