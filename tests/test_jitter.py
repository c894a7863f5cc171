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


def test_zero_copy_ring_batch_under_jitter():
    import torch

    from recv_fifo_plane_amd import workloads as W
    cfg = dict(W.W4_RING, slice_bytes=3 << 20)
    log("case: zero-copy ring under jitter")
    ring = W.make_ring(cfg)
    for i, e in enumerate(ring.edges.values()):
        e.set_jitter(0xA11CE + i)
    n = 8 * cfg["slice_bytes"]
    a = torch.from_numpy(synth.uint8_uniform(n, 5)).to("cuda")
    b = torch.zeros_like(a)
    for _ in range(2):
        ring.run(a, b)
    torch.cuda.synchronize()
    S = cfg["slice_bytes"]
    for r in range(8):
        d = (r + 1) % 8
        assert torch.equal(a[r * S:(r + 1) * S], b[d * S:(d + 1) * S]), r
    for e in ring.edges.values():
        for ch in range(cfg["channels_per_edge"]):
            st = e.query(ch)
            assert st["error"] == 0 and st["head"] == st["tail"] and st["ptr_exchange"] == 0
    ring.close()
