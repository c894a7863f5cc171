"""Connections created with xfer_attr.cooperative = 1 launch their grids
cooperatively (every workgroup resident at once, or the launch is refused).
The kernels are the same, so every result must still equal the oracle's
byte for byte, counters and FIFO included; a batch or ping-pong must not
mix cooperative and ordinary connections."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import compare_state, log, run_transfers, to_dev, to_host
import recv_fifo_plane_amd as xf
from recv_fifo_plane_amd import workloads as W
from recv_fifo_plane_amd import xfer as X

pytestmark = pytest.mark.gpu

SIZES = [1, 4097, 300_001]


@pytest.mark.parametrize("proto,fifo_loc,slot,lanes,block", [
    ("simple", "device", 65536, 4, 768),
    ("simple", "host", 16384, 2, 256),
    ("simple", "relay", 65536, 2, 256),
    ("ll", "device", 8192, 2, 1024),   # striped lines, groups of 2 steps
    ("ll", "device", 32768, 2, 256),   # block layout
    ("zc", "device", 65536, 4, 128),
    ("zcd", "device", 65536, 4, 128),
])
def test_cooperative_transfers_match_oracle(proto, fifo_loc, slot, lanes, block):
    run_transfers(proto, 4, 4 if proto in ("simple", "ll") else 1, slot, SIZES, fifo_loc=fifo_loc,
                  lanes=lanes, block=block, cooperative=1, label="cooperative")


def test_cooperative_ring_batch_matches_oracle():
    import torch
    cfg = dict(W.W4_RING, slice_bytes=4 << 20, cooperative=1)
    log("case: cooperative ring " + str(cfg))
    ring = W.make_ring(cfg)
    n, sl = cfg["endpoints"], cfg["slice_bytes"]
    A = synth.fp32_uniform_bytes(n * sl, 31)
    a = to_dev(A)
    b = torch.zeros_like(a)
    try:
        for _ in range(2):
            ring.run(a, b)
            torch.cuda.synchronize()
        got = to_host(b)
        for r in range(n):
            d = (r + 1) % n
            assert np.array_equal(got[d * sl:(d + 1) * sl], A[r * sl:(r + 1) * sl]), r
            ocn = oracle.Conn("zc", cfg["channels_per_edge"], 1, cfg["slot_bytes"])
            B = np.zeros(sl, dtype=np.uint8)
            for _ in range(2):
                ocn.run(np.ascontiguousarray(A[r * sl:(r + 1) * sl]), B)
            compare_state(ring.edges[(r, d)], ocn, cfg["channels_per_edge"], "cooperative ring %d" % r)
            ocn.close()
    finally:
        torch.cuda.synchronize()
        ring.close()


@pytest.mark.parametrize("proto", ["simple", "ll"])
def test_cooperative_pingpong_matches_oracle(proto):
    import torch
    size, iters = 70_001, 20
    log("case: cooperative %s ping-pong" % proto)
    A = synth.int32_uniform_bytes(size, 5)
    conns = [xf.Conn(proto, 2, 4, 16384, wgs_per_channel=4, block_threads=1024, cooperative=1)
             for _ in range(2)]
    ocs = [oracle.Conn(proto, 2, 4, 16384) for _ in range(2)]
    a = to_dev(A)
    b = torch.zeros_like(a)
    c = torch.zeros_like(a)
    try:
        X.run_pingpong(conns[0], conns[1], a, b, c, size, iters)
        torch.cuda.synchronize()
        ob, oc = np.zeros_like(A), np.zeros_like(A)
        oracle.run_pingpong(ocs[0], ocs[1], A, ob, oc, size, iters)
        assert np.array_equal(to_host(b), ob) and np.array_equal(to_host(c), oc)
        compare_state(conns[0], ocs[0], 2, "cooperative fwd")
        compare_state(conns[1], ocs[1], 2, "cooperative rev")
    finally:
        torch.cuda.synchronize()
        for x in conns + ocs:
            x.close()


def test_batch_and_pingpong_refuse_mixed_launch_kinds():
    import torch
    a = torch.zeros(8192, dtype=torch.uint8, device="cuda")
    b = torch.zeros_like(a)
    c = torch.zeros_like(a)
    coop = xf.Conn("simple", 1, 4, 4096, cooperative=1)
    plain = xf.Conn("simple", 1, 4, 4096)
    try:
        with pytest.raises(xf.XferError) as e:
            X.run_batch([coop, plain], [a.data_ptr(), a.data_ptr() + 4096],
                        [b.data_ptr(), b.data_ptr() + 4096], [4096, 4096])
        assert e.value.status == X.XFER_ERR_INVALID_ARG
        with pytest.raises(xf.XferError) as e:
            X.run_pingpong(coop, plain, a, b, c, 4096, 1)
        assert e.value.status == X.XFER_ERR_INVALID_ARG
        for x in (coop, plain):
            st = x.query(0)
            assert (st["head"], st["tail"], st["error"]) == (0, 0, 0), st
    finally:
        torch.cuda.synchronize()
        coop.close()
        plain.close()
