"""One connection driven from several streams in turn.  Each hardware queue
deals a launch's blocks to the XCDs from a start XCD of its own, and the
paired launch shape places its workgroups by the XCD id each block reads;
whatever the stream, every transfer must match the oracle byte for byte,
counters and FIFO included."""
import re

import numpy as np
import pytest

import oracle
from gpu_cases import compare_state, log, oracle_proto, payload, to_dev, to_host
import recv_fifo_plane_amd as xf

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("proto,nch,nslots,slot,lanes,pairing", [
    ("simple", 4, 4, 4096, 2, 1),
    ("ll", 3, 8, 4096, 1, 1),
    ("zc", 4, 1, 4096, 2, 1),
    ("zcd", 5, 1, 4096, 1, 1),
    ("simple", 4, 4, 4096, 2, -1),
])
def test_same_connection_from_several_streams(proto, nch, nslots, slot, lanes, pairing):
    import torch
    log("case: streams %s nch=%d lanes=%d pairing=%d" % (proto, nch, lanes, pairing))
    conn = xf.Conn(proto, nch, nslots, slot, "device", wgs_per_channel=lanes,
                   block_threads=128, xcd_pairing=pairing)
    ocn = oracle.Conn(oracle_proto(proto, "device"), nch, nslots, slot)
    streams = [torch.cuda.Stream() for _ in range(6)] + [torch.cuda.current_stream()]
    try:
        for t, st in enumerate(streams):
            n = 50000 + 977 * t
            A = payload("uint8", n, 4242 + t)
            a = to_dev(A)
            b = torch.zeros_like(a)
            torch.cuda.synchronize()
            conn.run(a, b, n, st)
            st.synchronize()
            B = np.zeros_like(A)
            ocn.run(A, B, n)
            assert np.array_equal(to_host(b), B), (proto, "stream", t)
        compare_state(conn, ocn, nch, "streams " + proto)
    finally:
        torch.cuda.synchronize()
        conn.close()
        ocn.close()


def _resident_capacity(block: int) -> int:
    """Workgroups of `block` threads the GPU holds resident, from the
    refusal of a grid that cannot be (the refusal names the capacity)."""
    import torch
    c = xf.Conn("simple", 64, 1, 4096, wgs_per_channel=16, block_threads=block, xcd_pairing=-1)
    a = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    b = torch.zeros_like(a)
    try:
        with pytest.raises(xf.XferError) as e:
            c.run(a, b, 1 << 20)
    finally:
        c.close()
    m = re.search(r"exceed the (\d+)", str(e.value))
    assert m, str(e.value)
    return int(m.group(1))


def test_launches_whose_grids_do_not_fit_together():
    # Two connections on two streams, each grid fitting the GPU alone but
    # not both at once: the library's launches run one at a time on a
    # device, so neither is left partly resident waiting on the other.
    import torch
    block = 1024
    cap = _resident_capacity(block)
    pairs = cap * 3 // 8  # each grid 3/4 of the capacity
    lanes = min(16, pairs)
    nch = min(64, pairs // lanes)
    grid = 2 * nch * lanes
    log("case: two grids of %d workgroups on two streams, capacity %d" % (grid, cap))
    assert grid <= cap < 2 * grid
    conns = [xf.Conn("simple", nch, 2, 65536, "device", wgs_per_channel=lanes,
                     block_threads=block, xcd_pairing=-1) for _ in range(2)]
    ocns = [oracle.Conn("simple", nch, 2, 65536) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    try:
        for rnd in range(3):
            n = (8 << 20) + 4099 * rnd
            As = [payload("uint8", n, 777 + 2 * rnd + k) for k in range(2)]
            ds = [to_dev(A) for A in As]
            bs = [torch.zeros_like(d) for d in ds]
            torch.cuda.synchronize()
            for k in range(2):  # queued back to back, no synchronisation between them
                conns[k].run(ds[k], bs[k], n, streams[(k + rnd) % 2])
            torch.cuda.synchronize()
            for k in range(2):
                B = np.zeros_like(As[k])
                ocns[k].run(As[k], B, n)
                assert np.array_equal(to_host(bs[k]), B), ("round", rnd, "connection", k)
        for k in range(2):
            compare_state(conns[k], ocns[k], nch, "grids that do not fit together %d" % k)
    finally:
        torch.cuda.synchronize()
        for c in conns:
            c.close()
        for o in ocns:
            o.close()


def _hip_runtime():
    """The HIP runtime this process already runs on (torch's), by path, so
    no second copy is loaded."""
    import ctypes
    with open("/proc/self/maps", encoding="utf-8") as f:
        for line in f:
            if "libamdhip64" in line:
                return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("no HIP runtime mapped")


def test_launches_on_streams_destroyed_right_after_use():
    # Each launch goes to a new stream that is destroyed at once; a new
    # stream may reuse a destroyed one's handle.  Grids again fit the GPU
    # one at a time only.
    import ctypes
    import torch
    hip = _hip_runtime()
    block = 1024
    cap = _resident_capacity(block)
    pairs = cap * 3 // 8
    lanes = min(16, pairs)
    nch = min(64, pairs // lanes)
    log("case: launches on destroyed streams, grids of %d of %d" % (2 * nch * lanes, cap))
    conns = [xf.Conn("simple", nch, 2, 65536, "device", wgs_per_channel=lanes,
                     block_threads=block, xcd_pairing=-1) for _ in range(2)]
    ocns = [oracle.Conn("simple", nch, 2, 65536) for _ in range(2)]
    try:
        n = 4 << 20
        As, bs = [], []
        for i in range(6):
            A = payload("uint8", n, 900 + i)
            d = to_dev(A)
            b = torch.zeros_like(d)
            torch.cuda.synchronize()
            h = ctypes.c_void_p()
            assert hip.hipStreamCreate(ctypes.byref(h)) == 0
            conns[i % 2].run(d, b, n, h.value)
            assert hip.hipStreamDestroy(h) == 0
            As.append((A, d))
            bs.append(b)
        torch.cuda.synchronize()
        for i in range(6):
            B = np.zeros_like(As[i][0])
            ocns[i % 2].run(As[i][0], B, n)
            assert np.array_equal(to_host(bs[i]), B), ("launch", i)
        for k in range(2):
            compare_state(conns[k], ocns[k], nch, "destroyed streams %d" % k)
    finally:
        torch.cuda.synchronize()
        for c in conns:
            c.close()
        for o in ocns:
            o.close()
