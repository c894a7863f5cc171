"""The entry point that allocates nothing (xfer_run_noalloc), through the C
ABI: two calls in a row, the second with a smaller input, each compared
byte for byte with xfer_run on a new connection of the same shape and with
the source, guard bytes around the destination included."""
import numpy as np
import pytest

import recv_fifo_plane_amd as xf
from recv_fifo_plane_amd import xfer as X
from gpu_cases import GUARD, log, payload, to_dev, to_host
import synth

pytestmark = pytest.mark.gpu

# (proto, nchannels, nslots, slot_bytes, lanes, block): FIFOs of 1 MiB
# (SIMPLE), 512 KiB (LL) and none (zero-copy), several steps per channel.
SHAPES = [
    ("simple", 4, 4, 65536, 2, 256),
    ("ll", 4, 4, 32768, 2, 256),
    ("ll", 2, 4, 8192, 2, 1024),  # striped lines: 512-line stripes, groups of 2 steps
    ("zc", 4, 1, 65536, 2, 128),
    ("zcd", 3, 1, 65536, 1, 256),
]


def _run_both(proto, nch, nslots, slot, lanes, block, n, src_off, dst_off, seed):
    import torch
    A = payload("uint8", n, seed)
    src = np.zeros(n + 32, dtype=np.uint8)
    src[src_off:src_off + n] = A
    dstb = synth.guard_pattern(n + 2 * GUARD + 16, seed=seed)
    ds = to_dev(src)
    d_noalloc = to_dev(dstb)
    d_run = to_dev(dstb)
    status = torch.full((1,), 0x7777, dtype=torch.int32, device="cuda")
    X.run_noalloc(proto, nch, nslots, slot, ds.data_ptr() + src_off,
                  d_noalloc.data_ptr() + GUARD + dst_off, n, status=status,
                  wgs_per_channel=lanes, block_threads=block)
    conn = xf.Conn(proto, nch, nslots, slot, wgs_per_channel=lanes, block_threads=block)
    conn.run(ds.data_ptr() + src_off, d_run.data_ptr() + GUARD + dst_off, n)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, (proto, n, int(status.item()))
    got, want = to_host(d_noalloc), to_host(d_run)
    expect = dstb.copy()
    expect[GUARD + dst_off:GUARD + dst_off + n] = A
    assert np.array_equal(want, expect), (proto, n, "xfer_run")
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (proto, n, "xfer_run_noalloc differs from xfer_run", bad.size, bad[:8])
    for c in range(nch):
        assert conn.query(c)["error"] == 0
    conn.close()


@pytest.mark.parametrize("shape", SHAPES, ids=["-".join(map(str, s)) for s in SHAPES])
def test_noalloc_matches_run_on_two_calls(shape):
    proto, nch, nslots, slot, lanes, block = shape
    log("case: noalloc %s nch=%d nslots=%d slot=%d lanes=%d" % shape[:5])
    # the first call larger (several steps per channel, ragged tail), the
    # second smaller and at odd offsets (the unaligned kernel variant)
    _run_both(proto, nch, nslots, slot, lanes, block, (3 << 20) + 37, 0, 0, 101)
    _run_both(proto, nch, nslots, slot, lanes, block, 70001, 3, 5, 202)


def test_noalloc_rejects_a_fifo_beyond_its_array():
    import torch
    a = torch.randint(0, 256, (4096,), dtype=torch.uint8, device="cuda")
    b = torch.zeros_like(a)
    room = X.NOALLOC_SCRATCH_BYTES - (1 << 20)
    with pytest.raises(xf.XferError) as e:
        X.run_noalloc("simple", 2, 8, room // 8, a, b, 4096)  # 2x the room
    assert e.value.status == X.XFER_ERR_INVALID_ARG
    X.run_noalloc("simple", 1, 8, room // 8, a, b, 4096)  # exactly the room: accepted
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# The callers the entry point is for include code under HIP graph capture:
# one call captured (its clearing kernel, the transfer and the report kernel
# become graph nodes) must redo the whole transfer on every replay, with the
# program's own eager work and synchronisations between the replays.
@pytest.mark.parametrize("proto,nch,nslots,slot,lanes,block", [
    ("simple", 4, 4, 65536, 2, 256),
    ("ll", 2, 4, 8192, 2, 1024),
    ("zc", 4, 1, 65536, 2, 128),
])
def test_noalloc_replays_in_a_captured_graph(proto, nch, nslots, slot, lanes, block):
    import torch
    n = (1 << 20) + 37
    log("case: graph %s" % proto)
    a = to_dev(synth.uint8_uniform(n, 9))
    b = torch.zeros_like(a)
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    kw = dict(wgs_per_channel=lanes, block_threads=block)
    # the first call on a device takes the array's address and the capacity
    X.run_noalloc(proto, nch, nslots, slot, a, b, n, status=status, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and int(status.item()) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        X.run_noalloc(proto, nch, nslots, slot, a, b, n, status=status, **kw)
    for r in range(4):
        # eager work between replays: new source bytes, cleared destination
        a.copy_(to_dev(synth.uint8_uniform(n, 100 + r)))
        b.zero_()
        status.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(a, b), (proto, "replay", r)
        assert int(status.item()) == 0, (proto, "replay", r, int(status.item()))
