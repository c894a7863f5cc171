"""GPU parity of the copy-engine relay (the shm transport's memcpy mode): the
producer fills a send FIFO in HBM, a host send proxy moves each step into a
pinned staging FIFO with a device-to-host copy, a host receive proxy moves it
on into a receive FIFO in HBM with a host-to-device copy, and the consumer
drains that.  Destination (with guards), counters, all three FIFOs and both
proxy tails must equal the oracle's relay mode."""
import time

import numpy as np
import pytest

import oracle
import synth
from gpu_cases import log, run_message_list, run_transfers

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 15, 16, 17, 4095, 4096, 4097, 65536 + 13, 300_001]


@pytest.mark.parametrize("nch,nslots,lanes", [(1, 1, 1), (1, 3, 2), (3, 2, 1), (4, 8, 3)])
def test_relay(nch, nslots, lanes):
    run_transfers("simple", nch, nslots, 4096, SIZES, fifo_loc="relay", lanes=lanes)


@pytest.mark.parametrize("src_off,dst_off", [(1, 0), (5, 11), (15, 1)])
def test_relay_misaligned(src_off, dst_off):
    run_transfers("simple", 2, 3, 512, [1, 100, 5000, 33333], fifo_loc="relay", lanes=2,
                  src_off=src_off, dst_off=dst_off)


@pytest.mark.parametrize("block", [64, 1024])
def test_relay_block_sizes(block):
    run_transfers("simple", 2, 4, 8192, [100_000, 7], fifo_loc="relay", block=block, lanes=2)


def test_relay_many_steps_through_few_slots():
    # every slot of all three FIFOs is reused many times
    run_transfers("simple", 4, 1, 1024, [1 << 20], fifo_loc="relay", lanes=2)
    run_transfers("simple", 8, 2, 64 << 10, [16 << 20, 5], fifo_loc="relay", lanes=4, block=512)


def test_relay_message_list():
    sizes = synth.log_uniform_message_sizes(6 << 20, 21, lo_exp=0, hi_exp=17)[:200]
    run_message_list("simple", 4, 3, 16 << 10, sizes, fifo_loc="relay", lanes=2, base_off=3,
                     repeat=2)


def test_relay_in_a_batch_with_plain_connections():
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    n = 3 << 20
    A = synth.uint8_uniform(2 * n, 31)
    a = torch.from_numpy(A).to("cuda")
    b = torch.zeros_like(a)
    r = xf.Conn("simple", 4, 4, 64 << 10, "relay", wgs_per_channel=2, ctrl_loc=2)
    d = xf.Conn("simple", 4, 4, 64 << 10, "device", wgs_per_channel=2, ctrl_loc=2)
    for _ in range(2):
        X.run_batch([r, d], [a.data_ptr(), a.data_ptr() + n], [b.data_ptr(), b.data_ptr() + n],
                    [n, n])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    o = oracle.Conn("relay", 4, 4, 64 << 10)
    B = np.zeros(n, dtype=np.uint8)
    for _ in range(2):
        o.run(np.ascontiguousarray(A[:n]), B)
    for ch in range(4):
        st, want = r.query(ch), o.state(ch)
        assert (st["head"], st["tail"], st["error"]) == (want["head"], want["tail"], 0)
        assert r.query_relay(ch)["recv_proxy_tail"] == o.relay_state(ch)["recv_proxy_tail"]
        for which in range(3):
            assert np.array_equal(r.read_fifo(ch, which), o.fifo(ch, which)), (ch, which)
    r.close()
    d.close()
    o.close()


def test_relay_lone_producer_times_out_and_the_proxies_let_go():
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    log("case: relay lone producer")
    c = xf.Conn("simple", 2, 2, 4096, "relay", timeout_ms=50, roles=1)
    a = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    b = torch.zeros_like(a)
    t0 = time.time()
    c.run(a, b, 1 << 16)
    torch.cuda.synchronize()
    assert time.time() - t0 < 5.0
    st = c.query(0)
    assert st["error"] == X.XFER_ERR_TIMEOUT
    # the proxies relayed what the producer published: its two credited steps
    assert c.query_relay(0)["recv_proxy_tail"] == 2
    with pytest.raises(xf.XferError) as e:
        c.run(a, b, 1 << 16)
    assert e.value.status == X.XFER_ERR_STATE
    c.close()  # joins the proxies


def test_relay_abort_ends_waits():
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    c = xf.Conn("simple", 1, 2, 4096, "relay", timeout_ms=4000, roles=2)
    a = torch.zeros(1 << 14, dtype=torch.uint8, device="cuda")
    b = torch.zeros_like(a)
    c.abort()
    t0 = time.time()
    c.run(a, b, 1 << 14)
    torch.cuda.synchronize()
    assert time.time() - t0 < 3.0
    assert c.query(0)["error"] == X.XFER_ERR_ABORTED
    c.close()


def test_relay_connections_come_and_go():
    # the proxy threads start with each connection and are joined by its
    # destruction, also with runs queued behind each other
    import torch

    import recv_fifo_plane_amd as xf
    a = torch.from_numpy(synth.uint8_uniform(1 << 20, 8)).to("cuda")
    for i in range(12):
        b = torch.zeros_like(a)
        c = xf.Conn("simple", 2, 2, 16 << 10, "relay")
        for _ in range(3):
            c.run(a, b, a.numel() - i)
        torch.cuda.synchronize()
        assert torch.equal(a[:a.numel() - i], b[:a.numel() - i])
        c.close()


def test_relay_refuses_pingpong_and_bad_reads():
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    f = xf.Conn("simple", 1, 2, 4096, "relay")
    r = xf.Conn("simple", 1, 2, 4096, "relay")
    a = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(xf.XferError) as e:
        X.run_pingpong(f, r, a, torch.zeros_like(a), torch.zeros_like(a), 64, 1)
    assert e.value.status == X.XFER_ERR_INVALID_ARG
    d = xf.Conn("simple", 1, 2, 4096, "device")
    with pytest.raises(xf.XferError):
        d.read_fifo(0, 1)  # a plain connection has one FIFO
    with pytest.raises(xf.XferError):
        d.query_relay(0)
    for c in (f, r, d):
        c.close()
