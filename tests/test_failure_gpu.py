"""Failure handling, forced from the host so every kernel still exits
normally: one side switched off makes the other side's bounded wait end
with XFER_ERR_TIMEOUT (or XFER_ERR_ABORTED once the host abort word is set);
the connection then refuses further runs."""
import time

import pytest

import recv_fifo_plane_amd as xf
from recv_fifo_plane_amd import xfer as X
from gpu_cases import log

pytestmark = pytest.mark.gpu


def _bufs(n):
    import torch
    return torch.zeros(n, dtype=torch.uint8, device="cuda"), torch.zeros(n, dtype=torch.uint8,
                                                                          device="cuda")


@pytest.mark.parametrize("proto,roles", [("simple", 1), ("simple", 2), ("ll", 1), ("ll", 2),
                                         ("zc", 1), ("zc", 2), ("zcd", 2)])
def test_lone_side_times_out(proto, roles):
    import torch
    log("case: lone side %s roles=%d" % (proto, roles))
    c = xf.Conn(proto, 2, 2, 4096, timeout_ms=20, roles=roles)
    a, b = _bufs(1 << 16)
    t0 = time.time()
    c.run(a, b, 1 << 16)
    torch.cuda.synchronize()
    assert time.time() - t0 < 5.0
    # a lone producer runs out of credit (16 steps per channel, 2 slots) or
    # waits for an address; a lone consumer waits for data
    assert c.query(0)["error"] == X.XFER_ERR_TIMEOUT
    with pytest.raises(xf.XferError) as e:
        c.run(a, b, 1 << 16)
    assert e.value.status == X.XFER_ERR_STATE
    c.close()


def test_lone_direct_zero_copy_producer_needs_no_receiver():
    # the destination is known before the launch: the producer writes every
    # step and publishes tail without waiting for its receiver
    import torch
    c = xf.Conn("zcd", 2, 1, 4096, timeout_ms=20, roles=1)
    a, b = _bufs(1 << 16)
    a.copy_(torch.arange(1 << 16, device="cuda").to(torch.uint8))
    c.run(a, b, 1 << 16)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for ch in range(2):
        st = c.query(ch)
        assert st["error"] == 0 and st["tail"] == 8 and st["head"] == 0
    c.close()


@pytest.mark.parametrize("proto", ["simple", "ll", "zc", "zcd"])
def test_abort_word_ends_waits(proto):
    import torch
    log("case: abort %s" % proto)
    c = xf.Conn(proto, 1, 2, 4096, timeout_ms=4000, roles=2)
    a, b = _bufs(1 << 14)
    c.abort()
    t0 = time.time()
    c.run(a, b, 1 << 14)
    torch.cuda.synchronize()
    assert time.time() - t0 < 3.0  # well before the 4 s timeout
    assert c.query(0)["error"] == X.XFER_ERR_ABORTED
    c.close()


def test_healthy_connection_unaffected_by_a_failed_one():
    import torch
    bad = xf.Conn("simple", 1, 2, 4096, timeout_ms=10, roles=2)
    good = xf.Conn("simple", 1, 2, 4096)
    a, b = _bufs(1 << 15)
    a.random_(0, 255)
    bad.run(a, b, 1 << 15)
    torch.cuda.synchronize()
    good.run(a, b, 1 << 15)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert good.query(0)["error"] == 0 and bad.query(0)["error"] == X.XFER_ERR_TIMEOUT
    bad.close()
    good.close()


def test_run_validation_on_device_buffers():
    c = xf.Conn("simple", 1, 2, 4096)
    a, b = _bufs(4096)
    with pytest.raises(xf.XferError) as e:
        c.run(a.data_ptr(), a.data_ptr() + 100, 1000)  # overlap
    assert e.value.status == X.XFER_ERR_INVALID_ARG
    with pytest.raises(xf.XferError):
        c.run(0, b, 10)
    c.run(0, 0, 0)  # nothing to move: no launch
    c.close()


def test_grid_that_cannot_be_resident_is_refused():
    c = xf.Conn("simple", 64, 1, 4096, wgs_per_channel=16, block_threads=1024)
    a, b = _bufs(1 << 20)
    g, blk = c.launch_shape()
    assert (g, blk) == (64 * 16 * 2, 1024)
    with pytest.raises(xf.XferError) as e:
        c.run(a, b, 1 << 20)
    assert e.value.status == X.XFER_ERR_INVALID_ARG
    c.close()


def test_batch_rejects_transfers_that_overlap_each_other():
    import torch
    c0, c1 = xf.Conn("simple", 1, 2, 4096), xf.Conn("simple", 1, 2, 4096)
    a, b = _bufs(1 << 16)
    pa, pb = a.data_ptr(), b.data_ptr()
    n = 4096
    bad = [([pa, pa + n], [pb, pb + n // 2]),          # destinations overlap
           ([pa, pb], [pb, pb + 2 * n]),               # 1 reads 0's destination
           ([pa, pa + 2 * n], [pb, pa + n // 2])]      # 1 writes into 0's source
    for src, dst in bad:
        with pytest.raises(xf.XferError) as e:
            X.run_batch([c0, c1], src, dst, [n, n])
        assert e.value.status == X.XFER_ERR_INVALID_ARG
        assert "overlaps" in str(e.value)
    # nothing was launched and no step was counted
    assert c0.query(0)["steps"] == 0 and c1.query(0)["steps"] == 0
    # disjoint transfers, and an empty one next to any range, are accepted
    a.copy_(torch.arange(1 << 16, device="cuda").to(torch.uint8))
    X.run_batch([c0, c1], [pa, pa + n], [pb, pb + n], [n, n])
    X.run_batch([c0, c1], [pa + 2 * n, pb], [pb + 2 * n, pb + 2 * n], [n, 0])
    torch.cuda.synchronize()
    assert torch.equal(a[:3 * n], b[:3 * n])
    c0.close()
    c1.close()


@pytest.mark.parametrize("proto,roles", [("zc", 2), ("simple", 1), ("ll", 1), ("zcd", 2)])
def test_run_queued_behind_a_failed_one_changes_nothing(proto, roles):
    # The second run is queued before the first has failed, so the host
    # accepts it; on the device it must find the failure on entry and leave
    # every word where the failed run left it (a lone zero-copy receiver
    # leaves its first address in ptrExchange: a producer of a later run
    # must never take it).  `ref` shows where the failed run alone leaves
    # the words.
    import torch
    log("case: run queued behind a failure %s roles=%d" % (proto, roles))
    n = 1 << 16
    ref = xf.Conn(proto, 2, 2, 4096, timeout_ms=200, roles=roles)
    c = xf.Conn(proto, 2, 2, 4096, timeout_ms=200, roles=roles)
    a1, b1 = _bufs(n)
    a2, b2 = _bufs(n)
    a1.random_(0, 255)
    a2.random_(0, 255)
    ref.run(a1, b1, n)
    torch.cuda.synchronize()
    b1.zero_()
    c.run(a1, b1, n)
    c.run(a2, b2, n)
    torch.cuda.synchronize()
    for ch in range(2):
        qr, qc = ref.query(ch), c.query(ch)
        assert qr["error"] == X.XFER_ERR_TIMEOUT and qc["error"] == X.XFER_ERR_TIMEOUT, (qr, qc)
        for k in ("head", "tail", "ptr_exchange", "lanes_agree"):
            assert qc[k] == qr[k], (proto, ch, k, qr, qc)
        if proto in ("simple", "ll"):
            assert (c.read_fifo(ch) == ref.read_fifo(ch)).all(), (proto, ch)
    if proto == "zc":
        assert c.query(0)["ptr_exchange"] == b1.data_ptr()  # the failed run's first address
    assert not b2.any()
    ref.close()
    c.close()
