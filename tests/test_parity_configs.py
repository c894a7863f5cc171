"""GPU parity on the five workloads at full size, in the launch
configuration the benchmark times.  The oracle runs the same seeded inputs on
the CPU; destination bytes, counters and FIFO bytes must match exactly."""
import numpy as np
import pytest

import oracle
import synth
from recv_fifo_plane_amd import workloads as W
from gpu_cases import compare_state, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def test_w1_simple_single_channel_4mib():
    torch = _torch()
    cfg = W.W1
    log("case: W1 " + str(cfg))
    A = synth.uint8_uniform(cfg["nbytes"], synth.workload_seed(1))
    conn = W.make_conn(cfg)
    ocn = oracle.Conn("simple", 1, 8, 128 << 10)
    a = to_dev(A)
    b = torch.zeros_like(a)
    conn.run(a, b, A.size)
    torch.cuda.synchronize()
    B = np.zeros_like(A)
    ocn.run(A, B)
    assert np.array_equal(to_host(b), B)
    st = conn.query(0)
    assert st["head"] == st["tail"] == 32  # 4 MiB / 128 KiB steps
    compare_state(conn, ocn, 1, "W1")
    conn.close()


@pytest.mark.parametrize("size", W.W2_SIZES)
def test_w2_ll_pingpong(size):
    torch = _torch()
    cfg = W.W2
    iters = cfg["iters"]
    log("case: W2 LL ping-pong size=%d iters=%d" % (size, iters))
    A = synth.int32_uniform_bytes(size, synth.workload_seed(2) + size)
    fwd, rev = W.make_conn(cfg), W.make_conn(cfg)
    of, orv = oracle.Conn("ll", 1, 8, 32 << 10), oracle.Conn("ll", 1, 8, 32 << 10)
    a = to_dev(A)
    b = torch.zeros_like(a)
    c = torch.zeros_like(a)
    W.run_pingpong(fwd, rev, a, b, c, size, iters)
    torch.cuda.synchronize()
    ob, oc = np.zeros_like(A), np.zeros_like(A)
    oracle.run_pingpong(of, orv, A, ob, oc, size, iters)
    assert np.array_equal(to_host(b), ob) and np.array_equal(to_host(c), oc)
    compare_state(fwd, of, 1, "W2 fwd")
    compare_state(rev, orv, 1, "W2 rev")
    fwd.close()
    rev.close()


@pytest.mark.parametrize("cfg", [W.W3, W.W3R], ids=["write", "p2p_read"])
def test_w3_simple_32_channels_1gib(cfg):
    torch = _torch()
    log("case: W3 " + str(cfg))
    A = synth.bf16_normal_bytes(cfg["nbytes"], synth.workload_seed(3))
    conn = W.make_conn(cfg)
    ocn = oracle.Conn("simple", 32, 8, 512 << 10)
    a = to_dev(A)
    b = torch.zeros_like(a)
    conn.run(a, b, A.size)
    torch.cuda.synchronize()
    B = np.zeros_like(A)
    ocn.run(A, B)
    got = to_host(b)
    assert np.array_equal(got, B)
    del got
    for ch in range(32):
        assert conn.query(ch)["head"] == 64
    compare_state(conn, ocn, 32, "W3")
    conn.close()


@pytest.mark.parametrize("proto", ["zc", "zcd"])
def test_w4_zero_copy_single_pair(proto):
    torch = _torch()
    cfg = W.W4_PAIR if proto == "zc" else W.W4D_PAIR
    log("case: W4 pair " + str(cfg))
    A = synth.fp32_uniform_bytes(cfg["nbytes"], synth.workload_seed(4))
    conn = W.make_conn(cfg)
    ocn = oracle.Conn(proto, cfg["nchannels"], 1, cfg["slot_bytes"])
    a = to_dev(A)
    b = torch.zeros_like(a)
    conn.run(a, b, A.size)
    torch.cuda.synchronize()
    B = np.zeros_like(A)
    ocn.run(A, B)
    assert np.array_equal(to_host(b), B)
    compare_state(conn, ocn, cfg["nchannels"], "W4 pair")
    conn.close()


@pytest.mark.parametrize("proto", ["zc", "zcd"])
def test_w4_eight_endpoint_ring(proto):
    torch = _torch()
    cfg = W.W4_RING if proto == "zc" else W.W4D_RING
    n = cfg["endpoints"]
    log("case: W4 ring " + str(cfg))
    ring = W.make_ring(cfg)
    assert sorted(ring.edges) == [(r, (r + 1) % n) for r in range(n)]
    A = synth.fp32_uniform_bytes(n * cfg["slice_bytes"], synth.workload_seed(4) + 100)
    a = to_dev(A)
    b = torch.zeros_like(a)
    ring.run(a, b)
    torch.cuda.synchronize()
    got = to_host(b)
    S = cfg["slice_bytes"]
    for r in range(n):
        d = (r + 1) % n
        ocn = oracle.Conn(proto, cfg["channels_per_edge"], 1, cfg["slot_bytes"])
        Bd = np.zeros(S, dtype=np.uint8)
        ocn.run(np.ascontiguousarray(A[r * S:(r + 1) * S]), Bd)
        assert np.array_equal(got[d * S:(d + 1) * S], Bd), ("edge", r, d)
        compare_state(ring.edges[(r, d)], ocn, cfg["channels_per_edge"], "W4 ring edge %d" % r)
    ring.close()


@pytest.mark.parametrize("one_launch_per_message", [True, False])
def test_w5_host_fifo_mixed_messages(one_launch_per_message):
    torch = _torch()
    cfg = W.W5
    log("case: W5 launch per message=%s %s" % (one_launch_per_message, cfg))
    sizes = synth.log_uniform_message_sizes(cfg["total_bytes"], synth.workload_seed(5))
    A = synth.uint8_uniform(cfg["total_bytes"], synth.workload_seed(5))
    conn = W.make_conn(cfg)
    ocn = oracle.Conn("simple", 16, 8, 256 << 10)
    a = to_dev(A)
    b = torch.zeros_like(a)
    if one_launch_per_message:
        W.run_messages(conn, a, b, sizes)
    else:
        W.run_message_list(conn, a, b, sizes)
    torch.cuda.synchronize()
    B = np.zeros_like(A)
    off = 0
    for s in sizes:
        ocn.run(np.ascontiguousarray(A[off:off + s]), B[off:off + s])
        off += s
    assert np.array_equal(to_host(b), B)
    compare_state(conn, ocn, 16, "W5")
    conn.close()


def test_w5r_copy_engine_relay_full_size():
    # the relay at the benchmark's shape: one 512 MiB transfer, then the
    # host-FIFO message mix, on one connection; every FIFO and tail checked
    torch = _torch()
    cfg = W.W5R
    log("case: W5R relay " + str(cfg))
    n = cfg["nbytes"]
    sizes = synth.log_uniform_message_sizes(cfg["total_bytes"], synth.workload_seed(5))
    A = synth.uint8_uniform(cfg["total_bytes"], synth.workload_seed(5))
    conn = W.make_conn(cfg)
    ocn = oracle.Conn("relay", cfg["nchannels"], cfg["nslots"], cfg["slot_bytes"])
    a = to_dev(A)
    b = torch.zeros_like(a)
    conn.run(a, b, n)
    W.run_message_list(conn, a, b, sizes)
    torch.cuda.synchronize()
    B = np.zeros_like(A)
    ocn.run(np.ascontiguousarray(A[:n]), B[:n], n)
    off = 0
    for s_ in sizes:
        ocn.run(np.ascontiguousarray(A[off:off + s_]), B[off:off + s_], s_)
        off += s_
    assert np.array_equal(to_host(b), B)
    compare_state(conn, ocn, cfg["nchannels"], "W5R")
    conn.close()
