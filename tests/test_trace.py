"""GPU tests of the step trace (xfer_conn_set_trace).  Each side's first
thread stamps an ACQUIRE and a PUBLISH event per step with the device's
constant wall clock, so the records must:
- be complete: both events of every step, in their ring slots, with the
  right channel, lane and side;
- be ordered in time: a producer's PUBLISH of step g before the consumer's
  ACQUIRE of it; a consumer's PUBLISH of step g - nslots (its head) before
  the producer's ACQUIRE of step g (the credit);
- for zero-copy, carry exactly the destination offsets of the oracle's
  publication sequence (reading R7): taken by the producer, published by
  the receiver."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import log, to_dev

pytestmark = pytest.mark.gpu

FILL = 0xAB


def traced_run(proto, nch, nslots, slot, lanes, n, fifo_loc="device", runs=1, per=None,
               block=256, jitter=0):
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    conn = xf.Conn(proto, nch, nslots, slot, fifo_loc, wgs_per_channel=lanes,
                   block_threads=block)
    S = oracle.step_bytes("ll" if proto == "ll" else "simple", slot)
    k_max = max((ln + S - 1) // S for ln in oracle.partition(n, nch)[1]) * runs
    per = per or 2 * max(1, k_max)
    rings = nch * lanes * 2
    buf = torch.full((rings * per * X.TRACE_REC_BYTES,), FILL, dtype=torch.uint8, device="cuda")
    conn.set_trace(buf)
    if jitter:
        conn.set_jitter(jitter)
    A = synth.uint8_uniform(n, 4000 + n)
    a = to_dev(A)
    b = torch.zeros_like(a)
    for _ in range(runs):
        conn.run(a, b, n)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for ch in range(nch):
        assert conn.query(ch)["error"] == 0
    recs = X.trace_records(buf.cpu().numpy())
    conn.close()
    return recs.reshape(nch, lanes, 2, per), int(b.data_ptr()), S


def steps_of(n, nch, S):
    return [(ln + S - 1) // S for ln in oracle.partition(n, nch)[1]]


def check_complete(R, n, nch, lanes, S, runs=1):
    per = R.shape[-1]
    ks = steps_of(n, nch, S)
    for c in range(nch):
        for w in range(lanes):
            for side in (0, 1):
                ring = R[c, w, side]
                for g in range(ks[c] * runs):
                    for ev in (0, 1):
                        r = ring[(2 * g + ev) % per]
                        assert (r["step"], r["event"], r["channel"], r["lane"], r["side"]) == \
                            (g, ev, c, w, side), (c, w, side, g, ev, r)
                    assert ring[(2 * g) % per]["time"] <= ring[(2 * g + 1) % per]["time"]
    return ks


def ev(R, c, w, side, g, e):
    return R[c, w, side][(2 * g + e) % R.shape[-1]]


@pytest.mark.parametrize("jitter", [0, 0x5EED])
@pytest.mark.parametrize("proto,fifo_loc", [("simple", "device"), ("simple", "host"),
                                            ("simple", "relay"), ("ll", "device")])
def test_trace_fifo_protocols(proto, fifo_loc, jitter):
    nch, nslots, lanes, n = 3, 2, 2, 300_001
    slot = 16384 if proto == "ll" else 8192
    log("case: trace %s %s jitter=%#x" % (proto, fifo_loc, jitter))
    R, _, S = traced_run(proto, nch, nslots, slot, lanes, n, fifo_loc=fifo_loc, jitter=jitter)
    ks = check_complete(R, n, nch, lanes, S)
    for c in range(nch):
        for w in range(lanes):
            for g in range(ks[c]):
                if proto == "ll":
                    # a lane whose first line lies past the step's chunk has
                    # no line to wait for, and the producer stamps before its
                    # first thread's line
                    L = min(S, oracle.partition(n, nch)[1][c] - g * S)
                    if w * 256 >= (L + 3) // 4:
                        continue
                assert ev(R, c, w, 0, g, 1)["time"] < ev(R, c, w, 1, g, 0)["time"], (c, w, g)
                if g >= nslots:
                    assert ev(R, c, w, 1, g - nslots, 1)["time"] < ev(R, c, w, 0, g, 0)["time"]


@pytest.mark.parametrize("jitter", [0, 0x5EED])
@pytest.mark.parametrize("nslots", [1, 3, 8, 12])
def test_trace_ll_one_line_per_thread(nslots, jitter):
    # steps of at most one line per thread (the one-pass path), many per
    # transfer: every step is stamped, a step's lines are seen after the
    # producer published them, and its slot's previous step was handed back
    # before the producer took it again
    nch, lanes, slot, n = 2, 2, 4096, 60_001
    log("case: trace ll one line per thread nslots=%d jitter=%#x" % (nslots, jitter))
    R, _, S = traced_run("ll", nch, nslots, slot, lanes, n, jitter=jitter)
    ks = check_complete(R, n, nch, lanes, S)
    for c in range(nch):
        for w in range(lanes):
            for g in range(ks[c]):
                L = min(S, oracle.partition(n, nch)[1][c] - g * S)
                if w * 256 >= (L + 3) // 4:
                    continue
                assert ev(R, c, w, 0, g, 1)["time"] < ev(R, c, w, 1, g, 0)["time"], (c, w, g)
                if g >= nslots:
                    assert ev(R, c, w, 1, g - nslots, 1)["time"] < ev(R, c, w, 0, g, 0)["time"]


@pytest.mark.parametrize("jitter", [0, 0x5EED])
@pytest.mark.parametrize("proto", ["zc", "zcd"])
def test_trace_zero_copy_offsets_match_the_oracle(proto, jitter):
    nch, lanes, slot, n = 4, 2, 4096, 100_003
    log("case: trace %s offsets jitter=%#x" % (proto, jitter))
    R, dst, S = traced_run(proto, nch, 8, slot, lanes, n, jitter=jitter)
    ks = check_complete(R, n, nch, lanes, S)
    want = oracle.zero_copy_offsets(proto, n, nch, slot)
    for c in range(nch):
        assert len(want[c]) == ks[c]
        for w in range(lanes):
            got = [int(ev(R, c, w, 0, g, 0)["value"]) - dst for g in range(ks[c])]
            assert got == want[c], (c, w, got[:4], want[c][:4])
            for g in range(ks[c]):
                assert ev(R, c, w, 0, g, 1)["time"] < ev(R, c, w, 1, g, 1)["time"]
                if proto == "zc":
                    pub = ev(R, c, w, 1, g, 0)
                    assert int(pub["value"]) - dst == want[c][g]
                    assert pub["time"] < ev(R, c, w, 0, g, 0)["time"], (c, w, g)


def test_trace_ring_keeps_the_latest_steps_over_runs():
    # 3 runs of 8 steps per channel through rings of 6 records: each ring
    # holds the last 3 steps, numbered globally across the runs
    nch, lanes = 1, 1
    R, _, S = traced_run("simple", nch, 2, 4096, lanes, 8 * 4096, runs=3, per=6)
    for side in (0, 1):
        ring = R[0, 0, side]
        assert sorted(set(int(x) for x in ring["step"])) == [21, 22, 23]
        for i in range(6):
            assert (2 * int(ring[i]["step"]) + int(ring[i]["event"])) % 6 == i


def test_trace_off_writes_nothing():
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    conn = xf.Conn("simple", 2, 2, 4096, wgs_per_channel=1)
    buf = torch.full((2 * 2 * 8 * X.TRACE_REC_BYTES,), FILL, dtype=torch.uint8, device="cuda")
    conn.set_trace(buf)
    conn.set_trace(None)
    a = torch.from_numpy(synth.uint8_uniform(50_000, 1)).to("cuda")
    b = torch.zeros_like(a)
    conn.run(a, b, a.numel())
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert bool((buf == FILL).all())
    with pytest.raises(xf.XferError):
        conn.set_trace(buf[:X.TRACE_REC_BYTES * 4])  # fewer than 2 records per ring
    conn.close()


def test_jitter_lengthens_the_traced_steps():
    # the producer's acquire-to-publish span of a step holds its jitter (two
    # points of 0..15 sleeps of 512 cycles each, several microseconds in
    # all, hundreds of ticks of the 100 MHz clock); without jitter it is the
    # copy alone
    nch, lanes, n = 2, 1, 64 * 4096

    def mean_span(jitter):
        R, _, S = traced_run("simple", nch, 4, 4096, lanes, n, jitter=jitter)
        ks = check_complete(R, n, nch, lanes, S)
        spans = [int(ev(R, c, 0, 0, g, 1)["time"]) - int(ev(R, c, 0, 0, g, 0)["time"])
                 for c in range(nch) for g in range(ks[c])]
        return sum(spans) / len(spans)

    plain, jittered = mean_span(0), mean_span(0xC0FFEE)
    log("producer step span: %.1f ticks plain, %.1f with jitter" % (plain, jittered))
    assert jittered > plain + 100


def test_trace_in_a_batch_where_only_some_connections_trace():
    # one launch for both: the traced connection records every step, the
    # other runs through the same (debug) kernel with no buffer and no seed
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    n, nch, lanes, slot = 200_000, 2, 2, 8192
    traced = xf.Conn("simple", nch, 4, slot, wgs_per_channel=lanes)
    plain = xf.Conn("simple", nch, 4, slot, wgs_per_channel=lanes)
    S = oracle.step_bytes("simple", slot)
    k = max(steps_of(n, nch, S))
    per = 2 * k
    buf = torch.full((nch * lanes * 2 * per * X.TRACE_REC_BYTES,), FILL, dtype=torch.uint8,
                     device="cuda")
    traced.set_trace(buf)
    A = synth.uint8_uniform(2 * n, 9)
    a = to_dev(A)
    b = torch.zeros_like(a)
    X.run_batch([traced, plain], [a.data_ptr(), a.data_ptr() + n], [b.data_ptr(), b.data_ptr() + n],
                [n, n])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    R = X.trace_records(buf.cpu().numpy()).reshape(nch, lanes, 2, per)
    check_complete(R, n, nch, lanes, S)
    for ch in range(nch):
        assert traced.query(ch)["error"] == 0 and plain.query(ch)["error"] == 0
    traced.close()
    plain.close()


def test_trace_pingpong_orders_the_round_trips():
    # X sends on fwd then receives on rev; Y the other way round.  Round i's
    # reply can only start after its request landed: on each channel and
    # lane, fwd's consumer ACQUIRE of step i precedes rev's producer PUBLISH
    # of step i, which precedes rev's consumer ACQUIRE of it.
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    size, iters, nch, lanes, slot = 4096, 12, 1, 1, 16384
    conns = [xf.Conn("ll", nch, 8, slot, wgs_per_channel=lanes, block_threads=256)
             for _ in range(2)]
    per = 2 * iters
    bufs = [torch.full((nch * lanes * 2 * per * X.TRACE_REC_BYTES,), FILL, dtype=torch.uint8,
                       device="cuda") for _ in range(2)]
    for c, buf in zip(conns, bufs):
        c.set_trace(buf)
    a = torch.from_numpy(synth.uint8_uniform(size, 3)).to("cuda")
    b = torch.zeros_like(a)
    cc = torch.zeros_like(a)
    X.run_pingpong(conns[0], conns[1], a, b, cc, size, iters)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, cc)
    F, Rv = (X.trace_records(buf.cpu().numpy()).reshape(nch, lanes, 2, per) for buf in bufs)
    for i in range(iters):
        fwd_ready = ev(F, 0, 0, 1, i, 0)["time"]
        rev_pub = ev(Rv, 0, 0, 0, i, 1)["time"]
        rev_ready = ev(Rv, 0, 0, 1, i, 0)["time"]
        assert ev(F, 0, 0, 0, i, 1)["time"] < fwd_ready <= rev_pub < rev_ready, i
        if i + 1 < iters:
            assert rev_ready <= ev(F, 0, 0, 0, i + 1, 1)["time"], i
    for c in conns:
        c.close()


@pytest.mark.parametrize("jitter", [0, 0x5EED])
def test_trace_ll_striped_groups(jitter):
    # the striped layout (1024-thread lanes, a 512-line stripe each, groups
    # of 2 steps with 3 slots): every step is stamped once per lane and side,
    # a step's lines are seen after the producer published them, and a slot
    # is taken again only after the head that handed it back
    nch, nslots, lanes, slot, n, q = 2, 3, 2, 8192, 90_001, 512
    log("case: trace ll striped jitter=%#x" % jitter)
    R, _, S = traced_run("ll", nch, nslots, slot, lanes, n, block=1024, jitter=jitter)
    ks = check_complete(R, n, nch, lanes, S)
    for c in range(nch):
        for w in range(lanes):
            for g in range(ks[c]):
                L = min(S, oracle.partition(n, nch)[1][c] - g * S)
                if w * q >= (L + 3) // 4:
                    continue
                assert ev(R, c, w, 0, g, 1)["time"] < ev(R, c, w, 1, g, 0)["time"], (c, w, g)
                if g >= nslots:
                    assert ev(R, c, w, 1, g - nslots, 1)["time"] < ev(R, c, w, 0, g, 0)["time"]
