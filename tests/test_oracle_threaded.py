"""The oracle's threaded mode against its sequential simulator: real threads
handing off through C11 atomics must end in exactly the state the
sequential run reaches (destination, head, tail, ptrExchange, step base and
every FIFO byte), for every protocol, thread count and run history.  The
sequential simulator is pinned by test_oracle_protocol.py; every
interleaving of its actions is proven to end in that one state, so any
correct concurrent execution must too."""
import numpy as np
import pytest

import oracle
import synth


def _end_state(conn, B, nch):
    relay = conn.proto == oracle.RELAY
    return (B.tobytes(), [sorted(conn.state(ch).items()) for ch in range(nch)],
            [conn.fifo(ch, w).tobytes() for ch in range(nch) for w in range(3 if relay else 1)],
            [sorted(conn.relay_state(ch).items()) for ch in range(nch)] if relay else None)


CASES = [
    ("simple", 1, 1, 16), ("simple", 3, 2, 64), ("simple", 8, 4, 4096), ("simple", 16, 8, 1024),
    ("ll", 1, 1, 8), ("ll", 2, 3, 64), ("ll", 8, 4, 2048),
    ("zc", 1, 1, 16), ("zc", 4, 1, 256), ("zc", 16, 1, 4096),
    ("zcd", 1, 1, 16), ("zcd", 4, 1, 256), ("zcd", 16, 1, 4096),
    ("relay", 1, 1, 16), ("relay", 3, 2, 64), ("relay", 8, 4, 4096),
]


@pytest.mark.parametrize("proto,nch,nslots,slot_bytes", CASES)
def test_threaded_mode_ends_in_the_sequential_state(proto, nch, nslots, slot_bytes):
    sizes = [0, 1, 15, 17, 4 * slot_bytes * nch + 3, 100_003]
    for nthreads in sorted({1, 2, 3, 2 * nch, (4 if proto == "relay" else 2) * nch}):
        seq = oracle.Conn(proto, nch, nslots, slot_bytes)
        thr = oracle.Conn(proto, nch, nslots, slot_bytes)
        for i, n in enumerate(sizes):
            A = synth.uint8_uniform(n, 5000 + i)
            Bs = np.zeros(n, dtype=np.uint8)
            Bt = np.zeros(n, dtype=np.uint8)
            seq.run(A, Bs)
            thr.run_threaded(A, Bt, nthreads)
            assert _end_state(thr, Bt, nch) == _end_state(seq, Bs, nch), (nthreads, n)
        seq.close()
        thr.close()


def test_threaded_runs_interleave_with_sequential_runs():
    # one connection, alternating modes: the step base and the FIFO carry over
    seq = oracle.Conn("simple", 4, 2, 128)
    mix = oracle.Conn("simple", 4, 2, 128)
    for i, n in enumerate([5000, 123, 0, 7777, 4096]):
        A = synth.uint8_uniform(n, 6000 + i)
        Bs, Bm = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
        seq.run(A, Bs)
        if i % 2:
            mix.run(A, Bm)
        else:
            mix.run_threaded(A, Bm, 8)
        assert _end_state(mix, Bm, 4) == _end_state(seq, Bs, 4)


@pytest.mark.parametrize("proto", ["simple", "ll"])
@pytest.mark.parametrize("nch", [1, 2])
def test_threaded_pingpong_matches_sequential(proto, nch):
    slot = 64 if proto == "ll" else 128
    n, iters = 300, 25
    a = synth.uint8_uniform(n, 7000)
    ends = []
    for mode in ("seq", "thr"):
        f = oracle.Conn(proto, nch, 2, slot)
        r = oracle.Conn(proto, nch, 2, slot)
        b = np.zeros(n, np.uint8)
        c = np.zeros(n, np.uint8)
        if mode == "seq":
            oracle.run_pingpong(f, r, a, b, c, n, iters)
        else:
            sec = oracle.pingpong_threaded(f, r, a, b, c, n, iters)
            assert sec > 0
        ends.append((b.tobytes(), c.tobytes(), _end_state(f, b, nch)[1:], _end_state(r, c, nch)[1:]))
        f.close()
        r.close()
    assert ends[0] == ends[1]
    assert ends[1][1] == a.tobytes()


def test_threaded_rejects_bad_arguments():
    c = oracle.Conn("simple", 2, 2, 64)
    A = np.zeros(10, np.uint8)
    with pytest.raises(oracle.OracleError):
        c.run_threaded(A, A.copy(), 0)
    c.close()
    f, r = oracle.Conn("zc", 1, 1, 16), oracle.Conn("zc", 1, 1, 16)
    with pytest.raises(oracle.OracleError):
        oracle.pingpong_threaded(f, r, A, A.copy(), A.copy(), 10, 1)
    f.close()
    r.close()
