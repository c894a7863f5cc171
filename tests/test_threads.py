"""Connections driven from several host threads at once, each thread with
its own connections and stream (the library's shared per-device state is
locked; ctypes releases the GIL during each call).  Every transfer must
match the oracle byte for byte, counters included."""
import threading

import numpy as np
import pytest

import oracle
from gpu_cases import compare_state, log, payload, to_dev, to_host
import recv_fifo_plane_amd as xf

pytestmark = pytest.mark.gpu


def _worker(k, proto, errors):
    import torch
    try:
        st = torch.cuda.Stream()
        nch, nslots, slot = 2 + k % 3, 4, 4096
        conn = xf.Conn(proto, nch, nslots, slot, wgs_per_channel=1 + k % 2, block_threads=128,
                       place_trials=2 if proto in ("simple", "ll") and k % 2 else 0)
        ocn = oracle.Conn(proto, nch, nslots, slot)
        for t in range(6):
            n = 30000 + 4099 * t + 17 * k
            A = payload("uint8", n, 1000 * k + t)
            with torch.cuda.stream(st):
                a = to_dev(A)
                b = torch.zeros_like(a)
            st.synchronize()
            conn.run(a, b, n, st)
            st.synchronize()
            B = np.zeros_like(A)
            ocn.run(A, B, n)
            assert np.array_equal(to_host(b), B), (k, proto, t)
        compare_state(conn, ocn, nch, "thread %d %s" % (k, proto))
        conn.close()
        ocn.close()
    except Exception as e:  # reported by the main thread
        errors.append((k, proto, repr(e)))


def test_connections_from_several_threads():
    import torch
    log("case: 8 threads, 2 each of simple, ll, zc, zcd")
    errors = []
    protos = ["simple", "ll", "zc", "zcd"] * 2
    threads = [threading.Thread(target=_worker, args=(k, p, errors)) for k, p in enumerate(protos)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    torch.cuda.synchronize()
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
