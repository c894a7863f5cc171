"""One connection driven from several streams in turn.  Each hardware queue
deals a launch's blocks to the XCDs from a start XCD of its own, and the
paired launch shape places its workgroups by the XCD id each block reads;
whatever the stream, every transfer must match the oracle byte for byte,
counters and FIFO included."""
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
