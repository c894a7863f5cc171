"""Connections placed by measured latency (xfer_attr.place_trials): the kept
candidate starts from the state of a new connection (FIFO, counters and
status zeroed, no steps counted) and then matches the oracle byte for byte,
counters and FIFO included.  The LL ping-pong workload uses such
connections, so its parity tests cover them at full size as well."""
import pytest

from gpu_cases import run_transfers

pytestmark = pytest.mark.gpu

SIZES = [1, 15, 4096, 20000, 65536 + 24, 5000]


@pytest.mark.parametrize("proto,nch,nslots,slot,lanes,trials,read", [
    ("ll", 1, 8, 4096, 1, 4, 0),
    ("ll", 4, 8, 4096, 2, 3, 0),
    ("ll", 3, 3, 1032, 1, 2, 0),
    ("simple", 2, 8, 4096, 1, 8, 0),
    ("simple", 4, 4, 4096, 2, 2, 0),
    ("simple", 1, 2, 1 << 16, 1, 8, 0),
])
def test_placed_connection_matches_oracle(proto, nch, nslots, slot, lanes, trials, read):
    run_transfers(proto, nch, nslots, slot, SIZES, lanes=lanes, place_trials=trials, p2p_read=read,
                  label="placed")
