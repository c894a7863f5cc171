"""LL steps of at most one line per thread (a whole step's lines fit the
lanes' threads: the one-pass path) over transfers of many steps.  Parity
with the oracle on shapes at the edges: one slot, slot counts below and
above 8, ragged last steps, odd step sizes, misaligned buffers, and the LL
ping-pong workload's own shape (16 lanes of 256 threads on 16 KiB steps)."""
import pytest

from gpu_cases import run_transfers

pytestmark = pytest.mark.gpu


def sizes_for(slot):
    S = slot // 2
    return [1, 17, 3 * S + 5, 8 * S, 11 * S + 3, 100_003, 4 * S]


@pytest.mark.parametrize("nch,nslots,slot,lanes,block", [
    (1, 1, 2048, 1, 256),      # 256 lines per step on 256 threads
    (2, 2, 2048, 2, 128),
    (3, 3, 1032, 1, 256),      # 129 lines, a 516-byte step
    (1, 8, 4096, 4, 128),
    (2, 12, 4096, 2, 256),
    (1, 8, 32768, 16, 256),    # the LL ping-pong workload's shape
])
@pytest.mark.parametrize("offs", [(0, 0), (3, 5)])
def test_ll_one_pass_matches_oracle(nch, nslots, slot, lanes, block, offs):
    run_transfers("ll", nch, nslots, slot, sizes_for(slot), lanes=lanes, block=block,
                  src_off=offs[0], dst_off=offs[1], label="ll one pass")
