"""GPU parity of message lists (xfer_run_messages): one launch carries up to
128 messages; the result, counters and FIFO bytes must equal those of the
same messages sent as separate transfers, as the oracle runs them."""
import pytest

import synth
from gpu_cases import run_message_list

pytestmark = pytest.mark.gpu


def _sizes(n, total, seed, lo=0, hi=16):
    return synth.log_uniform_message_sizes(total, seed, lo_exp=lo, hi_exp=hi)[:n]


@pytest.mark.parametrize("fifo_loc", ["device", "host"])
@pytest.mark.parametrize("proto", ["simple", "ll", "zc", "zcd"])
def test_message_list_matches_separate_transfers(proto, fifo_loc):
    sizes = _sizes(300, 6 << 20, 11, lo=0, hi=17)  # > 128 messages: several launches
    sizes[3] = 0  # a zero-size message is skipped
    run_message_list(proto, 4, 3, 4096, sizes, fifo_loc=fifo_loc, lanes=2, base_off=3,
                     kind="uint8", repeat=2)


@pytest.mark.parametrize("lanes,block", [(1, 64), (4, 256), (16, 128)])
def test_message_list_shapes(lanes, block):
    sizes = [1, 15, 16, 17, 4095, 100_003, 1 << 20, 7, (1 << 20) + 9]
    run_message_list("simple", 8, 2, 64 << 10, sizes, lanes=lanes, block=block, base_off=0)
    run_message_list("zc", 8, 1, 64 << 10, sizes, lanes=lanes, block=block, base_off=5)
    run_message_list("zcd", 8, 1, 64 << 10, sizes, lanes=lanes, block=block, base_off=7)


def test_message_list_rejects_bad_arguments():
    import torch

    import recv_fifo_plane_amd as xf
    from recv_fifo_plane_amd import xfer as X
    c = xf.Conn("simple", 2, 2, 4096)
    a = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    b = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(xf.XferError) as e:
        c.run_messages(a, a.data_ptr() + 100, [0, 200], [100, 100])  # src and dst spans overlap
    assert e.value.status == X.XFER_ERR_INVALID_ARG
    with pytest.raises(xf.XferError) as e:
        c.run_messages(a, b, [0, 50], [100, 100])  # two messages write the same bytes
    assert e.value.status == X.XFER_ERR_INVALID_ARG
    assert "overlap" in str(e.value)
    c.run_messages(a, b, [100, 0], [100, 100])  # out of order but disjoint: accepted
    torch.cuda.synchronize()
    c.run_messages(a, a, [], [])  # nothing to move
    c.run_messages(0, 0, [0], [0])  # only empty messages
    c.close()
