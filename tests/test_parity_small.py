"""GPU parity on seeded small cases: every protocol x FIFO location, several
tiles and a ragged tail, misaligned buffers, 1..4 channels, 1..3 lanes,
1..8 slots; the destination (with guard bytes), counters and FIFO bytes must
equal the oracle's with 0 differing bytes."""
import pytest

from gpu_cases import run_transfers

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 15, 16, 17, 255, 4095, 4096, 4097, 65536 + 13, 300_001]


@pytest.mark.parametrize("fifo_loc", ["device", "host"])
@pytest.mark.parametrize("nch,nslots,lanes", [(1, 1, 1), (1, 2, 2), (3, 3, 1), (4, 8, 3)])
def test_simple(fifo_loc, nch, nslots, lanes):
    run_transfers("simple", nch, nslots, 4096, SIZES, fifo_loc=fifo_loc, lanes=lanes)


@pytest.mark.parametrize("fifo_loc", ["device", "host"])
@pytest.mark.parametrize("nch,nslots,lanes", [(1, 1, 1), (1, 3, 2), (2, 8, 1), (4, 2, 3)])
def test_ll(fifo_loc, nch, nslots, lanes):
    run_transfers("ll", nch, nslots, 2048, SIZES, fifo_loc=fifo_loc, lanes=lanes, kind="int32")


@pytest.mark.parametrize("proto", ["zc", "zcd"])
@pytest.mark.parametrize("fifo_loc", ["device", "host"])
@pytest.mark.parametrize("nch,lanes", [(1, 1), (2, 2), (4, 3)])
def test_zerocopy(proto, fifo_loc, nch, lanes):
    run_transfers(proto, nch, 8, 4096, SIZES, fifo_loc=fifo_loc, lanes=lanes)


@pytest.mark.parametrize("proto", ["simple", "ll", "zc", "zcd"])
@pytest.mark.parametrize("src_off,dst_off", [(1, 0), (0, 3), (5, 11), (8, 8), (15, 1)])
def test_misaligned(proto, src_off, dst_off):
    run_transfers(proto, 2, 3, 512, [1, 100, 5000, 33333], src_off=src_off, dst_off=dst_off,
                  lanes=2)


@pytest.mark.parametrize("block", [64, 512, 1024])
def test_block_sizes(block):
    for proto in ("simple", "ll", "zc", "zcd"):
        run_transfers(proto, 2, 4, 8192, [100_000, 7], block=block, lanes=2)


@pytest.mark.parametrize("ctrl_loc", [1, 2])
def test_control_words_either_side(ctrl_loc):
    for proto in ("simple", "ll", "zc", "zcd"):
        for fifo_loc in ("device", "host"):
            run_transfers(proto, 2, 2, 1024, [20_000, 3], fifo_loc=fifo_loc, ctrl_loc=ctrl_loc)


@pytest.mark.parametrize("xcd_pairing", [-1, 1])
def test_xcd_pairing_either_way(xcd_pairing):
    # 8 channels x 1 lane -> 16 workgroups: the pairing remap is active when on
    for proto in ("simple", "ll", "zc", "zcd"):
        run_transfers(proto, 8, 2, 4096, [1 << 20, 4097], xcd_pairing=xcd_pairing)


@pytest.mark.parametrize("fifo_loc", ["device", "host"])
@pytest.mark.parametrize("proto", ["simple", "ll", "zc", "zcd"])
def test_fenced_ordering(proto, fifo_loc):
    # the scoped-fence ordering must give the same bytes and counters
    run_transfers(proto, 3, 2, 4096, SIZES, fifo_loc=fifo_loc, lanes=2, ordering=1,
                  src_off=0, dst_off=0)
    run_transfers(proto, 2, 3, 512, [5000, 33], fifo_loc=fifo_loc, lanes=2, ordering=1,
                  src_off=3, dst_off=7)


def test_many_steps_through_few_slots():
    # long runs over 1-2 slots exercise slot reuse: every byte of every step
    # must come from its own step
    for proto in ("simple", "ll"):
        run_transfers(proto, 4, 1, 1024, [4 << 20], lanes=4)
        run_transfers(proto, 8, 2, 4096, [16 << 20], lanes=2, block=512)


@pytest.mark.parametrize("proto", ["simple", "zc", "zcd"])
@pytest.mark.parametrize("src_off,dst_off", [(3, 7), (1, 1), (0, 9), (12, 0)])
def test_misaligned_large_pipelined(proto, src_off, dst_off):
    # lane slices that fit one register batch take the pipelined producer
    run_transfers(proto, 8, 4, 64 << 10, [(8 << 20) + 5, 4097], src_off=src_off,
                  dst_off=dst_off, lanes=4, block=256)


@pytest.mark.parametrize("fifo_loc", ["device", "host"])
def test_messages_at_arbitrary_offsets(fifo_loc):
    # consecutive messages of odd sizes on one connection, as the host-FIFO
    # workload issues them: every message after the first starts misaligned
    import synth
    sizes = synth.log_uniform_message_sizes(24 << 20, 77, lo_exp=4, hi_exp=22)
    run_transfers("simple", 16, 8, 256 << 10, sizes[:40], fifo_loc=fifo_loc, lanes=4,
                  src_off=5, dst_off=11, ctrl_loc=1)


@pytest.mark.parametrize("fifo_loc", ["device", "host"])
@pytest.mark.parametrize("nslots", [1, 2])
def test_ll_lanes_that_own_no_lines(fifo_loc, nslots):
    # a 2 KiB LL slot holds 256 lines = one block of a 256-thread workgroup,
    # so lanes 1..3 never own a line: their consumers free every step at once
    # and run ahead of their producers, whose credit test must still hold
    run_transfers("ll", 2, nslots, 2048, [100_000, 5, 40_000], fifo_loc=fifo_loc, lanes=4,
                  kind="int32")


@pytest.mark.parametrize("proto", ["zc", "zcd"])
@pytest.mark.parametrize("lanes,block", [(16, 128), (2, 64)])
def test_zero_copy_destination_with_bit31_of_the_low_word_set(proto, lanes, block):
    # Destination addresses travel through ptrExchange and are made
    # wave-uniform 32 bits at a time; an address whose low word has bit 31
    # set must come back whole (a sign-extended half would point nowhere).
    import numpy as np
    import torch

    import recv_fifo_plane_amd as xf
    import synth
    from gpu_cases import log
    n, guard = 8 << 20, 4096
    big = torch.zeros((2 << 30) + n + 2 * guard, dtype=torch.uint8, device="cuda")
    low = big.data_ptr() & 0xFFFFFFFF
    off = guard + (0 if low + guard >= 1 << 31 else (1 << 31) - low)
    dst = big.data_ptr() + off
    assert (dst & 0xFFFFFFFF) >= 1 << 31 and off + n + guard <= big.numel()
    log("case: %s lanes=%d block=%d dst=%#x" % (proto, lanes, block, dst))
    A = synth.uint8_uniform(n, 2024)
    a = torch.from_numpy(A).to("cuda")
    conn = xf.Conn(proto, 4, 1, 512 << 10, wgs_per_channel=lanes, block_threads=block)
    for _ in range(2):
        conn.run(a, dst, n)
    torch.cuda.synchronize()
    assert conn.query(0)["error"] == 0
    assert np.array_equal(big[off:off + n].cpu().numpy(), A)
    assert int(big[off - guard:off].count_nonzero()) == 0
    assert int(big[off + n:off + n + guard].count_nonzero()) == 0
    conn.close()
    del big
