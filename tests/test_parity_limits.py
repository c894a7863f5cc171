"""GPU parity at the size limits: a transfer past 4 GiB (64-bit offsets in
every mode's addressing), the largest slot (1 GiB; LL steps of 512 MiB), and
a relay run in a loop.  Large inputs are generated on the device from a
seeded generator; the result is checked by properties the oracle fixes at
any size (B equals A byte for byte, guard bytes untouched, and each
channel's head/tail/steps equal the closed form of the oracle's partition),
small ones against the oracle itself."""
import numpy as np
import pytest

import oracle
from gpu_cases import log, run_transfers

pytestmark = pytest.mark.gpu


def _device_bytes(n, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)


def _closed_form_steps(proto, n, nch, slot_bytes):
    S = oracle.step_bytes(oracle.PROTO_NAMES[proto], slot_bytes)
    beg, ln = oracle.partition(n, nch)
    return [(l + S - 1) // S for l in ln]


@pytest.mark.parametrize("proto,nch,lanes", [("simple", 2, 4), ("zc", 4, 4), ("zcd", 2, 2)])
def test_transfer_past_4gib(proto, nch, lanes):
    import torch

    import recv_fifo_plane_amd as xf
    n = (5 << 30) + 12345  # chunk offsets run past 4 GiB in every channel
    guard = 64
    log("case: %s %d bytes over %d channels" % (proto, n, nch))
    a = _device_bytes(n, 77)
    b = torch.full((n + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    c = xf.Conn(proto, nch, 4, 4 << 20, wgs_per_channel=lanes, block_threads=512)
    c.run(a, b[guard:guard + n], n)
    torch.cuda.synchronize()
    assert torch.equal(a, b[guard:guard + n])
    assert bool((b[:guard] == 0xA5).all()) and bool((b[guard + n:] == 0xA5).all())
    want = _closed_form_steps(proto, n, nch, 4 << 20)
    for ch in range(nch):
        st = c.query(ch)
        assert st["error"] == 0 and st["lanes_agree"]
        assert st["head"] == st["tail"] == st["steps"] == want[ch], (ch, st, want[ch])
    c.close()


@pytest.mark.parametrize("proto,n", [("simple", (2 << 30) + (1 << 29) + 7), ("ll", (1 << 30) + 99)])
def test_largest_slot(proto, n):
    import torch

    import recv_fifo_plane_amd as xf
    slot = 1 << 30  # the largest slot the library accepts
    log("case: %s slot 1 GiB, %d bytes" % (proto, n))
    a = _device_bytes(n, 5)
    b = torch.zeros_like(a)
    c = xf.Conn(proto, 1, 2, slot, wgs_per_channel=4, block_threads=1024)
    c.run(a, b, n)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    st = c.query(0)
    want = _closed_form_steps(proto, n, 1, slot)[0]
    assert st["error"] == 0 and st["head"] == st["tail"] == st["steps"] == want
    c.close()


def test_relay_run_loop_matches_separate_runs():
    import torch

    import recv_fifo_plane_amd as xf
    from gpu_cases import compare_state, to_dev, to_host
    import synth
    n, iters = 3 << 20, 4
    A = synth.uint8_uniform(n, 12)
    a = to_dev(A)
    b = torch.zeros_like(a)
    c = xf.Conn("simple", 3, 2, 256 << 10, "relay", wgs_per_channel=2)
    c.run_loop(a, b, n, iters)
    torch.cuda.synchronize()
    o = oracle.Conn("relay", 3, 2, 256 << 10)
    B = np.zeros(n, dtype=np.uint8)
    for _ in range(iters):
        o.run(A, B)
    assert np.array_equal(to_host(b), B)
    compare_state(c, o, 3, "relay loop")
    c.close()
    o.close()
