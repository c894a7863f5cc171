"""Pins of the oracle's protocol simulation.

What fixes the expected values (none of them comes from the GPU library):
  * the result of every mode is a plain copy, B[0:n] == A[0:n], with the
    bytes around B untouched;
  * closed forms for the counters: head == tail == the number of steps,
    ceil(len_c / S) summed per channel over the transfers so far;
    the 4 MiB / 128 KiB single-channel SIMPLE workload takes 32 steps;
  * the FIFO bytes by replay: each slot position holds the last step that
    wrote it, and an LL line's flag is that step's 1-based number;
  * every interleaving of producer and consumer actions on tiny inputs keeps
    the protocol's invariants and ends in one state, and each deliberate
    protocol mistake is caught.
Sources: "【NCCL】transport数据传输（二）" (p2pTransport zero-copy and copy
sequences; shmTransport normal mode), "Intra-Node Transport (P2P)" section 4
(POST / POLL), "RDMA and GPUDirect" section 四.1 (flag carried in the data).
"""
import numpy as np
import pytest

import oracle
import synth


def _chunks(n, nch, S):
    """Brute-force list of (channel, step-in-run, offset, length): the channel
    ranges tile [0, n) in order with 16-byte-aligned starts and equal sizes
    except the tail, and every channel cuts its range into S-byte steps."""
    beg, ln = oracle.partition(n, nch)
    out = []
    for c in range(nch):
        j, off = 0, beg[c]
        while off < beg[c] + ln[c]:
            L = min(S, beg[c] + ln[c] - off)
            out.append((c, j, off, L))
            off += L
            j += 1
    return out


def _steps_per_channel(n, nch, S):
    cnt = [0] * nch
    for c, _, _, _ in _chunks(n, nch, S):
        cnt[c] += 1
    return cnt


@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 100, 4096, 65535, 1 << 20, (1 << 20) + 3])
@pytest.mark.parametrize("nch", [1, 2, 3, 7, 32, 64])
def test_partition_properties(n, nch):
    beg, ln = oracle.partition(n, nch)
    assert sum(ln) == n
    pos = 0
    sizes = []
    for c in range(nch):
        assert beg[c] == pos  # contiguous, in channel order
        assert beg[c] % 16 == 0 or ln[c] == 0
        pos += ln[c]
        sizes.append(ln[c])
    nonempty = [s for s in sizes if s]
    if len(nonempty) >= 2:
        per = nonempty[0]
        # every non-empty channel but the last carries the same multiple of 16 ...
        assert per % 16 == 0 and all(s == per for s in nonempty[:-1])
        assert 0 < nonempty[-1] <= per
        # ... which is the smallest such size that fits n into nch channels
        assert per * nch >= n and (per - 16) * nch < n
    elif nonempty:
        # one channel holds everything only when no 16-multiple below n fits n into nch
        assert sizes[0] == n
        assert all(p * nch < n for p in range(16, n, 16))
    # empty channels only at the end
    k = len(nonempty)
    assert all(s == 0 for s in sizes[k:]) and all(s > 0 for s in sizes[:k])


def test_workload_one_closed_form():
    """SIMPLE, 1 channel, 8 x 128 KiB FIFO, 4 MiB: B == A and head == tail == 32."""
    A = synth.uint8_uniform(4 << 20, synth.workload_seed(1))
    B = np.zeros_like(A)
    c = oracle.Conn("simple", 1, 8, 128 << 10)
    c.run(A, B)
    assert np.array_equal(A, B)
    st = c.state(0)
    assert st == {"head": 32, "tail": 32, "ptr_exchange": 0, "steps": 32}


def _replay_fifo(proto, nslots, slot_bytes, transfers, nch):
    """Writes every chunk of every transfer into its slot, in step order,
    without any protocol: the FIFO a correct protocol must leave behind."""
    S = oracle.step_bytes(proto, slot_bytes)
    fifo = [bytearray(nslots * slot_bytes) for _ in range(nch)]
    base = [0] * nch
    for A in transfers:
        A = bytes(A)
        for c, j, off, L in _chunks(len(A), nch, S):
            g = base[c] + j
            s0 = (g % nslots) * slot_bytes
            if proto in (oracle.SIMPLE, oracle.RELAY):
                fifo[c][s0:s0 + L] = A[off:off + L]
            else:
                for i in range(0, L, 4):
                    word = A[off + i:off + min(i + 4, L)].ljust(4, b"\0")
                    fifo[c][s0 + 2 * i:s0 + 2 * i + 4] = word
                    fifo[c][s0 + 2 * i + 4:s0 + 2 * i + 8] = (g + 1).to_bytes(4, "little")
        for c, k in enumerate(_steps_per_channel(len(A), nch, S)):
            base[c] += k
    return fifo, base


CASES = [
    # proto, nch, nslots, slot_bytes, sizes of consecutive transfers
    ("simple", 1, 8, 128, [4096]),
    ("simple", 1, 3, 48, [1, 47, 48, 49, 500]),
    ("simple", 3, 2, 32, [1000, 17, 0, 333]),
    ("simple", 4, 8, 64, [4096 + 5, 64]),
    ("ll", 1, 8, 64, [8, 9, 31, 32, 33, 1000]),
    ("ll", 2, 3, 24, [77, 5, 256]),
    ("ll", 5, 1, 8, [100, 3]),
    ("zc", 1, 8, 64, [1000, 1]),
    ("zc", 3, 1, 16, [555, 16, 0]),
    ("zcd", 1, 8, 64, [1000, 1]),
    ("zcd", 3, 1, 16, [555, 16, 0]),
    ("relay", 1, 8, 64, [1000, 1]),
    ("relay", 3, 2, 32, [1000, 17, 0, 333]),
    ("relay", 2, 1, 16, [555, 16]),
]


@pytest.mark.parametrize("proto,nch,nslots,slot_bytes,sizes", CASES)
def test_counters_result_and_fifo_by_replay(proto, nch, nslots, slot_bytes, sizes):
    conn = oracle.Conn(proto, nch, nslots, slot_bytes)
    transfers = []
    for t, n in enumerate(sizes):
        A = synth.uint8_uniform(n, 100 + t)
        guard = 64
        Bfull = synth.guard_pattern(n + 2 * guard, seed=t)
        before = Bfull.copy()
        conn.run(A, Bfull[guard:guard + n] if n else Bfull[guard:guard], n)
        assert np.array_equal(Bfull[guard:guard + n], A)
        assert np.array_equal(Bfull[:guard], before[:guard])
        assert np.array_equal(Bfull[guard + n:], before[guard + n:])
        transfers.append(A)
    pid = oracle.PROTO_NAMES[proto]
    fifo, base = _replay_fifo(pid, nslots, slot_bytes, transfers, nch)
    for c in range(nch):
        st = conn.state(c)
        assert st["head"] == st["tail"] == st["steps"] == base[c]
        assert st["ptr_exchange"] == 0
        if pid in (oracle.ZC, oracle.ZCD):
            assert conn.fifo(c).size == 0
        elif pid == oracle.RELAY:
            # every step passes through all three FIFOs, so each holds the replay
            for which in range(3):
                assert bytes(conn.fifo(c, which)) == bytes(fifo[c]), which
            rs = conn.relay_state(c)
            assert rs["send_proxy_tail"] == rs["recv_proxy_tail"] == base[c]
        else:
            assert bytes(conn.fifo(c)) == bytes(fifo[c])


def test_simple_fifo_is_the_payload_when_it_fits():
    """A single transfer no longer than the FIFO leaves the payload laid out
    verbatim in a fresh FIFO (slots in step order), the rest still zero."""
    A = synth.uint8_uniform(8 * 64 - 5, 3)
    c = oracle.Conn("simple", 1, 8, 64)
    c.run(A, np.zeros_like(A))
    f = c.fifo(0)
    assert np.array_equal(f[:A.size], A) and not f[A.size:].any()


def test_ll_lines_interleave_payload_and_step_flags():
    """LL on a fresh FIFO: word w of the payload sits in line w, with the
    1-based number of its step as the flag; a trailing partial word is
    zero-padded.  The 16-byte slot below carries 8 payload bytes per step."""
    A = np.arange(1, 24, dtype=np.uint8)  # 23 bytes -> 3 steps of 8, 8, 7
    c = oracle.Conn("ll", 1, 4, 16)
    c.run(A, np.zeros_like(A))
    f = c.fifo(0).view(np.uint32).reshape(-1, 2)  # (data, flag) per line
    want_flags = [1, 1, 2, 2, 3, 3, 0, 0]
    assert list(f[:, 1]) == want_flags
    words = np.frombuffer(np.concatenate([A, [0]]).astype(np.uint8).tobytes(), dtype=np.uint32)
    assert list(f[:6, 0]) == list(words)
    assert c.state(0)["head"] == c.state(0)["tail"] == 3


@pytest.mark.parametrize("proto,slot_sizes", [("simple", [16, 32, 48]), ("ll", [8, 24]),
                                              ("zc", [16, 48]), ("zcd", [16, 48]),
                                              ("relay", [16, 32])])
def test_edge_sizes_brute_force(proto, slot_sizes):
    pid = oracle.PROTO_NAMES[proto]
    for slot_bytes in slot_sizes:
        S = oracle.step_bytes(pid, slot_bytes)
        for nslots in (1, 2, 3):
            for nch in (1, 2, 3):
                conn = oracle.Conn(proto, nch, nslots, slot_bytes)
                total = [0] * nch
                for n in range(0, 4 * nslots * S + 18, 1 if S <= 16 else 3):
                    A = synth.uint8_uniform(n, n)
                    B = np.zeros(n, dtype=np.uint8)
                    conn.run(A, B)
                    assert np.array_equal(A, B)
                    for c, k in enumerate(_steps_per_channel(n, nch, S)):
                        total[c] += k
                for c in range(nch):
                    st = conn.state(c)
                    assert st["head"] == st["tail"] == st["steps"] == total[c]


def test_pingpong_composes_two_connections():
    a = synth.int32_uniform_bytes(1000, 9)
    b = np.zeros_like(a)
    cc = np.zeros_like(a)
    fwd = oracle.Conn("ll", 1, 8, 32 << 10)
    rev = oracle.Conn("ll", 1, 8, 32 << 10)
    oracle.run_pingpong(fwd, rev, a, b, cc, a.size, 25)
    assert np.array_equal(a, b) and np.array_equal(a, cc)
    for conn in (fwd, rev):
        st = conn.state(0)
        assert st["head"] == st["tail"] == 25


# ------------------------------------------------------------ interleavings
ENUM_CASES = []
for _p, _slots in (("simple", (16, 32)), ("ll", (8, 16)), ("zc", (16,)), ("zcd", (16,)),
                   ("relay", (16,))):
    for _ns in (1, 2, 3):
        for _sb in _slots:
            for _nch in (1, 2):
                ENUM_CASES.append((_p, _nch, _ns, _sb))


@pytest.mark.parametrize("proto,nch,nslots,slot_bytes", ENUM_CASES)
def test_every_interleaving_is_safe_and_confluent(proto, nch, nslots, slot_bytes):
    pid = oracle.PROTO_NAMES[proto]
    S = oracle.step_bytes(pid, slot_bytes)
    # up to 6 steps per channel (fewer with two channels or per-line LL actions)
    max_steps = 6 if nch == 1 else 3
    if pid == oracle.LL:
        max_steps = min(max_steps, 4 if nch == 1 else 2)
    for n in sorted({1, S - 1, S, S + 1, max_steps * S * nch - 3, max_steps * S * nch}):
        if n <= 0:
            continue
        A = synth.uint8_uniform(n, 1000 + n)
        for prior in (0, 1):
            r = oracle.enumerate_interleavings(proto, nch, nslots, slot_bytes, A, prior_runs=prior)
            assert r["violation"] == "ok", (n, prior, r)
            assert r["terminals"] == 1, r
            assert r["states"] > 1


MUTATION_CASES = [
    ("simple", "weak_credit", {"window", "overwrite"}),
    ("simple", "early_tail", {"read_unfilled"}),
    ("simple", "no_acquire", {"read_unfilled", "read_early"}),
    ("simple", "early_head", {"overwrite"}),
    ("ll", "weak_credit", {"window", "overwrite"}),
    ("ll", "torn_line", {"read_unfilled"}),
    ("ll", "early_head", {"overwrite", "deadlock"}),
    ("zc", "zc_no_wait", {"wrong_ptr"}),
    ("zc", "zc_no_reset", {"wrong_ptr", "counters"}),
    ("zcd", "early_tail", {"read_unfilled"}),
    ("relay", "relay_early", {"read_unfilled"}),
    ("relay", "weak_credit", {"window", "overwrite"}),
    ("relay", "early_tail", {"read_unfilled"}),
]


@pytest.mark.parametrize("proto,mutation,expected", MUTATION_CASES)
@pytest.mark.parametrize("nslots", [1, 2])
def test_enumerator_catches_each_broken_rule(proto, mutation, expected, nslots):
    pid = oracle.PROTO_NAMES[proto]
    slot_bytes = 16 if pid != oracle.LL else 8
    S = oracle.step_bytes(pid, slot_bytes)
    A = synth.uint8_uniform(4 * S + 3, 77)
    r = oracle.enumerate_interleavings(proto, 1, nslots, slot_bytes, A, mutation=mutation)
    assert r["violation"] in expected, r


def test_correct_protocol_is_clean_under_the_same_inputs_as_the_mutations():
    for proto in ("simple", "ll", "zc", "zcd", "relay"):
        pid = oracle.PROTO_NAMES[proto]
        slot_bytes = 16 if pid != oracle.LL else 8
        S = oracle.step_bytes(pid, slot_bytes)
        A = synth.uint8_uniform(4 * S + 3, 77)
        for nslots in (1, 2):
            r = oracle.enumerate_interleavings(proto, 1, nslots, slot_bytes, A)
            assert r["violation"] == "ok" and r["terminals"] == 1


# The zero-copy kernels take step g+1's address while step g's stores drain,
# before tail = g+1: a producer program order the pages do not print.  It
# must be as safe and confluent as theirs, end in the same state, and the
# enumerator must still catch the broken rules under it.
@pytest.mark.parametrize("nch,nslots", [(1, 1), (1, 2), (2, 1), (2, 3)])
def test_zc_take_ahead_order_is_safe_and_confluent(nch, nslots):
    S = 16
    max_steps = 6 if nch == 1 else 3
    for n in sorted({1, S - 1, S, S + 1, 2 * S, max_steps * S * nch - 3, max_steps * S * nch}):
        A = synth.uint8_uniform(n, 3000 + n)
        for prior in (0, 1):
            pages = oracle.enumerate_interleavings("zc", nch, nslots, S, A, prior_runs=prior)
            ahead = oracle.enumerate_interleavings("zc", nch, nslots, S, A, prior_runs=prior,
                                                   order="zc_take_ahead")
            assert ahead["violation"] == "ok" and ahead["terminals"] == 1, (n, prior, ahead)
            assert pages["violation"] == "ok"


def test_zc_take_ahead_ends_in_the_pages_state():
    for n in (0, 5, 16, 100, 1000):
        A = synth.uint8_uniform(n, 4000 + n)
        ends = []
        for order in ("pages", "zc_take_ahead"):
            c = oracle.Conn("zc", 3, 1, 32)
            c.set_order(order)
            B = np.zeros(n, dtype=np.uint8)
            for _ in range(2):
                c.run(A, B)
            ends.append((B.tobytes(), [sorted(c.state(ch).items()) for ch in range(3)]))
            c.close()
        assert ends[0] == ends[1]
        assert ends[1][0] == A.tobytes()


@pytest.mark.parametrize("mutation,expected", [("zc_no_wait", {"wrong_ptr"}),
                                               ("zc_no_reset", {"wrong_ptr", "counters"}),
                                               ("zc_ahead_past_end", {"deadlock"})])
def test_enumerator_catches_broken_rules_under_take_ahead(mutation, expected):
    A = synth.uint8_uniform(4 * 16 + 3, 77)
    r = oracle.enumerate_interleavings("zc", 1, 1, 16, A, mutation=mutation,
                                       order="zc_take_ahead")
    assert r["violation"] in expected, r


# The striped LL kernels take a transfer's steps in aligned groups of m <=
# nslots: step j is written by sub-producer j mod m (its own waves, each step
# on its own credit) and read by sub-consumer j mod m; the readers of a group
# meet at a barrier and one head store frees the whole group.  That order
# must be as safe and confluent as the pages' step-at-a-time order, end in
# the same state, and the enumerator must catch the mistakes it invites.
@pytest.mark.parametrize("nch,nslots,m,slot", [(1, 1, 1, 16), (1, 2, 2, 16), (1, 3, 2, 16),
                                               (1, 3, 3, 16), (1, 4, 4, 16), (1, 8, 4, 8),
                                               (1, 6, 3, 16), (2, 2, 2, 16), (2, 4, 2, 16)])
def test_ll_group_order_is_safe_and_confluent(nch, nslots, m, slot):
    S = slot // 2
    steps = (3 * m + 1) if nch == 1 else (2 * m + 1)
    for n in sorted({1, S - 1, S, S + 1, m * S, m * S + 1, nch * (steps * S - 3),
                     nch * steps * S}):
        A = synth.uint8_uniform(n, 5000 + n)
        for prior in (0, 2):
            r = oracle.enumerate_interleavings("ll", nch, nslots, slot, A, prior_runs=prior,
                                               order="ll_group%d" % m)
            assert r["violation"] == "ok" and r["terminals"] == 1, (n, prior, r)


def test_ll_group_of_one_step_is_the_pages_order():
    # With m = 1 the group order is the pages' order action for action: the
    # enumerator visits exactly as many states and transitions.
    for nch, nslots, slot in [(1, 1, 16), (1, 2, 16), (1, 3, 32), (2, 2, 16)]:
        for n in (1, 9, 40, 77):
            A = synth.uint8_uniform(n, 6000 + n)
            a = oracle.enumerate_interleavings("ll", nch, nslots, slot, A)
            b = oracle.enumerate_interleavings("ll", nch, nslots, slot, A, order="ll_group1")
            assert (a["states"], a["transitions"]) == (b["states"], b["transitions"]), (nch, n)
            assert a["violation"] == b["violation"] == "ok"


@pytest.mark.parametrize("nslots,m", [(8, 4), (4, 4), (3, 2), (16, 4)])
def test_ll_group_order_ends_in_the_pages_state(nslots, m):
    for n in (0, 5, 16, 100, 1000, 4099):
        A = synth.uint8_uniform(n, 7000 + n)
        ends = []
        for order in ("pages", "ll_group%d" % m):
            c = oracle.Conn("ll", 3, nslots, 64)
            c.set_order(order)
            B = np.zeros(n, dtype=np.uint8)
            for _ in range(3):
                B[:] = 0
                c.run(A, B)
            ends.append((B.tobytes(), [sorted(c.state(ch).items()) for ch in range(3)],
                         [c.fifo(ch).tobytes() for ch in range(3)]))
            c.close()
        assert ends[0] == ends[1], (nslots, m, n)
        assert ends[1][0] == A.tobytes()


@pytest.mark.parametrize("nslots,m", [(1, 2), (2, 3), (3, 4)])
def test_ll_group_larger_than_the_fifo_deadlocks(nslots, m):
    # A group's head comes only after all of its steps are read, and its last
    # step needs credit from that head once m > nslots: no group may
    # outnumber the slots (the kernels cap m at nslots).
    A = synth.uint8_uniform((m + 1) * 8, 8)
    r = oracle.enumerate_interleavings("ll", 1, nslots, 16, A, order="ll_group%d" % m)
    assert r["violation"] == "deadlock", r
    # a transfer of at most nslots steps (one partial group) still goes through
    r = oracle.enumerate_interleavings("ll", 1, nslots, 16, A[: nslots * 8],
                                       order="ll_group%d" % m)
    assert r["violation"] == "ok", r


@pytest.mark.parametrize("nslots,m", [(2, 2), (3, 2), (4, 4), (8, 4)])
def test_enumerator_catches_a_group_head_without_its_barrier(nslots, m):
    # head for the group stored once its first step is read, the others
    # still being read: the producer then refills one of their slots.
    A = synth.uint8_uniform((2 * m + 2) * 8 + 3, 9)
    r = oracle.enumerate_interleavings("ll", 1, nslots, 16, A, mutation="group_no_barrier",
                                       order="ll_group%d" % m)
    assert r["violation"] == "overwrite", r
    r = oracle.enumerate_interleavings("ll", 1, nslots, 16, A, mutation="weak_credit",
                                       order="ll_group%d" % m)
    assert r["violation"] in {"overwrite", "window"}, r


def test_ll_group_order_is_for_ll_on_the_sequential_modes_only():
    A = synth.uint8_uniform(40, 1)
    with pytest.raises(oracle.OracleError):
        oracle.enumerate_interleavings("simple", 1, 2, 16, A, order="ll_group2")
    c = oracle.Conn("ll", 1, 4, 16)
    try:
        c.set_order("ll_group2")
        with pytest.raises(oracle.OracleError):
            c.run_threaded(A, np.zeros_like(A), 2)
    finally:
        c.close()


def test_conn_rejects_bad_shapes():
    for args in [("simple", 0, 8, 16), ("simple", 65, 8, 16), ("simple", 1, 0, 16),
                 ("simple", 1, 8, 24), ("ll", 1, 8, 12), ("zc", 1, 8, 8), ("zcd", 1, 8, 8),
                 ("relay", 1, 8, 8)]:
        with pytest.raises(oracle.OracleError):
            oracle.Conn(*args)


@pytest.mark.parametrize("proto", ["zc", "zcd"])
@pytest.mark.parametrize("n,nch,slot", [(0, 1, 16), (1, 1, 16), (100, 3, 16), (4097, 4, 64),
                                        (100_003, 4, 4096), (65536, 64, 16)])
def test_zero_copy_offsets_tile_the_transfer(proto, n, nch, slot):
    # the published offsets of all channels, each step covering its chunk,
    # tile [0, n) exactly once, in increasing order within a channel (the
    # simulator holds its producer to this sequence: the zc_no_wait mutation
    # above, a receiver offering an address out of turn, is caught as
    # wrong_ptr)
    offs = oracle.zero_copy_offsets(proto, n, nch, slot)
    S = oracle.step_bytes(proto, slot)
    assert len(offs) == nch
    covered = np.zeros(n, dtype=np.int32)
    beg, ln = oracle.partition(n, nch)
    for c in range(nch):
        assert offs[c] == sorted(offs[c])
        for o in offs[c]:
            covered[o:min(o + S, beg[c] + ln[c])] += 1
    assert bool((covered == 1).all())

