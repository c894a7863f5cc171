"""Pins of the oracle's host schedule (peer loop, ring masks, connect batching).

Sources: page "transport建立" (NCCL v2.25.1-1), section 具体说明: the
8-rank peer example, the per-channel receive-then-send setup listings, the
ring rule that only the first loop carries channels, and connect phases
every maxPeers (default 128) peers.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "peer_order_8ranks.txt")


def _golden_rows():
    rows = []
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(tuple(int(x) for x in line.split()))
    return rows


def test_page_example_peer_order():
    rows = _golden_rows()
    assert len(rows) == 2
    for n, rank, loop, rp, sp in rows:
        assert oracle.peers(rank, n, loop) == (rp, sp)


@pytest.mark.parametrize("n", list(range(1, 65)))
def test_peer_loop_brute_force(n):
    for i in range(1, n):
        sends = [oracle.peers(r, n, i)[1] for r in range(n)]
        recvs = [oracle.peers(r, n, i)[0] for r in range(n)]
        # every loop pairs the ranks by a permutation ...
        assert sorted(sends) == list(range(n))
        assert sorted(recvs) == list(range(n))
        for r in range(n):
            # ... and my send peer receives from me in the same loop
            assert recvs[sends[r]] == r
            assert sends[r] != r and recvs[r] != r
    for r in range(n):
        # over the loops a rank meets every other rank exactly once per role
        got_s = sorted(oracle.peers(r, n, i)[1] for i in range(1, n))
        got_r = sorted(oracle.peers(r, n, i)[0] for i in range(1, n))
        others = sorted(set(range(n)) - {r})
        assert got_s == others and got_r == others


@pytest.mark.parametrize("n", [1, 2, 3, 8, 17, 64])
@pytest.mark.parametrize("nch", [1, 4, 64])
def test_ring_masks_only_first_loop(n, nch):
    for r in range(n):
        rm, sm = oracle.ring_masks(r, n, nch)
        full = (1 << nch) - 1
        if n == 1:
            assert not rm.any() and not sm.any()
            continue
        rp1, sp1 = oracle.peers(r, n, 1)
        assert int(rm[rp1]) == full and int(sm[sp1]) == full
        for i in range(2, n):
            rp, sp = oracle.peers(r, n, i)
            if rp != rp1:
                assert int(rm[rp]) == 0
            if sp != sp1:
                assert int(sm[sp]) == 0
        # the whole mask array holds exactly one non-zero entry per direction
        assert np.count_nonzero(rm) == 1 and np.count_nonzero(sm) == 1


def test_ring_plan_8_ranks_4_channels():
    rm, sm = oracle.ring_masks(0, 8, 4)
    ops = oracle.plan(0, 8, rm, sm, 128)
    R, S, K = oracle.OP_RECV_SETUP, oracle.OP_SEND_SETUP, oracle.OP_CONNECT_BATCH
    assert ops == [(R, 7, 0), (R, 7, 1), (R, 7, 2), (R, 7, 3),
                   (S, 1, 0), (S, 1, 1), (S, 1, 2), (S, 1, 3), (K, -1, -1)]


@pytest.mark.parametrize("max_peers", [1, 2, 7, 128])
def test_connect_phase_count(max_peers):
    for n in range(1, 301):
        rm = np.zeros(n, dtype=np.uint64)
        sm = np.zeros(n, dtype=np.uint64)
        ops = oracle.plan(0, n, rm, sm, max_peers)
        batches = [k for k, op in enumerate(ops) if op[0] == oracle.OP_CONNECT_BATCH]
        assert len(batches) == math.ceil((n - 1) / max_peers)
        assert len(ops) == len(batches)  # empty masks: only connect phases


def test_plan_covers_masks_exactly():
    rng = np.random.default_rng(5)
    for trial in range(60):
        n = int(rng.integers(2, 40))
        rank = int(rng.integers(0, n))
        mp = int(rng.choice([1, 3, 5, 128]))
        rm = rng.integers(0, 2**63, size=n, dtype=np.int64).astype(np.uint64) & np.uint64(0xF0F0FFFF0000F00F)
        sm = rng.integers(0, 2**63, size=n, dtype=np.int64).astype(np.uint64)
        rm[rank] = sm[rank] = 0
        ops = oracle.plan(rank, n, rm, sm, mp)
        want_r = {(p, c) for p in range(n) for c in range(64) if p != rank and (int(rm[p]) >> c) & 1}
        want_s = {(p, c) for p in range(n) for c in range(64) if p != rank and (int(sm[p]) >> c) & 1}
        got_r = [(p, c) for k, p, c in ops if k == oracle.OP_RECV_SETUP]
        got_s = [(p, c) for k, p, c in ops if k == oracle.OP_SEND_SETUP]
        assert sorted(got_r) == sorted(want_r) and len(got_r) == len(want_r)
        assert sorted(got_s) == sorted(want_s) and len(got_s) == len(want_s)
        # within one loop: all receive setups (channels ascending) before the send setups
        loop_of = {oracle.peers(rank, n, i)[0]: i for i in range(1, n)}
        prev = None
        seen_send_in_loop = set()
        for k, p, c in ops:
            if k == oracle.OP_CONNECT_BATCH:
                continue
            i = loop_of[p] if k == oracle.OP_RECV_SETUP else [j for j in range(1, n)
                                                               if oracle.peers(rank, n, j)[1] == p][0]
            if k == oracle.OP_RECV_SETUP:
                assert i not in seen_send_in_loop
            else:
                seen_send_in_loop.add(i)
            key = (i, k, c)
            if prev is not None:
                assert key > prev
            prev = key


def test_plan_rejects_bad_arguments():
    z = np.zeros(4, dtype=np.uint64)
    with pytest.raises(oracle.OracleError):
        oracle.plan(4, 4, z, z, 128)
    with pytest.raises(oracle.OracleError):
        oracle.plan(0, 4, z, z, 0)
