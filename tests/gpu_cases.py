"""Helpers of the GPU parity tests: run a sequence of transfers on the HIP
path and on the oracle with the same seeded inputs and compare every byte
of the destination (with guard zones), the counters and the FIFO bytes."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

GUARD = 64


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def to_dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def to_host(t) -> np.ndarray:
    return t.cpu().numpy()


def payload(kind: str, n: int, seed: int) -> np.ndarray:
    if kind == "uint8":
        return synth.uint8_uniform(n, seed)
    if kind == "int32":
        return synth.int32_uniform_bytes(n, seed)
    if kind == "bf16":
        return synth.bf16_normal_bytes(n, seed)
    if kind == "fp32":
        return synth.fp32_uniform_bytes(n, seed)
    raise ValueError(kind)


def describe_mismatch(got, want, before, bad, base) -> str:
    """Contiguous runs of differing bytes (offsets relative to the start of
    the destination) and how many of them still hold their initial bytes."""
    runs = []
    start = prev = int(bad[0])
    for i in bad[1:]:
        i = int(i)
        if i != prev + 1:
            runs.append((start - base, prev - start + 1))
            start = i
        prev = i
    runs.append((start - base, prev - start + 1))
    untouched = int(np.count_nonzero(got[bad] == before[bad]))
    return "%d bytes differ in %d runs %s; %d still hold their initial value" % (
        bad.size, len(runs), runs[:12], untouched)


def oracle_proto(proto: str, fifo_loc: str) -> str:
    """The oracle's mode for a GPU connection: a relay FIFO is its own mode."""
    return "relay" if fifo_loc == "relay" else proto


def compare_state(conn, oconn, nch: int, what: str) -> None:
    for c in range(nch):
        g = conn.query(c)
        o = oconn.state(c)
        assert g["error"] == 0, (what, c, g)
        assert g["lanes_agree"], (what, c, g)
        for k in ("head", "tail", "steps"):
            assert g[k] == o[k], (what, c, k, g, o)
        assert g["ptr_exchange"] == 0 and o["ptr_exchange"] == 0, (what, c, g, o)
        relay = oconn.proto == oracle.RELAY
        for which in range(3 if relay else 1):
            gf = conn.read_fifo(c, which)
            of = oconn.fifo(c, which)
            assert gf.size == of.size, (what, c, which)
            if gf.size:
                bad = np.flatnonzero(gf != of)
                assert bad.size == 0, (what, "fifo", which, c, bad.size, bad[:8])
        if relay:
            gr = conn.query_relay(c)
            orr = oconn.relay_state(c)
            assert gr["send_proxy_tail"] == orr["send_proxy_tail"], (what, c, gr, orr)
            assert gr["recv_proxy_tail"] == orr["recv_proxy_tail"], (what, c, gr, orr)


def run_transfers(proto: str, nch: int, nslots: int, slot_bytes: int, sizes, *,
                  fifo_loc="device", lanes=1, block=0, src_off=0, dst_off=0, kind="uint8",
                  seed=1, ctrl_loc=0, xcd_pairing=0, ordering=0, p2p_read=0, jitter=0,
                  place_trials=0, cooperative=0, label="") -> None:
    """Each size is one xfer_run on the same connection; after every run the
    whole destination buffer (guards included) must equal the oracle's."""
    import recv_fifo_plane_amd as xf
    torch = torch_mod()
    what = "%s %s nch=%d nslots=%d slot=%d lanes=%d block=%d off=(%d,%d) %s ord=%d read=%d" % (
        label, proto, nch, nslots, slot_bytes, lanes, block, src_off, dst_off, fifo_loc, ordering,
        p2p_read) + (" jitter=%#x" % jitter if jitter else "") + (
        " place_trials=%d" % place_trials if place_trials else "") + (
        " cooperative" if cooperative else "")
    log("case: " + what + " sizes=" + str(list(sizes)[:6]))
    conn = xf.Conn(proto, nch, nslots, slot_bytes, fifo_loc, wgs_per_channel=lanes,
                   block_threads=block, ctrl_loc=ctrl_loc, xcd_pairing=xcd_pairing,
                   ordering=ordering, p2p_read=p2p_read, place_trials=place_trials,
                   cooperative=cooperative)
    if place_trials:
        # the kept candidate must look like a new connection
        for c in range(nch):
            st = conn.query(c)
            assert (st["head"], st["tail"], st["steps"], st["error"]) == (0, 0, 0, 0), (what, st)
            assert not conn.read_fifo(c).any(), (what, "FIFO not zeroed", c)
    if jitter:
        conn.set_jitter(jitter)
    ocn = oracle.Conn(oracle_proto(proto, fifo_loc), nch, nslots, slot_bytes)
    try:
        for t, n in enumerate(sizes):
            A = payload(kind, n, seed * 7919 + t)
            srcb = np.zeros(n + 32, dtype=np.uint8)
            srcb[src_off:src_off + n] = A
            dstb = synth.guard_pattern(n + 2 * GUARD + 16, seed=t)
            ob = dstb.copy()
            ds = to_dev(srcb)
            dd = to_dev(dstb)
            conn.run(ds.data_ptr() + src_off, dd.data_ptr() + GUARD + dst_off, n)
            torch.cuda.synchronize()
            view = ob[GUARD + dst_off:GUARD + dst_off + n]
            ocn.run(np.ascontiguousarray(A), view, n)
            got = to_host(dd)
            bad = np.flatnonzero(got != ob)
            assert bad.size == 0, (what, "transfer", t, n,
                                   describe_mismatch(got, ob, dstb, bad, GUARD + dst_off),
                                   [conn.query(c)["error"] for c in range(nch)])
        compare_state(conn, ocn, nch, what)
    finally:
        torch.cuda.synchronize()
        conn.close()
        ocn.close()


def run_message_list(proto: str, nch: int, nslots: int, slot_bytes: int, sizes, *,
                     fifo_loc="device", lanes=1, block=0, base_off=0, kind="uint8", seed=5,
                     ctrl_loc=0, repeat=1) -> None:
    """The messages go through xfer_run_messages (consecutive offsets from
    base_off); the oracle runs them as separate transfers in order.  The
    whole destination buffer, the counters and the FIFO bytes must match."""
    import recv_fifo_plane_amd as xf
    torch = torch_mod()
    total = int(sum(sizes))
    what = "messages %s n=%d total=%d nch=%d nslots=%d slot=%d lanes=%d %s" % (
        proto, len(sizes), total, nch, nslots, slot_bytes, lanes, fifo_loc)
    log("case: " + what)
    offs, off = [], base_off
    for s_ in sizes:
        offs.append(off)
        off += s_
    conn = xf.Conn(proto, nch, nslots, slot_bytes, fifo_loc, wgs_per_channel=lanes,
                   block_threads=block, ctrl_loc=ctrl_loc)
    ocn = oracle.Conn(oracle_proto(proto, fifo_loc), nch, nslots, slot_bytes)
    try:
        for r in range(repeat):
            A = payload(kind, base_off + total + 16, seed + r)
            dstb = synth.guard_pattern(base_off + total + 2 * GUARD, seed=r)
            ob = dstb.copy()
            da = to_dev(A)
            dd = to_dev(dstb)
            conn.run_messages(da, dd.data_ptr() + GUARD, offs, sizes)
            torch.cuda.synchronize()
            for o, s_ in zip(offs, sizes):
                ocn.run(np.ascontiguousarray(A[o:o + s_]), ob[GUARD + o:GUARD + o + s_], s_)
            got = to_host(dd)
            bad = np.flatnonzero(got != ob)
            assert bad.size == 0, (what, "repeat", r, describe_mismatch(got, ob, dstb, bad, GUARD))
        compare_state(conn, ocn, nch, what)
    finally:
        torch.cuda.synchronize()
        conn.close()
        ocn.close()
