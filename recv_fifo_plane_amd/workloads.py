"""Launch configurations of the five workloads, shared by the benchmark and
the GPU parity tests (so the tests check exactly what the benchmark times).

W1  SIMPLE, 1 channel, 8 x 128 KiB HBM FIFO, one producer/consumer pair, 4 MiB.
W2  LL, 1 channel, 8 x 32 KiB, messages 8 B .. 64 KiB, in-kernel ping-pong.
W3  SIMPLE, 32 channels x 8 x 512 KiB HBM, 1 GiB, 4 workgroups per channel side.
    W3R: the same under P2P read (the FIFO in the send side's memory).
W4  zero-copy through ptrExchange: one pair on 128 MiB, and a ring of 8
    logical endpoints built by the host schedule, endpoint r sending its
    128 MiB slice to (r + 1) mod 8, all edges in one launch.  W4D: the same
    with the destination known before the launch (zero-copy direct).
W5  host FIFO: 16 channels x 8 x 256 KiB in pinned host memory, 2 GiB of
    messages with log-uniform sizes 1 KiB .. 64 MiB at consecutive offsets;
    the head/tail words sit in HBM, next to the side that polls them.
W5R the copy-engine relay: host proxies move each step through a pinned
    staging FIFO with device-to-host and host-to-device DMA copies.
"""
from __future__ import annotations

from . import xfer as X

# One producer and one consumer workgroup; 512 threads measured 32.9 GB/s
# (0.98 of one 512-thread workgroup's straight copy) against 27.7 at 256.
W1 = dict(name="simple_1ch_4MiB", proto="simple", nchannels=1, nslots=8, slot_bytes=128 << 10,
          fifo_loc="device", wgs_per_channel=1, block_threads=512, nbytes=4 << 20)

# 16 workgroup pairs of 1024 threads: each lane owns a 256-line stripe of
# every slot (the 4096 lines of a 16 KiB step over 16 lanes), and its 16
# waves cover 4 steps at once, so a 64 KiB message is one group of 4 steps
# handed back by one head store (measured 1.65 us one-way at 64 KiB and
# 0.92 us at 8 B, against 3.39 and 0.99 us with 256-thread lanes that take
# the steps one after another).  Each connection's FIFO and counters are
# placed by measured latency at the fastest of eight offsets 2 KiB apart
# (place_trials): the time of a hand-off depends on the physical granule of
# the polled lines.
W2 = dict(name="ll_pingpong", proto="ll", nchannels=1, nslots=8, slot_bytes=32 << 10,
          fifo_loc="device", wgs_per_channel=16, block_threads=1024, iters=10000, place_trials=8)
W2_SIZES = [8 << i for i in range(14)]  # 8 B .. 64 KiB

# 4 workgroups per channel side as the workload fixes them; the block size
# and dispatch order were swept (0.911-0.914 of the roofline at 704-832
# threads in dispatch order; with pairs placed on one XCD by XCD id, 0.890
# at 768, 0.904 at 512 and 0.873 at 1024 threads).
W3 = dict(name="simple_32ch_1GiB", proto="simple", nchannels=32, nslots=8, slot_bytes=512 << 10,
          fifo_loc="device", wgs_per_channel=4, block_threads=768, xcd_pairing=-1,
          nbytes=1 << 30)

# The same workload with P2P read: the FIFO in the send side's memory.
W3R = dict(W3, name="simple_32ch_1GiB_p2p_read", p2p_read=1)

# Zero-copy launches run one producer workgroup per lane and a few receiver
# workgroups (one thread per lane).  Shapes swept (fraction of HBM, 2 x
# payload): the pair at 16 x 128 with each channel's lanes grouped on one
# XCD, 0.72 (0.58 in dispatch order); the ring at 8 x 512 in dispatch
# order, 0.765 (0.72 grouped by XCD, 0.73 at 16 x 128).
W4_PAIR = dict(name="zc_pair_128MiB", proto="zc", nchannels=32, nslots=1, slot_bytes=512 << 10,
               fifo_loc="device", wgs_per_channel=16, block_threads=128, nbytes=128 << 20)

W4_RING = dict(name="zc_ring_8x128MiB", proto="zc", endpoints=8, channels_per_edge=4,
               nslots=1, slot_bytes=512 << 10, fifo_loc="device", wgs_per_channel=8,
               block_threads=512, xcd_pairing=-1, slice_bytes=128 << 20, max_peers=128)

# The same two zero-copy workloads with the destination known before the
# launch (no ptrExchange hand-off): the pair 0.76 grouped, the ring 0.75 at
# 16 x 128 in dispatch order.
W4D_PAIR = dict(W4_PAIR, name="zcd_pair_128MiB", proto="zcd")
W4D_RING = dict(W4_RING, name="zcd_ring_8x128MiB", proto="zcd", wgs_per_channel=16,
                block_threads=128)

W5 = dict(name="host_fifo_16ch_2GiB", proto="simple", nchannels=16, nslots=8,
          slot_bytes=256 << 10, fifo_loc="host", wgs_per_channel=8, block_threads=1024,
          ctrl_loc=1, total_bytes=2 << 30)

# The copy-engine relay (SIMPLE through send FIFO -> pinned staging FIFO ->
# receive FIFO, moved by two host proxies on the DMA engines): one 512 MiB
# transfer, and the host-FIFO workload's message mix.  Every step is one DMA
# copy per direction, and a copy has a fixed cost (about 4 us at the least),
# so the mix's many small messages want few channels: swept, one channel of
# 8 x 8 MiB slots moved the mix at 42 GB/s and 512 MiB at 46 GB/s, two
# channels 41 and 45, four channels of 4 MiB 34 and 42, sixteen 16 and 26.
W5R = dict(name="relay_1ch_8MiB", proto="simple", nchannels=1, nslots=8, slot_bytes=8 << 20,
           fifo_loc="relay", wgs_per_channel=8, block_threads=1024, nbytes=512 << 20,
           total_bytes=2 << 30)

_ATTRS = ("wgs_per_channel", "block_threads", "ctrl_loc", "timeout_ms", "xcd_pairing", "ordering",
          "p2p_read", "place_trials", "cooperative")


def make_conn(cfg: dict, **override) -> X.Conn:
    c = dict(cfg, **override)
    attrs = {k: c[k] for k in _ATTRS if k in c}
    return X.Conn(c["proto"], c.get("nchannels", 1), c["nslots"], c["slot_bytes"], c["fifo_loc"],
                  **attrs)


class Ring:
    """Logical endpoints on one GPU connected by the host schedule's ring
    plan; one edge per (r, (r + 1) mod n), each with its own channels."""

    def __init__(self, cfg: dict):
        import numpy as np
        n = cfg["endpoints"]
        rm = np.zeros((n, n), dtype=np.uint64)
        sm = np.zeros((n, n), dtype=np.uint64)
        for r in range(n):
            rm[r], sm[r] = X.sched_ring_masks(r, n, cfg["channels_per_edge"])
        attrs = {k: cfg[k] for k in _ATTRS if k in cfg}
        self.n = n
        self.slice = cfg["slice_bytes"]
        self.edges = X.endpoints_connect(n, rm, sm, cfg.get("max_peers", 128), cfg["proto"],
                                         cfg["nslots"], cfg["slot_bytes"], cfg["fifo_loc"], **attrs)

    def run(self, a, b, stream=None) -> None:
        """Endpoint r's slice of a goes to endpoint (r+1) mod n's slice of b."""
        keys = sorted(self.edges)
        conns = [self.edges[k] for k in keys]
        dev = conns[0].device if conns else None
        pa = X._buf(a, self.n * self.slice, dev, "Ring.run: a")
        pb = X._buf(b, self.n * self.slice, dev, "Ring.run: b")
        src = [pa + s * self.slice for s, _ in keys]
        dst = [pb + d * self.slice for _, d in keys]
        X.run_batch(conns, src, dst, [self.slice] * len(keys), stream)

    def close(self) -> None:
        for c in self.edges.values():
            c.close()


def make_ring(cfg: dict) -> Ring:
    return Ring(cfg)


def run_pingpong(fwd: X.Conn, rev: X.Conn, a, b, c, nbytes: int, iters: int, stream=None) -> None:
    X.run_pingpong(fwd, rev, a, b, c, nbytes, iters, stream)


def message_offsets(sizes) -> list[int]:
    offs, off = [], 0
    for s in sizes:
        offs.append(off)
        off += s
    return offs


def run_messages(conn: X.Conn, a, b, sizes, stream=None) -> None:
    """One transfer (one launch) per message, at consecutive offsets of a and b."""
    off = 0
    total = sum(int(s) for s in sizes)
    pa = X._buf(a, total, conn.device, "run_messages: a")
    pb = X._buf(b, total, conn.device, "run_messages: b")
    for s in sizes:
        conn.run(pa + off, pb + off, s, stream)
        off += s


def run_message_list(conn: X.Conn, a, b, sizes, stream=None) -> None:
    """The same messages through xfer_run_messages (up to 128 per launch)."""
    conn.run_messages(a, b, message_offsets(sizes), sizes, stream)
