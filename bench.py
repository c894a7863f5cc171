"""Benchmark of the MI355X FIFO send/recv data plane; prints ONE JSON line.

value: payload GB/s of the SIMPLE copy workload with 32 channels x 8 slots x
512 KiB in HBM moving 1 GiB (4 workgroups per channel side), inputs resident
in HBM.  A step is one such transfer (one kernel launch holding both
endpoints).  The other modes are measured in the same run and reported under
"modes": the single-pair SIMPLE transfer, the LL ping-pong latency sweep,
zero-copy (pair and 8-endpoint ring, with the destination exchanged per step
or known before the launch), the host-memory FIFO, and the copy-engine relay.

Real bytes per payload byte: SIMPLE 4 (read A, write FIFO, read FIFO, write
B), zero-copy 2, LL 6 (read A, 8-byte lines for 4 payload bytes written and
read, write B); host FIFO: 1 byte down and 1 byte up the PCIe link.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "payload GB/s + % of HBM/PCIe roofline per mode; LL small-msg latency (µs)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
PCIE_PEAK_GBS = 64.0           # PCIe 5.0 x16, per direction, nominal
KERNEL_SRC = os.path.join(ROOT, "recv_fifo_plane_amd", "csrc", "kernels.hip")
PMC_FILE = os.path.join(ROOT, "profiles", "simple_32ch_1GiB_pmc.txt")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def pmc_traffic() -> float | None:
    """HBM bytes per launch of the headline kernel from the committed
    rocprofv3 counter summary, or None when absent or taken on other code."""
    if not os.path.exists(PMC_FILE):
        return None
    vals = {}
    with open(PMC_FILE, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events on the stream the kernels are launched on."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        self.last = []  # ms of each timed launch of the last call, in order

    def median(self) -> float:
        return statistics.median(self.last)

    def time_launches(self, fn, warmup: int, steps: int) -> tuple[float, float]:
        """Returns (ms per step over the whole timed region, mean ms per launch
        from per-launch event pairs).  torch work inside fn is queued on the
        same stream."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            return self._time(fn, warmup, steps)

    def _time(self, fn, warmup: int, steps: int) -> tuple[float, float]:
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(self.stream)
        for a, b in evs:
            a.record(self.stream)
            fn()
            b.record(self.stream)
        t1.record(self.stream)
        torch.cuda.synchronize()
        total = t0.elapsed_time(t1) / steps
        self.last = [a.elapsed_time(b) for a, b in evs]
        per = sum(self.last) / steps
        return total, per


def check_no_error(conn, nch: int, what: str) -> None:
    for c in range(nch):
        st = conn.query(c)
        if st["error"] or not st["lanes_agree"]:
            raise RuntimeError("%s: channel %d state %s" % (what, c, st))


def chan_steps(n: int, nch: int, step: int) -> list[int]:
    """Steps of each channel in one transfer of n bytes: contiguous channel
    ranges of ceil(n / nch) rounded up to 16 bytes, cut into steps."""
    per = -(-n // nch)
    per = (per + 15) & ~15
    out = []
    for c in range(nch):
        b = min(n, c * per)
        e = min(n, b + per)
        out.append(-(-(e - b) // step))
    return out


def check_counters(conn, nch: int, step: int, transfers, what: str) -> None:
    """Every launch moved what it was given: each channel's head and tail
    (every lane's) equal the steps of all transfers run on the connection,
    transfers = [(nbytes, times)], and the address word is clear."""
    exp = [0] * nch
    for n, times in transfers:
        for c, k in enumerate(chan_steps(n, nch, step)):
            exp[c] += k * times
    for c in range(nch):
        st = conn.query(c)
        if (st["error"] or not st["lanes_agree"] or st["ptr_exchange"] or
                (st["head"], st["tail"], st["steps"]) != (exp[c], exp[c], exp[c])):
            raise RuntimeError("%s: channel %d state %s, expected head = tail = %d"
                               % (what, c, st, exp[c]))


def final_check(torch, T, launch, a, b) -> bool:
    """One more launch into a cleared destination, then B == A."""
    with torch.cuda.stream(T.stream):
        b.zero_()
        launch()
    torch.cuda.synchronize()
    return bool(torch.equal(a, b))


def bench_w3(torch, T, W, synth, steps, warmup, cfg=None):
    cfg = cfg or W.W3
    n = cfg["nbytes"]
    A = synth.bf16_normal_bytes(n, synth.workload_seed(3))
    a = torch.from_numpy(A).to("cuda")
    b = torch.empty_like(a)
    conn = W.make_conn(cfg)
    s = T.stream
    total, per = T.time_launches(lambda: conn.run(a, b, n, s), warmup, steps)
    med = T.median()
    torch.cuda.synchronize()
    ok = bool(torch.equal(a, b)) and final_check(torch, T, lambda: conn.run(a, b, n, s), a, b)
    check_counters(conn, cfg["nchannels"], cfg["slot_bytes"], [(n, warmup + steps + 1)],
                   cfg["name"])
    g, blk = conn.launch_shape()
    conn.close()
    del a, b
    return A, {"ms_per_step": total, "kernel_ms": per, "kernel_ms_median": med,
               "payload_gbs": n / (total * 1e-3) / 1e9,
               "b_equals_a": ok, "workgroups": g, "block_threads": blk,
               "self_check": "B == A after every timed launch and after one more launch into a "
                             "cleared B; every channel's head = tail = %d (64 steps x %d launches)"
                             % (64 * (warmup + steps + 1), warmup + steps + 1)}


def bench_w1(torch, T, W, synth):
    cfg = W.W1
    n = cfg["nbytes"]
    a = torch.from_numpy(synth.uint8_uniform(n, synth.workload_seed(1))).to("cuda")
    b = torch.empty_like(a)
    conn = W.make_conn(cfg)
    total, per = T.time_launches(lambda: conn.run(a, b, n, T.stream), 5, 100)
    med, low = T.median(), min(T.last)
    ok = bool(torch.equal(a, b)) and final_check(torch, T, lambda: conn.run(a, b, n, T.stream),
                                                 a, b)
    check_counters(conn, 1, cfg["slot_bytes"], [(n, 106)], cfg["name"])
    conn.close()
    gbs = n / (per * 1e-3) / 1e9
    # Ceiling of one workgroup copying A -> B straight (zero-copy, one channel,
    # one 4 MiB step: a single address hand-off, then a plain copy).
    zc = W.make_conn(dict(cfg, proto="zc", nslots=1, slot_bytes=n))
    b.zero_()
    _, per_zc = T.time_launches(lambda: zc.run(a, b, n, T.stream), 5, 100)
    check_counters(zc, 1, n, [(n, 105)], "W1 single-workgroup copy")
    ok = ok and bool(torch.equal(a, b))
    zc.close()
    wg = n / (per_zc * 1e-3) / 1e9
    return {"payload_gbs": round(gbs, 2), "real_gbs": round(4 * gbs, 2),
            "hbm_frac": round(4 * gbs / HBM_PEAK_GBS, 4), "kernel_us": round(per * 1e3, 2),
            "kernel_us_median": round(med * 1e3, 2), "kernel_us_min": round(low * 1e3, 2),
            "b_equals_a": ok, "note": "one producer/consumer workgroup pair",
            "single_wg_copy_ceiling": {
                "payload_gbs": round(wg, 2), "kernel_us": round(per_zc * 1e3, 2),
                "vs_ceiling": round(gbs / wg, 3),
                "note": "one %d-thread workgroup copying the 4 MiB straight into B; each side of "
                        "the FIFO pair is one such copy" % cfg["block_threads"]}}


def bench_w2(torch, T, W, synth):
    cfg = W.W2
    iters = cfg["iters"]
    out = {}
    # One pair of connections for every size, so that the curve shows the
    # size alone: the latency also depends on where the connections' FIFO
    # and control words sit in HBM, which place_trials picks by measurement
    # (the spread over placements is measured below).
    fwd, rev = W.make_conn(cfg), W.make_conn(cfg)
    done = []  # (bytes, messages) each connection has carried
    for size in W.W2_SIZES:
        A = synth.int32_uniform_bytes(size, synth.workload_seed(2) + size)
        a = torch.from_numpy(A).to("cuda")
        b = torch.zeros_like(a)
        c = torch.zeros_like(a)
        total, per = T.time_launches(
            lambda: W.run_pingpong(fwd, rev, a, b, c, size, iters, T.stream), 1, 3)
        done.append((size, 4 * iters))
        check_counters(fwd, 1, cfg["slot_bytes"] // 2, done, "W2 forward")
        check_counters(rev, 1, cfg["slot_bytes"] // 2, done, "W2 reverse")
        ok = bool(torch.equal(a, b) and torch.equal(a, c))
        one_way_us = per * 1e3 / (2 * iters)
        out[str(size)] = {"one_way_us": round(one_way_us, 3),
                          "payload_gbs": round(size / (one_way_us * 1e-6) / 1e9, 3),
                          "ok": ok}
    fwd.close()
    rev.close()
    # 8 B over eight pairs of connections alive at once (so at different
    # addresses): with one allocation each, and with the workload's
    # placement by measurement.
    A = synth.int32_uniform_bytes(8, synth.workload_seed(2) + 8)
    a = torch.from_numpy(A).to("cuda")
    for key, trials in (("placement_8B_one_allocation", 0),
                        ("placement_8B_place_trials", cfg["place_trials"])):
        pairs = [(W.make_conn(cfg, place_trials=trials), W.make_conn(cfg, place_trials=trials))
                 for _ in range(8)]
        spread, ok = [], True
        for f, r in pairs:
            b = torch.zeros_like(a)
            c = torch.zeros_like(a)
            _, per = T.time_launches(lambda: W.run_pingpong(f, r, a, b, c, 8, iters, T.stream),
                                     1, 3)
            check_no_error(f, 1, "W2 placement")
            check_no_error(r, 1, "W2 placement")
            ok = ok and bool(torch.equal(a, b) and torch.equal(a, c))
            spread.append(per * 1e3 / (2 * iters))
        for f, r in pairs:
            f.close()
            r.close()
        spread.sort()
        out[key] = {"pairs": len(spread), "place_trials": trials,
                    "min_us": round(spread[0], 3),
                    "median_us": round(statistics.median(spread), 3),
                    "max_us": round(spread[-1], 3), "ok": ok}
    big = out[str(W.W2_SIZES[-1])]
    big["real_gbs_6x"] = round(6 * big["payload_gbs"], 2)
    big["hbm_frac_6x"] = round(6 * big["payload_gbs"] / HBM_PEAK_GBS, 4)
    # Secondary: messages back to back on one connection in one launch (the
    # pipeline never drains), and one host-issued launch per message.
    sec = {}
    for size in (8, 1024, 65536):
        A = synth.int32_uniform_bytes(size, synth.workload_seed(2) + size)
        a = torch.from_numpy(A).to("cuda")
        b = torch.zeros_like(a)
        conn = W.make_conn(cfg)
        _, per_loop = T.time_launches(lambda: conn.run_loop(a, b, size, iters, T.stream), 1, 3)
        ok = bool(torch.equal(a, b))
        b.zero_()
        nrun = 1000
        _, per_runs = T.time_launches(
            lambda: [conn.run(a, b, size, T.stream) for _ in range(nrun)], 1, 3)
        check_no_error(conn, 1, "W2 secondary")
        ok = ok and bool(torch.equal(a, b))
        conn.close()
        sec[str(size)] = {"in_launch_us_per_msg": round(per_loop * 1e3 / iters, 3),
                          "host_issued_us_per_msg": round(per_runs * 1e3 / nrun, 3), "ok": ok}
    out["serialized_one_connection"] = sec
    return out


def bench_w4(torch, T, W, synth):
    """Zero-copy through ptrExchange (pair and ring), and the same shapes with
    the destination known before the launch ("direct": no pointer hand-off)."""
    res = {}
    for pair_cfg, ring_cfg, key in ((W.W4_PAIR, W.W4_RING, ""), (W.W4D_PAIR, W.W4D_RING, "direct_")):
        proto = pair_cfg["proto"]
        cfg = pair_cfg
        n = cfg["nbytes"]
        a = torch.from_numpy(synth.fp32_uniform_bytes(n, synth.workload_seed(4))).to("cuda")
        b = torch.empty_like(a)
        conn = W.make_conn(cfg)
        total, per = T.time_launches(lambda: conn.run(a, b, n, T.stream), 3, 20)
        med = T.median()
        ok = bool(torch.equal(a, b)) and final_check(
            torch, T, lambda: conn.run(a, b, n, T.stream), a, b)
        check_counters(conn, cfg["nchannels"], cfg["slot_bytes"], [(n, 24)], cfg["name"])
        conn.close()
        gbs = n / (per * 1e-3) / 1e9
        res[key + "pair"] = {"payload_gbs": round(gbs, 2), "real_gbs": round(2 * gbs, 2),
                             "hbm_frac": round(2 * gbs / HBM_PEAK_GBS, 4),
                             "kernel_ms": round(per, 4), "kernel_ms_median": round(med, 4),
                             "b_equals_a": ok}
        del a, b
        cfg = ring_cfg
        ring = W.make_ring(cfg)
        tot = cfg["endpoints"] * cfg["slice_bytes"]
        a = torch.from_numpy(synth.fp32_uniform_bytes(tot, synth.workload_seed(4) + 100)).to("cuda")
        b = torch.empty_like(a)
        total, per = T.time_launches(lambda: ring.run(a, b, T.stream), 3, 20)
        med = T.median()
        S = cfg["slice_bytes"]

        def edges_ok():
            return all(bool(torch.equal(a[r * S:(r + 1) * S],
                                        b[((r + 1) % 8) * S:((r + 1) % 8 + 1) * S]))
                       for r in range(8))

        ok = edges_ok()
        with torch.cuda.stream(T.stream):
            b.zero_()
            ring.run(a, b, T.stream)
        torch.cuda.synchronize()
        ok = ok and edges_ok()
        for e in ring.edges.values():
            check_counters(e, cfg["channels_per_edge"], cfg["slot_bytes"], [(S, 24)],
                           cfg["name"])
        ring.close()
        del a, b
        gbs = tot / (per * 1e-3) / 1e9
        res[key + "ring"] = {"payload_gbs": round(gbs, 2), "real_gbs": round(2 * gbs, 2),
                             "hbm_frac": round(2 * gbs / HBM_PEAK_GBS, 4),
                             "kernel_ms": round(per, 4), "kernel_ms_median": round(med, 4),
                             "edges_ok": ok}
    return res


def bench_w5(torch, T, W, synth):
    cfg = W.W5
    tot = cfg["total_bytes"]
    sizes = synth.log_uniform_message_sizes(tot, synth.workload_seed(5))
    a = torch.from_numpy(synth.uint8_uniform(tot, synth.workload_seed(5))).to("cuda")
    b = torch.empty_like(a)
    conn = W.make_conn(cfg)
    # each figure: the median over 5 runs of the whole message sequence
    T.time_launches(lambda: W.run_messages(conn, a, b, sizes, T.stream), 1, 5)
    each = T.median()
    check_counters(conn, cfg["nchannels"], cfg["slot_bytes"], [(s_, 6) for s_ in sizes],
                   cfg["name"])
    ok_each = bool(torch.equal(a, b))
    b.zero_()
    T.time_launches(lambda: W.run_message_list(conn, a, b, sizes, T.stream), 1, 5)
    total = T.median()
    check_counters(conn, cfg["nchannels"], cfg["slot_bytes"], [(s_, 12) for s_ in sizes],
                   cfg["name"])
    ok = ok_each and bool(torch.equal(a, b))
    conn.close()
    gbs = tot / (total * 1e-3) / 1e9
    gbs_each = tot / (each * 1e-3) / 1e9
    # pinned-memory copy ceilings of the same link, for context: one
    # direction at a time, and both at once (the FIFO's traffic pattern)
    m = 256 << 20
    h = torch.empty(m, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(m, dtype=torch.uint8, device="cuda")
    d2h, _ = T.time_launches(lambda: h.copy_(d, non_blocking=True), 2, 5)
    h2d, _ = T.time_launches(lambda: d.copy_(h, non_blocking=True), 2, 5)
    h2 = torch.empty(m, dtype=torch.uint8, pin_memory=True)
    d2 = torch.empty(m, dtype=torch.uint8, device="cuda")
    s_up, s_down = torch.cuda.Stream(), torch.cuda.Stream()

    def duplex():
        with torch.cuda.stream(s_up):
            h.copy_(d, non_blocking=True)
        with torch.cuda.stream(s_down):
            d2.copy_(h2, non_blocking=True)
        s_up.synchronize()
        s_down.synchronize()

    for _ in range(2):
        duplex()
    # a ceiling: the best of 5 trials of 5 (the runtime now and then places
    # both copies on one engine, which halves the rate)
    dup_gbs = 0.0
    for _ in range(5):
        t0 = time.perf_counter()
        for _ in range(5):
            duplex()
        dup_gbs = max(dup_gbs, m / ((time.perf_counter() - t0) / 5) / 1e9)
    d2h_gbs, h2d_gbs = m / (d2h * 1e-3) / 1e9, m / (h2d * 1e-3) / 1e9
    # When the runtime runs the two copies one after the other the reference
    # is no duplex rate at all: report it, but no ratio against it.
    serialized = dup_gbs < 0.75 * min(d2h_gbs, h2d_gbs)
    return {"payload_gbs": round(gbs, 2), "pcie_frac": round(gbs / PCIE_PEAK_GBS, 4),
            "messages": len(sizes), "ms": round(total, 3), "b_equals_a": ok,
            "launches": (len(sizes) + 127) // 128,
            "one_launch_per_message": {"payload_gbs": round(gbs_each, 2),
                                       "pcie_frac": round(gbs_each / PCIE_PEAK_GBS, 4),
                                       "ms": round(each, 3)},
            "pinned_copy_d2h_gbs": round(d2h_gbs, 2),
            "pinned_copy_h2d_gbs": round(h2d_gbs, 2),
            "pinned_copy_duplex_gbs_each_way": round(dup_gbs, 2),
            "pinned_copy_duplex_serialized": serialized,
            "vs_duplex_copy": None if serialized else round(gbs / dup_gbs, 3)}


def bench_relay(torch, T, W, synth, dup_gbs):
    """The copy-engine relay: one 512 MiB transfer and the host-FIFO message
    mix, against the link's full-duplex copy rate."""
    cfg = W.W5R
    tot = cfg["total_bytes"]
    n = cfg["nbytes"]
    sizes = synth.log_uniform_message_sizes(tot, synth.workload_seed(5))
    a = torch.from_numpy(synth.uint8_uniform(tot, synth.workload_seed(5))).to("cuda")
    b = torch.empty_like(a)
    conn = W.make_conn(cfg)
    one, _ = T.time_launches(lambda: conn.run(a, b, n, T.stream), 1, 3)
    check_counters(conn, cfg["nchannels"], cfg["slot_bytes"], [(n, 4)], cfg["name"])
    ok = bool(torch.equal(a[:n], b[:n]))
    b.zero_()
    lst, _ = T.time_launches(lambda: W.run_message_list(conn, a, b, sizes, T.stream), 1, 3)
    check_counters(conn, cfg["nchannels"], cfg["slot_bytes"],
                   [(n, 4)] + [(s_, 4) for s_ in sizes], cfg["name"])
    ok = ok and bool(torch.equal(a, b))
    conn.close()
    g1 = n / (one * 1e-3) / 1e9
    gl = tot / (lst * 1e-3) / 1e9
    return {"payload_gbs": round(g1, 2), "pcie_frac": round(g1 / PCIE_PEAK_GBS, 4),
            "vs_duplex_copy": round(g1 / dup_gbs, 3) if dup_gbs else None,
            "bytes": n, "ms": round(one, 3),
            "message_mix": {"payload_gbs": round(gl, 2), "pcie_frac": round(gl / PCIE_PEAK_GBS, 4),
                            "messages": len(sizes)},
            "b_equals_a": ok,
            "note": "send FIFO (HBM) -> staging FIFO (pinned host) -> receive FIFO (HBM), each "
                    "hop a DMA copy queued by a host proxy thread"}


def plain_copy_ceiling(torch, T) -> dict:
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(7)
    total, per = T.time_launches(lambda: b.copy_(a), 3, 20)
    return {"bytes": n, "ms": round(per, 4), "real_gbs": round(2 * n / (per * 1e-3) / 1e9, 1),
            "payload_gbs": round(n / (per * 1e-3) / 1e9, 1)}


def host_cpu() -> dict:
    """The host CPU the oracle runs on: model name and logical CPUs."""
    model = None
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = None
    return {"model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def _cpu_threads() -> int:
    """Host threads the threaded oracle may use: the CPUs this process may run
    on, capped at 16 (the host share of one GPU) and at 2 x 32 channels."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n, 64))


def cpu_baseline(A, budget_s: float = 8.0) -> dict:
    """The oracle as it is, on the same 1 GiB input: its threaded mode (one
    producer and one consumer actor per channel on the host's cores) is the
    value; the single-threaded sequential simulation and a two-thread LL
    ping-pong latency are reported beside it."""
    import numpy as np

    import oracle
    B = np.empty_like(A)

    def timed(run):
        runs, t0 = 0, time.perf_counter()
        while True:
            conn = oracle.Conn("simple", 32, 8, 512 << 10)
            run(conn)
            conn.close()
            runs += 1
            el = time.perf_counter() - t0
            if el >= budget_s or runs >= 20:
                return runs, el

    threads = _cpu_threads()
    runs_t, el_t = timed(lambda c: c.run_threaded(A, B, threads))
    runs_s, el_s = timed(lambda c: c.run(A, B))
    lat = {}
    for size in (8, 1024, 65536):
        a = np.ascontiguousarray(A[:size])
        b, c = np.zeros(size, np.uint8), np.zeros(size, np.uint8)
        f, r = oracle.Conn("ll", 1, 8, 32 << 10), oracle.Conn("ll", 1, 8, 32 << 10)
        iters = 10000 if size <= 1024 else 2000
        sec = oracle.pingpong_threaded(f, r, a, b, c, size, iters)
        f.close()
        r.close()
        lat[str(size)] = round(sec * 1e6 / (2 * iters), 3)
    return {"value": round(runs_t * A.size / el_t / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "host_cpu": host_cpu(),
            "sample": "%d full transfers of the 1 GiB bf16 input through 32 channels x 8 x 512 KiB "
                      "in the oracle's threaded mode (64 actors on %d threads, %.1f s)"
                      % (runs_t, threads, el_t),
            "single_thread": {"value": round(runs_s * A.size / el_s / 1e9, 3), "unit": "GB/s",
                              "cores": 1, "sample": "%d transfers, sequential simulation, %.1f s"
                                                    % (runs_s, el_s)},
            "ll_pingpong_one_way_us": lat,
            "ll_pingpong_note": "two host threads on two cores, LL 1 channel x 8 x 32 KiB"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", choices=["value", "all", "copy", "zerocopy", "relay", "ll", "host"],
                    default="all",
                    help="value: time only the headline workload; copy: only a plain 1 GiB "
                         "device copy (the calibration kernel of the HBM byte counters); "
                         "zerocopy, relay, ll, host: only that mode (for profiling it alone)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this data plane runs on one GPU (both endpoints in one launch); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2
    import torch

    import synth
    from recv_fifo_plane_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    stream = torch.cuda.Stream()
    T = Timer(torch, stream)
    if args.only == "copy":
        print(json.dumps({"plain_copy_1GiB_torch": plain_copy_ceiling(torch, T)}), flush=True)
        return 0
    if args.only == "zerocopy":
        print(json.dumps({"zerocopy": bench_w4(torch, T, W, synth)}), flush=True)
        return 0
    if args.only == "ll":
        print(json.dumps({"ll_pingpong": bench_w2(torch, T, W, synth)}), flush=True)
        return 0
    if args.only == "host":
        print(json.dumps({"host_fifo_16ch_2GiB": bench_w5(torch, T, W, synth)}), flush=True)
        return 0
    if args.only == "relay":
        # the duplex copy rate of the link is measured by the host-FIFO mode;
        # alone, the relay reports against PCIe only
        print(json.dumps({W.W5R["name"]: bench_relay(torch, T, W, synth, None)}),
              flush=True)
        return 0
    log("bench: W3 simple 32ch 1GiB, %d warmup + %d steps" % (args.warmup, args.steps))
    A, w3 = bench_w3(torch, T, W, synth, args.steps, args.warmup)
    payload = W.W3["nbytes"]
    algo_bytes = 4 * payload
    achieved = algo_bytes / (w3["kernel_ms"] * 1e-3) / 1e9
    traffic = pmc_traffic()
    log("bench: plain 1 GiB device copy (context for the value)")
    plain = plain_copy_ceiling(torch, T)
    line = {
        "metric": METRIC,
        "value": round(w3["payload_gbs"], 2),
        "unit": "GB/s",
        # The same 1 GiB moved by a plain device copy (read A, write B: half the
        # bytes of the FIFO round trip): what the FIFO costs against no FIFO.
        "plain_copy_payload_gbs": plain["payload_gbs"],
        "fifo_vs_plain_copy": round(w3["payload_gbs"] / plain["payload_gbs"], 3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(w3["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic: bf16 bit patterns of N(0,1) (seeded PCG64), resident in HBM",
        "config": {"workload": W.W3["name"], "proto": "simple", "nchannels": 32, "nslots": 8,
                   "slot_bytes": W.W3["slot_bytes"], "fifo": "hbm",
                   "wgs_per_channel_side": W.W3["wgs_per_channel"],
                   "block_threads": w3["block_threads"], "workgroups": w3["workgroups"],
                   "xcd_pairing": W.W3.get("xcd_pairing", 0),
                   "payload_bytes": payload, "b_equals_a": w3["b_equals_a"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel_ms": round(w3["kernel_ms"], 5),
                     "kernel_ms_median": round(w3["kernel_ms_median"], 5),
                     "algorithmic_bytes_per_launch": algo_bytes},
    }
    if args.only == "all":
        log("bench: W1 single pair")
        modes = {"simple_1ch_4MiB": bench_w1(torch, T, W, synth)}
        log("bench: W2 LL ping-pong sweep")
        modes["ll_pingpong"] = bench_w2(torch, T, W, synth)
        log("bench: W3 under P2P read")
        _, w3r = bench_w3(torch, T, W, synth, args.steps, args.warmup, W.W3R)
        real_r = 4 * W.W3R["nbytes"] / (w3r["kernel_ms"] * 1e-3) / 1e9  # as the roofline counts
        modes["simple_32ch_1GiB_p2p_read"] = {
            "payload_gbs": round(w3r["payload_gbs"], 2),
            "real_gbs": round(real_r, 1),
            "hbm_frac": round(real_r / HBM_PEAK_GBS, 4),
            "kernel_ms": round(w3r["kernel_ms"], 5), "b_equals_a": w3r["b_equals_a"],
            "note": "the FIFO in the send side's memory; on one GPU both sides share one HBM"}
        log("bench: W4 zero-copy")
        modes["zerocopy"] = bench_w4(torch, T, W, synth)
        log("bench: W5 host FIFO")
        modes["host_fifo_16ch_2GiB"] = bench_w5(torch, T, W, synth)
        log("bench: copy-engine relay")
        w5 = modes["host_fifo_16ch_2GiB"]
        modes[W.W5R["name"]] = bench_relay(
            torch, T, W, synth,
            None if w5["pinned_copy_duplex_serialized"] else w5["pinned_copy_duplex_gbs_each_way"])
        modes["plain_copy_1GiB_torch"] = plain
        line["modes"] = modes
    if not args.no_cpu_baseline:
        log("bench: CPU baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(A)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
