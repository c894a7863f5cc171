"""CPU oracle of the FIFO send/recv data plane (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It wraps ``oracle.c`` and ``threaded.c`` (plain
C, built with gcc into ``liboracle.so`` next to them) through ctypes and shares
no code with the GPU library.  See the header comment of ``oracle.c`` for what is modelled and
for every reading taken where the pages are silent.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, f) for f in ("oracle.c", "threaded.c", "oracle.h",
                                        "oracle_internal.h")]
LIB = os.path.join(HERE, "liboracle.so")

SIMPLE, LL, ZC, ZCD, RELAY = 0, 1, 2, 3, 4
PROTO_NAMES = {"simple": SIMPLE, "ll": LL, "zc": ZC, "zerocopy": ZC, "zcd": ZCD,
               "zerocopy_direct": ZCD, "relay": RELAY}

OP_RECV_SETUP, OP_SEND_SETUP, OP_CONNECT_BATCH = 0, 1, 2

# Producer program orders: the pages' order, and the kernels' where it differs.
ORDER = {
    "pages": 0,
    "zc_take_ahead": 1,  # ZC: take step g+1's address after writing step g, before tail = g+1
}
# LL, the striped kernels' order: aligned groups of m steps, step j written by
# sub-producer j mod m and read by sub-consumer j mod m, one head per group.
GROUP_MAX = 4
ORDER.update({"ll_group%d" % m: 0x100 + m for m in range(1, GROUP_MAX + 1)})

MUT = {
    "none": 0,
    "weak_credit": 1,
    "early_tail": 2,
    "no_acquire": 3,
    "torn_line": 4,
    "zc_no_wait": 5,
    "zc_no_reset": 6,
    "early_head": 7,
    "zc_ahead_past_end": 8,
    "relay_early": 9,
    "group_no_barrier": 10,
}
VIOLATIONS = {
    0: "ok",
    1: "overwrite",
    2: "read_unfilled",
    3: "read_early",
    4: "window",
    5: "wrong_ptr",
    6: "deadlock",
    7: "result",
    8: "counters",
    9: "confluence",
    10: "state_limit",
}

_lock = threading.Lock()
_lib = None


def _stale() -> bool:
    return not os.path.exists(LIB) or os.path.getmtime(LIB) < max(map(os.path.getmtime, SRCS))


def build(force: bool = True) -> str:
    """Compile the oracle's C sources into liboracle.so with gcc."""
    if not force and not _stale():
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp,
           *[f for f in SRCS if f.endswith(".c")], "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


class _EnumResult(C.Structure):
    _fields_ = [
        ("states", C.c_uint64),
        ("terminals", C.c_uint64),
        ("transitions", C.c_uint64),
        ("violation", C.c_int),
        ("channel", C.c_int),
        ("msg", C.c_char * 256),
    ]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if _stale():
                build()
            L = C.CDLL(LIB)
            u64p = C.POINTER(C.c_uint64)
            ip = C.POINTER(C.c_int)
            vp = C.c_void_p
            L.orc_peers.argtypes = [C.c_int, C.c_int, C.c_int, ip, ip]
            L.orc_ring_masks.argtypes = [C.c_int, C.c_int, C.c_int, u64p, u64p]
            L.orc_plan.argtypes = [C.c_int, C.c_int, u64p, u64p, C.c_int, ip, C.c_int, ip]
            L.orc_step_bytes.argtypes = [C.c_int, C.c_uint64]
            L.orc_step_bytes.restype = C.c_uint64
            L.orc_partition.argtypes = [C.c_uint64, C.c_int, u64p, u64p]
            L.orc_conn_new.argtypes = [C.c_int, C.c_int, C.c_int, C.c_uint64]
            L.orc_conn_new.restype = vp
            L.orc_conn_free.argtypes = [vp]
            L.orc_conn_set_mutation.argtypes = [vp, C.c_int]
            L.orc_conn_set_order.argtypes = [vp, C.c_int]
            L.orc_run.argtypes = [vp, vp, vp, C.c_uint64]
            L.orc_run_pingpong.argtypes = [vp, vp, vp, vp, vp, C.c_uint64, C.c_int]
            L.orc_run_threaded.argtypes = [vp, vp, vp, C.c_uint64, C.c_int]
            L.orc_pingpong_threaded.argtypes = [vp, vp, vp, vp, vp, C.c_uint64, C.c_int,
                                                C.POINTER(C.c_double)]
            L.orc_conn_state.argtypes = [vp, C.c_int, u64p]
            L.orc_conn_fifo.argtypes = [vp, C.c_int, u64p]
            L.orc_conn_fifo.restype = vp
            L.orc_conn_fifo_ex.argtypes = [vp, C.c_int, C.c_int, u64p]
            L.orc_conn_fifo_ex.restype = vp
            L.orc_conn_relay_state.argtypes = [vp, C.c_int, u64p]
            L.orc_enumerate.argtypes = [C.c_int, C.c_int, C.c_int, C.c_uint64, vp, C.c_uint64,
                                        C.c_int, C.c_int, C.c_int, C.c_uint64,
                                        C.POINTER(_EnumResult)]
            _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != 0:
        name = VIOLATIONS.get(rc, "error %d" % rc)
        raise OracleError("%s failed: %s (%d)" % (what, name, rc))


def _proto(p) -> int:
    return PROTO_NAMES[p] if isinstance(p, str) else int(p)


def _ptr(a: np.ndarray):
    return C.c_void_p(a.ctypes.data) if a.size else C.c_void_p(0)


# ---------------------------------------------------------------- schedule
def peers(rank: int, nranks: int, i: int) -> tuple[int, int]:
    r, s = C.c_int(), C.c_int()
    _check(lib().orc_peers(rank, nranks, i, C.byref(r), C.byref(s)), "orc_peers")
    return r.value, s.value


def ring_masks(rank: int, nranks: int, nchannels: int) -> tuple[np.ndarray, np.ndarray]:
    rm = np.zeros(nranks, dtype=np.uint64)
    sm = np.zeros(nranks, dtype=np.uint64)
    u64p = C.POINTER(C.c_uint64)
    _check(lib().orc_ring_masks(rank, nranks, nchannels, rm.ctypes.data_as(u64p),
                                sm.ctypes.data_as(u64p)), "orc_ring_masks")
    return rm, sm


def plan(rank: int, nranks: int, recv_mask, send_mask, max_peers: int = 128) -> list[tuple[int, int, int]]:
    rm = np.ascontiguousarray(recv_mask, dtype=np.uint64)
    sm = np.ascontiguousarray(send_mask, dtype=np.uint64)
    u64p = C.POINTER(C.c_uint64)
    n = C.c_int()
    rc = lib().orc_plan(rank, nranks, rm.ctypes.data_as(u64p), sm.ctypes.data_as(u64p), max_peers,
                        None, 0, C.byref(n))
    if rc not in (0, -4):
        _check(rc, "orc_plan")
    ops = np.zeros(3 * max(n.value, 1), dtype=np.int32)
    _check(lib().orc_plan(rank, nranks, rm.ctypes.data_as(u64p), sm.ctypes.data_as(u64p), max_peers,
                          ops.ctypes.data_as(C.POINTER(C.c_int)), n.value, C.byref(n)), "orc_plan")
    return [tuple(int(x) for x in ops[3 * k:3 * k + 3]) for k in range(n.value)]


# ---------------------------------------------------------------- partition
def step_bytes(proto, slot_bytes: int) -> int:
    return int(lib().orc_step_bytes(_proto(proto), slot_bytes))


def partition(nbytes: int, nchannels: int) -> tuple[list[int], list[int]]:
    b = np.zeros(nchannels, dtype=np.uint64)
    ln = np.zeros(nchannels, dtype=np.uint64)
    u64p = C.POINTER(C.c_uint64)
    _check(lib().orc_partition(nbytes, nchannels, b.ctypes.data_as(u64p), ln.ctypes.data_as(u64p)),
           "orc_partition")
    return [int(x) for x in b], [int(x) for x in ln]


# ---------------------------------------------------------------- protocol
def zero_copy_offsets(proto, nbytes: int, nchannels: int, slot_bytes: int) -> list[list[int]]:
    """Per channel, the destination offset of each step of one transfer, in
    step order: the addresses a zero-copy receiver publishes through
    ptrExchange, one per step, and the ones a zero-copy-direct producer
    writes to (transfer page, zero copy, both kinds; reading R7).  The
    simulator holds its producer to exactly this sequence: taking any other
    address is the violation "producer took an address not published for
    its step"."""
    beg, ln = partition(nbytes, nchannels)
    S = step_bytes(proto, slot_bytes)
    return [[b + j * S for j in range((n + S - 1) // S)] for b, n in zip(beg, ln)]


class Conn:
    """A simulated connection; its counters and FIFO persist across runs."""

    def __init__(self, proto, nchannels: int, nslots: int, slot_bytes: int):
        self.proto = _proto(proto)
        self.nchannels = nchannels
        self.nslots = nslots
        self.slot_bytes = slot_bytes
        self._h = lib().orc_conn_new(self.proto, nchannels, nslots, slot_bytes)
        if not self._h:
            raise OracleError("orc_conn_new rejected its arguments")

    def close(self) -> None:
        if self._h:
            lib().orc_conn_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_mutation(self, name: str) -> None:
        lib().orc_conn_set_mutation(self._h, MUT[name])

    def set_order(self, name: str) -> None:
        lib().orc_conn_set_order(self._h, ORDER[name])

    def run(self, A: np.ndarray, B: np.ndarray, nbytes: int | None = None) -> None:
        """Transfer A[:n] into B[:n] (both uint8 arrays, modified in place)."""
        n = A.size if nbytes is None else int(nbytes)
        assert A.dtype == np.uint8 and B.dtype == np.uint8 and A.size >= n and B.size >= n
        assert A.flags.c_contiguous and B.flags.c_contiguous
        _check(lib().orc_run(self._h, _ptr(A), _ptr(B), n), "orc_run")

    def run_threaded(self, A: np.ndarray, B: np.ndarray, nthreads: int,
                     nbytes: int | None = None) -> None:
        """The same transfer in the threaded mode: every channel's producer and
        consumer as actors on `nthreads` threads (clamped to 2 x channels)."""
        n = A.size if nbytes is None else int(nbytes)
        assert A.dtype == np.uint8 and B.dtype == np.uint8 and A.size >= n and B.size >= n
        assert A.flags.c_contiguous and B.flags.c_contiguous
        _check(lib().orc_run_threaded(self._h, _ptr(A), _ptr(B), n, int(nthreads)),
               "orc_run_threaded")

    def state(self, channel: int) -> dict:
        out = (C.c_uint64 * 4)()
        _check(lib().orc_conn_state(self._h, channel, out), "orc_conn_state")
        return {"head": out[0], "tail": out[1], "ptr_exchange": out[2], "steps": out[3]}

    def relay_state(self, channel: int) -> dict:
        """Relay connections: the send proxy's and the receive proxy's tails."""
        out = (C.c_uint64 * 2)()
        _check(lib().orc_conn_relay_state(self._h, channel, out), "orc_conn_relay_state")
        return {"send_proxy_tail": out[0], "recv_proxy_tail": out[1]}

    def fifo(self, channel: int, which: int = 0) -> np.ndarray:
        """FIFO bytes of a channel; relay connections: which = 0 send, 1 staging,
        2 receive."""
        n = C.c_uint64()
        p = lib().orc_conn_fifo_ex(self._h, int(which), channel, C.byref(n))
        if not p:
            return np.zeros(0, dtype=np.uint8)
        return np.ctypeslib.as_array((C.c_uint8 * n.value).from_address(p)).copy()


def run_pingpong(fwd: Conn, rev: Conn, a: np.ndarray, b: np.ndarray, c: np.ndarray,
                 nbytes: int, iters: int) -> None:
    _check(lib().orc_run_pingpong(fwd._h, rev._h, _ptr(a), _ptr(b), _ptr(c), nbytes, iters),
           "orc_run_pingpong")



def pingpong_threaded(fwd: Conn, rev: Conn, a: np.ndarray, b: np.ndarray, c: np.ndarray,
                      nbytes: int, iters: int) -> float:
    """iters round trips a -> b (fwd), b -> c (rev) with the two endpoints on two
    threads (on two distinct cores when possible); returns the wall seconds."""
    for x in (a, b, c):
        assert x.dtype == np.uint8 and x.flags.c_contiguous and x.size >= nbytes
    sec = C.c_double()
    _check(lib().orc_pingpong_threaded(fwd._h, rev._h, _ptr(a), _ptr(b), _ptr(c), int(nbytes),
                                       int(iters), C.byref(sec)), "orc_pingpong_threaded")
    return sec.value

def enumerate_interleavings(proto, nchannels: int, nslots: int, slot_bytes: int, A: np.ndarray,
                            mutation: str = "none", prior_runs: int = 0,
                            max_states: int = 2_000_000, order: str = "pages") -> dict:
    """Every interleaving of one transfer of A; returns counts and the first violation."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    res = _EnumResult()
    rc = lib().orc_enumerate(_proto(proto), nchannels, nslots, slot_bytes, _ptr(A), A.size,
                             MUT[mutation], ORDER[order], prior_runs, max_states, C.byref(res))
    if rc != 0:
        raise OracleError("orc_enumerate error %d" % rc)
    return {
        "states": res.states,
        "terminals": res.terminals,
        "transitions": res.transitions,
        "violation": VIOLATIONS.get(res.violation, str(res.violation)),
        "channel": res.channel,
        "msg": res.msg.decode(),
    }
