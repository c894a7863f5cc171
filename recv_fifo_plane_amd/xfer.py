"""ctypes binding of libxfer.so: the C ABI declared in include/xfer.h.

Argument marshalling only: every step of a transfer runs in the library's
HIP kernels.  PyTorch is used for device memory (tensors' data_ptr()) and
streams (cuda_stream handles).  The library must be built (``build.py``);
loading fails loudly when it is missing and cannot be built.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

from . import build as _build

XFER_OK = 0
XFER_ERR_INVALID_ARG = 1
XFER_ERR_NO_MEMORY = 2
XFER_ERR_HIP = 3
XFER_ERR_INTERNAL = 4
XFER_ERR_TIMEOUT = 5
XFER_ERR_ABORTED = 6
XFER_ERR_RANGE = 7
XFER_ERR_STATE = 8

XFER_PROTO_SIMPLE = 0
XFER_PROTO_LL = 1
XFER_PROTO_ZEROCOPY = 2
XFER_PROTO_ZEROCOPY_DIRECT = 3
XFER_FIFO_DEVICE = 0
XFER_FIFO_HOST = 1
XFER_FIFO_RELAY = 2
XFER_CTRL_DEFAULT = 0
XFER_CTRL_DEVICE = 1
XFER_CTRL_HOST = 2
XFER_ORDER_COHERENT = 0
XFER_ORDER_FENCED = 1
XFER_OP_RECV_SETUP = 0
XFER_OP_SEND_SETUP = 1
XFER_OP_CONNECT_BATCH = 2
XFER_MAX_BATCH = 16

PROTOS = {"simple": XFER_PROTO_SIMPLE, "ll": XFER_PROTO_LL, "zc": XFER_PROTO_ZEROCOPY,
          "zerocopy": XFER_PROTO_ZEROCOPY, "zcd": XFER_PROTO_ZEROCOPY_DIRECT,
          "zerocopy_direct": XFER_PROTO_ZEROCOPY_DIRECT}
FIFO_LOCS = {"device": XFER_FIFO_DEVICE, "host": XFER_FIFO_HOST, "relay": XFER_FIFO_RELAY}


class xfer_attr(C.Structure):
    _fields_ = [
        ("wgs_per_channel", C.c_int),
        ("block_threads", C.c_int),
        ("ctrl_loc", C.c_int),
        ("timeout_ms", C.c_uint32),
        ("xcd_pairing", C.c_int),
        ("roles", C.c_int),
        ("ordering", C.c_int),
        ("p2p_read", C.c_int),
        ("place_trials", C.c_int),
        ("cooperative", C.c_int),
    ]


def make_attr(**kw) -> xfer_attr:
    """An xfer_attr from keyword fields; absent ones are 0 (the defaults)."""
    names = [f[0] for f in xfer_attr._fields_]
    bad = set(kw) - set(names)
    if bad:
        raise TypeError("unknown connection attribute(s): " + ", ".join(sorted(bad)))
    return xfer_attr(*[int(kw.get(n, 0)) for n in names])


class xfer_chan_state(C.Structure):
    _fields_ = [
        ("head", C.c_uint64),
        ("tail", C.c_uint64),
        ("ptr_exchange", C.c_uint64),
        ("steps", C.c_uint64),
        ("lanes", C.c_int),
        ("lanes_agree", C.c_int),
        ("error", C.c_int),
        ("reserved", C.c_int),
    ]


class xfer_setup_op(C.Structure):
    _fields_ = [("kind", C.c_int), ("peer", C.c_int), ("channel", C.c_int)]


# Every symbol include/xfer.h declares, with its ctypes signature.
_vp = C.c_void_p
_u64p = C.POINTER(C.c_uint64)
_ip = C.POINTER(C.c_int)
SIGNATURES = {
    "xfer_conn_create": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_size_t, C.c_int, C.POINTER(_vp)]),
    "xfer_conn_create_ex": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_size_t, C.c_int,
                                      C.POINTER(xfer_attr), C.POINTER(_vp)]),
    "xfer_conn_destroy": (C.c_int, [_vp]),
    "xfer_run": (C.c_int, [_vp, _vp, _vp, C.c_size_t, _vp]),
    "xfer_run_batch": (C.c_int, [C.POINTER(_vp), C.POINTER(_vp), C.POINTER(_vp),
                                 C.POINTER(C.c_size_t), C.c_int, _vp]),
    "xfer_run_loop": (C.c_int, [_vp, _vp, _vp, C.c_size_t, C.c_int, _vp]),
    "xfer_run_messages": (C.c_int, [_vp, _vp, _vp, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t),
                                    C.c_int, _vp]),
    "xfer_run_pingpong": (C.c_int, [_vp, _vp, _vp, _vp, _vp, C.c_size_t, C.c_int, _vp]),
    "xfer_run_noalloc": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_size_t, C.POINTER(xfer_attr),
                                   _vp, _vp, C.c_size_t, _vp, _vp]),
    "xfer_conn_query": (C.c_int, [_vp, C.c_int, C.POINTER(xfer_chan_state)]),
    "xfer_conn_fifo": (C.c_int, [_vp, C.c_int, C.POINTER(_vp), C.POINTER(C.c_size_t)]),
    "xfer_conn_read_fifo": (C.c_int, [_vp, C.c_int, _vp, C.c_size_t]),
    "xfer_conn_read_fifo_ex": (C.c_int, [_vp, C.c_int, C.c_int, _vp, C.c_size_t]),
    "xfer_conn_query_relay": (C.c_int, [_vp, C.c_int, _u64p, _u64p]),
    "xfer_conn_abort": (C.c_int, [_vp]),
    "xfer_conn_set_trace": (C.c_int, [_vp, _vp, C.c_size_t]),
    "xfer_conn_set_jitter": (C.c_int, [_vp, C.c_uint32]),
    "xfer_conn_launch_shape": (C.c_int, [_vp, _ip, _ip]),
    "xfer_last_error": (C.c_char_p, []),
    "xfer_status_string": (C.c_char_p, [C.c_int]),
    "xfer_sched_peers": (C.c_int, [C.c_int, C.c_int, C.c_int, _ip, _ip]),
    "xfer_sched_ring_masks": (C.c_int, [C.c_int, C.c_int, C.c_int, _u64p, _u64p]),
    "xfer_sched_plan": (C.c_int, [C.c_int, C.c_int, _u64p, _u64p, C.c_int,
                                  C.POINTER(xfer_setup_op), C.c_int, _ip]),
    "xfer_endpoints_connect": (C.c_int, [C.c_int, _u64p, _u64p, C.c_int, C.c_int, C.c_int,
                                         C.c_size_t, C.c_int, C.POINTER(xfer_attr),
                                         C.POINTER(_vp), _ip]),
}

_lock = threading.Lock()
_lib = None


def lib() -> C.CDLL:
    """Loads libxfer.so (building it first only if it does not exist)."""
    global _lib
    if _lib is not None:  # loaded: no lock on the per-call path
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_build.LIB):
                _build.build()
            L = C.CDLL(_build.LIB)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


class XferError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (status_string(status), msg))
        self.status = status


def status_string(s: int) -> str:
    return lib().xfer_status_string(int(s)).decode()


def last_error() -> str:
    return lib().xfer_last_error().decode()


def check(rc: int) -> None:
    if rc != XFER_OK:
        raise XferError(rc, last_error())


def _stream_handle(stream) -> int | None:
    if stream is None:
        try:
            import torch
            return torch.cuda.current_stream().cuda_stream or None
        except Exception:
            return None
    if isinstance(stream, int):
        return stream or None
    return getattr(stream, "cuda_stream", stream) or None


def _addr(buf) -> int:
    """Device address of a torch tensor, or an integer address."""
    if buf is None:
        return 0
    if isinstance(buf, int):
        return buf
    return int(buf.data_ptr())


def _current_device() -> int | None:
    try:
        import torch
        return torch.cuda.current_device() if torch.cuda.is_available() else None
    except Exception:
        return None


def _buf(buf, nbytes: int, device: int | None, what: str) -> int:
    """Address of a buffer the kernels will access over [0, nbytes).

    An integer is taken as a raw device address: its extent is the caller's
    responsibility.  A tensor must live on the GPU, on the connection's
    device, be contiguous and hold at least nbytes bytes; otherwise
    ValueError is raised before the library is called (a kernel given a
    host address, another device's memory or too short a buffer would
    access memory outside it)."""
    if buf is None or isinstance(buf, int):
        return _addr(buf)
    if not hasattr(buf, "data_ptr"):
        raise TypeError("%s: expected a torch tensor or an integer address, got %s"
                        % (what, type(buf).__name__))
    if nbytes <= 0:
        return int(buf.data_ptr())
    if not getattr(buf, "is_cuda", False):
        raise ValueError("%s: tensor is not in GPU memory (device %s)" % (what, buf.device))
    if device is not None and buf.device.index != device:
        raise ValueError("%s: tensor is on cuda:%s, the connection on cuda:%d"
                         % (what, buf.device.index, device))
    if not buf.is_contiguous():
        raise ValueError("%s: tensor is not contiguous" % what)
    have = buf.numel() * buf.element_size()
    if have < nbytes:
        raise ValueError("%s: tensor holds %d bytes, the transfer touches %d" % (what, have, nbytes))
    return int(buf.data_ptr())


class Conn:
    """One connection (xfer_conn).  Destroy it only after its streams are idle."""

    def __init__(self, proto="simple", nchannels=1, nslots=8, slot_bytes=128 << 10,
                 fifo_loc="device", wgs_per_channel=0, block_threads=0, ctrl_loc=0,
                 timeout_ms=0, xcd_pairing=0, roles=0, ordering=0, p2p_read=0, place_trials=0,
                 cooperative=0, _handle=None):
        self.proto = PROTOS[proto] if isinstance(proto, str) else int(proto)
        self.nchannels = int(nchannels)
        self.nslots = int(nslots)
        self.slot_bytes = int(slot_bytes)
        self.fifo_loc = FIFO_LOCS[fifo_loc] if isinstance(fifo_loc, str) else int(fifo_loc)
        self._h = None
        self.device = _current_device()  # where the library allocated it (the current device)
        if _handle is not None:
            self._h = _handle
            return
        attr = make_attr(wgs_per_channel=wgs_per_channel, block_threads=block_threads,
                         ctrl_loc=ctrl_loc, timeout_ms=timeout_ms, xcd_pairing=xcd_pairing,
                         roles=roles, ordering=ordering, p2p_read=p2p_read,
                         place_trials=place_trials, cooperative=cooperative)
        h = _vp()
        check(lib().xfer_conn_create_ex(self.proto, self.nchannels, self.nslots, self.slot_bytes,
                                        self.fifo_loc, C.byref(attr), C.byref(h)))
        self._h = h.value

    @property
    def handle(self) -> int:
        return self._h

    def close(self) -> None:
        if self._h:
            lib().xfer_conn_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run(self, src, dst, nbytes: int, stream=None) -> None:
        n = int(nbytes)
        s = _buf(src, n, self.device, "run: src")
        d = _buf(dst, n, self.device, "run: dst")
        check(lib().xfer_run(self._h, s, d, n, _stream_handle(stream)))

    def run_loop(self, src, dst, nbytes: int, iters: int, stream=None) -> None:
        n = int(nbytes)
        s = _buf(src, n, self.device, "run_loop: src")
        d = _buf(dst, n, self.device, "run_loop: dst")
        check(lib().xfer_run_loop(self._h, s, d, n, int(iters), _stream_handle(stream)))

    def run_messages(self, src, dst, offsets, sizes, stream=None) -> None:
        n = len(sizes)
        if len(offsets) != n:
            raise ValueError("run_messages: %d offsets for %d sizes" % (len(offsets), n))
        offs_l = [int(x) for x in offsets]
        szs_l = [int(x) for x in sizes]
        if any(x < 0 for x in offs_l + szs_l):
            raise ValueError("run_messages: negative offset or size")
        extent = max([o + z for o, z in zip(offs_l, szs_l) if z] or [0])
        s = _buf(src, extent, self.device, "run_messages: src")
        d = _buf(dst, extent, self.device, "run_messages: dst")
        offs = (C.c_size_t * max(n, 1))(*offs_l)
        szs = (C.c_size_t * max(n, 1))(*szs_l)
        check(lib().xfer_run_messages(self._h, s, d, offs, szs, n, _stream_handle(stream)))

    def query(self, channel: int) -> dict:
        st = xfer_chan_state()
        check(lib().xfer_conn_query(self._h, int(channel), C.byref(st)))
        return {"head": st.head, "tail": st.tail, "ptr_exchange": st.ptr_exchange,
                "steps": st.steps, "lanes": st.lanes, "lanes_agree": bool(st.lanes_agree),
                "error": st.error}

    def fifo_bytes(self, channel: int) -> int:
        p, n = _vp(), C.c_size_t()
        check(lib().xfer_conn_fifo(self._h, int(channel), C.byref(p), C.byref(n)))
        return n.value

    def read_fifo(self, channel: int, which: int = 0):
        """One channel's FIFO bytes; a relay's which = 0 send, 1 staging, 2 receive."""
        import numpy as np
        n = self.fifo_bytes(channel)
        out = np.zeros(n, dtype=np.uint8)
        if n:
            check(lib().xfer_conn_read_fifo_ex(self._h, int(which), int(channel), out.ctypes.data,
                                               n))
        return out

    def query_relay(self, channel: int) -> dict:
        """A relay's proxy tails for one channel (after the stream is synchronised)."""
        y, g = C.c_uint64(), C.c_uint64()
        check(lib().xfer_conn_query_relay(self._h, int(channel), C.byref(y), C.byref(g)))
        return {"send_proxy_tail": y.value, "recv_proxy_tail": g.value}

    def abort(self) -> None:
        check(lib().xfer_conn_abort(self._h))

    def set_jitter(self, seed: int) -> None:
        """Random delays in the step loops (debug); 0 turns them off."""
        check(lib().xfer_conn_set_jitter(self._h, int(seed) & 0xFFFFFFFF))

    def set_trace(self, records, nrecords: int = 0) -> None:
        """Step trace into a device buffer (a torch tensor of TRACE_REC_BYTES x
        nrecords bytes, or an address with nrecords); None turns it off."""
        if records is None:
            check(lib().xfer_conn_set_trace(self._h, None, 0))
            return
        if not isinstance(records, int):
            nrecords = records.numel() * records.element_size() // TRACE_REC_BYTES
        addr = _buf(records, int(nrecords) * TRACE_REC_BYTES, self.device, "set_trace: records")
        check(lib().xfer_conn_set_trace(self._h, addr, int(nrecords)))

    def launch_shape(self) -> tuple[int, int]:
        g, b = C.c_int(), C.c_int()
        check(lib().xfer_conn_launch_shape(self._h, C.byref(g), C.byref(b)))
        return g.value, b.value


XFER_TRACE_ACQUIRE, XFER_TRACE_PUBLISH = 0, 1
TRACE_REC_BYTES = 32


def trace_records(raw):
    """Decodes a step-trace buffer (bytes as a numpy uint8 array) into a
    structured array of xfer_trace_rec."""
    import numpy as np
    dt = np.dtype([("time", "<u8"), ("step", "<u8"), ("value", "<u8"), ("channel", "<u4"),
                   ("lane", "<u2"), ("side", "u1"), ("event", "u1")])
    assert dt.itemsize == TRACE_REC_BYTES
    return np.frombuffer(np.ascontiguousarray(raw).tobytes(), dtype=dt)


def run_batch(conns, srcs, dsts, nbytes, stream=None) -> None:
    n = len(conns)
    if not (len(srcs) == len(dsts) == len(nbytes) == n):
        raise ValueError("run_batch: conns, srcs, dsts and nbytes differ in length")
    hs = (_vp * n)(*[c.handle for c in conns])
    ss = (_vp * n)(*[_buf(s, int(k), c.device, "run_batch: src[%d]" % i)
                     for i, (c, s, k) in enumerate(zip(conns, srcs, nbytes))])
    ds = (_vp * n)(*[_buf(d, int(k), c.device, "run_batch: dst[%d]" % i)
                     for i, (c, d, k) in enumerate(zip(conns, dsts, nbytes))])
    ns = (C.c_size_t * n)(*[int(x) for x in nbytes])
    check(lib().xfer_run_batch(hs, ss, ds, ns, n, _stream_handle(stream)))


def run_pingpong(fwd: Conn, rev: Conn, a, b, c, nbytes: int, iters: int, stream=None) -> None:
    n = int(nbytes)
    pa = _buf(a, n, fwd.device, "run_pingpong: a")
    pb = _buf(b, n, fwd.device, "run_pingpong: b")
    pc = _buf(c, n, fwd.device, "run_pingpong: c")
    check(lib().xfer_run_pingpong(fwd.handle, rev.handle, pa, pb, pc, n, int(iters),
                                  _stream_handle(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20  # XFER_NOALLOC_SCRATCH_BYTES


def run_noalloc(proto, nchannels: int, nslots: int, slot_bytes: int, src, dst, nbytes: int,
                status=None, stream=None, **attr) -> None:
    """xfer_run_noalloc: one transfer through the library's fixed device
    array (no connection, nothing allocated).  status: None, or a device
    tensor of at least 4 bytes (or an address) that receives the in-kernel
    failure code after the transfer."""
    p = PROTOS[proto] if isinstance(proto, str) else int(proto)
    a = make_attr(**attr)
    dev = _current_device()
    n = int(nbytes)
    s = _buf(src, n, dev, "run_noalloc: src")
    d = _buf(dst, n, dev, "run_noalloc: dst")
    st = _buf(status, 4, dev, "run_noalloc: status") if status is not None else None
    check(lib().xfer_run_noalloc(p, int(nchannels), int(nslots), int(slot_bytes), C.byref(a), s,
                                 d, n, st, _stream_handle(stream)))


# ---------------------------------------------------------------- schedule
def sched_peers(rank: int, nranks: int, i: int) -> tuple[int, int]:
    r, s = C.c_int(), C.c_int()
    check(lib().xfer_sched_peers(rank, nranks, i, C.byref(r), C.byref(s)))
    return r.value, s.value


def sched_ring_masks(rank: int, nranks: int, nchannels: int):
    import numpy as np
    rm = np.zeros(nranks, dtype=np.uint64)
    sm = np.zeros(nranks, dtype=np.uint64)
    check(lib().xfer_sched_ring_masks(rank, nranks, nchannels, rm.ctypes.data_as(_u64p),
                                      sm.ctypes.data_as(_u64p)))
    return rm, sm


def sched_plan(rank: int, nranks: int, recv_mask, send_mask, max_peers: int = 128):
    import numpy as np
    rm = np.ascontiguousarray(recv_mask, dtype=np.uint64)
    sm = np.ascontiguousarray(send_mask, dtype=np.uint64)
    n = C.c_int()
    rc = lib().xfer_sched_plan(rank, nranks, rm.ctypes.data_as(_u64p), sm.ctypes.data_as(_u64p),
                               max_peers, None, 0, C.byref(n))
    if rc not in (XFER_OK, XFER_ERR_INVALID_ARG) or n.value < 0:
        check(rc)
    if rc == XFER_ERR_INVALID_ARG and n.value == 0:
        check(rc)
    ops = (xfer_setup_op * max(n.value, 1))()
    check(lib().xfer_sched_plan(rank, nranks, rm.ctypes.data_as(_u64p), sm.ctypes.data_as(_u64p),
                                max_peers, ops, n.value, C.byref(n)))
    return [(ops[k].kind, ops[k].peer, ops[k].channel) for k in range(n.value)]


def endpoints_connect(nranks: int, recv_masks, send_masks, max_peers: int = 128, proto="zc",
                      nslots: int = 8, slot_bytes: int = 512 << 10, fifo_loc="device",
                      **attr) -> dict:
    """Connections of every directed edge the ranks' plans declare: {(s, d): Conn}."""
    import numpy as np
    rm = np.ascontiguousarray(recv_masks, dtype=np.uint64).reshape(nranks, nranks)
    sm = np.ascontiguousarray(send_masks, dtype=np.uint64).reshape(nranks, nranks)
    p = PROTOS[proto] if isinstance(proto, str) else int(proto)
    fl = FIFO_LOCS[fifo_loc] if isinstance(fifo_loc, str) else int(fifo_loc)
    a = make_attr(**attr)
    edges = (_vp * (nranks * nranks))()
    ne = C.c_int()
    check(lib().xfer_endpoints_connect(nranks, rm.ctypes.data_as(_u64p), sm.ctypes.data_as(_u64p),
                                       max_peers, p, nslots, slot_bytes, fl, C.byref(a), edges,
                                       C.byref(ne)))
    out = {}
    for s in range(nranks):
        for d in range(nranks):
            h = edges[s * nranks + d]
            if h:
                nch = bin(int(sm[s, d])).count("1")
                out[(s, d)] = Conn(p, nch, nslots, slot_bytes, fl, _handle=h)
    return out
