"""MI355X (gfx950) FIFO send/recv data plane.

A connection moves a device buffer A into a device buffer B through a ring of
FIFO slots per channel (SIMPLE copy, LL 8-byte flagged lines, or zero-copy
through a ptrExchange word), with both endpoints running as concurrent
workgroup sets in one kernel launch.  The compute path is libxfer.so (HIP
kernels + C++ runtime, C ABI in include/xfer.h); this package only binds it.
"""
from .xfer import (  # noqa: F401
    Conn,
    XferError,
    endpoints_connect,
    last_error,
    lib,
    run_batch,
    run_pingpong,
    sched_peers,
    sched_plan,
    sched_ring_masks,
    status_string,
)
from . import xfer  # noqa: F401
