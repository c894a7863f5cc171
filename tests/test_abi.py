"""CPU tests of the C ABI: the library loads, exports every symbol the
header declares, rejects bad arguments before touching a GPU, and its host
schedule agrees op-for-op with the oracle's (no GPU compute is called)."""
import os
import re

import numpy as np
import pytest

import oracle
import recv_fifo_plane_amd as xf
from recv_fifo_plane_amd import xfer as X

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "xfer.h")


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(xfer_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for must in ("xfer_conn_create", "xfer_run", "xfer_sched_peers", "xfer_sched_plan",
                 "xfer_sched_ring_masks", "xfer_conn_destroy", "xfer_run_batch"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = xf.lib()
    names = _declared()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(X.SIGNATURES) == names


@pytest.mark.parametrize("args", [
    (4, 1, 8, 128, 0),          # unknown protocol
    (-1, 1, 8, 128, 0),         # unknown protocol
    (0, 0, 8, 128, 0),          # no channels
    (0, 65, 8, 128, 0),         # too many channels (64-bit masks)
    (0, 1, 0, 128, 0),          # no slots
    (0, 1, 8, 24, 0),           # SIMPLE slot not a multiple of 16
    (1, 1, 8, 12, 0),           # LL slot not a multiple of 8
    (2, 1, 8, 8, 0),            # zero-copy step not a multiple of 16
    (3, 1, 8, 8, 0),            # zero-copy direct step not a multiple of 16
    (0, 1, 8, 128, 3),          # unknown FIFO location
    (1, 1, 8, 128, 2),          # the relay carries SIMPLE only
    (2, 1, 8, 128, 2),
])
def test_create_rejects_bad_arguments(args):
    with pytest.raises(xf.XferError) as e:
        xf.Conn(*args)
    assert e.value.status == X.XFER_ERR_INVALID_ARG
    assert xf.last_error()


def test_relay_needs_host_control_words():
    with pytest.raises(xf.XferError) as e:
        xf.Conn("simple", 1, 8, 128, "relay", ctrl_loc=X.XFER_CTRL_DEVICE)
    assert e.value.status == X.XFER_ERR_INVALID_ARG
    assert "host memory" in xf.last_error()


@pytest.mark.parametrize("proto,fifo_loc,attr", [
    ("simple", "device", dict(p2p_read=2)),
    ("simple", "device", dict(p2p_read=-1)),
    ("ll", "device", dict(p2p_read=1)),
    ("zc", "device", dict(p2p_read=1)),
    ("zcd", "device", dict(p2p_read=1)),
    ("simple", "host", dict(p2p_read=1)),
    ("simple", "relay", dict(p2p_read=1)),
    ("simple", "device", dict(p2p_read=1, ctrl_loc=X.XFER_CTRL_HOST)),
])
def test_p2p_read_is_simple_in_hbm_only(proto, fifo_loc, attr):
    # P2P read moves the SIMPLE buffer to the send side; the pages give it no
    # meaning for LL, zero-copy or host-memory FIFOs
    with pytest.raises(xf.XferError) as e:
        xf.Conn(proto, 1, 8, 128, fifo_loc, **attr)
    assert e.value.status == X.XFER_ERR_INVALID_ARG


@pytest.mark.parametrize("proto,fifo_loc,attr", [
    ("ll", "device", dict(place_trials=-1)),
    ("ll", "device", dict(place_trials=9)),
    ("zc", "device", dict(place_trials=2)),
    ("zcd", "device", dict(place_trials=4)),
    ("simple", "host", dict(place_trials=2)),
    ("ll", "host", dict(place_trials=2)),
    ("simple", "relay", dict(place_trials=2)),
    ("ll", "device", dict(place_trials=2, ctrl_loc=X.XFER_CTRL_HOST)),
    ("simple", "device", dict(place_trials=2, p2p_read=1)),
])
def test_place_trials_needs_a_polled_fifo_in_hbm(proto, fifo_loc, attr):
    # placement by measured latency times a ping-pong through the FIFO and
    # counters in HBM; zero-copy has no FIFO, host memory is not placed
    with pytest.raises(xf.XferError) as e:
        xf.Conn(proto, 1, 8, 128, fifo_loc, **attr)
    assert e.value.status == X.XFER_ERR_INVALID_ARG
    assert "place_trials" in xf.last_error()


def test_attribute_struct_matches_the_header():
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "xfer.h")).read()
    body = hdr[hdr.index("typedef struct {", hdr.index("Optional creation attributes")):
               hdr.index("} xfer_attr;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(?:int|uint32_t)\s+(\w+);", body)
    assert fields == [f[0] for f in X.xfer_attr._fields_]
    with pytest.raises(TypeError):
        X.make_attr(no_such_field=1)
    a = X.make_attr(place_trials=3, p2p_read=1)
    assert (a.place_trials, a.p2p_read, a.wgs_per_channel) == (3, 1, 0)


@pytest.mark.parametrize("attr", [dict(wgs_per_channel=17), dict(block_threads=96),
                                  dict(block_threads=2048), dict(ctrl_loc=3), dict(roles=3),
                                  dict(xcd_pairing=2), dict(cooperative=2),
                                  dict(cooperative=-1)])
def test_create_rejects_bad_attributes(attr):
    with pytest.raises(xf.XferError) as e:
        xf.Conn("simple", 1, 8, 128, **attr)
    assert e.value.status == X.XFER_ERR_INVALID_ARG


def test_run_rejects_null_connection():
    rc = xf.lib().xfer_run(None, 16, 32, 16, None)
    assert rc == X.XFER_ERR_INVALID_ARG


def test_status_strings():
    for code, name in [(0, "XFER_OK"), (5, "XFER_ERR_TIMEOUT"), (8, "XFER_ERR_STATE"),
                       (99, "XFER_ERR_UNKNOWN")]:
        assert xf.status_string(code) == name


@pytest.mark.parametrize("n", list(range(1, 40)) + [64, 100, 257])
def test_schedule_peers_and_ring_masks_match_oracle(n):
    for r in range(n):
        for i in range(0, n + 2):
            assert xf.sched_peers(r, n, i) == oracle.peers(r, n, i)
        for nch in (1, 4, 64):
            rm, sm = xf.sched_ring_masks(r, n, nch)
            orm, osm = oracle.ring_masks(r, n, nch)
            assert np.array_equal(rm, orm) and np.array_equal(sm, osm)


def test_schedule_plan_matches_oracle_op_for_op():
    rng = np.random.default_rng(11)
    for n in list(range(1, 20)) + [128, 129, 200, 300]:
        for mp in (1, 2, 7, 128):
            r = int(rng.integers(0, n))
            if rng.random() < 0.5:
                rm, sm = oracle.ring_masks(r, n, int(rng.integers(1, 65)))
            else:
                rm = rng.integers(0, 2**63, size=n, dtype=np.int64).astype(np.uint64)
                sm = rng.integers(0, 2**63, size=n, dtype=np.int64).astype(np.uint64)
                rm &= np.uint64(0x00FF00000000F0F1)
                sm &= np.uint64(0x8000000000000F0F)
            assert xf.sched_plan(r, n, rm, sm, mp) == oracle.plan(r, n, rm, sm, mp)


def test_schedule_rejects_bad_arguments():
    z = np.zeros(4, dtype=np.uint64)
    with pytest.raises(xf.XferError):
        xf.sched_plan(0, 4, z, z, 0)
    with pytest.raises(xf.XferError):
        xf.sched_peers(5, 4, 1)
    with pytest.raises(xf.XferError):
        xf.sched_ring_masks(0, 4, 65)


def test_set_trace_rejects_a_null_connection():
    from recv_fifo_plane_amd import xfer as X
    assert X.lib().xfer_conn_set_trace(None, None, 0) == X.XFER_ERR_INVALID_ARG


def test_set_jitter_rejects_a_null_connection():
    from recv_fifo_plane_amd import xfer as X
    assert X.lib().xfer_conn_set_jitter(None, 1) == X.XFER_ERR_INVALID_ARG


def test_library_loads_where_torch_brought_the_hip_runtime():
    # torch ships its own HIP runtime under the same soname; imported first,
    # it is the runtime libxfer.so binds to, so the library must not need a
    # symbol (or symbol version) newer than that runtime has
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import torch\n"
            "import recv_fifo_plane_amd as xf\n"
            "xf.lib()\n"
            "print('loaded')\n" % root)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "loaded" in r.stdout, r.stderr[-2000:]


@pytest.mark.parametrize("args,attr", [
    ((4, 1, 8, 4096), {}),                                  # unknown protocol
    ((0, 0, 8, 4096), {}),                                  # no channels
    ((0, 1, 8, 24), {}),                                    # SIMPLE slot not a multiple of 16
    ((0, 2, 8, (15 << 20) // 8), {}),                       # FIFO twice the array's room
    ((0, 1, 8, 4096), dict(roles=1)),                       # both sides always run
    ((0, 1, 8, 4096), dict(p2p_read=1)),
    ((0, 1, 8, 4096), dict(ctrl_loc=X.XFER_CTRL_HOST)),
    ((1, 1, 8, 4096), dict(place_trials=2)),
    ((0, 1, 8, 4096), dict(wgs_per_channel=17)),
    ((0, 1, 8, 4096), dict(cooperative=1)),                 # no cooperative grids
])
def test_noalloc_rejects_bad_arguments_before_touching_a_gpu(args, attr):
    a = X.make_attr(**attr)
    rc = xf.lib().xfer_run_noalloc(*args, C_byref(a), 1 << 20, 1 << 21, 4096, None, None)
    assert rc == X.XFER_ERR_INVALID_ARG, (args, attr, xf.last_error())
    assert "xfer_run_noalloc" in xf.last_error()


def C_byref(x):
    import ctypes
    return ctypes.byref(x)
