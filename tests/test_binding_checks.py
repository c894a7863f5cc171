"""CPU tests of the Python binding's argument checks: a tensor the kernels
would access outside its memory (host memory, another device, a strided
view, too few bytes) is refused before the library is called."""
import numpy as np
import pytest
import torch

import recv_fifo_plane_amd as xf
from recv_fifo_plane_amd import xfer as X


class FakeDeviceTensor:
    """Stands in for a GPU tensor on a machine without one: only the
    attributes the binding inspects."""

    def __init__(self, nbytes, device=0, contiguous=True, ptr=1 << 40):
        self._n = nbytes
        self.device = torch.device("cuda", device)
        self._contig = contiguous
        self._ptr = ptr
        self.is_cuda = True

    def data_ptr(self):
        return self._ptr

    def numel(self):
        return self._n

    def element_size(self):
        return 1

    def is_contiguous(self):
        return self._contig


class Unreachable:
    """A library stand-in that fails the test if any entry point is called."""

    def __getattr__(self, name):
        raise AssertionError("library called: " + name)


@pytest.fixture
def no_library(monkeypatch):
    monkeypatch.setattr(X, "_lib", Unreachable())
    conn = X.Conn("simple", 1, 8, 4096, _handle=0x1234)
    conn.device = 0
    yield conn
    conn._h = None  # nothing to destroy


def test_host_tensor_is_refused(no_library):
    a = torch.zeros(4096, dtype=torch.uint8)
    with pytest.raises(ValueError, match="not in GPU memory"):
        no_library.run(a, FakeDeviceTensor(4096), 4096)
    with pytest.raises(ValueError, match="not in GPU memory"):
        no_library.run(FakeDeviceTensor(4096), a, 4096)


def test_short_tensor_is_refused(no_library):
    with pytest.raises(ValueError, match="holds 4095 bytes"):
        no_library.run(FakeDeviceTensor(4096), FakeDeviceTensor(4095), 4096)
    with pytest.raises(ValueError, match="holds"):
        no_library.run_loop(FakeDeviceTensor(100), FakeDeviceTensor(4096), 4096, 3)


def test_other_device_and_strided_views_are_refused(no_library):
    with pytest.raises(ValueError, match="cuda:1"):
        no_library.run(FakeDeviceTensor(4096, device=1), FakeDeviceTensor(4096), 4096)
    with pytest.raises(ValueError, match="contiguous"):
        no_library.run(FakeDeviceTensor(4096), FakeDeviceTensor(4096, contiguous=False), 4096)


def test_message_list_extent_is_checked(no_library):
    # the last message ends at 3000 + 1200 = 4200 > 4096
    with pytest.raises(ValueError, match="touches 4200"):
        no_library.run_messages(FakeDeviceTensor(8192), FakeDeviceTensor(4096), [0, 3000],
                                [1000, 1200])
    with pytest.raises(ValueError, match="offsets"):
        no_library.run_messages(FakeDeviceTensor(8192), FakeDeviceTensor(8192), [0], [1, 2])


def test_batch_and_pingpong_are_checked(no_library):
    with pytest.raises(ValueError, match=r"dst\[1\]"):
        X.run_batch([no_library, no_library], [FakeDeviceTensor(64), FakeDeviceTensor(64)],
                    [FakeDeviceTensor(64), FakeDeviceTensor(63)], [64, 64])
    with pytest.raises(ValueError, match="run_pingpong: c"):
        X.run_pingpong(no_library, no_library, FakeDeviceTensor(64), FakeDeviceTensor(64),
                       torch.zeros(64, dtype=torch.uint8), 64, 10)


def test_noalloc_tensors_are_checked(monkeypatch):
    monkeypatch.setattr(X, "_lib", Unreachable())
    monkeypatch.setattr(X, "_current_device", lambda: 0)
    with pytest.raises(ValueError, match="not in GPU memory"):
        X.run_noalloc("simple", 1, 8, 4096, torch.zeros(64, dtype=torch.uint8),
                      FakeDeviceTensor(64), 64)
    with pytest.raises(ValueError, match="status"):
        X.run_noalloc("simple", 1, 8, 4096, FakeDeviceTensor(64), FakeDeviceTensor(64), 64,
                      status=FakeDeviceTensor(3))


def test_integer_addresses_and_empty_transfers_pass_through():
    # raw addresses are the caller's to get right; a zero-byte transfer
    # touches nothing, so any buffer passes
    assert X._buf(12345, 1 << 30, 0, "x") == 12345
    assert X._buf(None, 0, 0, "x") == 0
    assert X._buf(torch.zeros(1, dtype=torch.uint8), 0, 0, "x") != 0
    with pytest.raises(TypeError):
        X._buf(np.zeros(4, np.uint8), 4, 0, "x")
