"""Seeded synthetic inputs for the FIFO send/recv data plane.

Both the CPU oracle's tests and the GPU path's tests and benchmark draw their
inputs from here, so the two sides always see the same bytes.  This module
holds none of the protocol's arithmetic: it only produces payloads and
message-size lists.  Every payload is drawn from numpy PCG64 streams in blocks of 2**24 values,
block b from ``numpy.random.default_rng([seed, b])``; message-size lists
come from ``numpy.random.default_rng(seed)``.  The workload seeds are
1000 + the workload number.
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 1000


def workload_seed(k: int) -> int:
    """Seed of workload ``k`` (1-based)."""
    return SEED_BASE + int(k)


BLOCK = 1 << 24


def _blocked(n: int, dtype, seed: int, draw) -> np.ndarray:
    """n values of dtype; block b (BLOCK values) comes from default_rng([seed, b]),
    so large inputs are generated on several threads with a fixed result."""
    out = np.empty(int(n), dtype=dtype)
    nblocks = (int(n) + BLOCK - 1) // BLOCK

    def fill(b: int) -> None:
        s = b * BLOCK
        e = min(int(n), s + BLOCK)
        out[s:e] = draw(np.random.default_rng([seed, b]), e - s)

    if nblocks > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(8, nblocks)) as ex:
            list(ex.map(fill, range(nblocks)))
    elif nblocks:
        fill(0)
    return out


def uint8_uniform(nbytes: int, seed: int) -> np.ndarray:
    """``nbytes`` uniform random bytes."""
    return _blocked(nbytes, np.uint8, seed,
                    lambda g, m: g.integers(0, 256, size=m, dtype=np.uint8))


def int32_uniform_bytes(nbytes: int, seed: int) -> np.ndarray:
    """Full-range uniform int32 payload, returned as ``nbytes`` raw bytes.

    The message may end in a partial word: the words are drawn for
    ceil(nbytes/4) and the byte view is cut to ``nbytes``.
    """
    nwords = (int(nbytes) + 3) // 4
    w = _blocked(nwords, np.int32, seed,
                 lambda g, m: g.integers(-(2**31), 2**31, size=m, dtype=np.int64).astype(np.int32))
    return w.view(np.uint8)[: int(nbytes)].copy()


def _bf16_rne(g, m: int) -> np.ndarray:
    u = g.standard_normal(m, dtype=np.float32).view(np.uint32)
    # finite fp32 bit patterns stay below 2**32 after adding at most 0x8000
    lsb = (u >> 16) & 1
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= 16
    return u


def bf16_normal_bytes(nbytes: int, seed: int) -> np.ndarray:
    """bf16 bit patterns of N(0,1) samples, as ``nbytes`` raw bytes.

    fp32 normals are rounded to bf16 with round-to-nearest-even on the upper
    16 bits (the samples are finite, so no NaN handling is needed).  Only the
    bits matter to a byte copy; the payload type is opaque to the protocol.
    """
    nbytes = int(nbytes)
    out = _blocked((nbytes + 1) // 2, np.uint16, seed, _bf16_rne)
    return out.view(np.uint8)[:nbytes].copy()


def fp32_uniform_bytes(nbytes: int, seed: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """fp32 uniform[lo, hi) samples as ``nbytes`` raw bytes (nbytes % 4 == 0)."""
    nbytes = int(nbytes)
    if nbytes % 4:
        raise ValueError("fp32 payload must be a whole number of words")
    f = _blocked(nbytes // 4, np.float32, seed,
                 lambda g, m: g.uniform(lo, hi, size=m).astype(np.float32))
    return f.view(np.uint8)


def log_uniform_message_sizes(total: int, seed: int, lo_exp: float = 10.0,
                              hi_exp: float = 26.0, min_bytes: int = 1024) -> list[int]:
    """Message sizes floor(2**U(lo_exp, hi_exp)) drawn until they reach ``total``.

    The last draw is cut so the sizes sum to exactly ``total``; if that cut
    leaves less than ``min_bytes`` it is merged into the message before it.
    """
    rng = np.random.default_rng(seed)
    sizes: list[int] = []
    acc = 0
    while acc < total:
        s = int(np.floor(2.0 ** rng.uniform(lo_exp, hi_exp)))
        s = max(1, min(s, total - acc))
        sizes.append(s)
        acc += s
    if len(sizes) > 1 and sizes[-1] < min_bytes:
        last = sizes.pop()
        sizes[-1] += last
    assert sum(sizes) == total
    return sizes


def guard_pattern(nbytes: int, seed: int = 7) -> np.ndarray:
    """Bytes that fill destination buffers (and the guard zones around them)
    before a transfer, so an untouched byte is distinguishable from a copied one."""
    return np.random.default_rng(seed ^ 0x5A5A).integers(0, 256, size=int(nbytes), dtype=np.uint8)
