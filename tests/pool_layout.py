"""Test-side decoder: the library's pool image -> the oracle's plain image.

The library orders the bytes inside each page for its matrix-core loads;
``include/k8v4.h`` documents that order (the ``kv_pool`` comment).  The
oracle writes the plain order of the pages' statement (three runs for k8v4,
each ``[page][kv head][slot]``, one record per head-cell: 256 int8 codes,
2 fp32 scales, 8 conventional 18-byte Q4_0 blocks, or 256 fp16 values).
This module rearranges a library image into the plain one with numpy
reshapes written from the header's offsets, so pool images are compared
byte for byte without the oracle knowing the library's order.

Header offsets used (hc = (page*H + g)*P + slot, c = hc % 16):
  INT8 K codes    code d of hc at (hc/16)*4096 + (d/64)*1024 + c*64 + d%64
  INT8 V codes    plain rows, hc*256 + d (int8 format)
  INT8 scales     plain, (hc*2 + j)*4
  Q4_0 tile       per (page, head) tile t = hc / P of 144*P bytes: nibble
                  bytes of block b of slot s at s*128 + b*16, its fp16 scale
                  at 128*P + (s/16)*256 + b*32 + (s%16)*2
  fp16 K          element d at (hc/16)*8192 + (d/32)*1024 + ((d%32)/8)*256
                  + c*16 + (d%8)*2
  fp16 V          element d at (hc/16)*8192 + ((d%16)/2)*1024 + (c/4)*256
                  + (d/16)*16 + (d%2)*8 + (c%4)*2
``tests/test_pool_layout.py`` checks every rearrangement below against
these formulas evaluated element by element.
"""
from __future__ import annotations

import numpy as np

FMT_F16, FMT_INT8, FMT_Q4_0, FMT_K8V4 = 0, 1, 2, 3


def kcodes_to_plain(run: np.ndarray) -> np.ndarray:
    """INT8 K-code run -> [hc][256] plain rows (flat uint8)."""
    n16 = run.size // 4096
    return run.reshape(n16, 4, 16, 64).transpose(0, 2, 1, 3).reshape(-1)


def q4_to_plain(run: np.ndarray, P: int) -> np.ndarray:
    """Q4_0 tile run -> [hc][8][18] conventional blocks (flat uint8)."""
    tile = run.reshape(-1, 144 * P)
    T = tile.shape[0]
    nib = tile[:, :128 * P].reshape(T, P, 8, 16)
    sc = tile[:, 128 * P:].reshape(T, P // 16, 8, 16, 2).transpose(0, 1, 3, 2, 4).reshape(T, P, 8, 2)
    return np.concatenate([sc, nib], axis=-1).reshape(-1)


def f16k_to_plain(run: np.ndarray) -> np.ndarray:
    """fp16 K run -> [hc][256] fp16 rows (flat uint8)."""
    h = run.view(np.uint16)
    n16 = h.size // 4096
    # uint16 index: blk*4096 + (d/32)*512 + ((d%32)/8)*128 + c*8 + d%8
    return h.reshape(n16, 8, 4, 16, 8).transpose(0, 3, 1, 2, 4).reshape(-1).view(np.uint8)


def f16v_to_plain(run: np.ndarray) -> np.ndarray:
    """fp16 V run -> [hc][256] fp16 rows (flat uint8)."""
    h = run.view(np.uint16)
    n16 = h.size // 4096
    # uint16 index: blk*4096 + ((d%16)/2)*512 + (c/4)*128 + (d/16)*8 + (d%2)*4 + c%4
    # axes:         blk, A=(d%16)/2, B=c/4, C=d/16, D=d%2, E=c%4
    x = h.reshape(n16, 8, 4, 16, 2, 4)
    # plain [blk][c = 4B + E][d = 16C + 2A + D]
    return x.transpose(0, 2, 5, 3, 1, 4).reshape(-1).view(np.uint8)


def to_plain(fmt: int, runs, P: int):
    """Library runs (numpy uint8 arrays or None) -> the oracle's plain runs."""
    out = [None if r is None else np.asarray(r, np.uint8).reshape(-1) for r in runs]
    if fmt == FMT_F16:
        return [f16k_to_plain(out[0]), None, f16v_to_plain(out[2]), None]
    if fmt == FMT_Q4_0:
        return [q4_to_plain(out[0], P), None, q4_to_plain(out[2], P), None]
    if fmt == FMT_INT8:
        return [kcodes_to_plain(out[0]), out[1], out[2], out[3]]
    return [kcodes_to_plain(out[0]), out[1], q4_to_plain(out[2], P), None]


def gpu_plain_runs(gpool):
    """A device pool's runs copied to the host and rearranged to plain order."""
    runs = [None if t is None else t.cpu().numpy() for t in gpool.runs]
    return to_plain(gpool.fmt, runs, gpool.page_size)


def assert_pool_equal(gpool, opool, what: str = "") -> None:
    """Byte-for-byte equality of a device pool and an oracle pool image."""
    plain = gpu_plain_runs(gpool)
    for r in range(4):
        if opool.runs[r] is None:
            continue
        assert plain[r] is not None, f"{what} run {r} missing"
        if not np.array_equal(plain[r], opool.runs[r]):
            bad = np.flatnonzero(plain[r] != opool.runs[r])
            raise AssertionError(f"{what} run {r} differs at {bad.size} bytes, first at {bad[0]}")
