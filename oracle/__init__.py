"""CPU oracle for the k8v4 KV cache and its attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path
(``long_context_decode_append_amd``) never imports it, and this package never
imports the product: they share no code.

Everything arithmetic lives in ``k8v4_oracle.c`` (plain C, fp32 quantizers
rounded as written, fp64 attention by definition); this module only marshals
numpy arrays through ctypes.  Formats: 0 = fp16 K/V (unquantized), 1 = int8
K/V, 2 = q4_0 K/V (both rotated), 3 = k8v4 (INT8 K + rotated Q4_0 V),
following the pages
"#120 --kv k8v4: hybrid KV cache" (What, How, Tests) and
"kv: --kv k8v4 streams with --kv-resident" (How).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liborc_k8v4.so")
_lib = None

D = 256          # head_dim
KGROUP = 128     # INT8 scale group
QBLK = 32        # Q4_0 block length
QBYTES = 18      # Q4_0 block bytes
FMT_F16, FMT_INT8, FMT_Q4_0, FMT_K8V4 = 0, 1, 2, 3


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # rebuilt whenever the C source is newer than the library, so an edit to
    # the oracle can never be tested against a stale build
    if (not os.path.exists(_LIB_PATH)
            or os.path.getmtime(_LIB_PATH) < os.path.getmtime(os.path.join(_HERE, "k8v4_oracle.c"))):
        from . import build as _b
        _b.build()
    lib = C.CDLL(_LIB_PATH)
    P = C.c_void_p
    i, l, d = C.c_int, C.c_long, C.c_double
    lib.orc_f32_to_f16.argtypes = [C.c_float]
    lib.orc_f32_to_f16.restype = C.c_uint16
    lib.orc_f16_to_f32.argtypes = [C.c_uint16]
    lib.orc_f16_to_f32.restype = C.c_float
    for name, args in {
        "orc_f32_to_f16_array": [P, P, l],
        "orc_f16_to_f32_array": [P, P, l],
        "orc_fwht256_rows": [P, l],
        "orc_quant_int8_groups": [P, l, P, P],
        "orc_quant_q4_blocks": [P, l, P],
        "orc_dequant_int8": [P, P, l, P],
        "orc_dequant_q4": [P, l, P],
        "orc_hadamard_apply_f64": [P, P],
    }.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    lib.orc_cell_bytes.argtypes = [i, i, i]
    lib.orc_cell_bytes.restype = l
    lib.orc_append.argtypes = [i, i, i, i, P, P, P, P, P, i, P, P, i, i, i]
    lib.orc_append.restype = i
    lib.orc_gather.argtypes = [i, i, i, i, P, P, P, P, P, i, i, i, P, P, P, P]
    lib.orc_gather.restype = i
    lib.orc_attention.argtypes = [P, P, i, i, P, i, i, i, P, d, i, i, P]
    lib.orc_attention.restype = i
    lib.orc_attention_threads.argtypes = [P, P, i, i, P, i, i, i, P, d, i, i, P, i]
    lib.orc_attention_threads.restype = i
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- elementary rules

def f32_to_f16_bits(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().orc_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().orc_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


def fwht256(y) -> np.ndarray:
    """Rotate each 256-row by H/16 (fp32 butterflies, ascending strides)."""
    y = _c(y, np.float32).copy()
    assert y.shape[-1] == D
    _load().orc_fwht256_rows(_ptr(y), y.size // D)
    return y


def quant_int8(x):
    """INT8 rule per 128-group: returns (codes int8 like x, scales [..., n/128] fp32)."""
    x = _c(x, np.float32)
    assert x.shape[-1] % KGROUP == 0
    ng = x.size // KGROUP
    codes = np.empty(x.shape, np.int8)
    d = np.empty(x.shape[:-1] + (x.shape[-1] // KGROUP,), np.float32)
    _load().orc_quant_int8_groups(_ptr(x), ng, _ptr(codes), _ptr(d))
    return codes, d


def quant_q4(y):
    """Q4_0 rule per 32-block: returns canonical blocks [..., n/32, 18] uint8."""
    y = _c(y, np.float32)
    assert y.shape[-1] % QBLK == 0
    nb = y.size // QBLK
    out = np.empty(y.shape[:-1] + (y.shape[-1] // QBLK, QBYTES), np.uint8)
    _load().orc_quant_q4_blocks(_ptr(y), nb, _ptr(out))
    return out


def dequant_int8(codes, scales) -> np.ndarray:
    codes = _c(codes, np.int8)
    scales = _c(scales, np.float32)
    n = codes.size // D
    out = np.empty(codes.shape, np.float64)
    _load().orc_dequant_int8(_ptr(codes), _ptr(scales), n, _ptr(out))
    return out


def dequant_q4(blocks) -> np.ndarray:
    blocks = _c(blocks, np.uint8)
    n = blocks.size // ((D // QBLK) * QBYTES)
    out = np.empty(blocks.shape[:-2] + (D,), np.float64)
    _load().orc_dequant_q4(_ptr(blocks), n, _ptr(out))
    return out


def hadamard16(x) -> np.ndarray:
    """(1/16) H x in fp64 by the explicit matrix, row by row."""
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib = _load()
    for r in range(x.size // D):
        xi = x.reshape(-1, D)[r]
        oi = out.reshape(-1, D)[r]
        lib.orc_hadamard_apply_f64(_ptr(xi), _ptr(oi))
    return out


def cell_bytes(fmt: int, n_kv_heads: int, head_dim: int = D) -> int:
    return int(_load().orc_cell_bytes(fmt, n_kv_heads, head_dim))


# ---------------------------------------------------------------- pool image

class OraclePool:
    """Byte image of a paged pool in the plain order: every run is indexed
    [page][kv head][slot], one record per head-cell
    hc = (page*H + head)*P + slot (the pages fix the three runs of a k8v4
    block and the bytes per cell, not the order inside a page):

    INT8 codes   256 int8 at hc*256          INT8 scales  2 fp32 at hc*8
    Q4_0 blocks  8 x 18 bytes at hc*144      fp16 values  256 fp16 at hc*512

    run 0: K codes (k8v4, int8), K blocks (q4_0) or K values (fp16)
    run 1: K scales (k8v4, int8)
    run 2: V blocks (k8v4, q4_0), V codes (int8) or V values (fp16)
    run 3: V scales (int8)
    """

    def __init__(self, fmt: int, n_pages: int, page_size: int, n_kv_heads: int,
                 sentinel: int = 0xA5):
        self.fmt, self.n_pages, self.P, self.H = fmt, n_pages, page_size, n_kv_heads
        cells = n_pages * page_size * n_kv_heads
        int8_codes = cells * D
        int8_scales = cells * (D // KGROUP) * 4
        q4 = cells * 144
        sizes = {
            FMT_K8V4: [int8_codes, int8_scales, q4, 0],
            FMT_INT8: [int8_codes, int8_scales, int8_codes, int8_scales],
            FMT_Q4_0: [q4, 0, q4, 0],
            FMT_F16: [cells * D * 2, 0, cells * D * 2, 0],
        }[fmt]
        self.runs = [np.full(s, sentinel, np.uint8) if s else None for s in sizes]

    def append(self, page_table, k, v, pos0: int) -> None:
        """k, v: [n][H][256] float16 or float32 numpy arrays."""
        assert k.shape == v.shape and k.shape[1:] == (self.H, D)
        if k.dtype == np.float16:
            dtype, kb, vb = 0, _c(k, np.float16).view(np.uint16), _c(v, np.float16).view(np.uint16)
        else:
            dtype, kb, vb = 1, _c(k, np.float32), _c(v, np.float32)
        pt = _c(page_table, np.int32)
        rc = _load().orc_append(self.fmt, self.n_pages, self.P, self.H, *[_ptr(r) for r in self.runs],
                                _ptr(pt), pt.size, _ptr(kb), _ptr(vb), dtype, pos0, k.shape[0])
        if rc != 0:
            raise ValueError("oracle append: bad arguments")

    def gather(self, page_table, pos0: int, n: int):
        """Canonical bytes of cells [pos0, pos0+n) in logical order.

        k8v4 -> (k_codes [n][H][256] int8, k_scales [n][H][2] f32, v_blocks [n][H][8][18] u8)
        int8 -> (k_codes, k_scales, v_codes, v_scales)
        q4_0 -> (k_blocks, v_blocks)
        fp16 -> (k [n][H][256] float16, v [n][H][256] float16)
        """
        H = self.H
        codes = lambda: np.empty((n, H, D), np.int8)
        scales = lambda: np.empty((n, H, D // KGROUP), np.float32)
        blocks = lambda: np.empty((n, H, D // QBLK, QBYTES), np.uint8)
        if self.fmt == FMT_K8V4:
            outs = [codes(), scales(), blocks(), None]
        elif self.fmt == FMT_INT8:
            outs = [codes(), scales(), codes(), scales()]
        elif self.fmt == FMT_F16:
            outs = [np.empty((n, H, D), np.float16), None, np.empty((n, H, D), np.float16), None]
        else:
            outs = [blocks(), None, blocks(), None]
        pt = _c(page_table, np.int32)
        rc = _load().orc_gather(self.fmt, self.n_pages, self.P, self.H, *[_ptr(r) for r in self.runs],
                                _ptr(pt), pt.size, pos0, n, *[_ptr(o) for o in outs])
        if rc != 0:
            raise ValueError("oracle gather: bad arguments")
        return tuple(o for o in outs if o is not None)


def dequant_gathered(fmt: int, gathered):
    """fp64 K (in q's basis, or rotated for q4_0) and V (rotated unless int8)."""
    if fmt == FMT_K8V4:
        kc, ks, vb = gathered
        return dequant_int8(kc, ks), dequant_q4(vb)
    if fmt == FMT_INT8:
        kc, ks, vc, vs = gathered
        return dequant_int8(kc, ks), dequant_int8(vc, vs)
    if fmt == FMT_F16:
        kh, vh = gathered
        return kh.astype(np.float64), vh.astype(np.float64)
    kb, vb = gathered
    return dequant_q4(kb), dequant_q4(vb)


def default_threads() -> int:
    """Threads the oracle's attention uses by default: the host's cores
    (at most 16)."""
    return max(1, min(16, os.cpu_count() or 1))


def attention(kd, vd, q, n_visible, scale: float | None = None, *, q_rotate: bool = False,
              v_rotated: bool = True, threads: int | None = None) -> np.ndarray:
    """fp64 attention by definition.

    kd, vd: [n_cells][H][256] fp64.  q: [rows][Hq][256] fp16 or fp32.
    n_visible: [rows] leading cells each row attends to.  Returns [rows][Hq][256] fp64.
    threads: the (row, head) pairs are spread over this many threads
    (default: default_threads()); the result does not depend on it.
    """
    kd = _c(kd, np.float64)
    vd = _c(vd, np.float64)
    n_cells, H = kd.shape[0], kd.shape[1]
    rows, Hq = q.shape[0], q.shape[1]
    if q.dtype == np.float16:
        qd, qb = 0, _c(q, np.float16).view(np.uint16)
    else:
        qd, qb = 1, _c(q, np.float32)
    nv = _c(n_visible, np.int32)
    assert nv.size == rows
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((rows, Hq, D), np.float64)
    nt = default_threads() if threads is None else int(threads)
    rc = _load().orc_attention_threads(_ptr(kd), _ptr(vd), n_cells, H, _ptr(qb), qd, rows, Hq, _ptr(nv),
                                       float(scale), int(q_rotate), int(v_rotated), _ptr(out), nt)
    if rc != 0:
        raise ValueError("oracle attention: bad arguments")
    return out


def attention_from_pool(pool: OraclePool, page_table, q, n_visible, scale: float | None = None,
                        threads: int | None = None):
    """Gather the visible prefix, dequantize, attend (format rules of pool.fmt)."""
    n = int(np.max(n_visible))
    g = pool.gather(page_table, 0, n)
    kd, vd = dequant_gathered(pool.fmt, g)
    return attention(kd, vd, q, n_visible, scale, q_rotate=(pool.fmt == FMT_Q4_0),
                     v_rotated=(pool.fmt not in (FMT_INT8, FMT_F16)), threads=threads)
