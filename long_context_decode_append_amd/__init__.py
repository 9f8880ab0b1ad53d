"""MI355X-native k8v4 KV cache and fused long-context attention.

Thin Python binding over ``lib/libk8v4.so`` (the C ABI of
``include/k8v4.h``).  This module only marshals arguments: torch tensors
provide device memory and the current HIP stream, every step of the path
runs in the library's HIP kernels.  There is no CPU fallback: when the
library is missing every call raises.

The format and operations follow the pages "#120 --kv k8v4: hybrid KV cache
-- INT8 K + Hadamard-rotated Q4_0 V (816 B/cell)" (What, How, Tests) and
"kv: --kv k8v4 streams with --kv-resident" (How).
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libk8v4.so")

KV_FMT_F16, KV_FMT_INT8, KV_FMT_Q4_0, KV_FMT_K8V4 = 0, 1, 2, 3
KV_DTYPE_F16, KV_DTYPE_F32 = 0, 1
HEAD_DIM = 256
GQA = 8


class KvPoolStruct(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("n_pages", C.c_int32), ("page_size", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("reserved", C.c_int32),
                ("run", C.c_void_p * 4)]


class KvSeqStruct(C.Structure):
    _fields_ = [("page_table", C.c_void_p), ("n_table", C.c_int32), ("reserved", C.c_int32)]


class KvStreamStruct(C.Structure):
    _fields_ = [("window", KvPoolStruct), ("mirror", KvPoolStruct), ("mirror_table", C.c_void_p),
                ("window_map", C.c_void_p), ("window_owner", C.c_void_p), ("stats", C.c_void_p),
                ("fetch_list", C.c_void_p), ("n_table", C.c_int32), ("reserved", C.c_int32)]


# name -> (restype, argtypes); the exported symbols of include/k8v4.h
_P, _I, _SZ, _F = C.c_void_p, C.c_int, C.c_size_t, C.c_float
_PP, _PS = C.POINTER(KvPoolStruct), C.POINTER(KvSeqStruct)
_PST = C.POINTER(KvStreamStruct)
SIGNATURES = {
    "kv_cell_bytes": (_SZ, [_I, _I, _I]),
    "kv_run_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "kv_append_k8v4": (_I, [_PP, _PS, _P, _P, _I, C.c_int32, C.c_int32, _P]),
    "kv_gather": (_I, [_PP, _PS, C.c_int32, C.c_int32, _P, _P, _P, _P]),
    "attn_workspace_bytes": (_SZ, [_PP, _I, C.c_int32, C.c_int32]),
    "kv_workspace_init": (_I, [_P, _SZ, _P]),
    "kv_probe_read": (_I, [_P, _SZ, _P, _P]),
    "kv_copy_pages": (_I, [_PP, _PP, _P, _P, C.c_int32, _P]),
    "kv_append": (_I, [_PP, _PS, _P, _P, _I, C.c_int32, C.c_int32, _P]),
    "kv_gather_runs": (_I, [_PP, _PS, C.c_int32, C.c_int32, _P, _P, _P, _P, _P]),
    "attn_decode": (_I, [_PP, _PS, _P, _I, _I, C.c_int32, _F, _P, _P, _SZ, _P]),
    "attn_decode_noalloc": (_I, [_PP, _PS, _P, _I, _I, C.c_int32, _F, _P, _P]),
    "attn_decode_append": (_I, [_PP, _PS, _P, _P, _I, _P, _I, _I, C.c_int32, _F, _P, _P, _SZ, _P]),
    "attn_decode_batch": (_I, [_PP, _PS, C.c_int32, _P, _I, _I, _P, _F, _P, _P, _SZ, _P]),
    "attn_verify": (_I, [_PP, _PS, _P, _I, _I, C.c_int32, _P, _F, _P, _P, _SZ, _P]),
    "attn_prefill_chunk": (_I, [_PP, _PS, _P, _I, _I, C.c_int32, C.c_int32, _F, _P, _P, _SZ, _P]),
    "attn_prefill_workspace_bytes": (_SZ, [_PP, C.c_int32]),
    "kv_check_page_table": (_I, [_PP, _PS, C.c_int32, _P]),
    "kv_stream_append": (_I, [_PST, _P, _P, _I, C.c_int32, C.c_int32, _P]),
    "kv_stream_fetch": (_I, [_PST, C.c_int32, C.c_int32, _P]),
    "attn_decode_stream": (_I, [_PST, _P, _I, _I, C.c_int32, _F, _P, _P, _SZ, _P]),
    "attn_verify_stream": (_I, [_PST, _P, _I, _I, C.c_int32, _P, _F, _P, _P, _SZ, _P]),
    "kv_strerror": (C.c_char_p, [_I]),
    "kv_last_hip_error": (C.c_char_p, []),
    "kv_time_next_launch": (_I, [_P, _P]),
}

_lib = None


class KvError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        detail = ""
        if code == -8:
            detail = f" [{lib().kv_last_hip_error().decode()}]"
        super().__init__(f"{what}: {strerror(code)} ({code}){detail}")


def lib():
    """Load libk8v4.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime (same soname as the system one):
        # loading torch first makes libk8v4 bind to that runtime, so streams
        # and device pointers from torch are valid in the library.
        _torch()
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback path)")
        handle = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def strerror(code: int) -> str:
    return lib().kv_strerror(code).decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise KvError(rc, what)


def _torch():
    import torch
    return torch


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dev_ptr(t, name: str, dtypes=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return C.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return KV_DTYPE_F16
    if t.dtype == torch.float32:
        return KV_DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def cell_bytes(fmt: int = KV_FMT_K8V4, n_kv_heads: int = 2, head_dim: int = HEAD_DIM) -> int:
    return int(lib().kv_cell_bytes(fmt, n_kv_heads, head_dim))


class KvPool:
    """A paged pool of format fmt (KV_FMT_F16, KV_FMT_INT8, KV_FMT_Q4_0 or KV_FMT_K8V4):
    its runs as the header lays them out, in device memory, or with
    host=True in pinned host memory (the host side of a streamed cache, for
    kv_copy_pages only)."""

    def __init__(self, fmt: int, n_pages: int, page_size: int, n_kv_heads: int = 2, device="cuda",
                 fill: int | None = None, host: bool = False):
        torch = _torch()
        L = lib()
        self.n_pages, self.page_size, self.n_kv_heads = n_pages, page_size, n_kv_heads
        self.fmt = int(fmt)
        self.runs = []
        for r in range(4):
            nb = int(L.kv_run_bytes(self.fmt, r, n_pages, page_size, n_kv_heads, HEAD_DIM))
            if nb == 0:
                self.runs.append(None)
                continue
            if host:
                t = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
            else:
                t = torch.empty(nb, dtype=torch.uint8, device=device)
            if fill is not None:
                t.fill_(fill)
            self.runs.append(t)
        self._struct = KvPoolStruct(self.fmt, n_pages, page_size, n_kv_heads, HEAD_DIM, 0,
                                    (C.c_void_p * 4)(*[None if t is None else t.data_ptr()
                                                       for t in self.runs]))

    @property
    def struct(self) -> KvPoolStruct:
        return self._struct

    @property
    def nbytes(self) -> int:
        return sum(t.numel() for t in self.runs if t is not None)


class K8V4Pool(KvPool):
    """A k8v4 paged pool: three runs (K codes, K scales, V q4_0)."""

    def __init__(self, n_pages: int, page_size: int, n_kv_heads: int = 2, device="cuda",
                 fill: int | None = None):
        super().__init__(KV_FMT_K8V4, n_pages, page_size, n_kv_heads, device, fill)


class KvStream:
    """A streamed cache: the whole context in a pinned host mirror and a
    device window of fewer pages (include/k8v4.h, kv_stream).  mirror_table:
    int32 device tensor, logical page -> mirror page.  The window map and
    owner list start empty (-1); kv_stream_fetch places pages.  stats holds
    [lookups, misses] of the streamed attention calls."""

    def __init__(self, fmt: int, n_window: int, n_mirror: int, page_size: int, mirror_table,
                 n_kv_heads: int = 2, device="cuda", fill: int | None = None):
        torch = _torch()
        self.window = KvPool(fmt, n_window, page_size, n_kv_heads, device=device, fill=fill)
        self.mirror = KvPool(fmt, n_mirror, page_size, n_kv_heads, fill=fill, host=True)
        if mirror_table.dtype != torch.int32 or not mirror_table.is_cuda:
            raise ValueError("mirror_table must be an int32 device tensor")
        self.mirror_table = mirror_table
        n_table = int(mirror_table.numel())
        self.window_map = torch.full((n_table,), -1, dtype=torch.int32, device=device)
        self.window_owner = torch.full((n_window,), -1, dtype=torch.int32, device=device)
        self.stats = torch.zeros(2, dtype=torch.int32, device=device)
        self.fetch_list = torch.empty(2 * n_window, dtype=torch.int32, device=device)
        self.n_table = n_table
        self._struct = KvStreamStruct(self.window.struct, self.mirror.struct, mirror_table.data_ptr(),
                                      self.window_map.data_ptr(), self.window_owner.data_ptr(),
                                      self.stats.data_ptr(), self.fetch_list.data_ptr(), n_table, 0)

    @property
    def struct(self) -> KvStreamStruct:
        return self._struct


def kv_stream_append(s: KvStream, k, v, pos0: int, stream=None) -> None:
    """Quantize k, v ([n][H][256]) once and write cells [pos0, pos0+n) to the
    mirror, and to the window where their pages are resident."""
    if k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    _check(lib().kv_stream_append(C.byref(s.struct), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(k),
                                  int(pos0), int(k.shape[0]), _stream(stream)), "kv_stream_append")


def kv_stream_fetch(s: KvStream, first_page: int, n_pages: int, stream=None) -> None:
    """Make logical pages [first_page, first_page + n_pages) resident (ring
    placement, the last ones first when they do not all fit)."""
    _check(lib().kv_stream_fetch(C.byref(s.struct), int(first_page), int(n_pages), _stream(stream)),
           "kv_stream_fetch")


def attn_decode_stream(s: KvStream, q, n_ctx: int, ws, scale: float = 0.0, out=None, stream=None):
    """attn_decode over a streamed cache (window where resident, mirror otherwise)."""
    torch = _torch()
    if q.dim() != 2 or q.shape[1] != HEAD_DIM:
        raise ValueError("q must be [n_q_heads][256]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check(lib().attn_decode_stream(C.byref(s.struct), _dev_ptr(q, "q"), _dtype_code(q), int(q.shape[0]),
                                    int(n_ctx), float(scale), _dev_ptr(out, "out", (torch.float32,)),
                                    _dev_ptr(ws, "ws"), ws.numel(), _stream(stream)), "attn_decode_stream")
    return out


def attn_verify_stream(s: KvStream, q, n_visible, ws, scale: float = 0.0, out=None, stream=None):
    """attn_verify over a streamed cache."""
    torch = _torch()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [n_q][n_q_heads][256]")
    n_q = int(q.shape[0])
    if len(n_visible) != n_q:
        raise ValueError("n_visible must have one entry per query row")
    nv = (C.c_int32 * n_q)(*[int(x) for x in n_visible])
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check(lib().attn_verify_stream(C.byref(s.struct), _dev_ptr(q, "q"), _dtype_code(q), int(q.shape[1]), n_q, nv,
                                    float(scale), _dev_ptr(out, "out", (torch.float32,)), _dev_ptr(ws, "ws"),
                                    ws.numel(), _stream(stream)), "attn_verify_stream")
    return out


def _seq(page_table) -> KvSeqStruct:
    torch = _torch()
    if page_table.dtype != torch.int32:
        raise ValueError("page_table must be int32")
    return KvSeqStruct(_dev_ptr(page_table, "page_table"), page_table.numel(), 0)


def kv_append_k8v4(pool: K8V4Pool, page_table, k, v, pos0: int, stream=None) -> None:
    """Quantize and place k, v ([n][H][256], fp16 or fp32) at cells [pos0, pos0+n)."""
    if k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    if k.dim() != 3 or k.shape[1] != pool.n_kv_heads or k.shape[2] != HEAD_DIM:
        raise ValueError("k, v must be [n][n_kv_heads][256]")
    seq = _seq(page_table)
    rc = lib().kv_append_k8v4(C.byref(pool.struct), C.byref(seq), _dev_ptr(k, "k"),
                              _dev_ptr(v, "v"), _dtype_code(k), int(pos0), int(k.shape[0]),
                              _stream(stream))
    _check(rc, "kv_append_k8v4")


def kv_append(pool: KvPool, page_table, k, v, pos0: int, stream=None) -> None:
    """kv_append_k8v4 for a pool of any format."""
    if k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    if k.dim() != 3 or k.shape[1] != pool.n_kv_heads or k.shape[2] != HEAD_DIM:
        raise ValueError("k, v must be [n][n_kv_heads][256]")
    seq = _seq(page_table)
    rc = lib().kv_append(C.byref(pool.struct), C.byref(seq), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                         _dtype_code(k), int(pos0), int(k.shape[0]), _stream(stream))
    _check(rc, "kv_append")


def kv_gather_runs(pool: KvPool, page_table, pos0: int, n: int, stream=None):
    """Stored bytes of cells [pos0, pos0+n) for any format, as kv_gather_runs
    documents: int8-coded halves as (codes int8 [n][H][256], scales fp32
    [n][H][2]), q4_0-coded halves as blocks uint8 [n][H][8][18].  Returns
    (K..., V...) flattened: k8v4 (kc, ks, vb), int8 (kc, ks, vc, vs),
    q4_0 (kb, vb), fp16 (k, v) as float16 [n][H][256]."""
    torch = _torch()
    H = pool.n_kv_heads
    dev = pool.runs[0].device

    def codes():
        return torch.empty((n, H, HEAD_DIM), dtype=torch.int8, device=dev)

    def scales():
        return torch.empty((n, H, 2), dtype=torch.float32, device=dev)

    def blocks():
        return torch.empty((n, H, 8, 18), dtype=torch.uint8, device=dev)

    if pool.fmt == KV_FMT_F16:
        outs = [torch.empty((n, H, HEAD_DIM), dtype=torch.float16, device=dev) for _ in range(2)]
        ptrs = [outs[0], None, outs[1], None]
    elif pool.fmt == KV_FMT_INT8:
        outs = [codes(), scales(), codes(), scales()]
        ptrs = outs
    elif pool.fmt == KV_FMT_Q4_0:
        outs = [blocks(), blocks()]
        ptrs = [outs[0], None, outs[1], None]
    else:
        outs = [codes(), scales(), blocks()]
        ptrs = outs + [None]
    seq = _seq(page_table)
    args = [None if t is None else _dev_ptr(t, "out") for t in ptrs]
    rc = lib().kv_gather_runs(C.byref(pool.struct), C.byref(seq), int(pos0), int(n), *args,
                              _stream(stream))
    _check(rc, "kv_gather_runs")
    return tuple(outs)


def kv_gather(pool: K8V4Pool, page_table, pos0: int, n: int, stream=None):
    """Stored bytes of cells [pos0, pos0+n): (k_codes int8 [n][H][256],
    k_scales fp32 [n][H][2], v_blocks uint8 [n][H][8][18])."""
    torch = _torch()
    H = pool.n_kv_heads
    dev = pool.runs[0].device
    kc = torch.empty((n, H, HEAD_DIM), dtype=torch.int8, device=dev)
    ks = torch.empty((n, H, 2), dtype=torch.float32, device=dev)
    vb = torch.empty((n, H, 8, 18), dtype=torch.uint8, device=dev)
    seq = _seq(page_table)
    rc = lib().kv_gather(C.byref(pool.struct), C.byref(seq), int(pos0), int(n), _dev_ptr(kc, "kc"),
                         _dev_ptr(ks, "ks"), _dev_ptr(vb, "vb"), _stream(stream))
    _check(rc, "kv_gather")
    return kc, ks, vb


def attn_workspace(pool: KvPool, n_q: int, max_ctx: int, stream=None):
    """Allocate and zero a workspace for decode (n_q = 1) or verify calls."""
    torch = _torch()
    nb = int(lib().attn_workspace_bytes(C.byref(pool.struct), GQA * pool.n_kv_heads, n_q, max_ctx))
    if nb == 0:
        raise ValueError("bad workspace request")
    ws = torch.empty(nb, dtype=torch.uint8, device=pool.runs[0].device)
    _check(lib().kv_workspace_init(_dev_ptr(ws, "ws"), nb, _stream(stream)), "kv_workspace_init")
    return ws


def kv_copy_pages(dst: KvPool, src: KvPool, dst_pages, src_pages, stream=None) -> None:
    """Copy page src_pages[i] of src to page dst_pages[i] of dst, every run
    (device int32 page lists of one length; either pool may be host=True)."""
    torch = _torch()
    if dst_pages.dtype != torch.int32 or src_pages.dtype != torch.int32:
        raise ValueError("page lists must be int32")
    if dst_pages.numel() != src_pages.numel():
        raise ValueError("page lists differ in length")
    n = int(src_pages.numel())
    _check(lib().kv_copy_pages(C.byref(dst.struct), C.byref(src.struct),
                               _dev_ptr(dst_pages, "dst_pages"), _dev_ptr(src_pages, "src_pages"), n,
                               _stream(stream)), "kv_copy_pages")


def probe_read(buf, sink, stream=None):
    """One plain streaming read of the device tensor buf (a bandwidth yardstick)."""
    _check(lib().kv_probe_read(_dev_ptr(buf, "buf"), buf.numel() * buf.element_size(),
                               _dev_ptr(sink, "sink"), _stream(stream)), "kv_probe_read")


def attn_decode(pool: KvPool, page_table, q, n_ctx: int, ws, scale: float = 0.0, out=None,
                stream=None):
    """q: [Hq][256] fp16/fp32 -> out fp32 [Hq][256], attending cells [0, n_ctx)."""
    torch = _torch()
    if q.dim() != 2 or q.shape[1] != HEAD_DIM:
        raise ValueError("q must be [n_q_heads][256]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    seq = _seq(page_table)
    rc = lib().attn_decode(C.byref(pool.struct), C.byref(seq), _dev_ptr(q, "q"), _dtype_code(q),
                           int(q.shape[0]), int(n_ctx), float(scale),
                           _dev_ptr(out, "out", (torch.float32,)), _dev_ptr(ws, "ws"),
                           ws.numel(), _stream(stream))
    _check(rc, "attn_decode")
    return out


def attn_decode_noalloc(pool: KvPool, page_table, q, n_ctx: int, scale: float = 0.0, out=None,
                        stream=None):
    """attn_decode without a workspace: the library's per-device scratch
    array holds the split partials (calls on one GPU must be ordered)."""
    torch = _torch()
    if q.dim() != 2 or q.shape[1] != HEAD_DIM:
        raise ValueError("q must be [n_q_heads][256]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    seq = _seq(page_table)
    rc = lib().attn_decode_noalloc(C.byref(pool.struct), C.byref(seq), _dev_ptr(q, "q"), _dtype_code(q),
                                   int(q.shape[0]), int(n_ctx), float(scale),
                                   _dev_ptr(out, "out", (torch.float32,)), _stream(stream))
    _check(rc, "attn_decode_noalloc")
    return out


def attn_decode_append(pool: K8V4Pool, page_table, k, v, q, pos: int, ws, scale: float = 0.0,
                       out=None, stream=None):
    """Append token k, v ([H][256], fp16/fp32, same dtype) at cell pos of a
    k8v4 pool and attend q ([Hq][256]) over cells [0, pos] in one launch
    sequence -> out fp32 [Hq][256]."""
    torch = _torch()
    if q.dim() != 2 or q.shape[1] != HEAD_DIM:
        raise ValueError("q must be [n_q_heads][256]")
    if k.shape != v.shape or k.dim() != 2 or k.shape[1] != HEAD_DIM:
        raise ValueError("k, v must be [n_kv_heads][256]")
    if k.dtype != v.dtype:
        raise ValueError("k and v must share a dtype")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    seq = _seq(page_table)
    rc = lib().attn_decode_append(C.byref(pool.struct), C.byref(seq), _dev_ptr(k, "k"),
                                  _dev_ptr(v, "v"), _dtype_code(k), _dev_ptr(q, "q"), _dtype_code(q),
                                  int(q.shape[0]), int(pos), float(scale),
                                  _dev_ptr(out, "out", (torch.float32,)), _dev_ptr(ws, "ws"),
                                  ws.numel(), _stream(stream))
    _check(rc, "attn_decode_append")
    return out


def attn_decode_batch(pool: KvPool, page_tables, q, n_ctx, ws, scale: float = 0.0, out=None,
                      stream=None):
    """A batch of sequences in one launch sequence: q [n_seq][Hq][256],
    page_tables a list of n_seq int32 device tables, n_ctx a list of lengths
    -> out fp32 [n_seq][Hq][256]."""
    torch = _torch()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [n_seq][n_q_heads][256]")
    n_seq = int(q.shape[0])
    if len(page_tables) != n_seq or len(n_ctx) != n_seq:
        raise ValueError("one page table and one length per sequence")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    seqs = (KvSeqStruct * n_seq)(*[_seq(t) for t in page_tables])
    lens = (C.c_int32 * n_seq)(*[int(x) for x in n_ctx])
    rc = lib().attn_decode_batch(C.byref(pool.struct), seqs, n_seq, _dev_ptr(q, "q"), _dtype_code(q),
                                 int(q.shape[1]), lens, float(scale),
                                 _dev_ptr(out, "out", (torch.float32,)), _dev_ptr(ws, "ws"),
                                 ws.numel(), _stream(stream))
    _check(rc, "attn_decode_batch")
    return out


def attn_verify(pool: KvPool, page_table, q, n_visible, ws, scale: float = 0.0, out=None,
                stream=None):
    """q: [n_q][Hq][256]; row i attends cells [0, n_visible[i]) -> out fp32 [n_q][Hq][256]."""
    torch = _torch()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [n_q][n_q_heads][256]")
    n_q = int(q.shape[0])
    nv = (C.c_int32 * n_q)(*[int(x) for x in n_visible])
    if len(n_visible) != n_q:
        raise ValueError("n_visible must have one entry per query row")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    seq = _seq(page_table)
    rc = lib().attn_verify(C.byref(pool.struct), C.byref(seq), _dev_ptr(q, "q"), _dtype_code(q),
                           int(q.shape[1]), n_q, nv, float(scale),
                           _dev_ptr(out, "out", (torch.float32,)), _dev_ptr(ws, "ws"),
                           ws.numel(), _stream(stream))
    _check(rc, "attn_verify")
    return out


def attn_prefill_workspace(pool: KvPool, n_cells: int):
    """Allocate the workspace of attn_prefill_chunk over n_cells = pos0 + n_new
    cells (no initialisation needed)."""
    torch = _torch()
    nb = int(lib().attn_prefill_workspace_bytes(C.byref(pool.struct), int(n_cells)))
    if nb == 0:
        raise ValueError("bad workspace request")
    return torch.empty(nb, dtype=torch.uint8, device=pool.runs[0].device)


def attn_prefill_chunk(pool: KvPool, page_table, q, pos0: int, scale: float = 0.0, out=None,
                       ws=None, stream=None):
    """q: [n_new][Hq][256] at positions [pos0, pos0+n_new); row i attends [0, pos0+i].
    ws: attn_prefill_workspace(pool, pos0 + n_new), allocated here when None."""
    torch = _torch()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [n_new][n_q_heads][256]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if ws is None and q.shape[0] > 0:
        ws = attn_prefill_workspace(pool, int(pos0) + int(q.shape[0]))
    seq = _seq(page_table)
    rc = lib().attn_prefill_chunk(C.byref(pool.struct), C.byref(seq), _dev_ptr(q, "q"),
                                  _dtype_code(q), int(q.shape[1]), int(pos0), int(q.shape[0]),
                                  float(scale), _dev_ptr(out, "out", (torch.float32,)),
                                  None if ws is None else _dev_ptr(ws, "ws"),
                                  0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "attn_prefill_chunk")
    return out


def time_next_launch(start_event, stop_event) -> None:
    """Arm torch.cuda.Event pair (enable_timing=True, already recorded once so
    that torch has created the HIP events) around the next kernel this
    library launches on the calling thread."""
    if not start_event.cuda_event or not stop_event.cuda_event:
        raise ValueError("record the events once before arming them")
    _check(lib().kv_time_next_launch(C.c_void_p(start_event.cuda_event),
                                     C.c_void_p(stop_event.cuda_event)), "kv_time_next_launch")


def check_page_table(pool: K8V4Pool, page_table, n_cells: int) -> int:
    """Synchronous debug check: number of bad (out of range or repeated) entries."""
    seq = _seq(page_table)
    bad = C.c_int32(0)
    _check(lib().kv_check_page_table(C.byref(pool.struct), C.byref(seq), int(n_cells),
                                     C.byref(bad)), "kv_check_page_table")
    return int(bad.value)
