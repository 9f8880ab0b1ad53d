"""C-ABI checks that need no GPU: the library loads, exports every function
include/k8v4.h declares, and the host-side validation returns the documented
error codes before anything is launched."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "k8v4.h")


@pytest.fixture(scope="module")
def k8():
    import long_context_decode_append_amd as k8
    if not os.path.exists(k8.LIB_PATH):
        from long_context_decode_append_amd import build
        build.build()
    k8.lib()
    return k8


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kv_append_k8v4", "kv_gather", "attn_decode", "attn_verify", "attn_prefill_chunk"):
        assert n in names


def test_library_exports_every_declared_symbol(k8):
    lib = C.CDLL(k8.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) == set(k8.SIGNATURES)


def test_sizes_match_the_pages(k8):
    L = k8.lib()
    assert L.kv_cell_bytes(3, 2, 256) == 816
    assert L.kv_cell_bytes(1, 2, 256) == 1056
    assert L.kv_cell_bytes(2, 2, 256) == 576
    assert L.kv_cell_bytes(3, 2, 128) == 0 and L.kv_cell_bytes(7, 2, 256) == 0
    P, pages, H = 256, 10, 2
    runs = [L.kv_run_bytes(3, r, pages, P, H, 256) for r in range(4)]
    assert runs == [pages * P * H * 256, pages * P * H * 8, pages * P * H * 144, 0]
    assert sum(runs) == pages * P * 816
    # fp16 (no quantization): 2 heads x 256 dims x (K, V) x 2 bytes, runs 0 and 2
    assert L.kv_cell_bytes(0, 2, 256) == 2048
    runs = [L.kv_run_bytes(0, r, pages, P, H, 256) for r in range(4)]
    assert runs == [pages * P * H * 512, 0, pages * P * H * 512, 0]


def _pool(k8, fmt=3, P=16, pages=4, H=2, hd=256, ptrs=(16, 32, 48, 0)):
    return k8.KvPoolStruct(fmt, pages, P, H, hd, 0, (C.c_void_p * 4)(*[p or None for p in ptrs]))


def _seq(k8, n=4, ptr=64):
    return k8.KvSeqStruct(ptr, n, 0)


def test_validation_errors_before_launch(k8):
    L = k8.lib()
    pool, seq = _pool(k8), _seq(k8)
    P, S = C.byref, None
    dummy = C.c_void_p(16)
    # null pool / seq / inputs
    assert L.kv_append_k8v4(None, P(seq), dummy, dummy, 0, 0, 1, None) == -1
    assert L.kv_append_k8v4(P(pool), None, dummy, dummy, 0, 0, 1, None) == -1
    assert L.kv_append_k8v4(P(pool), P(seq), None, dummy, 0, 0, 1, None) == -1
    # a required run that is NULL is an error, never a skip
    bad = _pool(k8, ptrs=(16, 0, 48, 0))
    assert L.kv_append_k8v4(P(bad), P(seq), dummy, dummy, 0, 0, 1, None) == -1
    # unsupported shapes
    assert L.kv_append_k8v4(P(_pool(k8, fmt=1)), P(seq), dummy, dummy, 0, 0, 1, None) == -5
    assert L.kv_append_k8v4(P(_pool(k8, hd=128)), P(seq), dummy, dummy, 0, 0, 1, None) == -5
    assert L.kv_append_k8v4(P(_pool(k8, P=24)), P(seq), dummy, dummy, 0, 0, 1, None) == -5
    # dtype and ranges (4 pages of 16 cells -> 64 cells addressable)
    assert L.kv_append_k8v4(P(pool), P(seq), dummy, dummy, 5, 0, 1, None) == -4
    assert L.kv_append_k8v4(P(pool), P(seq), dummy, dummy, 0, 60, 5, None) == -3
    assert L.kv_append_k8v4(P(pool), P(seq), dummy, dummy, 0, -1, 1, None) == -3
    assert L.kv_append_k8v4(P(pool), P(seq), dummy, dummy, 0, 0, 0, None) == 0   # no-op
    # misaligned device pointer
    assert L.kv_append_k8v4(P(_pool(k8, ptrs=(17, 32, 48, 0))), P(seq), dummy, dummy, 0, 0, 1,
                            None) == -7
    # gather
    assert L.kv_gather(P(pool), P(seq), 0, 65, dummy, dummy, dummy, None) == -3
    assert L.kv_gather(P(pool), P(seq), 0, 4, None, dummy, dummy, None) == -1
    # attention
    out = C.c_void_p(256)
    assert L.attn_decode(P(pool), P(seq), dummy, 0, 16, 0, 0.0, out, dummy, 1 << 20, None) == -3
    assert L.attn_decode(P(pool), P(seq), dummy, 0, 16, 65, 0.0, out, dummy, 1 << 20, None) == -3
    assert L.attn_decode(P(pool), P(seq), dummy, 0, 12, 8, 0.0, out, dummy, 1 << 20, None) == -5
    assert L.attn_decode(P(pool), P(seq), dummy, 0, 16, 8, 0.0, out, None, 0, None) == -6
    assert L.attn_decode(P(pool), P(seq), dummy, 0, 16, 8, 0.0, out, dummy, 16, None) == -6
    nv = (C.c_int32 * 3)(10, 0, 12)
    assert L.attn_verify(P(pool), P(seq), dummy, 0, 16, 3, nv, 0.0, out, dummy, 1 << 20, None) == -3
    nv = (C.c_int32 * 3)(10, 11, 70)
    assert L.attn_verify(P(pool), P(seq), dummy, 0, 16, 3, nv, 0.0, out, dummy, 1 << 20, None) == -3
    assert L.attn_verify(P(pool), P(seq), dummy, 0, 16, 17, nv, 0.0, out, dummy, 1 << 20, None) == -2
    assert L.attn_verify(P(pool), P(seq), dummy, 0, 16, 3, None, 0.0, out, dummy, 1 << 20, None) == -1
    assert L.attn_prefill_chunk(P(pool), P(seq), dummy, 0, 16, 60, 5, 0.0, out, None, 0, None) == -3
    assert L.attn_prefill_chunk(P(pool), P(seq), dummy, 0, 16, 10, 0, 0.0, out, None, 0, None) == 0
    # prefill workspace: one 32,768-byte tile image per 32 cells and KV head
    nb = L.attn_prefill_workspace_bytes(P(pool), 15)
    assert nb == pool.n_kv_heads * 1 * 32768
    assert L.attn_prefill_workspace_bytes(P(pool), 33) == pool.n_kv_heads * 2 * 32768
    assert L.attn_prefill_workspace_bytes(P(pool), 0) == 0
    assert L.attn_prefill_workspace_bytes(None, 15) == 0
    assert L.attn_prefill_chunk(P(pool), P(seq), dummy, 0, 16, 10, 5, 0.0, out, None, 0, None) == -6
    assert L.attn_prefill_chunk(P(pool), P(seq), dummy, 0, 16, 10, 5, 0.0, out, dummy, nb - 16, None) == -6
    assert L.attn_prefill_chunk(P(pool), P(seq), dummy, 0, 16, 10, 5, 0.0, out, C.c_void_p(24), nb,
                                None) == -7
    assert L.kv_strerror(-6) == b"workspace missing or too small"
    # generic append / gather over the four formats
    for fmt, ptrs in ((0, (16, 0, 48, 0)), (1, (16, 32, 48, 64)), (2, (16, 0, 48, 0)), (3, (16, 32, 48, 0))):
        pl = _pool(k8, fmt=fmt, ptrs=ptrs)
        assert L.kv_append(P(pl), P(seq), dummy, dummy, 0, 0, 0, None) == 0
        assert L.kv_append(P(pl), P(seq), None, dummy, 0, 0, 1, None) == -1
        assert L.kv_gather_runs(P(pl), P(seq), 0, 65, dummy, dummy, dummy, dummy, None) == -3
        assert L.kv_gather_runs(P(pl), P(seq), 0, 4, dummy, dummy, None, dummy, None) == -1
    # int8 needs its fourth run (V scales) and a V-scales output
    assert L.kv_append(P(_pool(k8, fmt=1, ptrs=(16, 32, 48, 0))), P(seq), dummy, dummy, 0, 0, 1,
                       None) == -1
    assert L.kv_gather_runs(P(_pool(k8, fmt=1, ptrs=(16, 32, 48, 64))), P(seq), 0, 4, dummy, dummy,
                            dummy, None, None) == -1
    # q4_0 needs no scale outputs
    assert L.kv_gather_runs(P(_pool(k8, fmt=2, ptrs=(16, 0, 48, 0))), P(seq), 0, 0, dummy, None,
                            dummy, None, None) == 0
    # attention (decode, verify, prefill) accepts the three formats
    assert L.attn_decode(P(_pool(k8, fmt=2, ptrs=(16, 0, 48, 0))), P(seq), dummy, 0, 16, 65, 0.0,
                         out, dummy, 1 << 20, None) == -3
    assert L.attn_prefill_chunk(P(_pool(k8, fmt=1, ptrs=(16, 32, 48, 64))), P(seq), dummy, 0, 16, 0,
                                0, 0.0, out, None, 0, None) == 0
    assert L.attn_prefill_chunk(P(_pool(k8, fmt=2, ptrs=(16, 0, 48, 0))), P(seq), dummy, 0, 16, 60,
                                5, 0.0, out, None, 0, None) == -3
    # fp16: both runs required, aligned outputs
    assert L.kv_append(P(_pool(k8, fmt=0, ptrs=(16, 0, 0, 0))), P(seq), dummy, dummy, 0, 0, 1, None) == -1
    assert L.kv_gather_runs(P(_pool(k8, fmt=0, ptrs=(16, 0, 48, 0))), P(seq), 0, 4, C.c_void_p(24), None,
                            dummy, None, None) == -7
    assert L.attn_prefill_chunk(P(_pool(k8, fmt=0, ptrs=(16, 0, 48, 0))), P(seq), dummy, 0, 16, 60,
                                5, 0.0, out, None, 0, None) == -3
    assert L.attn_decode(P(_pool(k8, fmt=0, ptrs=(16, 0, 48, 0))), P(seq), dummy, 0, 16, 65, 0.0,
                         out, dummy, 1 << 20, None) == -3
    # the fused append + decode is k8v4 only
    assert L.attn_decode_append(P(_pool(k8, fmt=1, ptrs=(16, 32, 48, 64))), P(seq), dummy, dummy, 0,
                                dummy, 0, 16, 3, 0.0, out, dummy, 1 << 20, None) == -5
    # page copies: every run must be present (no silently skipped half), the
    # two pools must match in format and shape
    pl = C.c_void_p(64)
    assert L.kv_copy_pages(P(_pool(k8, fmt=3, ptrs=(16, 32, 0, 0))), P(_pool(k8, fmt=3, ptrs=(16, 32, 48, 0))),
                           pl, pl, 4, None) == -1
    assert L.kv_copy_pages(P(_pool(k8, fmt=3, ptrs=(16, 32, 48, 0))), P(_pool(k8, fmt=1, ptrs=(16, 32, 48, 64))),
                           pl, pl, 4, None) == -2
    assert L.kv_copy_pages(P(_pool(k8, fmt=3, ptrs=(16, 32, 48, 0))), P(_pool(k8, fmt=3, ptrs=(16, 32, 48, 0))),
                           None, pl, 4, None) == -1
    assert L.kv_copy_pages(P(_pool(k8, fmt=3, ptrs=(16, 32, 48, 0))), P(_pool(k8, fmt=3, ptrs=(16, 32, 48, 0))),
                           None, None, 0, None) == 0
    # the streaming-read yardstick
    assert L.kv_probe_read(None, 1024, dummy, None) == -1
    assert L.kv_probe_read(dummy, 1024, None, None) == -1
    assert L.kv_probe_read(C.c_void_p(24), 1024, dummy, None) == -7


def test_workspace_size_is_monotone_in_context(k8):
    L = k8.lib()
    pool = _pool(k8, P=256, pages=1024)
    sizes = [L.attn_workspace_bytes(C.byref(pool), 16, 1, n) for n in (1, 31, 1024, 32768, 240000)]
    assert all(s > 0 for s in sizes) and sizes == sorted(sizes)
    assert L.attn_workspace_bytes(C.byref(pool), 16, 5, 240000) > sizes[-1]
    assert L.attn_workspace_bytes(C.byref(pool), 16, 17, 100) == 0
    assert L.attn_workspace_bytes(C.byref(pool), 12, 1, 100) == 0


def _stream(k8, win=None, mir=None, n_table=4, ptrs=(80, 96, 112, 128, 144)):
    win = win or _pool(k8, pages=2)
    mir = mir or _pool(k8, pages=4, ptrs=(160, 176, 192, 0))
    mt, wm, wo, st, fl = [C.c_void_p(p) if p else None for p in ptrs]
    return k8.KvStreamStruct(win, mir, mt, wm, wo, st, fl, n_table, 0)


def test_stream_validation_errors_before_launch(k8):
    """The streamed cache refuses missing pieces and mismatched pools before
    launching: every run of both copies and every map is required."""
    L = k8.lib()
    P = C.byref
    dummy = C.c_void_p(16)
    s = _stream(k8)
    assert L.kv_stream_append(None, dummy, dummy, 0, 0, 1, None) == -1
    # the mirror's V run missing: an error, never a skipped host write
    s_nov = _stream(k8, mir=_pool(k8, pages=4, ptrs=(160, 176, 0, 0)))
    assert L.kv_stream_append(P(s_nov), dummy, dummy, 0, 0, 1, None) == -1
    s_nowin = _stream(k8, win=_pool(k8, pages=2, ptrs=(16, 32, 0, 0)))
    assert L.kv_stream_append(P(s_nowin), dummy, dummy, 0, 0, 1, None) == -1
    # maps and scratch are required
    for i in range(5):
        ptrs = [80, 96, 112, 128, 144]
        ptrs[i] = 0
        assert L.kv_stream_fetch(P(_stream(k8, ptrs=tuple(ptrs))), 0, 1, None) == -1
    # pools of different formats or page sizes
    assert L.kv_stream_append(P(_stream(k8, win=_pool(k8, fmt=1, pages=2, ptrs=(16, 32, 48, 64)))),
                              dummy, dummy, 0, 0, 1, None) == -2
    assert L.kv_stream_append(P(_stream(k8, win=_pool(k8, P=32, pages=2))), dummy, dummy, 0, 0, 1, None) == -2
    # ranges: cells beyond the table, pages beyond it
    assert L.kv_stream_append(P(s), dummy, dummy, 0, 60, 5, None) == -3
    assert L.kv_stream_fetch(P(s), 3, 2, None) == -3
    assert L.kv_stream_fetch(P(s), -1, 1, None) == -3
    assert L.kv_stream_fetch(P(s), 0, 0, None) == 0
    q = C.c_void_p(256)
    out = C.c_void_p(512)
    ws = C.c_void_p(1024)
    assert L.attn_decode_stream(P(s), q, 0, 16, 65, 0.0, out, ws, 1 << 20, None) == -3
    assert L.attn_decode_stream(P(s), q, 0, 16, 0, 0.0, out, ws, 1 << 20, None) == -3
    assert L.attn_decode_stream(P(s), q, 0, 16, 10, 0.0, out, None, 0, None) == -6
    nv = (C.c_int32 * 2)(10, 70)
    assert L.attn_verify_stream(P(s), q, 0, 16, 2, nv, 0.0, out, ws, 1 << 20, None) == -3
    assert L.attn_verify_stream(P(s), q, 0, 16, 0, nv, 0.0, out, ws, 1 << 20, None) == -2
