"""Streamed cache pieces on the GPU ("kv: --kv k8v4 streams with
--kv-resident", Tests): all pages mirrored to pinned host memory, the pages
of a context copied back into a device window at other slots, and attention
over the window through its own table bitwise equal to attention over the
resident pool (decode, verify, prefill), for the three formats.  Negative
control: a window missing one page is detected.
"""
import sys

import numpy as np
import pytest

from long_context_decode_append_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def k8():
    import long_context_decode_append_amd as k8
    k8.lib()
    return k8


def t_(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def page_block(pool, run, page):
    """The bytes of one page in one run (runs are [page][head][slot])."""
    nb = pool.runs[run].numel() // pool.n_pages
    return pool.runs[run][page * nb:(page + 1) * nb]


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_streamed_window_equals_resident_bitwise(k8, dev, fmt):
    import torch
    P, n_res, n_tab, n_win, ctx = 16, 80, 64, 70, 1000
    say(f"stream fmt={fmt}")
    res = k8.KvPool(fmt, n_res, P, 2, device=dev, fill=0x11)
    t_res = synth.page_table(61, n_tab, n_res)
    g_res = t_(t_res, dev)
    k, v = synth.kv_tokens(62, 0, 0, ctx, 2, 256, np.float16)
    k8.kv_append(res, g_res, t_(k, dev), t_(v, dev), 0)
    # every page to the pinned host mirror (same slots)
    host = k8.KvPool(fmt, n_res, P, 2, fill=0x22, host=True)
    allp = torch.arange(n_res, dtype=torch.int32, device=dev)
    k8.kv_copy_pages(host, res, allp, allp)
    torch.cuda.synchronize()
    for r in range(4):
        if res.runs[r] is not None:
            assert torch.equal(host.runs[r], res.runs[r].cpu()), f"mirror run {r}"
    # the context's pages into a smaller device window at other slots
    win = k8.KvPool(fmt, n_win, P, 2, device=dev, fill=0x33)
    t_win = synth.page_table(63, n_tab, n_win)
    k8.kv_copy_pages(win, host, t_(t_win, dev), t_(t_res, dev))
    g_win = t_(t_win, dev)
    torch.cuda.synchronize()
    for p in range(n_tab):
        for r in range(4):
            if res.runs[r] is not None:
                assert torch.equal(page_block(win, r, int(t_win[p])), page_block(res, r, int(t_res[p])))
    # attention through the two tables: bitwise equal
    q = t_(synth.queries(64, 0, 0, 5, 16, 256, np.float16), dev)
    ws = k8.attn_workspace(res, 5, ctx)
    for n in (1, 17, 600, ctx):
        a = k8.attn_decode(res, g_res, q[0], n, ws).cpu().numpy()
        b = k8.attn_decode(win, g_win, q[0], n, ws).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), n
    nv = [ctx, ctx - 1, 500, 33, 1]
    a = k8.attn_verify(res, g_res, q, nv, ws).cpu().numpy()
    b = k8.attn_verify(win, g_win, q, nv, ws).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    a = k8.attn_prefill_chunk(res, g_res, q, ctx - 5).cpu().numpy()
    b = k8.attn_prefill_chunk(win, g_win, q, ctx - 5).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # negative control: a window that misses one page of the context
    miss = k8.KvPool(fmt, n_win, P, 2, device=dev, fill=0x33)
    drop = n_tab // 2
    keep = [p for p in range(n_tab) if p != drop]
    k8.kv_copy_pages(miss, host, t_(t_win[keep], dev), t_(t_res[keep], dev))
    c = k8.attn_decode(miss, g_win, q[0], ctx, ws).cpu().numpy()
    a = k8.attn_decode(res, g_res, q[0], ctx, ws).cpu().numpy()
    assert not np.array_equal(a.view(np.uint32), c.view(np.uint32))


def test_copy_skips_out_of_range_entries(k8, dev):
    import torch
    a = k8.KvPool(3, 8, 16, 2, device=dev, fill=0x44)
    b = k8.KvPool(3, 8, 16, 2, device=dev, fill=0x55)
    before = [r.clone() for r in b.runs if r is not None]
    src = t_(np.array([0, 1, -1, 9, 2], np.int32), dev)
    dst = t_(np.array([100, -3, 4, 5, 6], np.int32), dev)
    k8.kv_copy_pages(b, a, dst, src)
    torch.cuda.synchronize()
    # only pair 4 (2 -> 6) is in range on both sides
    for r, old in zip([r for r in b.runs if r is not None], before):
        nb = r.numel() // 8
        for p in range(8):
            blk = r[p * nb:(p + 1) * nb]
            want = 0x44 if p == 6 else 0x55
            assert bool((blk == want).all()), (p, want)
