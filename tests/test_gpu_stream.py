"""The streamed cache on the GPU ("kv: --kv k8v4 streams with
--kv-resident", How and Tests): appends that write the pinned host mirror
and the device window from one quantization, miss service into a ring
window, and streamed decode / verify (window where resident, mirror where
not) bitwise equal to the same calls on a resident pool, whose output is
checked against the oracle, for the four formats; lookups and misses
counted on the device; negative controls (a mirror page's V half left out;
a mirror missing its V run is refused).  Also the page mover alone: all
pages mirrored to pinned host memory and copied back into a window at other
slots, attention through the window's table bitwise equal to the resident
pool (decode, verify, prefill), with a window missing one page detected.
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


TOL = 2e-3


def rel_err(out, ref):
    out, ref = np.asarray(out, np.float64), np.asarray(ref, np.float64)
    return float((np.abs(out - ref).max(-1) / np.abs(ref).max(-1)).max())


@pytest.mark.parametrize("fmt", [3, 0, 1, 2])
def test_streamed_cache_equals_resident_and_oracle(orc, k8, dev, fmt):
    """A streamed cache ("kv: --kv k8v4 streams with --kv-resident", How and
    Tests): the context grows in batches through kv_stream_append (one
    quantization, written to the pinned host mirror and to the window where
    resident), each batch followed by miss service (kv_stream_fetch: the
    newest pages into a 16-page window, ring placement).  After every batch
    the streamed decode and verify (window where resident, mirror where
    not) are bitwise equal to the same calls on a resident pool, whose
    output is checked against the oracle; the mirror image equals the
    oracle's; lookups and misses are counted on the device."""
    import torch
    from pool_layout import gpu_plain_runs
    P, ctx, n_mirror, W, n_res = 16, 1000, 70, 16, 80
    n_table = (ctx + P - 1) // P
    say(f"streamed cache fmt={fmt}")
    mt = synth.page_table(71, n_table, n_mirror)
    s = k8.KvStream(fmt, W, n_mirror, P, t_(mt, dev), fill=0x22)
    t_res = synth.page_table(72, n_table, n_res)
    res = k8.KvPool(fmt, n_res, P, 2, device=dev, fill=0x11)
    g_res = t_(t_res, dev)
    opool = orc.OraclePool(fmt, n_mirror, P, 2, sentinel=0x22)
    k, v = synth.kv_tokens(73, 0, 0, ctx, 2, 256, np.float16)
    q = synth.queries(74, 0, 0, 5, 16, 256, np.float16)
    qt = t_(q, dev)
    ws = k8.attn_workspace(res, 5, ctx)
    batches, lookups, misses, pos = 0, 0, 0, 0
    for n in (1, 15, 17, 100, 128, 250, 489):
        k8.kv_stream_append(s, t_(k[pos:pos + n], dev), t_(v[pos:pos + n], dev), pos)
        k8.kv_append(res, g_res, t_(k[pos:pos + n], dev), t_(v[pos:pos + n], dev), pos)
        opool.append(mt, k[pos:pos + n], v[pos:pos + n], pos)
        pos += n
        n_pages = (pos + P - 1) // P
        k8.kv_stream_fetch(s, 0, n_pages)
        torch.cuda.synchronize()
        wm = s.window_map.cpu().numpy()
        resident = [i for i in range(n_pages) if wm[i] >= 0]
        assert resident == list(range(max(0, n_pages - W), n_pages)), (pos, resident)
        assert all(wm[i] == i % W for i in resident)
        for nc in sorted({1, max(1, pos - 200), pos}):
            a = k8.attn_decode(res, g_res, qt[0], nc, ws).cpu().numpy()
            b = k8.attn_decode_stream(s, qt[0], nc, ws).cpu().numpy()
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (pos, nc)
            lookups += (nc + P - 1) // P
            misses += sum(1 for i in range((nc + P - 1) // P) if wm[i] < 0)
            batches += 1
        nv = [pos, max(1, pos - 1), max(1, pos // 2), 1, max(1, pos - 17)]
        a = k8.attn_verify(res, g_res, qt, nv, ws).cpu().numpy()
        b = k8.attn_verify_stream(s, qt, nv, ws).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (pos, nv)
        lookups += (max(nv) + P - 1) // P
        misses += sum(1 for i in range((max(nv) + P - 1) // P) if wm[i] < 0)
        batches += 1
    st = s.stats.cpu().numpy()
    say(f"  {batches} batches, {int(st[0])} page lookups, {int(st[1])} misses, 0 failures")
    assert int(st[0]) == lookups and int(st[1]) == misses and misses > 0
    # the resident side against the oracle's exact attention
    ref = orc.attention_from_pool(opool, mt, q, [ctx, ctx - 1, ctx // 2, 1, ctx - 17])
    out = k8.attn_verify(res, g_res, qt, [ctx, ctx - 1, ctx // 2, 1, ctx - 17], ws).cpu().numpy()
    err = rel_err(out, ref)
    say(f"  resident vs oracle rel err {err:.3e}")
    assert err <= TOL
    # the mirror holds the oracle's image (sentinels included); the window's
    # resident pages hold the same bytes as their mirror pages
    plain = gpu_plain_runs(s.mirror)
    for r in range(4):
        if opool.runs[r] is not None:
            assert np.array_equal(plain[r], opool.runs[r]), f"mirror run {r}"
    wm = s.window_map.cpu().numpy()
    for i in range(n_table):
        if wm[i] >= 0:
            for r in range(4):
                if s.window.runs[r] is not None:
                    assert torch.equal(page_block(s.window, r, int(wm[i])).cpu(),
                                       page_block(s.mirror, r, int(mt[i])).cpu()), (i, r)
    # negative control (the pages' trap: a V half whose host write was left
    # out): one non-resident page's V run in the mirror cleared
    gone = next(i for i in range(n_table) if wm[i] < 0)
    page_block(s.mirror, 2, int(mt[gone])).zero_()
    torch.cuda.synchronize()
    a = k8.attn_decode(res, g_res, qt[0], ctx, ws).cpu().numpy()
    b = k8.attn_decode_stream(s, qt[0], ctx, ws).cpu().numpy()
    assert not np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_stream_append_refuses_a_missing_run(k8, dev):
    """Every run of both copies is required: a mirror without its V run is
    an error before anything is written, never a skipped host write."""
    import ctypes as C
    mt = t_(synth.page_table(75, 8, 8), dev)
    s = k8.KvStream(3, 4, 8, 16, mt, fill=0)
    k = t_(np.zeros((3, 2, 256), np.float16), dev)
    st = s.struct
    saved = st.mirror.run[2]
    st.mirror.run[2] = None
    rc = k8.lib().kv_stream_append(C.byref(st), C.c_void_p(k.data_ptr()), C.c_void_p(k.data_ptr()), 0, 0, 3, None)
    st.mirror.run[2] = saved
    assert rc == -1  # KV_ERR_NULL



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


def test_streamed_int8_long_context_equals_resident_bitwise(k8, dev):
    """The int8 format's decode runs eight waves per workgroup once a split
    has at least 12 steps (65,536 cells: 16); the streamed call makes the
    same choice, so with half the pages read from the host mirror its output
    is still bitwise the resident call's, at that length and below the
    switch (32,768 cells)."""
    import torch
    P, ctx, W = 256, 65536, 128
    n_table = ctx // P
    say("streamed int8 at 65,536 cells")
    mt = synth.page_table(81, n_table, n_table)
    s = k8.KvStream(1, W, n_table, P, t_(mt, dev), fill=0)
    t_res = synth.page_table(82, n_table, n_table)
    res = k8.KvPool(1, n_table, P, 2, device=dev, fill=0)
    g_res = t_(t_res, dev)
    for c, st in enumerate(range(0, ctx, synth.CHUNK)):
        kk, vv = synth.kv_chunk_device(81, 0, c, synth.CHUNK, 2, 256, dev)
        k8.kv_stream_append(s, kk, vv, st)
        k8.kv_append(res, g_res, kk, vv, st)
    k8.kv_stream_fetch(s, n_table - W, W)
    q = synth.queries_device(81, 0, 0, 1, 16, 256, dev)[0]
    ws = k8.attn_workspace(res, 1, ctx)
    for nc in (ctx, 32768):
        a = k8.attn_decode(res, g_res, q, nc, ws).cpu().numpy()
        b = k8.attn_decode_stream(s, q, nc, ws).cpu().numpy()
        torch.cuda.synchronize()
        assert np.isfinite(a).all()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), nc
