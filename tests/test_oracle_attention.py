"""Pins for the oracle's pool placement, gather and fp64 attention.

Checks against: the direct quantization of the inputs (gather must return
exactly those bytes), page-table permutation invariance, sentinel bytes,
a negative control, pure-Python brute-force softmax on tiny contexts,
scipy's Hadamard matrix, closed forms (one cell, zero query, two cells),
the rotate-before / un-rotate-after identity on unquantized data, and the
GQA head mapping.
"""
import math

import numpy as np
import pytest
import scipy.linalg

from long_context_decode_append_amd import synth

H_SCI = scipy.linalg.hadamard(256).astype(np.float64)


def _pool_with(orc, fmt, P, n_pages, n_table, n_tok, seed, identity=False, dtype=np.float16):
    pt = synth.page_table(seed, n_table, n_pages, identity=identity)
    k, v = synth.kv_tokens(seed, 0, 0, n_tok, 2, 256, dtype)
    pool = orc.OraclePool(fmt, n_pages, P, 2)
    pool.append(pt, k, v, 0)
    return pool, pt, k, v


# ------------------------------------------------------------------ placement and gather

@pytest.mark.parametrize("fmt", [3, 1, 2])
def test_gather_returns_direct_quantization(orc, fmt):
    pool, pt, k, v = _pool_with(orc, fmt, P=16, n_pages=12, n_table=10, n_tok=150, seed=1)
    g = pool.gather(pt, 0, 150)
    kf, vf = k.astype(np.float32), v.astype(np.float32)
    if fmt == 3:
        kc, ks = orc.quant_int8(kf)
        vb = orc.quant_q4(orc.fwht256(vf))
        exp = (kc, ks, vb)
    elif fmt == 1:
        kc, ks = orc.quant_int8(kf)
        vc, vs = orc.quant_int8(vf)
        exp = (kc, ks, vc, vs)
    else:
        exp = (orc.quant_q4(orc.fwht256(kf)), orc.quant_q4(orc.fwht256(vf)))
    assert len(g) == len(exp)
    for a, b in zip(g, exp):
        assert a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("fmt", [3, 1, 2, 0])
def test_pool_image_is_the_quantized_inputs_placed_by_page(orc, fmt):
    """Each run is [physical page][kv head][slot][record]: logical page i's
    records, head-major, sit in physical page pt[i] (checked by numpy
    reshapes of the directly quantized inputs, not by offset formulas)."""
    P, H, n_pages, n_table = 16, 2, 7, 6
    n_tok = n_table * P
    pool, pt, k, v = _pool_with(orc, fmt, P=P, n_pages=n_pages, n_table=n_table, n_tok=n_tok, seed=2)
    kf, vf = k.astype(np.float32), v.astype(np.float32)
    if fmt == 3:
        kc, ks = orc.quant_int8(kf)
        recs = [kc, ks, orc.quant_q4(orc.fwht256(vf)), None]
    elif fmt == 1:
        kc, ks = orc.quant_int8(kf)
        vc, vs = orc.quant_int8(vf)
        recs = [kc, ks, vc, vs]
    elif fmt == 2:
        recs = [orc.quant_q4(orc.fwht256(kf)), None, orc.quant_q4(orc.fwht256(vf)), None]
    else:
        recs = [k.astype(np.float16), None, v.astype(np.float16), None]
    for r, rec in enumerate(recs):
        if rec is None:
            assert pool.runs[r] is None
            continue
        rb = np.ascontiguousarray(rec).view(np.uint8).reshape(n_table, P, H, -1)   # [logical page][slot][head][bytes]
        by_page = rb.transpose(0, 2, 1, 3).reshape(n_table, -1)                   # [logical page][head][slot][bytes]
        img = pool.runs[r].reshape(n_pages, -1)
        assert np.array_equal(img[pt], by_page), f"run {r}"
        unused = np.setdiff1d(np.arange(n_pages), pt)
        assert np.all(img[unused] == 0xA5)


def test_identity_vs_permuted_page_table(orc):
    a, pta, _, _ = _pool_with(orc, 3, P=16, n_pages=8, n_table=8, n_tok=128, seed=3, identity=True)
    b, ptb, _, _ = _pool_with(orc, 3, P=16, n_pages=8, n_table=8, n_tok=128, seed=3)
    assert not np.array_equal(pta, ptb)
    for x, y in zip(a.gather(pta, 0, 128), b.gather(ptb, 0, 128)):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    # the images are equal up to the page permutation
    per_page = [16 * 2 * 256, 16 * 2 * 8, 16 * 2 * 144]
    for r in range(3):
        ra = a.runs[r].reshape(8, per_page[r])
        rb = b.runs[r].reshape(8, per_page[r])
        assert np.array_equal(ra[pta], rb[ptb])


def test_unwritten_cells_keep_sentinel_and_wrong_table_is_detected(orc):
    P = 16
    pool, pt, _, _ = _pool_with(orc, 3, P=P, n_pages=10, n_table=6, n_tok=40, seed=4)
    used = set(int(x) for x in pt[:3])            # 40 tokens touch 3 pages, the third partly
    r0 = pool.runs[0].reshape(10, 2, P, 256)      # [page][head][slot][256 codes]
    for page in range(10):
        if page not in used:
            assert np.all(r0[page] == 0xA5)
    third = int(pt[2])
    assert np.all(r0[third, :, 8:] == 0xA5)
    assert not np.any(np.all(r0[third, :, :8] == 0xA5, axis=-1))
    # negative control: a table with two entries swapped reads other bytes
    bad = pt.copy()
    bad[[0, 1]] = bad[[1, 0]]
    good = pool.gather(pt, 0, 32)
    wrong = pool.gather(bad, 0, 32)
    assert not np.array_equal(good[0], wrong[0])


def test_append_in_pieces_equals_one_call(orc):
    pt = synth.page_table(5, 8, 8)
    k, v = synth.kv_tokens(5, 0, 0, 100, 2, 256)
    a = orc.OraclePool(3, 8, 16, 2)
    a.append(pt, k, v, 0)
    b = orc.OraclePool(3, 8, 16, 2)
    for s, e in ((0, 1), (1, 17), (17, 50), (50, 100)):
        b.append(pt, k[s:e], v[s:e], s)
    for x, y in zip(a.runs, b.runs):
        if x is not None:
            assert np.array_equal(x, y)


def test_out_of_range_append_is_rejected(orc):
    pool = orc.OraclePool(3, 4, 16, 2)
    pt = np.arange(4, dtype=np.int32)
    k = np.zeros((10, 2, 256), np.float16)
    with pytest.raises(ValueError):
        pool.append(pt, k, k, 60)


# ------------------------------------------------------------------ attention

def _brute(kd, vd, q, n, scale, rotated=True):
    """Pure-Python softmax attention for one (row, head) pair, fp64."""
    s = [scale * sum(float(q[c]) * kd[t][c] for c in range(256)) for t in range(n)]
    mx = max(s)
    w = [math.exp(x - mx) for x in s]
    W = sum(w)
    u = [sum(w[t] * vd[t][c] for t in range(n)) / W for c in range(256)]
    u = np.array(u)
    return H_SCI @ u / 16.0 if rotated else u


def test_attention_matches_brute_force_tiny(orc):
    pool, pt, _, _ = _pool_with(orc, 3, P=16, n_pages=2, n_table=2, n_tok=6, seed=6)
    q = synth.queries(6, 0, 0, 1, 16, 256, np.float16)
    kd, vd = orc.dequant_gathered(3, pool.gather(pt, 0, 6))
    for n in (1, 2, 3, 6):
        out = orc.attention(kd, vd, q, [n])
        for h in (0, 7, 8, 15):
            g = h // 8
            ref = _brute(kd[:, g].tolist(), vd[:, g].tolist(), q[0, h], n, 1 / 16)
            assert np.allclose(out[0, h], ref, rtol=0, atol=1e-12)


def test_one_cell_returns_unrotated_value(orc):
    rng = np.random.default_rng(0)
    kd = rng.standard_normal((5, 2, 256))
    vd = rng.standard_normal((5, 2, 256))
    q = rng.standard_normal((1, 16, 256)).astype(np.float32)
    out = orc.attention(kd, vd, q, [1])
    for h in range(16):
        assert np.allclose(out[0, h], H_SCI @ vd[0, h // 8] / 16, atol=1e-13)


def test_zero_query_averages_and_two_cell_closed_form(orc):
    rng = np.random.default_rng(1)
    kd = rng.standard_normal((9, 2, 256))
    vd = rng.standard_normal((9, 2, 256))
    q0 = np.zeros((1, 16, 256), np.float32)
    out = orc.attention(kd, vd, q0, [9], v_rotated=False)
    assert np.allclose(out[0, 3], vd[:, 0].mean(0), atol=1e-13)
    assert np.allclose(out[0, 12], vd[:, 1].mean(0), atol=1e-13)
    q = rng.standard_normal((1, 16, 256)).astype(np.float32)
    out = orc.attention(kd, vd, q, [2], scale=0.05, v_rotated=False)
    for h in (0, 9):
        g = h // 8
        s0 = 0.05 * float(q[0, h].astype(np.float64) @ kd[0, g])
        s1 = 0.05 * float(q[0, h].astype(np.float64) @ kd[1, g])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert np.allclose(out[0, h], w0 * vd[0, g] + (1 - w0) * vd[1, g], atol=1e-13)


def test_rotate_before_unrotate_after_identity(orc):
    """(1/16) H attn(q, K, (H/16) V) equals attn(q, K, V) on unquantized data."""
    rng = np.random.default_rng(2)
    kd = rng.standard_normal((40, 2, 256))
    vd = rng.standard_normal((40, 2, 256))
    q = rng.standard_normal((3, 16, 256)).astype(np.float32)
    vrot = vd @ H_SCI.T / 16
    a = orc.attention(kd, vd, q, [40, 17, 1], v_rotated=False)
    b = orc.attention(kd, vrot, q, [40, 17, 1], v_rotated=True)
    assert np.allclose(a, b, atol=1e-12)
    # q4_0 format: rotating both q and K leaves the scores unchanged
    krot = kd @ H_SCI.T / 16
    c = orc.attention(krot, vrot, q, [40, 17, 1], q_rotate=True, v_rotated=True)
    assert np.allclose(a, c, atol=1e-12)


def test_rows_with_step_limits_match_single_rows(orc):
    """Batched rows with a per-row step array equal one-row calls (the
    verify form against the decode form) and the prefill row rule."""
    rng = np.random.default_rng(3)
    kd = rng.standard_normal((30, 2, 256))
    vd = rng.standard_normal((30, 2, 256))
    q = rng.standard_normal((5, 16, 256)).astype(np.float32)
    nv = [26, 27, 28, 29, 30]
    batched = orc.attention(kd, vd, q, nv)
    for i in range(5):
        single = orc.attention(kd, vd, q[i:i + 1], [nv[i]])
        assert np.array_equal(batched[i], single[0])


def test_gqa_head_mapping(orc):
    rng = np.random.default_rng(4)
    kd = rng.standard_normal((7, 2, 256))
    vd = np.zeros((7, 2, 256))
    vd[:, 0] = 1.0
    vd[:, 1] = -2.0
    q = rng.standard_normal((1, 16, 256)).astype(np.float32)
    out = orc.attention(kd, vd, q, [7], v_rotated=False)
    assert np.allclose(out[0, :8], 1.0) and np.allclose(out[0, 8:], -2.0)


def test_quantized_attention_close_to_exact(orc):
    """Sanity: k8v4 attention stays near fp64 attention on the raw inputs."""
    n = 512
    pool, pt, k, v = _pool_with(orc, 3, P=16, n_pages=32, n_table=32, n_tok=n, seed=7)
    q = synth.queries(7, 0, 0, 1, 16, 256, np.float16)
    out = orc.attention_from_pool(pool, pt, q, [n])
    exact = orc.attention(k.astype(np.float64), v.astype(np.float64), q, [n], v_rotated=False)
    rel = np.abs(out - exact).max(-1) / np.abs(exact).max(-1)
    assert rel.max() < 0.25            # 4-bit V: about 8 % noise per element
    pool8, pt8, _, _ = _pool_with(orc, 1, P=16, n_pages=32, n_table=32, n_tok=n, seed=7)
    out8 = orc.attention_from_pool(pool8, pt8, q, [n])
    rel8 = np.abs(out8 - exact).max(-1) / np.abs(exact).max(-1)
    assert rel8.max() < 0.03 and rel8.max() < rel.max()


# ------------------------------------------------------------------ fp16 format (no quantization)

def test_f16_cell_bytes(orc):
    # 2 KV heads x 256 dims x (K and V) x 2 bytes
    assert orc.cell_bytes(0, 2) == 2048 and orc.cell_bytes(0, 1) == 1024


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_f16_gather_is_numpy_half_rounding(orc, dtype):
    # the stored values are the inputs rounded to fp16 (numpy's own
    # round-to-nearest-even cast), in logical order through a permuted table
    pool, pt, k, v = _pool_with(orc, 0, P=32, n_pages=6, n_table=5, n_tok=150, seed=11, dtype=dtype)
    gk, gv = pool.gather(pt, 0, 150)
    assert np.array_equal(gk.view(np.uint16), k.astype(np.float16).view(np.uint16))
    assert np.array_equal(gv.view(np.uint16), v.astype(np.float16).view(np.uint16))
    # untouched pages keep the sentinel
    used = set(int(x) for x in pt[:5])
    r0 = pool.runs[0].reshape(6, -1)
    for page in range(6):
        if page not in used:
            assert np.all(r0[page] == 0xA5)


def test_f16_values_placed_by_page(orc):
    P, H = 32, 2
    pool, pt, k, v = _pool_with(orc, 0, P=P, n_pages=4, n_table=3, n_tok=70, seed=12)
    for run, x in ((pool.runs[0], k), (pool.runs[2], v)):
        img = run.view(np.uint16).reshape(4, H, P, 256)   # [page][head][slot][256]
        for p in (0, 5, 16, 31, 32, 69):
            page, slot = pt[p // P], p % P
            for g in range(H):
                assert np.array_equal(img[page, g, slot], x[p, g].view(np.uint16))


def test_f16_attention_matches_brute_force_tiny(orc):
    # unrotated keys and values, the exact fp16 values: pure-Python softmax
    pool, pt, k, v = _pool_with(orc, 0, P=16, n_pages=2, n_table=2, n_tok=7, seed=13)
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 16, 256)).astype(np.float16)
    out = orc.attention_from_pool(pool, pt, q, np.array([7], np.int32))
    kd, vd = k.astype(np.float64), v.astype(np.float64)
    for h in (0, 7, 8, 15):
        ref = _brute(kd[:, h // 8].tolist(), vd[:, h // 8].tolist(), q[0, h], 7, 1 / 16, rotated=False)
        assert np.allclose(out[0, h], ref, rtol=0, atol=1e-12)


def test_threaded_attention_is_bitwise_the_single_thread_result(orc):
    """The (row, head) pairs spread over threads compute exactly what one
    thread computes (the threads only split the work)."""
    pool, pt, _, _ = _pool_with(orc, 3, P=16, n_pages=12, n_table=12, n_tok=180, seed=21)
    rng = np.random.default_rng(21)
    q = rng.standard_normal((5, 16, 256)).astype(np.float16)
    nv = np.array([180, 1, 57, 179, 100], np.int32)
    kd, vd = orc.dequant_gathered(3, pool.gather(pt, 0, 180))
    one = orc.attention(kd, vd, q, nv, threads=1)
    for nt in (2, 3, 7, 16):
        assert np.array_equal(orc.attention(kd, vd, q, nv, threads=nt).view(np.uint64), one.view(np.uint64))
