"""GPU parity of the comparison formats (int8: INT8 K and V, 1,056 B/cell;
q4_0: rotated Q4_0 K and V, 576 B/cell; fp16: K and V unquantized, 2,048
B/cell) through the C ABI against the CPU oracle: pool bytes and gathered
bytes bit-exact, decode and verify within 2e-3 max relative error per
(query row, head)."""
import sys

import numpy as np
import pytest

from long_context_decode_append_amd import synth
from pool_layout import assert_pool_equal

pytestmark = pytest.mark.gpu

TOL = 2e-3
FMT_F16, FMT_INT8, FMT_Q4_0, FMT_K8V4 = 0, 1, 2, 3


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


def rel_err(out, ref):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    return float((np.abs(out - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max())


class ArmCase:
    """The same seeded tokens appended to a GPU pool and an oracle pool of one format."""

    def __init__(self, orc, k8, dev, fmt, seed, ctx, P, n_pages, n_table, dtype=np.float16,
                 outlier_frac=0.0, chunk=8192, fill=0xA5):
        self.fmt = fmt
        self.pt = synth.page_table(seed, n_table, n_pages)
        outl = synth.outlier_channels(seed, 2, 256, outlier_frac) if outlier_frac else None
        self.gpool = k8.KvPool(fmt, n_pages, P, 2, device=dev, fill=fill)
        self.opool = orc.OraclePool(fmt, n_pages, P, 2, sentinel=fill)
        self.gpt = t_(self.pt, dev)
        for s in range(0, ctx, chunk):
            n = min(chunk, ctx - s)
            k, v = synth.kv_tokens(seed, 0, s, n, 2, 256, dtype, outl)
            k8.kv_append(self.gpool, self.gpt, t_(k, dev), t_(v, dev), s)
            self.opool.append(self.pt, k, v, s)


@pytest.mark.parametrize("fmt", [FMT_INT8, FMT_Q4_0, FMT_F16])
@pytest.mark.parametrize("dtype,ctx,P,n_pages", [(np.float32, 1024, 16, 64),
                                                 (np.float16, 1000, 16, 70),
                                                 (np.float16, 700, 256, 4)])
def test_arm_pool_bytes_and_gather_bitwise(orc, k8, dev, fmt, dtype, ctx, P, n_pages):
    say(f"arm append/gather fmt={fmt} dtype={dtype.__name__} ctx={ctx} P={P}")
    c = ArmCase(orc, k8, dev, fmt, 0, ctx, P, n_pages, (ctx + P - 1) // P, dtype=dtype, chunk=333)
    for r in range(4):
        assert (c.opool.runs[r] is None) == (c.gpool.runs[r] is None), f"run {r} presence"
    assert_pool_equal(c.gpool, c.opool)
    g = [x.cpu().numpy() for x in k8.kv_gather_runs(c.gpool, c.gpt, 0, ctx)]
    o = c.opool.gather(c.pt, 0, ctx)
    assert len(g) == len(o)
    for x, y in zip(g, o):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    w = [x.cpu().numpy() for x in k8.kv_gather_runs(c.gpool, c.gpt, 37, 101)]
    for x, y in zip(w, o):
        assert np.array_equal(x.view(np.uint8), y[37:138].view(np.uint8))


def test_k8v4_append_through_generic_entry_equals_k8v4_entry(k8, dev):
    pt = synth.page_table(1, 8, 8)
    k, v = synth.kv_tokens(1, 0, 0, 120, 2, 256, np.float16)
    a = k8.K8V4Pool(8, 16, 2, device=dev, fill=0)
    b = k8.KvPool(FMT_K8V4, 8, 16, 2, device=dev, fill=0)
    gpt = t_(pt, dev)
    k8.kv_append_k8v4(a, gpt, t_(k, dev), t_(v, dev), 0)
    k8.kv_append(b, gpt, t_(k, dev), t_(v, dev), 0)
    for r in range(3):
        assert np.array_equal(a.runs[r].cpu().numpy(), b.runs[r].cpu().numpy())


@pytest.fixture(scope="module", params=[FMT_INT8, FMT_Q4_0, FMT_F16])
def arm_tiny(request, orc, k8, dev):
    return ArmCase(orc, k8, dev, request.param, 0, 1024, 16, 64, 64, dtype=np.float32, chunk=1024)


@pytest.mark.parametrize("n_ctx", [1, 2, 31, 33, 300, 1000, 1024])
@pytest.mark.parametrize("qdtype", [np.float16, np.float32])
def test_arm_decode_parity_tiny(orc, k8, dev, arm_tiny, n_ctx, qdtype):
    say(f"arm decode fmt={arm_tiny.fmt} n_ctx={n_ctx} q={qdtype.__name__}")
    q = synth.queries(0, 0, n_ctx, 1, 16, 256, qdtype)
    ws = k8.attn_workspace(arm_tiny.gpool, 1, 1024)
    out = k8.attn_decode(arm_tiny.gpool, arm_tiny.gpt, t_(q[0], dev), n_ctx, ws).cpu().numpy()
    ref = orc.attention_from_pool(arm_tiny.opool, arm_tiny.pt, q, [n_ctx])[0]
    err = rel_err(out, ref)
    say(f"  rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("n_vis", [[1020, 1021, 1022, 1023, 1024], [700, 33, 1],
                                   [5, 1024, 64, 900, 17, 33, 1, 1000, 2]])
def test_arm_verify_parity_tiny(orc, k8, dev, arm_tiny, n_vis):
    say(f"arm verify fmt={arm_tiny.fmt} n_q={len(n_vis)}")
    q = synth.queries(0, 0, 77, len(n_vis), 16, 256, np.float16)
    ws = k8.attn_workspace(arm_tiny.gpool, len(n_vis), 1024)
    out = k8.attn_verify(arm_tiny.gpool, arm_tiny.gpt, t_(q, dev), n_vis, ws).cpu().numpy()
    ref = orc.attention_from_pool(arm_tiny.opool, arm_tiny.pt, q, n_vis)
    err = rel_err(out, ref)
    say(f"  rel err {err:.3e}")
    assert err <= TOL


def test_arm_verify_one_row_equals_decode_bitwise(k8, dev, arm_tiny):
    q = synth.queries(0, 0, 5, 1, 16, 256, np.float16)
    ws = k8.attn_workspace(arm_tiny.gpool, 1, 1024)
    a = k8.attn_decode(arm_tiny.gpool, arm_tiny.gpt, t_(q[0], dev), 999, ws).cpu().numpy()
    b = k8.attn_verify(arm_tiny.gpool, arm_tiny.gpt, t_(q, dev), [999], ws).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b[0].view(np.uint32))


@pytest.mark.parametrize("fmt", [FMT_INT8, FMT_Q4_0, FMT_F16])
def test_arm_decode_batch_parity(orc, k8, dev, fmt):
    """attn_decode_batch over a pool of each comparison format: three
    sequences with their own permuted tables and lengths (one of them a single
    cell), each output against the oracle and against attn_decode alone."""
    say(f"arm decode batch fmt={fmt}")
    lens, P, per = [700, 1, 333], 16, 48
    n_pages = len(lens) * per + 2
    perm = synth.page_table(61, n_pages, n_pages)
    gpool = k8.KvPool(fmt, n_pages, P, 2, device=dev, fill=0xA5)
    opool = orc.OraclePool(fmt, n_pages, P, 2, sentinel=0xA5)
    tabs, gtabs = [], []
    for b, n in enumerate(lens):
        pt = np.ascontiguousarray(perm[b * per:(b + 1) * per])
        tabs.append(pt)
        gtabs.append(t_(pt, dev))
        k, v = synth.kv_tokens(70 + b, 0, 0, n, 2, 256, np.float16)
        k8.kv_append(gpool, gtabs[b], t_(k, dev), t_(v, dev), 0)
        opool.append(pt, k, v, 0)
    q = synth.queries(62, 0, 0, len(lens), 16, 256, np.float16)
    ws = k8.attn_workspace(gpool, len(lens), max(lens))
    out = k8.attn_decode_batch(gpool, gtabs, t_(q, dev), lens, ws).cpu().numpy()
    for b, n in enumerate(lens):
        ref = orc.attention_from_pool(opool, tabs[b], q[b:b + 1], [n])[0]
        ws1 = k8.attn_workspace(gpool, 1, n)
        one = k8.attn_decode(gpool, gtabs[b], t_(q[b], dev), n, ws1).cpu().numpy()
        err, err1 = rel_err(out[b], ref), rel_err(out[b], one)
        say(f"  seq {b} len {n}: rel err {err:.3e}, vs single decode {err1:.3e}")
        assert err <= TOL
        assert err1 <= TOL


@pytest.mark.parametrize("v_scale", [1e-3, 3e-4])
def test_int8_small_values_decode_and_verify(orc, k8, dev, v_scale):
    """int8 format with V ~ N(0, v_scale^2): the V scales (max|V| / 127,
    ~3e-5 and ~1e-5) lie below fp16's normal range, where an fp16 copy of a
    scale loses its bits; the kernels form code * d in fp32 and round once
    (decode, verify and prefill).  The values themselves stay at or above
    the fp16 normal range for the most part: fp16 matrix-core operands
    cannot hold values far below 2^-14 to the attention tolerance."""
    say(f"int8 small V scale={v_scale}")
    P, n_pages, ctx = 16, 70, 1000
    pt = synth.page_table(14, 63, n_pages)
    gpt = t_(pt, dev)
    k, v = synth.kv_tokens(14, 0, 0, ctx, 2, 256, np.float32)
    v = (v * np.float32(v_scale)).astype(np.float32)
    gpool = k8.KvPool(FMT_INT8, n_pages, P, 2, device=dev, fill=0)
    opool = orc.OraclePool(FMT_INT8, n_pages, P, 2, sentinel=0)
    k8.kv_append(gpool, gpt, t_(k, dev), t_(v, dev), 0)
    opool.append(pt, k, v, 0)
    q = synth.queries(14, 0, 0, 3, 16, 256, np.float16)
    ws = k8.attn_workspace(gpool, 3, ctx)
    out = k8.attn_decode(gpool, gpt, t_(q[0], dev), ctx, ws).cpu().numpy()
    e1 = rel_err(out, orc.attention_from_pool(opool, pt, q[:1], [ctx])[0])
    nv = [ctx, 517, 33]
    outv = k8.attn_verify(gpool, gpt, t_(q, dev), nv, ws).cpu().numpy()
    e2 = rel_err(outv, orc.attention_from_pool(opool, pt, q, nv))
    outp = k8.attn_prefill_chunk(gpool, gpt, t_(q, dev), ctx - 3).cpu().numpy()
    e3 = rel_err(outp, orc.attention_from_pool(opool, pt, q, [ctx - 2, ctx - 1, ctx]))
    say(f"  rel err decode {e1:.3e} verify {e2:.3e} prefill {e3:.3e}")
    assert max(e1, e2, e3) <= TOL


@pytest.mark.parametrize("fmt", [FMT_K8V4, FMT_INT8, FMT_Q4_0, FMT_F16])
@pytest.mark.parametrize("k_scale", [1e-3, 64.0])
def test_k_magnitude_decode_verify_prefill(orc, k8, dev, fmt, k_scale):
    """K ~ N(0, k_scale^2) and queries divided by k_scale, so the scores keep
    their spread while K's magnitude moves: the prefill staging step rounds
    K times the softmax scale (times log2 e) to fp16, where K of 1e-3 lands
    partly in fp16's subnormal range, while decode and verify scale the
    scores in fp32.  All three stay within the tolerance of the oracle."""
    say(f"K magnitude fmt={fmt} k_scale={k_scale}")
    P, n_pages, ctx = 16, 70, 1000
    pt = synth.page_table(15, 63, n_pages)
    gpt = t_(pt, dev)
    k, v = synth.kv_tokens(15, 0, 0, ctx, 2, 256, np.float32)
    k = (k * np.float32(k_scale)).astype(np.float32)
    gpool = k8.KvPool(fmt, n_pages, P, 2, device=dev, fill=0)
    opool = orc.OraclePool(fmt, n_pages, P, 2, sentinel=0)
    k8.kv_append(gpool, gpt, t_(k, dev), t_(v, dev), 0)
    opool.append(pt, k, v, 0)
    q = (synth.queries(15, 0, 0, 3, 16, 256, np.float32) / np.float32(k_scale)).astype(np.float16)
    ws = k8.attn_workspace(gpool, 3, ctx)
    out = k8.attn_decode(gpool, gpt, t_(q[0], dev), ctx, ws).cpu().numpy()
    e1 = rel_err(out, orc.attention_from_pool(opool, pt, q[:1], [ctx])[0])
    nv = [ctx, 517, 33]
    outv = k8.attn_verify(gpool, gpt, t_(q, dev), nv, ws).cpu().numpy()
    e2 = rel_err(outv, orc.attention_from_pool(opool, pt, q, nv))
    outp = k8.attn_prefill_chunk(gpool, gpt, t_(q, dev), ctx - 3).cpu().numpy()
    e3 = rel_err(outp, orc.attention_from_pool(opool, pt, q, [ctx - 2, ctx - 1, ctx]))
    say(f"  rel err decode {e1:.3e} verify {e2:.3e} prefill {e3:.3e}")
    assert max(e1, e2, e3) <= TOL


@pytest.mark.parametrize("fmt", [FMT_INT8, FMT_Q4_0, FMT_K8V4, FMT_F16])
def test_arms_decode_32768_with_outlier_channels(orc, k8, dev, fmt):
    """The three formats on the same raw inputs: 32,768 cells, 3 outlier
    channels per KV head (x8 on K and V), P = 256, 128 pages drawn from a
    256-page pool."""
    say(f"arms 32768 fmt={fmt}")
    c = ArmCase(orc, k8, dev, fmt, 2, 32768, 256, 256, 128, outlier_frac=0.01)
    q = synth.queries(2, 0, 0, 1, 16, 256, np.float16)
    ws = k8.attn_workspace(c.gpool, 1, 32768)
    out = k8.attn_decode(c.gpool, c.gpt, t_(q[0], dev), 32768, ws).cpu().numpy()
    ref = orc.attention_from_pool(c.opool, c.pt, q, [32768])[0]
    err = rel_err(out, ref)
    say(f"  rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", [FMT_INT8, FMT_Q4_0, FMT_F16])
@pytest.mark.parametrize("n_new", [1, 17, 100])
@pytest.mark.parametrize("qdtype", [np.float16, np.float32])
def test_arm_prefill_parity(orc, k8, dev, fmt, n_new, qdtype):
    """Prefill chunks over the comparison formats: q4_0 scores the rotated
    query against rotated keys, int8 returns unrotated values."""
    say(f"arm prefill fmt={fmt} n_new={n_new} q={qdtype.__name__}")
    ctx = 1000
    c = ArmCase(orc, k8, dev, fmt, 5, ctx, 16, 70, 64, dtype=np.float32)
    pos0 = ctx - n_new
    q = synth.queries(5, 0, 3, n_new, 16, 256, qdtype)
    out = k8.attn_prefill_chunk(c.gpool, c.gpt, t_(q, dev), pos0).cpu().numpy()
    ref = orc.attention_from_pool(c.opool, c.pt, q, [pos0 + i + 1 for i in range(n_new)])
    err = rel_err(out, ref)
    say(f"  rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", [FMT_INT8, FMT_Q4_0, FMT_F16])
def test_arm_prefill_32768_outliers_matches_verify(orc, k8, dev, fmt):
    """64 queries at the end of 32,768 cells with outlier channels: against
    the oracle, and row by row against the verify kernel (same limits)."""
    say(f"arm prefill 32768 fmt={fmt}")
    ctx, n_new = 32768, 64
    c = ArmCase(orc, k8, dev, fmt, 6, ctx, 256, 256, 128, outlier_frac=0.01)
    pos0 = ctx - n_new
    q = synth.queries(6, 0, 4, n_new, 16, 256, np.float16)
    out = k8.attn_prefill_chunk(c.gpool, c.gpt, t_(q, dev), pos0).cpu().numpy()
    rows = [0, 31, 63]
    ref = orc.attention_from_pool(c.opool, c.pt, q[rows], [pos0 + i + 1 for i in rows])
    err = rel_err(out[rows], ref)
    say(f"  rel err vs oracle {err:.3e}")
    assert err <= TOL
    ws = k8.attn_workspace(c.gpool, 16, ctx)
    ver = k8.attn_verify(c.gpool, c.gpt, t_(q[48:], dev), [pos0 + i + 1 for i in range(48, 64)],
                         ws).cpu().numpy()
    err_v = rel_err(ver[[15]], ref[[2]])
    say(f"  verify rel err vs oracle (row 63) {err_v:.3e}")
    assert err_v <= TOL
    # two approximations of the same rows, each within TOL of the oracle
    err2 = rel_err(out[48:], ver)
    say(f"  rel diff vs verify {err2:.3e}")
    assert err2 <= 2 * TOL



@pytest.mark.parametrize("fmt", [FMT_F16, FMT_INT8, FMT_Q4_0])
def test_arm_240000_decode_and_prefill_sampled(orc, k8, dev, fmt):
    """The comparison formats at the bench's full size: 240,000 cells in a
    262,144-cell pool (permuted pages of 256).  The whole pool image
    bit-exact with the oracle's, a decode over all cells and sampled rows of
    the 8,192-query prefill chunk at [231,808, 240,000) against the oracle."""
    say(f"arm 240000 decode + prefill fmt={fmt}")
    ctx = 240000
    c = ArmCase(orc, k8, dev, fmt, 9, ctx, 256, 1024, 1024)
    assert_pool_equal(c.gpool, c.opool)
    q1 = synth.queries(9, 0, 0, 1, 16, 256, np.float16)
    ws = k8.attn_workspace(c.gpool, 1, ctx)
    out = k8.attn_decode(c.gpool, c.gpt, t_(q1[0], dev), ctx, ws).cpu().numpy()
    ref = orc.attention_from_pool(c.opool, c.pt, q1, [ctx])[0]
    err = rel_err(out, ref)
    say(f"  decode rel err {err:.3e}")
    assert err <= TOL
    pos0, n_new = 231808, 8192
    q = synth.queries(9, 0, 1, n_new, 16, 256, np.float16)
    outp = k8.attn_prefill_chunk(c.gpool, c.gpt, t_(q, dev), pos0).cpu().numpy()
    assert np.all(np.isfinite(outp))
    rows = [0, 4097, 8191]
    refp = orc.attention_from_pool(c.opool, c.pt, q[rows], [pos0 + i + 1 for i in rows])
    errp = rel_err(outp[rows], refp)
    say(f"  prefill rel err {errp:.3e}")
    assert errp <= TOL
