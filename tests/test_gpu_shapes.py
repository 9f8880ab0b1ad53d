"""GPU parity at page sizes that are not powers of two (the kernels' division
path for page lookups) and at 1 and 4 KV heads: append bytes, gather, decode,
verify, the fused append + decode and the prefill chunk, against the oracle.
"""
import sys

import numpy as np
import pytest

from long_context_decode_append_amd import synth
from pool_layout import assert_pool_equal

pytestmark = pytest.mark.gpu

TOL = 2e-3


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


@pytest.mark.parametrize("P,H,n_pages,n_table", [(48, 1, 30, 25), (80, 4, 20, 17), (144, 2, 12, 9)])
def test_odd_pages_and_head_counts(orc, k8, dev, P, H, n_pages, n_table):
    import torch
    cap = P * n_table
    ctx = cap - 37                      # ragged last page
    seed = 21 + P
    say(f"P={P} H={H} ctx={ctx}")
    pt = synth.page_table(seed, n_table, n_pages)
    gpt = t_(pt, dev)
    gpool = k8.K8V4Pool(n_pages, P, H, device=dev, fill=0x5A)
    opool = orc.OraclePool(3, n_pages, P, H, sentinel=0x5A)
    for s in range(0, ctx, 500):
        n = min(500, ctx - s)
        k, v = synth.kv_tokens(seed, 0, s, n, H, 256, np.float16)
        k8.kv_append_k8v4(gpool, gpt, t_(k, dev), t_(v, dev), s)
        opool.append(pt, k, v, s)
    # every stored byte (sentinels included) equals the oracle's image
    assert_pool_equal(gpool, opool)
    Hq = 8 * H
    # decode at a few lengths, incl. one ending inside a page and the full fill
    for n_ctx in (1, P - 1, P + 17, ctx):
        q = synth.queries(seed, 0, n_ctx, 1, Hq, 256, np.float16)
        ws = k8.attn_workspace(gpool, 1, n_ctx)
        out = k8.attn_decode(gpool, gpt, t_(q[0], dev), n_ctx, ws).cpu().numpy()
        ref = orc.attention_from_pool(opool, pt, q, [n_ctx])[0]
        err = rel_err(out, ref)
        say(f"  decode n_ctx={n_ctx} rel err {err:.3e}")
        assert err <= TOL
    # verify, 3 rows with mixed limits
    nv = [ctx, ctx - P, 2 * P + 1]
    q = synth.queries(seed, 0, 9, len(nv), Hq, 256, np.float16)
    ws = k8.attn_workspace(gpool, len(nv), ctx)
    out = k8.attn_verify(gpool, gpt, t_(q, dev), nv, ws).cpu().numpy()
    err = rel_err(out, orc.attention_from_pool(opool, pt, q, nv))
    say(f"  verify rel err {err:.3e}")
    assert err <= TOL
    # prefill of the last 40 cells' queries
    n_new = 40
    pos0 = ctx - n_new
    q = synth.queries(seed, 0, 11, n_new, Hq, 256, np.float16)
    out = k8.attn_prefill_chunk(gpool, gpt, t_(q, dev), pos0).cpu().numpy()
    err = rel_err(out, orc.attention_from_pool(opool, pt, q, [pos0 + i + 1 for i in range(n_new)]))
    say(f"  prefill rel err {err:.3e}")
    assert err <= TOL
    # fused append + decode at the next cell
    k, v = synth.kv_tokens(seed, 0, ctx, 1, H, 256, np.float16)
    q = synth.queries(seed, 0, ctx, 1, Hq, 256, np.float16)
    ws = k8.attn_workspace(gpool, 1, ctx + 1)
    out = k8.attn_decode_append(gpool, gpt, t_(k[0], dev), t_(v[0], dev), t_(q[0], dev), ctx, ws)
    torch.cuda.synchronize()
    opool.append(pt, k, v, ctx)
    assert_pool_equal(gpool, opool, "after the fused append")
    err = rel_err(out.cpu().numpy(), orc.attention_from_pool(opool, pt, q, [ctx + 1])[0])
    say(f"  decode_append rel err {err:.3e}")
    assert err <= TOL
