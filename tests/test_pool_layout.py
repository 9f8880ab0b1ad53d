"""The test-side decoder (tests/pool_layout.py) against the header's offsets.

Each rearrangement is checked on random bytes against the offset formulas
of include/k8v4.h evaluated element by element, and each is a permutation
of the run's bytes (so unwritten sentinel bytes stay visible).
"""
import numpy as np
import pytest

import pool_layout as PL


def _rand(n, seed):
    return np.random.default_rng(seed).integers(0, 256, n, dtype=np.uint8)


@pytest.mark.parametrize("P,H,pages", [(16, 2, 3), (48, 1, 2), (256, 2, 1)])
def test_kcodes_formula(P, H, pages):
    n_hc = pages * H * P
    run = _rand(n_hc * 256, 1)
    plain = PL.kcodes_to_plain(run).reshape(n_hc, 256)
    hc = np.arange(n_hc)[:, None]
    d = np.arange(256)[None, :]
    pos = (hc // 16) * 4096 + (d // 64) * 1024 + (hc % 16) * 64 + d % 64
    assert np.array_equal(plain, run[pos])
    assert np.array_equal(np.sort(pos.ravel()), np.arange(run.size))


@pytest.mark.parametrize("P,H,pages", [(16, 2, 3), (48, 1, 2), (256, 2, 1)])
def test_q4_formula(P, H, pages):
    n_hc = pages * H * P
    run = _rand(n_hc * 144, 2)
    plain = PL.q4_to_plain(run, P).reshape(n_hc, 8, 18)
    pos = np.empty((n_hc, 8, 18), np.int64)
    for hc in range(n_hc):
        t, s = divmod(hc, P)
        for b in range(8):
            so = t * 144 * P + 128 * P + (s // 16) * 256 + b * 32 + (s % 16) * 2
            pos[hc, b, 0:2] = [so, so + 1]
            pos[hc, b, 2:] = t * 144 * P + s * 128 + b * 16 + np.arange(16)
    assert np.array_equal(plain, run[pos])
    assert np.array_equal(np.sort(pos.ravel()), np.arange(run.size))


@pytest.mark.parametrize("P,H,pages", [(16, 2, 2), (80, 1, 1)])
def test_f16_formulas(P, H, pages):
    n_hc = pages * H * P
    run = _rand(n_hc * 512, 3)
    hc = np.arange(n_hc)[:, None]
    d = np.arange(256)[None, :]
    c = hc % 16
    kpos = (hc // 16) * 8192 + (d // 32) * 1024 + ((d % 32) // 8) * 256 + c * 16 + (d % 8) * 2
    vpos = (hc // 16) * 8192 + ((d % 16) // 2) * 1024 + (c // 4) * 256 + (d // 16) * 16 + (d % 2) * 8 + (c % 4) * 2
    for fn, pos in ((PL.f16k_to_plain, kpos), (PL.f16v_to_plain, vpos)):
        plain = fn(run).reshape(n_hc, 256, 2)
        assert np.array_equal(plain[..., 0], run[pos]) and np.array_equal(plain[..., 1], run[pos + 1])
        assert np.array_equal(np.sort(pos.ravel()), np.arange(0, run.size, 2))
