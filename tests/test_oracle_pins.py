"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    fails = pin(orc)
    assert not fails, "\n".join(fails)


def test_dense_formula_cross_check(orc):
    """Not a pin (it re-types the formula): the loop oracle agrees with a dense numpy
    evaluation of softmax(q k^T * scale + mask) v to rounding."""
    g = np.random.Generator(np.random.PCG64(7))
    B, H, N, d = 2, 3, 33, 16
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    lens = np.array([33, 20], np.int32)
    out = orc.attention(q, k, v, mask_kind=oracle.MASK_CAUSAL, key_lens=lens)
    s = q @ np.swapaxes(k, -1, -2) / np.sqrt(d)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = (j <= i)[None, None] & (j[None, None] < lens[:, None, None, None])
    s = np.where(vis, s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    np.testing.assert_allclose(out, p @ v, atol=1e-12, rtol=0)


def test_attention_rows_match_full(orc):
    g = np.random.Generator(np.random.PCG64(8))
    B, H, N, d = 2, 2, 40, 8
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    lens = np.array([40, 17], np.int32)
    full = orc.attention(q, k, v, mask_kind=oracle.MASK_CAUSAL, key_lens=lens)
    rows = np.array([[0, 0, 0], [1, 1, 39], [1, 0, 16], [0, 1, 21]], np.int32)
    got = orc.attention_rows(q, k, v, rows, mask_kind=oracle.MASK_CAUSAL, key_lens=lens)
    want = np.stack([full[b, h, i] for b, h, i in rows])
    assert np.array_equal(got, want)
