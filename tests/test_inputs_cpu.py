"""CPU checks of the seeded input generators that the GPU tests rely on."""
import numpy as np
import pytest

import oracle
from transformer_head_scaled_softmax_amd import synth


@pytest.mark.parametrize("scale", [0.125, 1.0, -0.5])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_planted_outliers_raise_the_row_maximum(scale, dtype):
    """plant_score_outliers does what the rescale tests need: rows that see the
    planted keys find, after the first 64-key tile, scores above that tile's
    maximum by more than the bf16 guard (64 in log2 units) at a 60-unit jump,
    and the two largest planted scores of a row stay within a few units."""
    inp = synth.core_inputs(2, 2, 300, 300, 64, 64, dtype, seed=5)
    synth.plant_score_outliers(inp["q"], inp["k"], [70, 150, 260], 60.0, scale, dtype, seed=6)
    s = oracle.scores(inp["q"], inp["k"], mask_kind=oracle.MASK_CAUSAL, scale=scale)
    rows = s[:, :, 280:, :]  # rows that see every planted slot
    first = rows[..., :64].max(axis=-1)
    assert np.mean((rows[..., 64:128].max(axis=-1) - first) / np.log(2.0) > 64.0) > 0.99
    top2 = np.sort(rows, axis=-1)[..., -2:]
    gap = top2[..., 1] - top2[..., 0]
    assert np.median(gap) < 3.0 and np.all(gap < 8.0)
    # rows above the first planted slot see only N(0,1)-like scores
    assert np.all(np.isfinite(s[:, :, :70, :70][np.isfinite(s[:, :, :70, :70])]))


def _rounded_projection_path(p, H, scale, dtype, cross):
    """The projection path with its projected Q, K, V and head outputs rounded
    to ``dtype`` (what the library stores), every other step the oracle's."""
    B, Nq, D = p["x_q"].shape
    xkv = p["x_kv"] if cross else p["x_q"]
    Nk = xkv.shape[1]

    def proj(x, W, n):
        y = synth.round_to((x.astype(np.float64) @ W.T.astype(np.float64)).astype(np.float32), dtype)
        return y.reshape(B, n, H, -1).transpose(0, 2, 1, 3)

    O = oracle.attention(proj(p["x_q"], p["W_Q"], Nq), proj(xkv, p["W_K"], Nk), proj(xkv, p["W_V"], Nk),
                         key_lens=p["key_lens"], scale=scale)
    O = synth.round_to(O.astype(np.float32), dtype).transpose(0, 2, 1, 3).reshape(B, Nq, -1)
    return O.astype(np.float64) @ p["W_O"].T.astype(np.float64)


@pytest.mark.parametrize("cross", [False, True])
def test_projection_rounding_budget(cross):
    """Rounding the projected Q, K, V to the input type costs about
    |scale| * |q| |k| * u in every score: at the pages' scale 1/8 it stays well
    inside the 2e-2 bound for bf16, at |scale| = 2 it does not (bf16) but does
    for f16 -- whatever the sign of the scale."""
    B, Nq, Nk, D, H = (8, 64, 80, 256, 4) if cross else (8, 64, 64, 256, 4)
    errs = {}
    for dtype in ("bf16", "f16"):
        p = synth.proj_inputs(B, Nq, Nk, D, H, 64, 64, dtype, seed=91 + cross, cross=cross, lens=(5, Nk))
        for scale in (0.125, -0.125, 2.0, -2.0):
            ref = oracle.mha_proj(p["x_q"], p["x_kv"], p["W_Q"], p["W_K"], p["W_V"], p["W_O"], H=H,
                                  key_lens=p["key_lens"], scale=scale)
            errs[dtype, scale] = np.abs(_rounded_projection_path(p, H, scale, dtype, cross) - ref).max()
    assert errs["bf16", 0.125] < 0.01 and errs["bf16", -0.125] < 0.01
    assert errs["bf16", 2.0] > 0.02 and errs["bf16", -2.0] > 0.02
    assert errs["f16", 2.0] < 0.015 and errs["f16", -2.0] < 0.015
