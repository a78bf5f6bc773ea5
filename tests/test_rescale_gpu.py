"""GPU parity of the streaming softmax when a row's maximum rises after its
first visible key tile, and with negative scales, against the fp64 oracle.

The kernels exponentiate each key tile against the row's current reference
maximum and only take a new reference -- rescaling the running sum and the
accumulators, then exponentiating the tile again -- when the partial sum
passes a guard (2^64 for bf16 weights, 2^15 for f16).  The bf16 kernel of
512-query workgroups first skips that guard after each row's first tile and
checks the pass at the end (row sums at most 2^100, accumulators finite),
redoing it with the guard otherwise; the inputs below take both outcomes.
N(0,1) data at the pages' scale never gets there after the first tile, so these inputs plant
keys whose scores jump far above everything before them in later tiles
(synth.plant_score_outliers): at 60 natural-log units (87 in log2) every
planted tile passes both guards; at 20 (29 in log2) f16 rows rescale while
bf16 rows keep the optimistic pass with weights up to ~2^29.  The planted
slots sit in the second, third and fifth key tile, so a row rescales up to
three times, and the last two planted keys carry nearly equal scores, so
the result mixes their values rather than selecting one.

Shapes run through both attention kernels (workgroups of 512 queries: eight
waves of 64 queries each; of 32: one wave, forced through
MHA_ATTENTION_BLOCK), causal and unmasked,
padded sequences (planted slots past a key length must not count), the
decoding kernel with caches cut between many waves (so the merging kernel
combines partial states whose references are far apart), and the fused
projection path.  Negative scales are checked in every kernel, since the
kernels fold the sign into q.  Tolerances are the suite's (gpu_util).
"""
import zlib

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, attention_block, lens_dev, to_dev, to_host
from transformer_head_scaled_softmax_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mha = pytest.importorskip("transformer_head_scaled_softmax_amd")

CAUSAL, NONE = mha.MASK_CAUSAL, mha.MASK_NONE
CODES = {"bf16": 1, "f16": 2}
SLOTS = (70, 150, 260)  # key tiles 1, 2 and 4 (the last one paired with slot 261)


def _seed(*parts) -> int:
    return zlib.crc32(repr(parts).encode()) % 1000


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mha.load()
    yield
    torch.cuda.synchronize()


def _attention_case(B, H, Nq, Nk, lens, dtype, scale, jump, seed):
    inp = synth.core_inputs(B, H, Nq, Nk, 64, 64, dtype, seed)
    synth.plant_score_outliers(inp["q"], inp["k"], [s for s in SLOTS if s + 1 < Nk], jump, scale, dtype,
                               seed + 1)
    inp["key_lens"] = None if lens is None else np.asarray(lens, np.int32)
    return inp


def _run_attention(inp, dtype, mask, scale, block):
    """mha.forward with the attention kernel of ``block`` (32, 256 or 512) queries
    per workgroup."""
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    with attention_block(block):
        B, H, Nq = q.shape[:3]
        assert mha.load().mha_forward_block_queries(B, H, Nq, mask, mha._dtype_code(q)) == block
        out = mha.forward(q, k, v, mask_kind=mask, key_lens=lens_dev(inp["key_lens"]), scale=scale)
        torch.cuda.synchronize()
    return to_host(out)


def _ref_attention(inp, mask, scale):
    return oracle.attention(inp["q"], inp["k"], inp["v"], mask_kind=mask, key_lens=inp["key_lens"], scale=scale)


ATTN_SHAPES = {
    # (B, H, Nq, Nk, key_lens, mask): several query sub-blocks per wave and
    # waves past the last query in the 512-query kernel
    "long_causal": (2, 2, 300, 300, [300, 157], CAUSAL),
    "long_cross": (2, 2, 200, 333, [333, 140], NONE),
    # few queries streaming several key tiles
    "short_cross": (3, 2, 40, 300, [300, 129, 262], NONE),
}


@pytest.mark.parametrize("block", [32, 256, 512])
@pytest.mark.parametrize("shape", sorted(ATTN_SHAPES))
@pytest.mark.parametrize("scale", [0.125, 1.0, -0.5])
@pytest.mark.parametrize("jump", [60.0, 20.0])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_attention_late_maximum(shape, scale, jump, dtype, block):
    B, H, Nq, Nk, lens, mask = ATTN_SHAPES[shape]
    inp = _attention_case(B, H, Nq, Nk, lens, dtype, scale, jump, seed=_seed(shape, dtype))
    got = _run_attention(inp, dtype, mask, scale, block)
    ref = _ref_attention(inp, mask, scale)
    # the planted keys decide most rows: the outputs must be far from the
    # unplanted mean and the last two planted values must both carry weight
    assert np.max(np.abs(ref)) > 0.5
    assert_close(got, ref, dtype, f"{shape} scale {scale} jump {jump} {dtype} block {block}")


@pytest.mark.parametrize("shape", ["long_causal", "long_cross"])
@pytest.mark.parametrize("scale", [0.125, -0.125])
def test_attention_bf16_large_weights_without_rescale(shape, scale):
    """bf16, more than 64 queries, at the pages' scale: a single planted key
    in the second tile (slot 70, paired with slot 71) raises a row's scaled
    score by t_i * 9 / 2 natural-log units, t_i = q_i . u mostly in [4, 12].
    Measured against each row's first-tile maximum, 13-20% of the rows get a
    weight above 2^64 (the guard of the streaming softmax) while every row
    sum stays below 2^90 (largest 2^89.2), so the bf16 kernel keeps its
    unguarded first pass of the 512-query kernel, with weights far above
    2^64, and must still match the oracle."""
    B, H, Nq, Nk, lens, mask = ATTN_SHAPES[shape]
    inp = synth.core_inputs(B, H, Nq, Nk, 64, 64, "bf16", _seed(shape, "wide"))
    synth.plant_score_outliers(inp["q"], inp["k"], [70], 9.0, scale, "bf16", _seed(shape, "wide") + 1)
    inp["key_lens"] = np.asarray(lens, np.int32)
    ref = _ref_attention(inp, mask, scale)
    # the planted key dominates: rows far from the unplanted mean
    assert np.max(np.abs(ref)) > 0.5
    assert_close(_run_attention(inp, "bf16", mask, scale, 512), ref, "bf16", f"{shape} scale {scale}")


@pytest.mark.parametrize("scale", [-0.5, -2.0])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(2, 3, 200, 200, CAUSAL), (3, 2, 50, 50, CAUSAL), (2, 2, 37, 150, NONE),
                                   (2, 2, 130, 70, NONE)])
@pytest.mark.parametrize("block", [32, 256, 512])
def test_attention_negative_scale(shape, scale, dtype, block):
    """N(0,1) data at negative scales: the row maximum of scale * q.k is its
    smallest q.k, which the kernels must take as the reference."""
    B, H, Nq, Nk, mask = shape
    inp = synth.core_inputs(B, H, Nq, Nk, 64, 64, dtype, seed=Nq * 7 + Nk)
    inp["key_lens"] = np.asarray([Nk] + [max(1, Nk // (b + 2)) for b in range(1, B)], np.int32)
    assert_close(_run_attention(inp, dtype, mask, scale, block), _ref_attention(inp, mask, scale), dtype,
                 f"{shape} scale {scale} {dtype} block {block}")


# ---------------------------------------------------------------------------
# Decoding: caches cut between waves, outliers inside one wave's piece and
# across pieces.

def _decode_case(B, H, Hkv, Nq, S, lens, dtype, scale, jump, seed, slots):
    inp = synth.decode_inputs(B, H, Hkv, Nq, S, 64, 64, dtype, seed)
    synth.plant_score_outliers(inp["q"], inp["k_cache"], slots, jump, scale, dtype, seed + 1)
    inp["cache_lens"] = None if lens is None else np.asarray(lens, np.int32)
    return inp


def _run_decode(inp, dtype, mask, scale):
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k_cache", "v_cache"))
    out = mha.decode_forward(q, k, v, cache_lens=lens_dev(inp["cache_lens"]), mask_kind=mask, scale=scale)
    torch.cuda.synchronize()
    return to_host(out)


DECODE_SHAPES = {
    # (B, H, Hkv, Nq, S, cache_lens, mask, planted slots): 4 x 2 caches of 16384
    # slots make 128 slots (four 32-slot blocks) per wave, so slot 40 rescales
    # inside a wave and the later slots sit in other waves' pieces
    "gqa_full": (4, 8, 2, 1, 16384, None, CAUSAL, (40, 500, 5000, 9000)),
    "gqa_ragged": (4, 8, 2, 1, 16384, [16384, 9001, 3000, 12000], CAUSAL, (40, 500, 5000, 9000)),
    "mha_two_new": (3, 4, 4, 2, 8192, [8192, 6000, 8100], CAUSAL, (33, 300, 4000, 6050)),
    "cross": (2, 4, 1, 3, 12000, [12000, 7777], NONE, (100, 2000, 7000, 7700)),
}


@pytest.mark.parametrize("shape", sorted(DECODE_SHAPES))
@pytest.mark.parametrize("scale", [0.125, -0.5])
@pytest.mark.parametrize("jump", [60.0, 20.0])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_late_maximum(shape, scale, jump, dtype):
    B, H, Hkv, Nq, S, lens, mask, slots = DECODE_SHAPES[shape]
    assert mha.decode_split(B, H, Hkv, Nq, S, 64, 64, CODES[dtype]) > 1
    inp = _decode_case(B, H, Hkv, Nq, S, lens, dtype, scale, jump, seed=_seed(shape, dtype),
                       slots=slots)
    got = _run_decode(inp, dtype, mask, scale)
    ref = oracle.decode(inp["q"], inp["k_cache"], inp["v_cache"], mask_kind=mask, cache_lens=inp["cache_lens"],
                        scale=scale)
    assert_close(got, ref, dtype, f"{shape} scale {scale} jump {jump} {dtype}")


@pytest.mark.parametrize("scale", [-0.5, -2.0])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_negative_scale(scale, dtype):
    inp = synth.decode_inputs(3, 8, 2, 2, 3000, 64, 64, dtype, seed=77)
    inp["cache_lens"] = np.asarray([3000, 1700, 45], np.int32)
    got = _run_decode(inp, dtype, CAUSAL, scale)
    ref = oracle.decode(inp["q"], inp["k_cache"], inp["v_cache"], mask_kind=CAUSAL, cache_lens=inp["cache_lens"],
                        scale=scale)
    assert_close(got, ref, dtype, f"decode scale {scale} {dtype}")


# ---------------------------------------------------------------------------
# Projection path (fused and unfused plans) at negative scales.

@pytest.mark.parametrize("dtype,scale", [("bf16", -0.125), ("f16", -0.5), ("f16", -2.0)])
@pytest.mark.parametrize("cross", [False, True])
def test_projection_negative_scale(scale, dtype, cross):
    """The projection path stores the projected Q and K in the input type, and
    that rounding moves every score by about |scale| * |q| |k| * u (u the
    type's unit roundoff), which the fp64 oracle does not do: the 2e-2 bound
    holds for bf16 at the pages' |scale| = 1/8 and for f16 up to |scale| = 2
    (tests/test_inputs_cpu.py measures this budget on the CPU), so bf16 is
    checked at -1/8 and f16 at larger negative scales."""
    B, Nq, Nk, D, H = (8, 64, 80, 256, 4) if cross else (8, 64, 64, 256, 4)
    p = synth.proj_inputs(B, Nq, Nk, D, H, 64, 64, dtype, seed=91 + cross, cross=cross, lens=(5, Nk))
    d = {n: to_dev(p[n], dtype) for n in ("x_q", "x_kv", "W_Q", "W_K", "W_V", "W_O")}
    out = mha.proj_forward(d["x_q"], d["x_kv"], d["W_Q"], d["W_K"], d["W_V"], d["W_O"], H=H,
                           key_lens=lens_dev(p["key_lens"]), scale=scale, plan=mha.PLAN_FUSED)
    torch.cuda.synchronize()
    ref = oracle.mha_proj(p["x_q"], p["x_kv"], p["W_Q"], p["W_K"], p["W_V"], p["W_O"], H=H,
                          key_lens=p["key_lens"], scale=scale)
    assert_close(to_host(out), ref, dtype, f"proj cross={cross} scale {scale} {dtype}")
