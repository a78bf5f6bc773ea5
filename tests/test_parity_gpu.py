"""GPU parity: libmha's kernels against the fp64 oracle on the same seeded inputs.

Every call goes through the C ABI (via the ctypes binding).  Element-by-element
comparisons use the suite tolerances of gpu_util (fp32: 1e-5 of the output
scale; bf16/f16: 2e-2 absolute); masking properties are checked bit-exactly.
"""
import math

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, attention_block, lens_dev, to_dev, to_host
from transformer_head_scaled_softmax_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mha = pytest.importorskip("transformer_head_scaled_softmax_amd")

CAUSAL, NONE = mha.MASK_CAUSAL, mha.MASK_NONE


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mha.load()
    yield
    torch.cuda.synchronize()


def run_core(inp, dtype, mask, scale=None, lens_override="keep", block=None):
    """mha.forward on the inputs; ``block`` (32, 256 or 512) forces the bf16/f16
    attention kernel of that many queries per workgroup, None takes the
    library's choice."""
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    lens = inp["key_lens"] if lens_override == "keep" else lens_override
    with attention_block(block):
        if block is not None and dtype != "f32":
            B, H, Nq = q.shape[:3]
            assert mha.load().mha_forward_block_queries(B, H, Nq, mask, mha._dtype_code(q)) == block
        out = mha.forward(q, k, v, mask_kind=mask, key_lens=lens_dev(lens), scale=scale)
        torch.cuda.synchronize()
    return to_host(out)


# The three bf16/f16 attention kernels (32, 256 and 512 queries per workgroup) for the
# low-precision types; fp32 has one kernel.
def with_blocks(dtypes):
    return [(d, b) for d in dtypes for b in ((None,) if d == "f32" else (32, 256, 512))]


def ref_core(inp, mask, scale=None, lens_override="keep"):
    lens = inp["key_lens"] if lens_override == "keep" else lens_override
    return oracle.attention(inp["q"], inp["k"], inp["v"], mask_kind=mask, key_lens=lens, scale=scale)


def check_core(B, H, Nq, Nk, d, dtype, mask, lens, seed, dv=None, scale=None, block=None):
    dv = d if dv is None else dv
    inp = synth.core_inputs(B, H, Nq, Nk, d, dv, dtype, seed)
    if lens is not None:
        inp["key_lens"] = np.asarray(lens, np.int32)
    got = run_core(inp, dtype, mask, scale, block=block)
    ref = ref_core(inp, mask, scale)
    return assert_close(got, ref, dtype,
                        f"B{B} H{H} Nq{Nq} Nk{Nk} d{d}/{dv} {dtype} mask{mask} lens{lens} block{block}")


# ---------------------------------------------------------------------------
# The workloads at full size.

def test_tiny_encoder_f32():
    w = synth.WORKLOADS["tiny_encoder_f32"]
    inp = synth.workload_inputs(w)
    assert_close(run_core(inp, "f32", w.mask), ref_core(inp, w.mask), "f32", w.name)


def test_base_decoder_causal_full():
    w = synth.WORKLOADS["base_decoder_causal"]
    inp = synth.workload_inputs(w)
    assert_close(run_core(inp, w.dtype, w.mask), ref_core(inp, w.mask), w.dtype, w.name)


@pytest.mark.parametrize("name,block", [("translation_decoder_causal", 32), ("mid_causal", 256)])
def test_mid_length_workloads_full(name, block):
    """The mid-length workloads in the launch configuration the benchmark times
    (one-wave workgroups at 100 tokens, 256-query workgroups at 256 tokens)."""
    w = synth.WORKLOADS[name]
    assert mha.load().mha_forward_block_queries(w.B, w.H, w.Nq, w.mask, mha.BF16) == block
    inp = synth.workload_inputs(w)
    assert_close(run_core(inp, w.dtype, w.mask), ref_core(inp, w.mask), w.dtype, w.name)


def _proj_dev(inp, dtype):
    return {n: to_dev(inp[n], dtype) for n in ("x_q", "x_kv", "W_Q", "W_K", "W_V", "W_O")}


def run_proj(inp, H, dtype, mask, biases=None, plan=None):
    """mha.proj_forward; ``plan`` (PLAN_FUSED / PLAN_UNFUSED) forces a kernel
    plan, None takes the library's."""
    d = _proj_dev(inp, dtype)
    b = {n: to_dev(x, dtype) for n, x in (biases or {}).items()}
    out = mha.proj_forward(d["x_q"], d["x_kv"], d["W_Q"], d["W_K"], d["W_V"], d["W_O"], H=H,
                           mask_kind=mask, key_lens=lens_dev(inp["key_lens"]), plan=plan, **b)
    torch.cuda.synchronize()
    return to_host(out)


def ref_proj(inp, H, mask, biases=None):
    return oracle.mha_proj(inp["x_q"], inp["x_kv"], inp["W_Q"], inp["W_K"], inp["W_V"], inp["W_O"],
                           H=H, mask_kind=mask, key_lens=inp["key_lens"], **(biases or {}))


def test_base_encoder_proj_full():
    """The benchmark's workload, in the launch configuration it times."""
    w = synth.WORKLOADS["base_encoder_proj"]
    inp = synth.workload_inputs(w)
    assert_close(run_proj(inp, w.H, w.dtype, w.mask), ref_proj(inp, w.H, w.mask), w.dtype, w.name)


def test_big_cross_proj_full():
    """The benchmark's big cross-attention workload, in the launch
    configuration it times (the three-kernel plan at this shape)."""
    w = synth.WORKLOADS["big_cross_proj"]
    assert mha.load().mha_proj_fused(w.B, w.Nq, w.Nk, w.D, 64, 64, 0) == 0
    inp = synth.workload_inputs(w)
    assert_close(run_proj(inp, w.H, w.dtype, w.mask), ref_proj(inp, w.H, w.mask), w.dtype, w.name)


def test_big_cross_proj_full_fused_plan():
    """The same workload forced through the fused projection+attention kernel,
    which takes these sizes although mha_proj_forward does not choose it."""
    w = synth.WORKLOADS["big_cross_proj"]
    inp = synth.workload_inputs(w)
    d = _proj_dev(inp, w.dtype)
    out = mha.proj_forward(d["x_q"], d["x_kv"], d["W_Q"], d["W_K"], d["W_V"], d["W_O"], H=w.H,
                           mask_kind=w.mask, key_lens=lens_dev(inp["key_lens"]), plan=mha.PLAN_FUSED)
    torch.cuda.synchronize()
    assert_close(to_host(out), ref_proj(inp, w.H, w.mask), w.dtype, w.name + " fused plan")


def test_long_causal_sampled_rows():
    """B=2, n=8192, h=16 causal: GPU output rows compared with the oracle one by one
    on tile-edge rows plus seeded random rows of every (b, h)."""
    w = synth.WORKLOADS["long_causal"]
    inp = synth.workload_inputs(w)
    got = run_core(inp, w.dtype, w.mask)
    rows = synth.sample_rows(w.B, w.H, w.Nq, seed=55)
    ref = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, mask_kind=w.mask)
    assert_close(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref, w.dtype, w.name)


# ---------------------------------------------------------------------------
# Shapes: tile edges, ragged tails, cross-attention, padding.

EDGE_N = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 80, 127, 128, 129, 200, 257]


@pytest.mark.parametrize("block", [32, 256, 512])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n", EDGE_N)
def test_causal_square_edges(dtype, n, block):
    g = synth.generator(1000 + n)
    lens = [n, int(g.integers(0, n + 1)), max(1, n // 3)]
    check_core(3, 2, n, n, 64, dtype, CAUSAL, lens, seed=n, block=block)


@pytest.mark.parametrize("block", [32, 256, 512])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 129), (7, 64), (64, 80), (65, 63), (130, 17),
                                   (33, 300), (17, 500), (64, 257), (200, 129), (128, 1)])
def test_cross_shapes(dtype, nq, nk, block):
    g = synth.generator(2000 + nq * 7 + nk)
    lens = [nk, int(g.integers(1, nk + 1)), 0]
    check_core(3, 2, nq, nk, 64, dtype, NONE, lens, seed=nq * 1000 + nk, block=block)


@pytest.mark.parametrize("nq,nk,dk,dv,mask", [
    (1, 1, 1, 1, NONE), (5, 9, 7, 3, NONE), (16, 16, 64, 64, CAUSAL), (65, 65, 100, 128, CAUSAL),
    (70, 130, 128, 64, NONE), (3, 200, 32, 96, NONE), (129, 129, 64, 64, CAUSAL)])
def test_f32_shapes(nq, nk, dk, dv, mask):
    g = synth.generator(3000 + nq + nk)
    lens = [nk, int(g.integers(0, nk + 1))]
    check_core(2, 3, nq, nk, dk, "f32", mask, lens, seed=nq + 17 * nk, dv=dv)


@pytest.mark.parametrize("block", [32, 256, 512])
def test_no_key_lens_and_single_head(block):
    check_core(1, 1, 100, 100, 64, "bf16", CAUSAL, None, seed=5, block=block)
    check_core(1, 1, 40, 90, 64, "bf16", NONE, None, seed=6, block=block)


def test_key_lens_out_of_range_are_clamped():
    inp = synth.core_inputs(3, 2, 20, 20, 64, 64, "bf16", seed=7)
    inp["key_lens"] = np.array([-5, 1000, 7], np.int32)
    got = run_core(inp, "bf16", NONE)
    assert np.all(got[0] == 0.0)
    assert_close(got, ref_core(inp, NONE), "bf16", "clamped lengths")


def test_scale_variants():
    for scale in (1.0, 0.0, -0.125, 0.37):
        inp = synth.core_inputs(2, 2, 70, 70, 64, 64, "bf16", seed=8)
        inp["key_lens"] = np.array([70, 33], np.int32)
        assert_close(run_core(inp, "bf16", CAUSAL, scale), ref_core(inp, CAUSAL, scale), "bf16",
                     f"scale {scale}")


def test_empty_key_set_gives_zeros():
    inp = synth.core_inputs(2, 2, 10, 0, 64, 64, "bf16", seed=9)
    assert np.all(run_core(inp, "bf16", NONE) == 0.0)
    inp = synth.core_inputs(2, 2, 10, 0, 64, 64, "f32", seed=9)
    assert np.all(run_core(inp, "f32", NONE) == 0.0)


# ---------------------------------------------------------------------------
# Masking is bit-exact.

@pytest.mark.parametrize("dtype,block", with_blocks(["bf16", "f32"]))
@pytest.mark.parametrize("nq,n,mask", [(64, 64, NONE), (64, 64, CAUSAL), (300, 300, NONE), (300, 300, CAUSAL),
                                       (40, 200, NONE)])
def test_padded_slots_never_reach_the_output(dtype, block, nq, n, mask):
    """Whatever sits in padded key/value rows j >= key_lens[b] -- huge finite values
    or NaN -- leaves every output bit unchanged."""
    inp = synth.core_inputs(3, 2, nq, n, 64, 64, dtype, seed=10 + n)
    inp["key_lens"] = np.array([n, n // 2 + 3, 1], np.int32)
    clean = run_core(inp, dtype, mask, block=block)
    big = 3.0e38
    for poison in (big, float("nan")):
        k, v = inp["k"].copy(), inp["v"].copy()
        for b, L in enumerate(inp["key_lens"]):
            k[b, :, L:] = poison
            v[b, :, L:] = -poison
        got = run_core(dict(inp, k=k, v=v), dtype, mask, block=block)
        assert np.array_equal(got, clean), f"poison {poison} changed the output"


@pytest.mark.parametrize("block", [32, 256, 512])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("nq,nk,mask,lens", [(65, 63, NONE, (63, 1, 40)), (100, 100, CAUSAL, (100, 37, 70)),
                                             (130, 200, NONE, (200, 150, 129))])
def test_stale_tile_memory_never_reaches_the_output(dtype, nq, nk, mask, lens, block):
    """A launch over all-NaN keys and values first leaves NaN in every compute
    unit's tile memory; a call whose last key tile is partial must still match
    the clean result bit for bit (rows past the key end read as zeros)."""
    import torch
    nan = torch.full((64, 16, 128, 64), float("nan"), dtype=torch.bfloat16 if dtype == "bf16" else torch.float16,
                     device="cuda")
    inp = synth.core_inputs(3, 2, nq, nk, 64, 64, dtype, seed=nq + nk)
    inp["key_lens"] = np.array(lens, np.int32)
    clean = run_core(inp, dtype, mask, block=block)
    with attention_block(block):  # the same kernel: every compute unit holds NaN tiles
        mha.forward(nan, nan, nan)
    got = run_core(inp, dtype, mask, block=block)
    assert np.array_equal(got, clean)
    assert_close(got, ref_core(inp, mask), dtype, f"stale-tile case Nq{nq} Nk{nk}")


@pytest.mark.parametrize("dtype,block", with_blocks(["bf16", "f32"]))
@pytest.mark.parametrize("n,cuts", [(300, (0, 31, 63, 64, 130, 298)), (64, (0, 17, 31, 32, 40, 62)),
                                    (50, (0, 31, 33, 48))])
def test_future_tokens_never_change_earlier_outputs(dtype, block, n, cuts):
    inp = synth.core_inputs(2, 2, n, n, 64, 64, dtype, seed=11)
    inp["key_lens"] = None
    base = run_core(inp, dtype, CAUSAL, block=block)
    g = synth.generator(12)
    for i0 in cuts:
        pert = {n_: inp[n_].copy() for n_ in ("q", "k", "v")}
        for t in pert.values():
            t[:, :, i0 + 1:] = synth.round_to(g.standard_normal(t[:, :, i0 + 1:].shape) * 30.0, dtype)
        got = run_core(dict(inp, **pert), dtype, CAUSAL, block=block)
        assert np.array_equal(got[:, :, :i0 + 1], base[:, :, :i0 + 1]), f"rows <= {i0} changed"


@pytest.mark.parametrize("dtype,block", with_blocks(["bf16", "f16", "f32"]))
def test_causal_first_row_is_first_value_row(dtype, block):
    inp = synth.core_inputs(2, 3, 150, 150, 64, 64, dtype, seed=13)
    inp["key_lens"] = np.array([150, 1], np.int32)
    got = run_core(inp, dtype, CAUSAL, block=block)
    assert np.array_equal(got[:, :, 0], inp["v"][:, :, 0].astype(np.float64))
    # with one visible key every row of the second sequence is V row 0
    assert np.array_equal(got[1], np.broadcast_to(inp["v"][1, :, :1], got[1].shape).astype(np.float64))


@pytest.mark.parametrize("dtype,block", with_blocks(["bf16", "f32"]))
def test_zero_queries_average_the_visible_values(dtype, block):
    n = 130
    inp = synth.core_inputs(2, 2, n, n, 64, 64, dtype, seed=14)
    inp["q"][:] = 0.0
    inp["key_lens"] = np.array([n, 45], np.int32)
    got = run_core(inp, dtype, CAUSAL, block=block)
    want = np.zeros_like(got)
    for b in range(2):
        for i in range(n):
            m = min(int(inp["key_lens"][b]), i + 1)
            want[b, :, i] = inp["v"][b, :, :m].astype(np.float64).mean(axis=1)
    tol = 1e-6 if dtype == "f32" else 8e-3  # bf16: rounding of the mean only
    assert np.max(np.abs(got - want)) <= tol


def test_deterministic():
    inp = synth.core_inputs(2, 4, 500, 500, 64, 64, "bf16", seed=15)
    a = run_core(inp, "bf16", CAUSAL)
    b = run_core(inp, "bf16", CAUSAL)
    assert np.array_equal(a, b)


def test_worked_example_on_the_gpu():
    """The pages' 3-token example (aicomputerinstitute.com, 'Worked example: attention
    weights and outputs by hand') through the GPU kernels: features zero-padded from
    2 to 64 leave every dot product unchanged, scale = 1/sqrt(2)."""
    import json
    import pathlib
    gold = json.loads((pathlib.Path(__file__).parent / "golden" / "worked_example.json").read_text())
    for case in gold["cases"]:
        x = np.zeros((1, 1, 3, 64), np.float32)
        x[0, 0, :, :2] = np.array(case["X"], np.float32)
        want = np.array([case["outputs"][t] for t in gold["tokens"] if t in case["outputs"]])
        idx = [i for i, t in enumerate(gold["tokens"]) if t in case["outputs"]]
        for dtype, tol in (("f32", 1e-6), ("bf16", 4e-3)):
            inp = {"q": x, "k": x, "v": x, "key_lens": None}
            got = run_core(inp, dtype, NONE, scale=case["scale"])
            assert np.max(np.abs(got[0, 0, idx, :2] - want)) <= tol, (case["name"], dtype)


# ---------------------------------------------------------------------------
# Projection path.

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,Nq,Nk,D,H,cross,mask", [
    (2, 5, 5, 64, 1, False, CAUSAL), (3, 17, 33, 128, 2, True, NONE), (2, 70, 70, 256, 4, False, NONE),
    (1, 130, 130, 192, 3, False, CAUSAL), (4, 64, 80, 1024, 16, True, NONE), (2, 9, 200, 200, 2, True, NONE)])
def test_proj_shapes_with_biases(dtype, B, Nq, Nk, D, H, cross, mask):
    inp = synth.proj_inputs(B, Nq, Nk, D, H, 64, 64, dtype, seed=B * 100 + Nq + D, cross=cross)
    g = synth.generator(D + Nq)
    inp["key_lens"] = g.integers(1, Nk + 1, size=B).astype(np.int32)
    biases = {n: synth.normal(g, (size,), dtype) * np.float32(0.5)
              for n, size in (("b_Q", H * 64), ("b_K", H * 64), ("b_V", H * 64), ("b_O", D))}
    biases = {n: synth.round_to(x, dtype) for n, x in biases.items()}
    got = run_proj(inp, H, dtype, mask, biases)
    ref = ref_proj(inp, H, mask, biases)
    assert_close(got, ref, dtype, f"proj B{B} Nq{Nq} Nk{Nk} D{D} H{H}")


@pytest.mark.parametrize("B,N,D,H", [
    (21, 130, 1000, 16),  # 528 tiles of 128 x 128 -> the 128 x 128 configuration; K tail 40
    (21, 130, 520, 8),    # 264 of 128 x 128, 528 of 128 x 64 -> the 128 x 64 one; K tail 8
    (3, 100, 200, 2),     # 48 of 128 x 64 -> the 64 x 64 one; K tail 8
])
def test_proj_gemm_tile_shapes(B, N, D, H):
    """Projection GEMMs large enough for the bigger tile shapes, with ragged row
    counts and a contraction that is not a multiple of 64 (cross-attention, so
    the projections run as separate GEMM launches)."""
    inp = synth.proj_inputs(B, N, N, D, H, 64, 64, "bf16", seed=B + N + D, cross=True, lens=(1, N))
    got = run_proj(inp, H, "bf16", NONE)
    ref = ref_proj(inp, H, NONE)
    assert_close(got, ref, "bf16", f"proj tiles B{B} N{N} D{D} H{H}")


def test_proj_worked_example_identity():
    """H = 1 with identity projections reproduces the printed example outputs."""
    import json
    import pathlib
    gold = json.loads((pathlib.Path(__file__).parent / "golden" / "worked_example.json").read_text())
    case = gold["cases"][0]
    D = 64
    x = np.zeros((1, 3, D), np.float32)
    x[0, :, :2] = np.array(case["X"], np.float32)
    eye = np.eye(D, dtype=np.float32)
    inp = {"x_q": x, "x_kv": None, "W_Q": eye, "W_K": eye, "W_V": eye, "W_O": eye, "key_lens": None}
    d = _proj_dev(inp, "bf16")
    out = mha.proj_forward(d["x_q"], None, d["W_Q"], d["W_K"], d["W_V"], d["W_O"], H=1,
                           scale=case["scale"])
    got = to_host(out)[0, :, :2]
    want = np.array([case["outputs"][t] for t in gold["tokens"]])
    assert np.max(np.abs(got - want)) <= 4e-3


# ---------------------------------------------------------------------------
# Fused Q/K/V projection + attention (D % 64 == 0; self-attention N <= 128,
# cross-attention Nq <= 64, Nk <= 128).

FUSED_CASES = [  # (B, Nq, Nk, D, H, cross, mask): every row padding, partial last groups
    (5, 1, 1, 64, 2, False, NONE), (5, 31, 31, 128, 2, False, CAUSAL), (3, 32, 32, 64, 3, False, NONE),
    (3, 33, 33, 192, 2, False, CAUSAL), (3, 64, 64, 256, 4, False, NONE), (1, 65, 65, 64, 1, False, CAUSAL),
    (2, 100, 100, 128, 2, False, NONE), (3, 128, 128, 64, 2, False, CAUSAL),
    (3, 1, 5, 64, 2, True, NONE), (5, 20, 40, 128, 2, True, NONE), (3, 32, 64, 64, 2, True, NONE),
    (3, 40, 70, 192, 3, True, NONE), (4, 64, 80, 256, 4, True, NONE), (1, 64, 96, 64, 1, True, NONE),
    (3, 50, 128, 128, 2, True, NONE), (2, 64, 64, 64, 2, True, CAUSAL),
    # grids on both sides of one round of 256 workgroups, where the kernel
    # switches between three and two pipeline stages: 128 x 2 = 256 (three),
    # 129 x 2 = 258 (two), and cross-attention over <= 32 keys with 257 (two)
    (256, 64, 64, 64, 2, False, NONE), (258, 64, 64, 64, 2, False, CAUSAL), (514, 8, 20, 64, 1, True, NONE)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,Nq,Nk,D,H,cross,mask", FUSED_CASES)
def test_fused_proj_attention(dtype, B, Nq, Nk, D, H, cross, mask):
    """The fused projection+attention kernel (forced: several of these batches
    are small enough that mha_proj_forward would take the three kernels)."""
    inp = synth.proj_inputs(B, Nq, Nk, D, H, 64, 64, dtype, seed=7 * B + Nq + Nk + D, cross=cross)
    g = synth.generator(31 * Nk + D)
    inp["key_lens"] = g.integers(0, Nk + 3, size=B).astype(np.int32)  # 0 and > Nk included
    biases = {n: synth.round_to(synth.normal(g, (size,), dtype) * np.float32(0.5), dtype)
              for n, size in (("b_Q", H * 64), ("b_K", H * 64), ("b_V", H * 64), ("b_O", D))}
    got = run_proj(inp, H, dtype, mask, biases, plan=mha.PLAN_FUSED)
    ref = ref_proj(inp, H, mask, biases)
    assert_close(got, ref, dtype, f"fused B{B} Nq{Nq} Nk{Nk} D{D} H{H} cross{cross}")


@pytest.mark.parametrize("Nq,Nk,cross,scale", [
    (17, 17, False, None), (64, 64, False, None), (40, 40, False, -0.3), (64, 64, False, 0.0),
    (100, 100, False, None), (33, 50, True, None), (64, 64, True, -0.5), (20, 120, True, None)])
def test_fused_matches_three_kernel_path(Nq, Nk, cross, scale):
    """Both plans round Q, K, V identically and, when every sequence's keys fit
    one 64-key tile, do the same arithmetic in the same order, so they agree bit
    for bit there; beyond that they agree to rounding."""
    B, D, H = 5, 128, 2
    lib = mha.load()
    inp = synth.proj_inputs(B, Nq, Nk, D, H, 64, 64, "bf16", seed=Nq + Nk, cross=cross, lens=(1, Nk))
    d = _proj_dev(inp, "bf16")
    lens = lens_dev(inp["key_lens"])
    w = (d["W_Q"], d["W_K"], d["W_V"], d["W_O"])
    mask = NONE if cross and Nq != Nk else CAUSAL
    runs = {p: mha.proj_forward(d["x_q"], d["x_kv"], *w, H=H, mask_kind=mask, key_lens=lens, scale=scale, plan=p)
            for p in (mha.PLAN_FUSED, mha.PLAN_UNFUSED)}
    torch.cuda.synchronize()
    fused, three = runs[mha.PLAN_FUSED], runs[mha.PLAN_UNFUSED]
    if Nk <= 64:
        assert torch.equal(fused, three)
    else:
        assert_close(to_host(fused), to_host(three), "bf16", f"fused vs three-kernel Nq{Nq} Nk{Nk}")


def test_fused_plan_rejected_when_unsupported():
    inp = synth.proj_inputs(2, 70, 70, 128, 2, 64, 64, "bf16", seed=3, cross=True)
    d = _proj_dev(inp, "bf16")
    with pytest.raises(mha.MhaError) as e:
        mha.proj_forward(d["x_q"], d["x_kv"], d["W_Q"], d["W_K"], d["W_V"], d["W_O"], H=2, plan=mha.PLAN_FUSED)
    assert e.value.status == -2  # MHA_ERR_UNSUPPORTED: 70 queries exceed the cross-attention tile


def test_graph_replays_match_eager():
    """Both entry points captured in one HIP graph: every replay, with eager work
    and synchronisations in between, reproduces the eager result bit for bit."""
    w = synth.WORKLOADS["base_encoder_proj"]
    inp = synth.workload_inputs(w)
    d = _proj_dev(inp, "bf16")
    lens = lens_dev(inp["key_lens"])
    core = synth.core_inputs(2, 2, 200, 200, 64, 64, "bf16", seed=21)
    q, k, v = (to_dev(core[n], "bf16") for n in ("q", "k", "v"))
    ws = torch.empty(mha.proj_workspace_bytes(w.B, w.Nq, w.Nk, w.D, w.H, 64, 64), dtype=torch.uint8,
                     device="cuda")
    out_p = torch.empty((w.B, w.Nq, w.D), dtype=torch.bfloat16, device="cuda")
    out_c = torch.empty((2, 2, 200, 64), dtype=torch.bfloat16, device="cuda")

    def run():
        mha.proj_forward(d["x_q"], None, d["W_Q"], d["W_K"], d["W_V"], d["W_O"], H=w.H,
                         key_lens=lens, out=out_p, workspace=ws)
        mha.forward(q, k, v, mask_kind=CAUSAL, out=out_c)

    run()
    torch.cuda.synchronize()
    want_p, want_c = out_p.clone(), out_c.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    for _ in range(4):
        out_p.zero_()
        out_c.zero_()
        run_eager_noise = torch.randn(1000, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_p, want_p)
        assert torch.equal(out_c, want_c)
        del run_eager_noise


def test_longest_key_sequence_at_the_offset_limit():
    """The most keys one head may have (the kernels address one head with 32-bit
    byte offsets, including the tile read past its end: (Nk + 128) * 128 bytes
    < 2^31).  Cross-attention of 64 queries over 16,777,087 keys, a padded tail;
    sampled rows against the oracle."""
    Nk = (1 << 24) - 128 - 1
    lens = np.array([Nk - 5], np.int32)
    inp = synth.core_inputs(1, 1, 64, Nk, 64, 64, "bf16", seed=21)
    got = run_core(inp, "bf16", NONE, lens_override=lens)
    rows = np.array([(0, 0, 0), (0, 0, 31), (0, 0, 32), (0, 0, 63)], np.int32)
    ref = oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, mask_kind=NONE, key_lens=lens)
    assert_close(got[0, 0, rows[:, 2]], ref, "bf16", "Nk at the offset limit")


@pytest.mark.parametrize("dtype,mask,Nq,Nk,lens", [
    ("bf16", CAUSAL, 150, 150, (20, 150)),
    ("f16", NONE, 37, 101, (1, 101)),
    ("bf16", NONE, 300, 64, None),
    ("f32", CAUSAL, 70, 70, (5, 70)),
])
def test_strided_views_of_token_major_storage(dtype, mask, Nq, Nk, lens):
    """q, k, v and out stored token-major [B, N, H, d] (the layout of a projection's
    output) and passed as [B, H, N, d] views: the same result as the oracle on the
    logical tensors, and bit-identical to the dense call."""
    B, H = 2, 3
    inp = synth.core_inputs(B, H, Nq, Nk, 64, 64, dtype, seed=22, lens=lens)
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    qt, kt, vt = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    assert not qt.is_contiguous()
    out_store = torch.full((B, Nq, H, 64), 7.0, dtype=q.dtype, device="cuda")
    out = out_store.transpose(1, 2)
    kl = lens_dev(inp["key_lens"])
    mha.forward(qt, kt, vt, mask_kind=mask, key_lens=kl, out=out)
    dense = mha.forward(q, k, v, mask_kind=mask, key_lens=kl)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)
    assert_close(to_host(out), ref_core(inp, mask), dtype, f"strided {dtype} {Nq}x{Nk}")


def test_strided_broadcast_key_value_heads():
    """Zero head strides share one key/value head among all query heads (the
    multi-query arrangement): the oracle on the repeated tensors."""
    B, H, Nq, Nk = 2, 4, 96, 130
    inp = synth.core_inputs(B, 1, Nq, Nk, 64, 64, "bf16", seed=23, lens=(40, 130))
    q_full = synth.core_inputs(B, H, Nq, Nk, 64, 64, "bf16", seed=24)["q"]
    q = to_dev(q_full, "bf16")
    k1, v1 = to_dev(inp["k"], "bf16"), to_dev(inp["v"], "bf16")
    k = k1.expand(B, H, Nk, 64)
    v = v1.expand(B, H, Nk, 64)
    out, lse = mha.forward_lse(q, k, v, mask_kind=NONE, key_lens=lens_dev(inp["key_lens"]))
    torch.cuda.synchronize()
    k_rep = np.repeat(inp["k"], H, axis=1)
    v_rep = np.repeat(inp["v"], H, axis=1)
    ref = oracle.attention(q_full, k_rep, v_rep, mask_kind=NONE, key_lens=inp["key_lens"])
    assert_close(to_host(out), ref, "bf16", "broadcast key/value heads")
    ref_lse = oracle.attention_lse(q_full, k_rep, mask_kind=NONE, key_lens=inp["key_lens"])
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 4e-3
