"""GPU parity of mha_proj_ln_forward -- the attention sublayer followed by the
residual connection and layer normalisation -- against the oracle's
oracle_mha_proj_ln, through the C ABI.  The residual and the row statistics run
in the output projection's epilogue (per tile), a second pass merges them and
normalises; every output tile configuration and both kernel plans of the
projection path are covered.  Tolerance: the suite's
bf16/f16 bound (gpu_util)."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close_scaled, lens_dev, to_dev, to_host
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


def _norm_params(D, seed, affine=True):
    if not affine:
        return None, None
    g = synth.generator(seed)
    gamma = synth.round_to(g.uniform(0.5, 1.5, size=D).astype(np.float32), "bf16")
    beta = synth.round_to((g.standard_normal(D) * 0.5).astype(np.float32), "bf16")
    return gamma, beta


def check(B, Nq, Nk, D, H, cross, mask, dtype="bf16", seed=1, biases=False, affine=True, eps=1e-5, plan=None,
          lens=(1, None), x_scale=1.0, b_O=None):
    """``x_scale`` multiplies the inputs x_q, x_kv (then rounded again);
    ``b_O`` = (mean, std) draws the output projection's bias N(mean, std^2)
    per feature, which moves every residual row by that much."""
    lo, hi = lens
    inp = synth.proj_inputs(B, Nq, Nk, D, H, 64, 64, dtype, seed, cross, (lo, hi or (Nk if cross else Nq)))
    if x_scale != 1.0:
        for n in ("x_q", "x_kv"):
            if inp[n] is not None:
                inp[n] = synth.round_to((inp[n] * x_scale).astype(np.float32), dtype)
    g = synth.generator(seed + 1000)
    bs = {}
    if biases:
        for n, size in (("b_Q", H * 64), ("b_K", H * 64), ("b_V", H * 64), ("b_O", D)):
            bs[n] = synth.round_to((g.standard_normal(size) * 0.1).astype(np.float32), dtype)
    if b_O is not None:
        bs["b_O"] = synth.round_to((b_O[0] + b_O[1] * g.standard_normal(D)).astype(np.float32), dtype)
    gamma, beta = _norm_params(D, seed + 2000, affine)
    d = {n: to_dev(inp[n], dtype) for n in ("x_q", "x_kv", "W_Q", "W_K", "W_V", "W_O")}
    out = mha.proj_ln_forward(d["x_q"], d["x_kv"], d["W_Q"], d["W_K"], d["W_V"], d["W_O"], H=H,
                              ln_gamma=to_dev(gamma, dtype), ln_beta=to_dev(beta, dtype), ln_eps=eps,
                              mask_kind=mask, key_lens=lens_dev(inp["key_lens"]), plan=plan,
                              **{n: to_dev(v, dtype) for n, v in bs.items()})
    torch.cuda.synchronize()
    ref = oracle.mha_proj_ln(inp["x_q"], inp["x_kv"], inp["W_Q"], inp["W_K"], inp["W_V"], inp["W_O"], H=H,
                             gamma=gamma, beta=beta, eps=eps, mask_kind=mask, key_lens=inp["key_lens"], **bs)
    return assert_close_scaled(to_host(out), ref, dtype,
                        f"B{B} Nq{Nq} Nk{Nk} D{D} H{H} cross{cross} mask{mask} {dtype} plan{plan}")


def test_base_encoder_layer_full_size():
    """The base encoder workload's sublayer with its norm (D = 512)."""
    w = synth.WORKLOADS["base_encoder_proj"]
    check(w.B, w.Nq, w.Nk, w.D, w.H, False, w.mask, seed=w.seed, lens=w.lens)


def test_big_cross_layer_full_size():
    """The big cross-attention workload's sublayer with its norm (D = 1024)."""
    w = synth.WORKLOADS["big_cross_proj"]
    check(w.B, w.Nq, w.Nk, w.D, w.H, True, w.mask, seed=w.seed, lens=w.lens)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,Nq,Nk,D,H,cross,mask", [
    (3, 17, 17, 64, 1, False, NONE),      # rows not a multiple of the 32-row tile
    (2, 40, 40, 256, 4, False, CAUSAL),
    (5, 31, 45, 512, 8, True, NONE),
    (2, 70, 70, 384, 6, False, NONE),     # D a multiple of 64 below the tile width
    (3, 9, 13, 520, 1, True, NONE),       # D % 64 != 0: a partial last column tile (unfused projections)
    (2, 33, 33, 768, 12, False, CAUSAL),
    (24, 64, 64, 2048, 32, False, NONE),  # 128 x 128 output tiles (>= 384 of them)
    (7, 40, 40, 1024, 16, False, NONE),   # 64 x 64 output tiles, bands of 64 rows
])
def test_shapes(dtype, B, Nq, Nk, D, H, cross, mask):
    if D % 64:
        H, D = 1, D  # one head of 64 features cannot fill D = 520; project 520 -> 64 -> 520
    check(B, Nq, Nk, D, H, cross, mask, dtype=dtype, seed=B * 100 + D, biases=True)


@pytest.mark.parametrize("plan", [mha.PLAN_UNFUSED, mha.PLAN_FUSED])
def test_both_projection_plans(plan):
    check(4, 64, 64, 512, 8, False, NONE, seed=77, biases=True, plan=plan)
    check(4, 64, 80, 512, 8, True, NONE, seed=78, biases=True, plan=plan)


def test_repeated_calls_reuse_the_workspace():
    """Calls in a row on one workspace, with different sizes, stay correct and
    bit-identical (nothing carries over in the workspace)."""
    w = synth.WORKLOADS["base_encoder_proj"]
    inp = synth.proj_inputs(8, 64, 64, 512, 8, 64, 64, "bf16", 5, False, (10, 64))
    gamma, beta = _norm_params(512, 6)
    d = {n: to_dev(inp[n], "bf16") for n in ("x_q", "W_Q", "W_K", "W_V", "W_O")}
    ws = torch.zeros(mha.load().mha_proj_ln_workspace_bytes(8, 64, 64, 512, 8, 64, 64, 1), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for n in (8, 3, 8, 8):
        o = mha.proj_ln_forward(d["x_q"][:n].contiguous(), None, d["W_Q"], d["W_K"], d["W_V"], d["W_O"], H=8,
                                ln_gamma=to_dev(gamma, "bf16"), ln_beta=to_dev(beta, "bf16"),
                                key_lens=lens_dev(inp["key_lens"][:n]), workspace=ws)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[0], outs[3])
    assert torch.equal(outs[1], outs[0][:3])
    ref = oracle.mha_proj_ln(inp["x_q"], None, inp["W_Q"], inp["W_K"], inp["W_V"], inp["W_O"], H=8, gamma=gamma,
                             beta=beta, key_lens=inp["key_lens"])
    assert_close_scaled(to_host(outs[3]), ref, "bf16", "fourth call")


def test_without_scale_and_shift_and_large_eps():
    check(3, 50, 50, 512, 8, False, NONE, seed=90, affine=False)
    check(3, 50, 50, 1024, 16, False, NONE, seed=91, affine=False, eps=0.25)
    check(3, 50, 50, 512, 8, False, CAUSAL, seed=92, eps=0.25)


@pytest.mark.parametrize("dtype,mean,std", [("bf16", 3e5, 1e5), ("bf16", -2e6, 4e5), ("f16", 2e4, 1e4)])
@pytest.mark.parametrize("D,H", [(512, 8), (1024, 16)])
def test_rows_of_large_spread(dtype, mean, std, D, H):
    """Residual rows that differ from their tile means by far more than fp16's
    largest value (bf16: ~1e5-1e6): the stored differences are scaled into
    fp16's range, so the rows still normalise to the oracle's values."""
    check(4, 64, 64, D, H, False, NONE, dtype=dtype, seed=D + int(std), b_O=(mean, std))


@pytest.mark.parametrize("x_scale", [1e-5, 1e-6])
def test_rows_of_tiny_spread(x_scale):
    """bf16 rows whose features differ by ~1e-5-1e-6 (below fp16's normal
    range), normalised with eps = 0 so the outputs are of unit size: the
    differences are scaled up into fp16's normal range before they are stored."""
    check(4, 64, 64, 512, 8, False, NONE, seed=31, x_scale=x_scale, eps=0.0)
    check(4, 64, 80, 512, 8, True, NONE, seed=32, x_scale=x_scale, eps=0.0, affine=False)
