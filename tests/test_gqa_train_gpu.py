"""GPU parity of training with shared key/value heads (mha_forward_gqa,
mha_backward_gqa) against the fp64 oracle, through the C ABI.

The oracle repeats each key/value head over its H / H_kv query heads, runs
per-head attention and its gradients, and sums the gradients of the copies of a
shared head (oracle.attention_backward_gqa, pinned by finite differences).

Tolerances: lse and dq as for mha_backward (tests/test_bwd_gpu.py).  A shared
head's dk, dv is the sum of G = H / H_kv per-head gradients, each within the
per-head bound 2e-2 + 2u * A_h, so the sum is held to the sum of the bounds,
G * 2e-2 + 2u * sum_h A_h (fp32: 1e-5 of the largest reference value).
"""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import (ROUNDING_UNIT, TOL_LOWP_ABS, assert_close, assert_close_grad, attention_block, grad_bounds,
                      lens_dev,
                      to_dev, to_host)
from transformer_head_scaled_softmax_amd import _binding as mb, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mha = pytest.importorskip("transformer_head_scaled_softmax_amd")

CAUSAL, NONE = mha.MASK_CAUSAL, mha.MASK_NONE
LSE_TOL = {"bf16": 4e-3, "f16": 1e-3}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mha.load()
    yield
    torch.cuda.synchronize()


def gpu_train(inp, dtype, mask, block=None):
    """Forward (through the attention kernel of ``block`` queries per
    workgroup, or the library's choice for None), then backward."""
    q, k, v, dout = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "dout"))
    lens = lens_dev(inp["key_lens"])
    with attention_block(block):
        out, lse = mha.forward_lse(q, k, v, mask_kind=mask, key_lens=lens)
        plain = mha.forward(q, k, v, mask_kind=mask, key_lens=lens)
    dq, dk, dv = mha.backward(q, k, v, out, dout, lse, mask_kind=mask, key_lens=lens)
    torch.cuda.synchronize()
    assert torch.equal(out, plain), "forward with and without the row statistic differ"
    assert dk.shape == k.shape and dv.shape == v.shape
    return {"out": to_host(out), "lse": lse.cpu().numpy().astype(np.float64), "dq": to_host(dq),
            "dk": to_host(dk), "dv": to_host(dv)}


def check_gqa(B, H, Hkv, Nq, Nk, dtype, mask, lens, seed, lens_override=None, block=None):
    inp = synth.train_inputs(B, H, Nq, Nk, 64, 64, dtype, seed, lens, Hkv=Hkv)
    if lens_override is not None:
        inp["key_lens"] = np.asarray(lens_override, np.int32)
    what = f"B{B} H{H} Hkv{Hkv} Nq{Nq} Nk{Nk} {dtype} mask{mask} lens{inp['key_lens']} block{block}"
    got = gpu_train(inp, dtype, mask, block)
    kw = dict(mask_kind=mask, key_lens=inp["key_lens"])
    G = H // Hkv

    out_ref = oracle.attention_gqa(inp["q"], inp["k"], inp["v"], **kw)
    lse_ref = oracle.attention_lse_gqa(inp["q"], inp["k"], **kw)
    assert np.array_equal(np.isneginf(got["lse"]), np.isneginf(lse_ref)), what
    fin = ~np.isneginf(lse_ref)
    if dtype == "f32":
        assert_close(got["out"], out_ref, "f32", f"out {what}")
        assert np.all(np.abs(got["lse"][fin] - lse_ref[fin]) <= 1e-5 * np.maximum(1.0, np.abs(lse_ref[fin])))
    else:
        assert np.max(np.abs(got["out"] - out_ref), initial=0.0) <= TOL_LOWP_ABS, what
        assert np.max(np.abs(got["lse"][fin] - lse_ref[fin]), initial=0.0) <= LSE_TOL[dtype], what

    ref = oracle.attention_backward_gqa(inp["q"], inp["k"], inp["v"], inp["dout"], **kw)
    if dtype == "f32":
        for n, r in zip(("dq", "dk", "dv"), ref):
            assert_close(got[n], r, "f32", f"{n} {what}")
    else:
        kx = np.repeat(inp["k"].astype(np.float64), G, axis=1)
        vx = np.repeat(inp["v"].astype(np.float64), G, axis=1)
        out, P = oracle.attention(inp["q"], kx, vx, return_weights=True, **kw)
        A_dq, A_dk, A_dv = grad_bounds(inp["q"], kx, vx, inp["dout"], P, out, 1.0 / np.sqrt(64))
        assert_close_grad(got["dq"], ref[0], A_dq, dtype, f"dq {what}")
        for n, r, A in (("dk", ref[1], A_dk), ("dv", ref[2], A_dv)):
            A = A.reshape(B, Hkv, G, Nk, -1).sum(axis=2)
            bound = G * TOL_LOWP_ABS + 2.0 * ROUNDING_UNIT[dtype] * A
            ratio = float(np.max(np.abs(got[n] - r) / bound, initial=0.0))
            assert ratio <= 1.0, f"{n} {what}: error reaches {ratio:.3g} x the bound"
    if inp["key_lens"] is not None:
        for b, L in enumerate(np.clip(inp["key_lens"], 0, Nk)):
            assert not np.any(got["dk"][b, :, L:]) and not np.any(got["dv"][b, :, L:]), f"padded keys {what}"
    return got


@pytest.mark.parametrize("dtype,block", [("bf16", 32), ("bf16", 256), ("bf16", 512), ("f16", 32), ("f16", 256), ("f16", 512), ("f32", None)])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,mask,lens", [
    (2, 8, 2, 150, 150, CAUSAL, (20, 150)),  # groups of 4, several tiles, ragged tail, padding
    (2, 6, 1, 64, 200, NONE, (1, 200)),      # multi-query: one key/value head, cross-shaped
    (3, 4, 2, 37, 101, NONE, None),          # groups of 2, Nq < Nk
    (1, 6, 3, 300, 300, CAUSAL, None),       # long query blocks, groups of 2
    (2, 2, 1, 1, 1, NONE, None),             # one query, one key
])
def test_gqa_training_matches_oracle(dtype, block, B, H, Hkv, Nq, Nk, mask, lens):
    check_gqa(B, H, Hkv, Nq, Nk, dtype, mask, lens, seed=41, block=block)


def test_gqa_training_empty_sequences():
    # key length 0 (no visible key: zero output and gradients), 37, clamped 500 -> Nk
    got = check_gqa(3, 4, 1, 80, 80, "bf16", NONE, None, seed=42, lens_override=[0, 37, 500])
    for n in ("out", "dq", "dk", "dv"):
        assert not np.any(got[n][0]), n
    assert np.all(np.isneginf(got["lse"][0]))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def test_gqa_with_one_head_per_group_is_mha_backward():
    """H_kv == H through the shared-head entry points gives the per-head entry
    points' results bit for bit."""
    inp = synth.train_inputs(2, 4, 150, 150, 64, 64, "bf16", 43, (60, 150))
    q, k, v, dout = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "dout"))
    lens = lens_dev(inp["key_lens"])
    out, lse = mha.forward_lse(q, k, v, mask_kind=CAUSAL, key_lens=lens)
    dq, dk, dv = mha.backward(q, k, v, out, dout, lse, mask_kind=CAUSAL, key_lens=lens)
    lib = mha.load()
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    ws = torch.empty(mha.backward_workspace_bytes(2, 4, 150, 150, 64, 64), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.mha_forward_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(out2), _ptr(lse2), 2, 4, 4, 150, 150, 64, 64, CAUSAL,
                             _ptr(lens), 0.125, mha.BF16, stream)
    assert st == mb.OK, lib.mha_last_error_message()
    st = lib.mha_backward_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(out2), _ptr(dout), _ptr(lse2), _ptr(dq2), _ptr(dk2),
                              _ptr(dv2), 2, 4, 4, 150, 150, 64, 64, CAUSAL, _ptr(lens), 0.125, mha.BF16, _ptr(ws),
                              ws.numel(), stream)
    assert st == mb.OK, lib.mha_last_error_message()
    torch.cuda.synchronize()
    for a, b in ((out, out2), (lse, lse2), (dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b)


def test_gqa_backward_is_deterministic():
    inp = synth.train_inputs(2, 8, 300, 300, 64, 64, "bf16", 44, (100, 300), Hkv=2)
    a = gpu_train(inp, "bf16", CAUSAL)
    b = gpu_train(inp, "bf16", CAUSAL)
    for n in ("dq", "dk", "dv", "lse"):
        assert np.array_equal(a[n], b[n]), n


def _r256(n):
    return (n + 255) // 256 * 256


def split_runs(B, H, Hkv, Nq, Nk):
    """Number of runs the dK/dV pass splits each head group into, read off the
    workspace size (D, then two fp32 [runs][B*Hkv][Nk][64] buffers)."""
    extra = mha.backward_workspace_bytes(B, H, Nq, Nk, 64, 64, mha.BF16, H_kv=Hkv) - _r256(B * H * Nq * 4)
    return 1 if extra == 0 else extra // (2 * B * Hkv * Nk * 64 * 4)


def check_sampled_groups(inp, got, Hkv, mask, dtype, picks):
    """Whole key/value-head groups (b, g) against the oracle element by element,
    and on every shared head sum_j dv_j = sum of dout over the group's rows (each
    weight row sums to 1) and sum_j dk_j = 0 up to the rounding of out in D (each
    dS row sums to 0)."""
    B, H, Nq, d = inp["q"].shape
    Nk = inp["k"].shape[2]
    G = H // Hkv
    for n in ("dq", "dk", "dv"):
        assert np.all(np.isfinite(got[n])), n
    if inp["key_lens"] is None:
        sdv = got["dv"].sum(axis=2)
        sdo = inp["dout"].astype(np.float64).reshape(B, Hkv, G, Nq, d).sum(axis=(2, 3))
        assert np.max(np.abs(sdv - sdo)) <= 0.05 * np.sqrt(G * Nq), np.max(np.abs(sdv - sdo))
        assert np.max(np.abs(got["dk"].sum(axis=2))) <= 0.05 * np.sqrt(G * Nk)
    scale = 1.0 / np.sqrt(d)
    for b, g in picks:
        lens = None if inp["key_lens"] is None else inp["key_lens"][b:b + 1]
        st = {"q": inp["q"][b:b + 1, g * G:(g + 1) * G], "dout": inp["dout"][b:b + 1, g * G:(g + 1) * G],
              "k": inp["k"][b:b + 1, g:g + 1], "v": inp["v"][b:b + 1, g:g + 1]}
        ref = oracle.attention_backward_gqa(st["q"], st["k"], st["v"], st["dout"], mask_kind=mask, key_lens=lens)
        A_dk = np.zeros((1, 1, Nk, d))
        A_dv = np.zeros((1, 1, Nk, d))
        for s in range(G):  # the weights for the bound, one slice at a time
            h = g * G + s
            sl = {n: st[n][:, s:s + 1] for n in ("q", "dout")}
            out, P = oracle.attention(sl["q"], st["k"], st["v"], mask_kind=mask, key_lens=lens, return_weights=True)
            A = grad_bounds(sl["q"], st["k"], st["v"], sl["dout"], P, out, scale)
            del P
            assert_close_grad(got["dq"][b:b + 1, h:h + 1], ref[0][:, s:s + 1], A[0], dtype, f"dq slice ({b},{h})")
            A_dk += A[1]
            A_dv += A[2]
        for n, r, A in (("dk", ref[1], A_dk), ("dv", ref[2], A_dv)):
            bound = G * TOL_LOWP_ABS + 2.0 * ROUNDING_UNIT[dtype] * A
            ratio = float(np.max(np.abs(got[n][b:b + 1, g:g + 1] - r) / bound))
            print(f"group ({b},{g}) {n} error/bound {ratio:.3f}", flush=True)
            assert ratio <= 1.0, f"{n} group ({b},{g}): {ratio:.3g} x the bound"


def test_long_causal_gqa_bwd_full_size():
    """The long-context grouped-query workload at full size (B=2, n=8192, 16 query
    heads over 4 key/value heads) in the launch configuration the benchmark times
    (each group's four query heads in runs of one): two whole groups against the
    oracle, and the exact sums on every shared head."""
    w = synth.WORKLOADS["long_causal_gqa_bwd"]
    assert split_runs(w.B, w.H, w.Hkv, w.Nq, w.Nk) == 4
    inp = synth.workload_inputs(w)
    got = gpu_train(inp, w.dtype, w.mask)
    check_sampled_groups(inp, got, w.Hkv, w.mask, w.dtype, ((0, 1), (1, 3)))


@pytest.mark.parametrize("B,H,Hkv,N,mask,lens,runs", [
    (32, 16, 8, 1024, CAUSAL, None, 1),        # enough key blocks: one run, sums in registers
    (32, 16, 8, 1024, NONE, (100, 1024), 1),   # the same, unmasked with key padding
    (32, 16, 4, 1024, CAUSAL, (500, 1024), 2), # runs of two query heads
    (4, 8, 2, 512, CAUSAL, (60, 512), 4),      # few key blocks: one run per query head
    (8, 12, 2, 320, NONE, None, 6),            # groups of six, ragged key blocks
])
def test_gqa_runs_match_oracle(B, H, Hkv, N, mask, lens, runs):
    """Both ways the dK/dV pass sums a shared head's gradients -- in registers over
    the whole group, or over runs of query heads added by a second kernel -- on
    sampled whole groups against the oracle."""
    assert split_runs(B, H, Hkv, N, N) == runs
    inp = synth.train_inputs(B, H, N, N, 64, 64, "bf16", 45, lens, Hkv=Hkv)
    got = gpu_train(inp, "bf16", mask)
    picks = ((0, 0), (B - 1, Hkv - 1), (B // 2, Hkv // 2))
    check_sampled_groups(inp, got, Hkv, mask, "bf16", picks)
    if lens is not None:
        for b, L in enumerate(np.clip(inp["key_lens"], 0, N)):
            assert not np.any(got["dk"][b, :, L:]) and not np.any(got["dv"][b, :, L:]), b


def test_gqa_training_step_graph_replays_match_eager():
    """Forward and backward with shared heads -- including the run-splitting dK/dV
    pass and its combining kernel -- captured in one HIP graph: every replay,
    with eager work and synchronisations in between, reproduces the eager
    results bit for bit."""
    B, H, Hkv, N = 2, 8, 2, 300
    assert split_runs(B, H, Hkv, N, N) > 1
    inp = synth.train_inputs(B, H, N, N, 64, 64, "bf16", 46, (100, N), Hkv=Hkv)
    q, k, v, dout = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "dout"))
    lens = lens_dev(inp["key_lens"])
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(mha.backward_workspace_bytes(B, H, N, N, 64, 64, H_kv=Hkv), dtype=torch.uint8, device="cuda")

    def run():
        mha.forward_lse(q, k, v, mask_kind=CAUSAL, key_lens=lens, out=out, lse=lse)
        mha.backward(q, k, v, out, dout, lse, mask_kind=CAUSAL, key_lens=lens, dq=dq, dk=dk, dv=dv, workspace=ws)

    run()
    torch.cuda.synchronize()
    want = [t.clone() for t in (out, lse, dq, dk, dv)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    for _ in range(4):
        for t in (out, lse, dq, dk, dv, ws):
            t.zero_()
        noise = torch.ones(1 << 20, device="cuda").cumsum(0)  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, w in zip((out, lse, dq, dk, dv), want):
            assert torch.equal(t, w)
        del noise


def test_gqa_one_sided_problems():
    """Shared heads with no queries (every shared key gets zero gradient) and with
    no keys (zero output, lse -inf, zero query gradient)."""
    B, H, Hkv = 2, 6, 2
    k = to_dev(synth.train_inputs(B, H, 4, 70, 64, 64, "bf16", 48, Hkv=Hkv)["k"], "bf16")
    q0 = torch.empty(B, H, 0, 64, device="cuda", dtype=torch.bfloat16)
    lse0 = torch.empty(B, H, 0, device="cuda", dtype=torch.float32)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(k, 7.0)
    mha.backward(q0, k, k, q0, q0, lse0, dk=dk, dv=dv)
    inp = synth.train_inputs(B, H, 45, 1, 64, 64, "bf16", 49, Hkv=Hkv)
    q, dout = to_dev(inp["q"], "bf16"), to_dev(inp["dout"], "bf16")
    k0 = torch.empty(B, Hkv, 0, 64, device="cuda", dtype=torch.bfloat16)
    out, lse = mha.forward_lse(q, k0, k0)
    dq = torch.full_like(q, 7.0)
    mha.backward(q, k0, k0, out, dout, lse, dq=dq)
    torch.cuda.synchronize()
    assert not torch.any(dk) and not torch.any(dv) and not torch.any(dq) and not torch.any(out)
    assert bool(torch.all(torch.isneginf(lse)))
