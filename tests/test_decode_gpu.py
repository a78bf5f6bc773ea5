"""GPU parity of mha_decode_forward (one decoding step against a key/value
cache, with shared key/value heads) against the fp64 oracle's decode.

Every call goes through the C ABI.  Shapes cover the balanced decoding kernel
(caches cut between waves and merged, caches covered whole by one wave, waves
spanning many short caches, 32-slot blocks, 1..64 query rows per cache head)
and the attention-kernel path it hands larger row counts and fp32 to; cache
lengths cover 0, 1, block edges, clamping past S, and more new queries than
filled slots.  Tolerances are the suite's (gpu_util).
"""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, lens_dev, to_dev, to_host
from transformer_head_scaled_softmax_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mha = pytest.importorskip("transformer_head_scaled_softmax_amd")

CAUSAL, NONE = mha.MASK_CAUSAL, mha.MASK_NONE
CODES = {"bf16": 1, "f16": 2, "f32": 0}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mha.load()
    yield
    torch.cuda.synchronize()


def run_decode(inp, dtype, mask, lens="keep", scale=None, poison=False):
    lens = inp["cache_lens"] if isinstance(lens, str) else lens
    q = to_dev(inp["q"], dtype)
    k = to_dev(inp["k_cache"], dtype)
    v = to_dev(inp["v_cache"], dtype)
    if poison:  # unfilled slots hold NaN: the kernels must never read them
        S = k.shape[2]
        Ls = [S] * k.shape[0] if lens is None else [min(max(int(x), 0), S) for x in lens]
        for b, L in enumerate(Ls):
            k[b, :, L:] = float("nan")
            v[b, :, L:] = float("nan")
    out = mha.decode_forward(q, k, v, cache_lens=lens_dev(lens), mask_kind=mask, scale=scale)
    torch.cuda.synchronize()
    return to_host(out)


def ref_decode(inp, mask, lens="keep", scale=None):
    lens = inp["cache_lens"] if isinstance(lens, str) else lens
    return oracle.decode(inp["q"], inp["k_cache"], inp["v_cache"], mask_kind=mask, cache_lens=lens, scale=scale)


def check(B, H, Hkv, Nq, S, dtype, mask, lens, seed, scale=None, poison=True, expect_split=None):
    inp = synth.decode_inputs(B, H, Hkv, Nq, S, 64 if dtype != "f32" else 48, 64 if dtype != "f32" else 40,
                              dtype, seed)
    if lens is not None:
        lens = np.asarray(lens, np.int32)
    split = mha.decode_split(B, H, Hkv, Nq, S, inp["q"].shape[3], inp["v_cache"].shape[3], CODES[dtype])
    if expect_split is not None:
        assert (split > 0) == expect_split, split
    got = run_decode(inp, dtype, mask, lens, scale, poison)
    ref = ref_decode(inp, mask, lens, scale)
    return assert_close(got, ref, dtype, f"B{B} H{H}/{Hkv} Nq{Nq} S{S} {dtype} mask{mask} lens{lens} split{split}")


# ---------------------------------------------------------------------------
# Split decoding kernel.

EDGE_S = [1, 2, 31, 32, 33, 127, 128, 129, 255, 256, 257, 1000, 1024, 1025, 3000]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("S", EDGE_S)
def test_single_token_cache_edges(dtype, S):
    """One new token per sequence, full caches of every block/chunk edge size."""
    check(3, 4, 4, 1, S, dtype, CAUSAL, None, 10 + S, expect_split=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mask", [CAUSAL, NONE])
@pytest.mark.parametrize("H,Hkv,Nq", [(4, 4, 1), (8, 2, 1), (8, 2, 3), (8, 1, 4), (16, 1, 4), (3, 1, 11),
                                      (6, 3, 5), (4, 4, 16), (2, 1, 32)])
def test_ragged_caches_and_head_groups(dtype, mask, H, Hkv, Nq):
    """Ragged fills (empty, one slot, fewer slots than new queries, block and
    chunk edges, past the capacity) with every grouping of query rows."""
    S = 1100
    lens = [0, 1, 2, Nq, 31, 32, 33, 256, 257, 1024, 1099, 1100, 5000]
    check(len(lens), H, Hkv, Nq, S, dtype, mask, lens, 100 + H + 7 * Hkv + Nq, expect_split=True)


@pytest.mark.parametrize("Nq,lens", [
    (4, [255, 256, 257, 258, 259, 260]),  # chunk boundaries (256) inside the last 4 positions
    (3, [1, 2, 3, 4]),                    # queries whose position is negative
    (8, [0, 0, 0]),                       # empty caches
])
def test_causal_positions_near_edges(Nq, lens):
    check(len(lens), 8, 8, Nq, 4096, "bf16", CAUSAL, lens, 200 + Nq, expect_split=True)


def test_long_caches_cut_between_waves():
    """Few long caches: each is cut between many waves and merged."""
    assert mha.decode_split(2, 8, 8, 1, 16384, 64, 64, 1) > 1
    check(2, 8, 8, 1, 16384, "bf16", CAUSAL, [16384, 9000], 300, expect_split=True)


@pytest.mark.parametrize("B,S,Hkv,H,Nq", [(300, 20, 8, 8, 1), (1000, 40, 2, 8, 2), (70, 3, 1, 4, 3)])
def test_many_short_caches_per_wave(B, S, Hkv, H, Nq):
    """Many short caches: waves span several caches (whole and cut ones), and
    more than 64 batch entries exercise the lane-blocked prefix sums."""
    lens = synth.key_lengths(synth.generator(800 + B), B, 0, S + 2)
    check(B, H, Hkv, Nq, S, "bf16", CAUSAL, lens, 810 + B, expect_split=True)
    check(B, H, Hkv, Nq, S, "bf16", NONE, lens, 820 + B, expect_split=True)


def test_scale_variants():
    for scale in (0.0, -0.125, 1.0):
        check(3, 8, 2, 2, 700, "bf16", CAUSAL, [700, 350, 5], 310, scale=scale)


def test_no_cache_lens_means_full():
    check(2, 4, 2, 2, 513, "bf16", CAUSAL, None, 320)
    check(2, 4, 2, 2, 513, "bf16", NONE, None, 321)


# ---------------------------------------------------------------------------
# Attention-kernel path (more than 64 rows per cache head, and fp32).

@pytest.mark.parametrize("mask", [CAUSAL, NONE])
@pytest.mark.parametrize("H,Hkv,Nq", [(4, 4, 65), (8, 2, 40), (2, 1, 200)])
def test_many_rows_use_attention_kernels(mask, H, Hkv, Nq):
    lens = [0, 3, Nq - 1, Nq, 300, 512]
    check(len(lens), H, Hkv, Nq, 512, "bf16", mask, lens, 400 + Nq, expect_split=False)


@pytest.mark.parametrize("mask", [CAUSAL, NONE])
@pytest.mark.parametrize("H,Hkv,Nq", [(4, 4, 1), (6, 2, 3), (4, 1, 9)])
def test_f32(mask, H, Hkv, Nq):
    check(4, H, Hkv, Nq, 300, "f32", mask, [300, 1, 0, 77], 500 + Nq, expect_split=False)


# ---------------------------------------------------------------------------
# Properties.

def test_decode_equals_prefill_rows():
    """The last Nq rows of causal self-attention over a full sequence (the
    prefill path, mha_forward) equal decoding those rows against the whole
    sequence as the cache."""
    B, H, N, Nq = 2, 8, 300, 3
    inp = synth.core_inputs(B, H, N, N, 64, 64, "bf16", 600)
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    full = to_host(mha.forward(q, k, v, mask_kind=CAUSAL))
    dec = to_host(mha.decode_forward(q[:, :, N - Nq:].contiguous(), k, v, mask_kind=CAUSAL))
    torch.cuda.synchronize()
    assert np.max(np.abs(full[:, :, N - Nq:] - dec)) <= 2e-2
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], mask_kind=CAUSAL)[:, :, N - Nq:]
    assert_close(dec, ref, "bf16", "decode of the last rows")


def test_deterministic_and_timed_entry_agree():
    """Repeated calls are bit-identical, and the timed entry point computes the
    same result while its events time both kernels."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    events = []
    for _ in range(4):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        events.append(e.value)
    try:
        inp = synth.decode_inputs(4, 16, 4, 1, 5000, 64, 64, "bf16", 700, lens=(1, 5000))
        assert mha.decode_split(4, 16, 4, 1, 5000, 64, 64, 1) > 1
        q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k_cache", "v_cache"))
        lens = lens_dev(inp["cache_lens"])
        a = mha.decode_forward(q, k, v, cache_lens=lens)
        b = mha.decode_forward(q, k, v, cache_lens=lens)
        c = mha.decode_forward(q, k, v, cache_lens=lens, events=events)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(a, c)
        for i in (0, 2):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), events[i], events[i + 1]) == 0
            assert ms.value > 0.0
    finally:
        for e in events:
            hip.hipEventDestroy(e)


def test_full_size_workloads():
    for name in ("long_decode", "long_decode_gqa"):
        w = synth.WORKLOADS[name]
        inp = synth.workload_inputs(w)
        got = run_decode(inp, w.dtype, w.mask)
        ref = ref_decode(inp, w.mask)
        assert_close(got, ref, w.dtype, name)
