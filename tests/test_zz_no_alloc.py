"""mha_decode_forward_noalloc through the C ABI: the same results as
mha_decode_forward with a caller's workspace, bit for bit, on consecutive
calls that reuse the library's built-in scratch (the second call smaller than
the first, and a third back at the first's size), and within the suite's
tolerance of the fp64 oracle.
"""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, to_dev, to_host
from transformer_head_scaled_softmax_amd import _binding as mb
from transformer_head_scaled_softmax_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mha = pytest.importorskip("transformer_head_scaled_softmax_amd")

CODES = {"bf16": mb.BF16, "f16": mb.F16}


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return mha.load()


def _case(B, H, Hkv, Nq, S, lens, dtype, seed):
    inp = synth.decode_inputs(B, H, Hkv, Nq, S, 64, 64, dtype, seed, lens=lens)
    dev = {n: to_dev(inp[n], dtype) for n in ("q", "k_cache", "v_cache")}
    dev["lens"] = torch.from_numpy(inp["cache_lens"]).to("cuda")
    return inp, dev


def _call(lib, dev, B, H, Hkv, Nq, S, mask, dtype, noalloc):
    out = torch.full((B, H, Nq, 64), float("nan"), dtype=dev["q"].dtype, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    head = (dev["q"].data_ptr(), dev["k_cache"].data_ptr(), dev["v_cache"].data_ptr(), out.data_ptr(),
            B, H, Hkv, Nq, S, 64, 64, mask, dev["lens"].data_ptr(), ctypes.c_float(0.125), CODES[dtype])
    if noalloc:
        st = lib.mha_decode_forward_noalloc(*head, stream)
    else:
        need = lib.mha_decode_workspace_bytes(B, H, Hkv, Nq, S, 64, 64, CODES[dtype])
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        st = lib.mha_decode_forward(*head, ws.data_ptr(), need, stream)
    assert st == mb.OK, lib.mha_last_error_message().decode()
    torch.cuda.synchronize()
    return to_host(out)


# (B, H, H_kv, Nq, S, cache length range, mask): the long decoding workload's
# shape, then a smaller grouped-query step with two new tokens, then the
# first again (the array keeps the previous call's states).
CALLS = [
    (16, 16, 16, 1, 8192, (1024, 8192), mb.MASK_CAUSAL),
    (3, 8, 2, 2, 3000, (1, 3000), mb.MASK_CAUSAL),
    (16, 16, 16, 1, 8192, (1024, 8192), mb.MASK_CAUSAL),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_noalloc_matches_workspace_entry_point(lib, dtype):
    for n, (B, H, Hkv, Nq, S, lens, mask) in enumerate(CALLS):
        assert lib.mha_decode_split(B, H, Hkv, Nq, S, 64, 64, CODES[dtype]) > 1
        need = lib.mha_decode_workspace_bytes(B, H, Hkv, Nq, S, 64, 64, CODES[dtype])
        assert 0 < need <= 16 << 20
        inp, dev = _case(B, H, Hkv, Nq, S, lens, dtype, seed=40 + n)
        got = _call(lib, dev, B, H, Hkv, Nq, S, mask, dtype, noalloc=True)
        want = _call(lib, dev, B, H, Hkv, Nq, S, mask, dtype, noalloc=False)
        assert np.array_equal(got, want), f"call {n}: results differ from mha_decode_forward"
        ref = oracle.decode(inp["q"], inp["k_cache"], inp["v_cache"], mask_kind=mask,
                            cache_lens=inp["cache_lens"])
        assert_close(got, ref, dtype, f"noalloc call {n} {dtype}")
