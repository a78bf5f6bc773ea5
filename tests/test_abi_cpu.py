"""The C ABI without a GPU: the library loads, exports every symbol include/mha.h
declares, and rejects bad arguments on the host before any HIP call.

Pointers here are fake, aligned addresses that are never dereferenced: every call
below fails validation first.  Nothing in this file launches a kernel.
"""
import ctypes
import os
import pathlib
import re
import subprocess
import sys

import pytest

from transformer_head_scaled_softmax_amd import _binding as mb

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "mha.h"
P = 0x100000  # fake, 256-byte aligned device address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    # MHA_TEST_LIB: another build of the same ABI (the sanitized CPU build of
    # the host layer, tests/test_sanitize_cpu.py); default: libmha.so.
    return mb.load(os.environ.get("MHA_TEST_LIB") or None)


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(mha_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(mb.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", str(mb.LIB_PATH)], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert hasattr(lib, name)


def test_status_strings_and_version(lib):
    for code in (mb.OK, mb.ERR_INVALID_ARG, mb.ERR_UNSUPPORTED, mb.ERR_WORKSPACE, mb.ERR_HIP):
        assert lib.mha_status_string(code).decode()
    assert lib.mha_status_string(12345).decode() == "unknown status"
    assert lib.mha_version() >= 100


def fwd(lib, q=P, k=P, v=P, out=P, B=2, H=3, Nq=5, Nk=5, dk=64, dv=64, mask=0, lens=None,
        scale=0.125, dtype=mb.BF16):
    return lib.mha_forward(q, k, v, out, B, H, Nq, Nk, dk, dv, mask, lens, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), mb.ERR_INVALID_ARG),
    (dict(H=-2), mb.ERR_INVALID_ARG),
    (dict(Nq=-1), mb.ERR_INVALID_ARG),
    (dict(Nk=-1), mb.ERR_INVALID_ARG),
    (dict(dk=0), mb.ERR_INVALID_ARG),
    (dict(dv=-4), mb.ERR_INVALID_ARG),
    (dict(mask=2), mb.ERR_INVALID_ARG),
    (dict(mask=1, Nq=4, Nk=5), mb.ERR_INVALID_ARG),
    (dict(dtype=3), mb.ERR_INVALID_ARG),
    (dict(scale=float("nan")), mb.ERR_INVALID_ARG),
    (dict(scale=float("inf")), mb.ERR_INVALID_ARG),
    (dict(dk=32, dv=32), mb.ERR_UNSUPPORTED),
    (dict(dk=64, dv=128), mb.ERR_UNSUPPORTED),
    (dict(dtype=mb.F16, dk=128, dv=128), mb.ERR_UNSUPPORTED),
    (dict(dtype=mb.F32, dk=129), mb.ERR_UNSUPPORTED),
    (dict(q=None), mb.ERR_INVALID_ARG),
    (dict(out=None), mb.ERR_INVALID_ARG),
    (dict(k=None), mb.ERR_INVALID_ARG),
    (dict(v=None), mb.ERR_INVALID_ARG),
    (dict(q=P + 8), mb.ERR_INVALID_ARG),
    (dict(out=P + 2), mb.ERR_INVALID_ARG),
    (dict(dtype=mb.F32, q=P + 2), mb.ERR_INVALID_ARG),
    (dict(Nq=64, Nk=(1 << 24) - 128), mb.ERR_UNSUPPORTED),   # one key past the 32-bit offset limit
    (dict(lens=P + 2), mb.ERR_INVALID_ARG),
])
def test_forward_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert lib.mha_last_error_message().decode()
    # the earlier name is an alias of the same thread-local message
    assert lib.mha_last_error().decode() == lib.mha_last_error_message().decode()


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Nq=0), dict(B=0, q=None, out=None)])
def test_forward_empty_problems_are_ok_without_launch(lib, kw):
    assert fwd(lib, **kw) == mb.OK
    assert lib.mha_last_error_message().decode() == ""


def test_workspace_bytes(lib):
    # Q, K, V, O regions of B*N*H*d bf16 values, each rounded up to 256 bytes.
    assert lib.mha_proj_workspace_bytes(64, 64, 64, 512, 8, 64, 64, mb.BF16) == 4 * 64 * 64 * 512 * 2
    q = 32 * 64 * 1024 * 2
    kv = 32 * 80 * 1024 * 2
    assert lib.mha_proj_workspace_bytes(32, 64, 80, 1024, 16, 64, 64, mb.BF16) == 2 * q + 2 * kv
    # 3*64*2 = 384 -> 512; 5*64*2 = 640 -> 768 (twice); 384 -> 512
    assert lib.mha_proj_workspace_bytes(1, 3, 5, 8, 1, 64, 64, mb.BF16) == 512 + 768 + 768 + 512
    assert lib.mha_proj_workspace_bytes(-1, 3, 5, 8, 1, 64, 64, mb.BF16) == 0
    assert lib.mha_proj_workspace_bytes(1, 3, 5, 8, 0, 64, 64, mb.BF16) == 0
    assert lib.mha_proj_workspace_bytes(1, 3, 5, 8, 1, 64, 64, 9) == 0


def proj(lib, x_q=P, x_kv=P, W_Q=P, W_K=P, W_V=P, W_O=P, out=P, B=2, Nq=4, Nk=6, D=64, H=1,
         dk=64, dv=64, mask=0, lens=None, scale=0.125, dtype=mb.BF16, ws=P, ws_bytes=1 << 30,
         biases=(None, None, None, None)):
    return lib.mha_proj_forward(x_q, x_kv, W_Q, W_K, W_V, W_O, *biases, out, B, Nq, Nk, D, H, dk,
                                dv, mask, lens, scale, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), mb.ERR_INVALID_ARG),
    (dict(D=0), mb.ERR_INVALID_ARG),
    (dict(H=0), mb.ERR_INVALID_ARG),
    (dict(x_kv=None), mb.ERR_INVALID_ARG),              # self-attention needs Nk == Nq
    (dict(mask=1), mb.ERR_INVALID_ARG),                 # causal cross-attention
    (dict(mask=7), mb.ERR_INVALID_ARG),
    (dict(scale=float("nan")), mb.ERR_INVALID_ARG),
    (dict(dtype=mb.F32), mb.ERR_UNSUPPORTED),
    (dict(dk=32), mb.ERR_UNSUPPORTED),
    (dict(D=60), mb.ERR_UNSUPPORTED),
    (dict(x_q=None), mb.ERR_INVALID_ARG),
    (dict(W_O=None), mb.ERR_INVALID_ARG),
    (dict(out=None), mb.ERR_INVALID_ARG),
    (dict(W_K=P + 8), mb.ERR_INVALID_ARG),
    (dict(biases=(P + 1, None, None, None)), mb.ERR_INVALID_ARG),
    (dict(ws=None), mb.ERR_WORKSPACE),
    (dict(ws=P + 16), mb.ERR_WORKSPACE),
    (dict(ws_bytes=1000), mb.ERR_WORKSPACE),
])
def test_proj_rejects(lib, kw, status):
    assert proj(lib, **kw) == status
    assert lib.mha_last_error_message().decode()


def test_proj_workspace_exact_size_passes_validation_check(lib):
    need = lib.mha_proj_workspace_bytes(2, 4, 6, 64, 1, 64, 64, mb.BF16)
    assert proj(lib, ws_bytes=need - 1) == mb.ERR_WORKSPACE
    assert "needed" in lib.mha_last_error_message().decode()


def test_proj_empty_is_ok(lib):
    assert proj(lib, B=0) == mb.OK
    assert proj(lib, Nq=0, x_kv=P) == mb.OK


@pytest.mark.parametrize("args,fused", [
    ((64, 64, 64, 512, 64, 64, 1), 1),     # sentence-length self-attention
    ((64, 128, 128, 64, 64, 64, 1), 1),    # longest fused sequence
    ((3, 129, 129, 64, 64, 64, 1), 0),     # too long for one tile
    ((64, 64, 80, 512, 64, 64, 0), 1),     # sentence-length cross-attention
    ((32, 64, 80, 1024, 64, 64, 0), 0),    # d_model >= 768 over 65..96 keys: three kernels measured faster
    ((32, 64, 96, 768, 64, 64, 0), 0),
    ((64, 64, 80, 640, 64, 64, 0), 1),     # d_model below 768
    ((32, 64, 64, 1024, 64, 64, 0), 1),    # one key tile
    ((32, 64, 97, 1024, 64, 64, 0), 1),    # more than 96 keys
    ((32, 64, 64, 1024, 64, 64, 1), 1),    # self-attention at d_model 1024
    ((8, 64, 64, 512, 64, 64, 1), 0),      # small batch: 32 fused workgroups < D / 8
    ((16, 64, 64, 512, 64, 64, 1), 1),     # 64 fused workgroups
    ((8, 64, 64, 1024, 64, 64, 1), 0),     # 64 < 1024 / 8
    ((16, 64, 128, 512, 64, 64, 0), 0),    # cross-attention: 64 fused workgroups < 256
    ((32, 65, 80, 1024, 64, 64, 0), 0),    # cross-attention with more than 64 queries
    ((32, 64, 129, 1024, 64, 64, 0), 0),   # cross-attention with more than 128 keys
    ((2, 64, 64, 200, 64, 64, 1), 0),      # D not a multiple of 64
    ((2, 64, 64, 512, 32, 32, 1), 0),      # head size other than 64
    ((2, 64, 32, 512, 64, 64, 1), 0),      # Nq != Nk
])
def test_proj_fused_plan(lib, args, fused):
    assert lib.mha_proj_fused(*args) == fused


@pytest.mark.parametrize("args,block", [
    ((64, 8, 64, mb.MASK_CAUSAL, mb.BF16), 32),      # sentence length: one-wave workgroups
    ((64, 8, 128, mb.MASK_CAUSAL, mb.BF16), 32),     # u(256) = 0.5 < 0.7 under the causal mask
    ((64, 8, 128, mb.MASK_NONE, mb.BF16), 256),      # u(256) = 0.5 >= 0.45 without it
    ((128, 8, 192, mb.MASK_NONE, mb.F16), 256),      # u(256) = 0.75
    ((64, 16, 256, mb.MASK_CAUSAL, mb.BF16), 256),   # u(256) = 1
    ((32, 8, 256, mb.MASK_CAUSAL, mb.BF16), 32),     # 256 workgroups of 256 queries: half a round
    ((16, 16, 1024, mb.MASK_CAUSAL, mb.BF16), 256),  # below 4096 queries
    ((2, 8, 1024, mb.MASK_CAUSAL, mb.BF16), 32),     # few heads: one-wave workgroups fill the chip
    ((1, 4, 8192, mb.MASK_CAUSAL, mb.BF16), 256),    # beyond 2048 queries, 512-query blocks under-used
    ((2, 16, 8192, mb.MASK_CAUSAL, mb.BF16), 512),   # the long causal workload
    ((2, 16, 8192, mb.MASK_CAUSAL, mb.F32), 4),      # fp32: vector-ALU kernel
    ((0, 16, 8192, mb.MASK_CAUSAL, mb.BF16), 0),     # invalid sizes
    ((2, 16, 8192, 7, mb.BF16), 0),                  # unknown mask
    ((2, 16, 8192, mb.MASK_CAUSAL, 9), 0),           # unknown dtype
])
def test_forward_block_queries(lib, args, block, monkeypatch):
    monkeypatch.delenv("MHA_ATTENTION_BLOCK", raising=False)
    assert lib.mha_forward_block_queries(*args) == block


def test_forward_block_queries_override(lib, monkeypatch):
    """MHA_ATTENTION_BLOCK forces either bf16/f16 kernel, read on every call;
    other values leave the choice to the library."""
    args = (2, 16, 8192, mb.MASK_CAUSAL, mb.BF16)
    monkeypatch.setenv("MHA_ATTENTION_BLOCK", "32")
    assert lib.mha_forward_block_queries(*args) == 32
    monkeypatch.setenv("MHA_ATTENTION_BLOCK", "512")
    assert lib.mha_forward_block_queries(64, 8, 64, mb.MASK_NONE, mb.BF16) == 512
    monkeypatch.setenv("MHA_ATTENTION_BLOCK", "256")
    assert lib.mha_forward_block_queries(*args) == 256
    monkeypatch.setenv("MHA_ATTENTION_BLOCK", "64")
    assert lib.mha_forward_block_queries(*args) == 512
    assert lib.mha_forward_block_queries(2, 16, 8192, mb.MASK_CAUSAL, mb.F32) == 4


def test_proj_timed_rejects_unknown_plan(lib):
    import ctypes
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first
    args = [fake, None, fake, fake, fake, fake, None, None, None, None, fake, 2, 8, 8, 64, 1, 64, 64, 0, None,
            ctypes.c_float(0.125), 1, fake, 1 << 20, None, None]
    assert lib.mha_proj_forward_timed(*args, 3) == mb.ERR_INVALID_ARG
    assert lib.mha_proj_forward_timed(*args, -1) == mb.ERR_INVALID_ARG


def test_last_error_is_per_thread(lib):
    import threading
    assert fwd(lib, B=-1) == mb.ERR_INVALID_ARG
    seen = {}

    def other():
        seen["msg"] = lib.mha_last_error_message().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert lib.mha_last_error_message().decode()


_NO_DEVICE_SCRIPT = r"""
import ctypes, sys
hip = ctypes.CDLL("libamdhip64.so")
n = ctypes.c_int(0)
hip.hipGetDeviceCount(ctypes.byref(n))
if n.value != 0:
    print("SKIP device present"); sys.exit(0)
sys.path.insert(0, sys.argv[1])
from transformer_head_scaled_softmax_amd import _binding as mb
lib = mb.load()
P = 0x100000
st = lib.mha_forward(P, P, P, P, 1, 1, 4, 4, 64, 64, 0, None, 0.125, mb.BF16, None)
print("STATUS", st, lib.mha_last_error_message().decode())
"""


def test_valid_call_without_a_device_reports_hip_error():
    """With no GPU, a call that passes validation must return MHA_ERR_HIP rather than
    abort.  Runs in a child process that first confirms no device is visible (so no
    kernel can be launched with the fake pointers)."""
    res = subprocess.run([sys.executable, "-c", _NO_DEVICE_SCRIPT, str(ROOT)], capture_output=True,
                         text=True, timeout=120, env={"HIP_VISIBLE_DEVICES": "-1",
                                                      "PATH": "/usr/bin:/bin",
                                                      "LD_LIBRARY_PATH": "/opt/rocm/lib"})
    if "SKIP" in res.stdout:
        pytest.skip("a device is visible")
    assert res.returncode == 0, res.stderr
    assert f"STATUS {mb.ERR_HIP}" in res.stdout, res.stdout + res.stderr


# --------------------------------------------------------------------------
# Decoding against a key/value cache.

def dec(lib, q=P, k=P, v=P, out=P, B=2, H=4, Hkv=2, Nq=1, S=300, dk=64, dv=64, mask=1, lens=None,
        scale=0.125, dtype=mb.BF16, ws=P, ws_bytes=1 << 30):
    return lib.mha_decode_forward(q, k, v, out, B, H, Hkv, Nq, S, dk, dv, mask, lens, scale, dtype, ws,
                                  ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), mb.ERR_INVALID_ARG),
    (dict(Nq=-1), mb.ERR_INVALID_ARG),
    (dict(S=-1), mb.ERR_INVALID_ARG),
    (dict(H=0, Hkv=0), mb.ERR_INVALID_ARG),
    (dict(Hkv=0), mb.ERR_INVALID_ARG),
    (dict(Hkv=3), mb.ERR_INVALID_ARG),        # 4 query heads do not split over 3 cache heads
    (dict(Hkv=8), mb.ERR_INVALID_ARG),        # more cache heads than query heads
    (dict(dk=0), mb.ERR_INVALID_ARG),
    (dict(mask=2), mb.ERR_INVALID_ARG),
    (dict(dtype=5), mb.ERR_INVALID_ARG),
    (dict(scale=float("nan")), mb.ERR_INVALID_ARG),
    (dict(dk=128, dv=128), mb.ERR_UNSUPPORTED),
    (dict(dtype=mb.F32, dk=160), mb.ERR_UNSUPPORTED),
    (dict(S=1 << 24), mb.ERR_UNSUPPORTED),    # past 32-bit offsets within one cache head
    (dict(q=None), mb.ERR_INVALID_ARG),
    (dict(out=None), mb.ERR_INVALID_ARG),
    (dict(k=None), mb.ERR_INVALID_ARG),
    (dict(v=P + 8), mb.ERR_INVALID_ARG),
    (dict(lens=P + 1), mb.ERR_INVALID_ARG),
])
def test_decode_rejects(lib, kw, status):
    assert dec(lib, **kw) == status
    assert lib.mha_last_error_message().decode()


def test_decode_workspace_checked(lib):
    need = lib.mha_decode_workspace_bytes(2, 4, 2, 1, 300, 64, 64, mb.BF16)
    assert need > 0
    assert dec(lib, ws=None) == mb.ERR_WORKSPACE
    assert dec(lib, ws=P + 16) == mb.ERR_WORKSPACE
    assert dec(lib, ws_bytes=need - 1) == mb.ERR_WORKSPACE
    assert "needed" in lib.mha_last_error_message().decode()


@pytest.mark.parametrize("kw", [dict(B=0), dict(Nq=0), dict(B=0, q=None, out=None)])
def test_decode_empty_is_ok(lib, kw):
    assert dec(lib, **kw) == mb.OK
    assert lib.mha_last_error_message().decode() == ""


@pytest.mark.parametrize("args,waves", [
    ((16, 16, 16, 1, 8192, 64, 64, mb.BF16), 768),    # three waves on each of the 256 CUs
    ((64, 8, 8, 1, 100, 64, 64, mb.BF16), 768),
    ((1, 8, 1, 4, 4096, 64, 64, mb.F16), 768),       # multi-query, 32 rows
    ((2, 64, 1, 1, 1000, 64, 64, mb.BF16), 768),     # 64 rows share the single cache head
    ((2, 64, 1, 2, 1000, 64, 64, mb.BF16), 0),        # 128 rows: attention kernels
    ((2, 8, 8, 1, 1000, 64, 64, mb.F32), 0),          # fp32: attention kernels
    ((2, 8, 8, 1, 0, 64, 64, mb.BF16), 768),         # empty caches
    ((2, 8, 3, 1, 100, 64, 64, mb.BF16), 0),          # invalid head split
])
def test_decode_split_plan(lib, args, waves):
    assert lib.mha_decode_split(*args) == waves


def _r256(n):
    return (n + 255) // 256 * 256


def test_decode_workspace_bytes(lib):
    # one partial state (68 fp32) per (cache + wave) and row, then an int2 span per cache
    assert lib.mha_decode_workspace_bytes(16, 16, 16, 1, 8192, 64, 64, mb.BF16) == \
        _r256((256 + 768) * 1 * 68 * 4) + _r256(256 * 8)
    assert lib.mha_decode_workspace_bytes(1, 8, 1, 4, 4096, 64, 64, mb.F16) == \
        _r256((1 + 768) * 32 * 68 * 4) + _r256(8)
    assert lib.mha_decode_workspace_bytes(2, 64, 1, 1, 1000, 64, 64, mb.BF16) == \
        _r256((2 + 768) * 64 * 68 * 4) + _r256(16)
    assert lib.mha_decode_workspace_bytes(2, 8, 8, 1, 1000, 64, 64, mb.F32) == 0
    assert lib.mha_decode_workspace_bytes(2, 8, 3, 1, 1000, 64, 64, mb.BF16) == 0
    assert lib.mha_decode_workspace_bytes(2, 8, 8, 1, 1000, 64, 64, 9) == 0


# --------------------------------------------------------------------------
# The sublayer with its residual connection and layer normalisation.

def proj_ln(lib, x_q=P, x_kv=P, W=(P, P, P, P), biases=(None, None, None, None), gamma=None, beta=None,
            eps=1e-5, out=P, B=2, Nq=4, Nk=6, D=64, H=1, dk=64, dv=64, mask=0, lens=None, scale=0.125,
            dtype=mb.BF16, ws=P, ws_bytes=1 << 30):
    return lib.mha_proj_ln_forward(x_q, x_kv, *W, *biases, gamma, beta, eps, out, B, Nq, Nk, D, H, dk, dv,
                                   mask, lens, scale, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(eps=float("nan")), mb.ERR_INVALID_ARG),
    (dict(eps=-1e-5), mb.ERR_INVALID_ARG),
    (dict(eps=float("inf")), mb.ERR_INVALID_ARG),
    (dict(gamma=P + 8), mb.ERR_INVALID_ARG),
    (dict(beta=P + 2), mb.ERR_INVALID_ARG),
    (dict(biases=(None, None, None, P + 4)), mb.ERR_INVALID_ARG),   # b_O needs 8-byte alignment here
    (dict(dtype=mb.F32), mb.ERR_UNSUPPORTED),
    (dict(x_q=None), mb.ERR_INVALID_ARG),
    (dict(ws=None), mb.ERR_WORKSPACE),
    (dict(mask=1), mb.ERR_INVALID_ARG),
])
def test_proj_ln_rejects(lib, kw, status):
    assert proj_ln(lib, **kw) == status
    assert lib.mha_last_error_message().decode()


def test_proj_ln_empty_is_ok(lib):
    assert proj_ln(lib, B=0) == mb.OK
    assert proj_ln(lib, Nq=0) == mb.OK


def test_proj_ln_workspace_bytes(lib):
    base = lib.mha_proj_workspace_bytes(64, 64, 64, 512, 8, 64, 64, mb.BF16)
    # + per row 512/64 tiles of (sum, centred sum of squares) fp32
    assert lib.mha_proj_ln_workspace_bytes(64, 64, 64, 512, 8, 64, 64, mb.BF16) == base + 4096 * 8 * 8
    base = lib.mha_proj_workspace_bytes(3, 5, 7, 520, 1, 64, 64, mb.BF16)
    # 15 rows x 9 tiles x 8 B = 1080 -> 1280
    assert lib.mha_proj_ln_workspace_bytes(3, 5, 7, 520, 1, 64, 64, mb.BF16) == base + 1280
    assert lib.mha_proj_ln_workspace_bytes(3, 5, 7, 0, 1, 64, 64, mb.BF16) == 0


def test_proj_ln_workspace_checked(lib):
    need = lib.mha_proj_ln_workspace_bytes(2, 4, 6, 64, 1, 64, 64, mb.BF16)
    assert need > lib.mha_proj_workspace_bytes(2, 4, 6, 64, 1, 64, 64, mb.BF16)
    assert proj_ln(lib, ws_bytes=need - 1) == mb.ERR_WORKSPACE
    assert "needed" in lib.mha_last_error_message().decode()


# --------------------------------------------------------------------------
# Training: the forward row statistic and the backward pass.

def fwd_lse(lib, q=P, k=P, v=P, out=P, lse=P, B=2, H=3, Nq=5, Nk=5, dk=64, dv=64, mask=0, lens=None,
            scale=0.125, dtype=mb.BF16):
    return lib.mha_forward_lse(q, k, v, out, lse, B, H, Nq, Nk, dk, dv, mask, lens, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(lse=None), mb.ERR_INVALID_ARG),
    (dict(lse=P + 2), mb.ERR_INVALID_ARG),
    (dict(mask=1, Nq=4, Nk=5), mb.ERR_INVALID_ARG),
    (dict(dk=32, dv=32), mb.ERR_UNSUPPORTED),
    (dict(q=None), mb.ERR_INVALID_ARG),
])
def test_forward_lse_rejects(lib, kw, status):
    assert fwd_lse(lib, **kw) == status
    assert lib.mha_last_error_message().decode()


def test_forward_lse_empty_is_ok(lib):
    assert fwd_lse(lib, Nq=0, lse=None) == mb.OK
    assert fwd_lse(lib, B=0, lse=None) == mb.OK


def bwd(lib, q=P, k=P, v=P, out=P, dout=P, lse=P, dq=P, dk=P, dv=P, B=2, H=3, Nq=5, Nk=7, d_k=64, d_v=64,
        mask=0, lens=None, scale=0.125, dtype=mb.BF16, ws=P, ws_bytes=1 << 20):
    return lib.mha_backward(q, k, v, out, dout, lse, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, mask, lens, scale,
                            dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), mb.ERR_INVALID_ARG),
    (dict(Nk=-1), mb.ERR_INVALID_ARG),
    (dict(d_k=0), mb.ERR_INVALID_ARG),
    (dict(mask=2), mb.ERR_INVALID_ARG),
    (dict(mask=1), mb.ERR_INVALID_ARG),              # causal needs Nq == Nk
    (dict(dtype=7), mb.ERR_INVALID_ARG),
    (dict(scale=float("nan")), mb.ERR_INVALID_ARG),
    (dict(dtype=mb.F32, d_k=129), mb.ERR_UNSUPPORTED),
    (dict(dtype=mb.F32, q=P + 2), mb.ERR_INVALID_ARG),
    (dict(d_k=128, d_v=128), mb.ERR_UNSUPPORTED),
    (dict(d_v=32), mb.ERR_UNSUPPORTED),
    (dict(q=None), mb.ERR_INVALID_ARG),
    (dict(out=None), mb.ERR_INVALID_ARG),
    (dict(dout=None), mb.ERR_INVALID_ARG),
    (dict(lse=None), mb.ERR_INVALID_ARG),
    (dict(dq=None), mb.ERR_INVALID_ARG),
    (dict(k=None), mb.ERR_INVALID_ARG),
    (dict(v=None), mb.ERR_INVALID_ARG),
    (dict(dk=None), mb.ERR_INVALID_ARG),
    (dict(dv=None), mb.ERR_INVALID_ARG),
    (dict(dq=P + 8), mb.ERR_INVALID_ARG),
    (dict(dout=P + 2), mb.ERR_INVALID_ARG),
    (dict(lse=P + 2), mb.ERR_INVALID_ARG),
    (dict(lens=P + 2), mb.ERR_INVALID_ARG),
    (dict(ws=None), mb.ERR_WORKSPACE),
    (dict(ws=P + 16), mb.ERR_WORKSPACE),
    (dict(ws_bytes=255), mb.ERR_WORKSPACE),
    (dict(Nq=1 << 24, Nk=1 << 24, ws_bytes=1 << 40), mb.ERR_UNSUPPORTED),
])
def test_backward_rejects(lib, kw, status):
    assert bwd(lib, **kw) == status
    assert lib.mha_last_error_message().decode()


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Nq=0, Nk=0),
                                dict(B=0, q=None, k=None, v=None, out=None, dout=None, lse=None, dq=None,
                                     dk=None, dv=None, ws=None)])
def test_backward_empty_is_ok(lib, kw):
    assert bwd(lib, **kw) == mb.OK


_ONE_SIDED_SCRIPT = r"""
import ctypes, sys
hip = ctypes.CDLL("libamdhip64.so")
n = ctypes.c_int(0)
hip.hipGetDeviceCount(ctypes.byref(n))
if n.value != 0:
    print("SKIP device present"); sys.exit(0)
sys.path.insert(0, sys.argv[1])
from transformer_head_scaled_softmax_amd import _binding as mb
lib = mb.load()
P = 0x100000
# Nq == 0: no query-side tensor and no workspace (dk, dv are zeros).
st = lib.mha_backward(None, P, P, None, None, None, None, P, P, 2, 3, 0, 7, 64, 64, 0, None, 0.125, mb.BF16,
                      None, 0, None)
print("STATUS", st, lib.mha_last_error_message().decode())
# Nk == 0: no key-side tensor (dq is zeros).
st = lib.mha_backward(P, None, None, P, P, P, P, None, None, 2, 3, 5, 0, 64, 64, 0, None, 0.125, mb.BF16,
                      P, 1 << 20, None)
print("STATUS", st, lib.mha_last_error_message().decode())
"""


def test_backward_one_sided_problems_need_only_that_side():
    """Pointers of a side with zero rows may be NULL: such calls pass validation and
    fail only at the launch, for want of a device.  Runs in a child process that
    first confirms no device is visible (so nothing is launched with fake pointers)."""
    res = subprocess.run([sys.executable, "-c", _ONE_SIDED_SCRIPT, str(ROOT)], capture_output=True,
                         text=True, timeout=120, env={"HIP_VISIBLE_DEVICES": "-1",
                                                      "PATH": "/usr/bin:/bin",
                                                      "LD_LIBRARY_PATH": "/opt/rocm/lib"})
    if "SKIP" in res.stdout:
        pytest.skip("a device is visible")
    assert res.returncode == 0, res.stderr
    assert res.stdout.count(f"STATUS {mb.ERR_HIP}") == 2, res.stdout + res.stderr


def test_backward_workspace_bytes(lib):
    # D_i per row, fp32 [B, H, Nq], rounded up to 256 bytes
    assert lib.mha_backward_workspace_bytes(2, 16, 8192, 8192, 64, 64, mb.BF16) == 2 * 16 * 8192 * 4
    assert lib.mha_backward_workspace_bytes(3, 5, 7, 9, 64, 64, mb.F16) == _r256(3 * 5 * 7 * 4)
    assert lib.mha_backward_workspace_bytes(3, 5, 0, 9, 64, 64, mb.BF16) == 0
    assert lib.mha_backward_workspace_bytes(-1, 5, 7, 9, 64, 64, mb.BF16) == 0
    assert lib.mha_backward_workspace_bytes(3, 5, 7, 9, 64, 64, 9) == 0
    need = lib.mha_backward_workspace_bytes(2, 3, 5, 7, 64, 64, mb.BF16)
    assert bwd(lib, ws_bytes=need - 1) == mb.ERR_WORKSPACE
    assert "needed" in lib.mha_last_error_message().decode()


def fwd_strided(lib, qs=(3 * 5 * 64, 5 * 64, 64), ks=(3 * 5 * 64, 5 * 64, 64), vs=(3 * 5 * 64, 5 * 64, 64),
                os_=(3 * 5 * 64, 5 * 64, 64), q=P, k=P, v=P, out=P, lse=None, B=2, H=3, Nq=5, Nk=5, dk=64, dv=64,
                mask=0, dtype=mb.BF16):
    arr = [None if x is None else (ctypes.c_int64 * 3)(*x) for x in (qs, ks, vs, os_)]
    return lib.mha_forward_strided(q, arr[0], k, arr[1], v, arr[2], out, arr[3], lse, B, H, Nq, Nk, dk, dv, mask,
                                   None, 0.125, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qs=None), mb.ERR_INVALID_ARG),
    (dict(os_=None), mb.ERR_INVALID_ARG),
    (dict(ks=(-64, 64, 64)), mb.ERR_INVALID_ARG),
    (dict(qs=(960, 320, 68)), mb.ERR_INVALID_ARG),            # bf16 row stride not a multiple of 8
    (dict(os_=(960, 320, 32)), mb.ERR_INVALID_ARG),           # output rows overlap
    (dict(os_=(960, 0, 64)), mb.ERR_INVALID_ARG),             # output heads overlap
    (dict(ks=(0, 0, 1 << 24), Nk=3), mb.ERR_UNSUPPORTED),     # a head spans more than 2^31 bytes
    (dict(mask=1, Nk=6), mb.ERR_INVALID_ARG),
    (dict(dtype=mb.BF16, dk=32, dv=32), mb.ERR_UNSUPPORTED),
    (dict(lse=P + 2), mb.ERR_INVALID_ARG),                    # optional lse, misaligned
])
def test_forward_strided_rejects(lib, kw, status):
    assert fwd_strided(lib, **kw) == status
    assert lib.mha_last_error_message().decode()


def test_forward_strided_empty_is_ok(lib):
    assert fwd_strided(lib, Nq=0) == mb.OK
    assert fwd_strided(lib, B=0, q=None, out=None) == mb.OK


# --------------------------------------------------------------------------
# Shared key/value heads in training.

def fwd_gqa(lib, q=P, k=P, v=P, out=P, lse=None, B=2, H=4, Hkv=2, Nq=5, Nk=5, dk=64, dv=64, mask=0,
            dtype=mb.BF16):
    return lib.mha_forward_gqa(q, k, v, out, lse, B, H, Hkv, Nq, Nk, dk, dv, mask, None, 0.125, dtype, None)


def bwd_gqa(lib, B=2, H=4, Hkv=2, Nq=5, Nk=7, d_k=64, d_v=64, dtype=mb.BF16, ws=P, ws_bytes=1 << 20, **ptrs):
    p = dict(q=P, k=P, v=P, out=P, dout=P, lse=P, dq=P, dk=P, dv=P)
    p.update(ptrs)
    return lib.mha_backward_gqa(*p.values(), B, H, Hkv, Nq, Nk, d_k, d_v, 0, None, 0.125, dtype, ws, ws_bytes,
                                None)


@pytest.mark.parametrize("Hkv", [0, -1, 3, 5])
def test_gqa_head_counts_checked(lib, Hkv):
    """H_kv must divide H (1 <= H_kv <= H)."""
    assert fwd_gqa(lib, Hkv=Hkv) == mb.ERR_INVALID_ARG
    assert "H_kv" in lib.mha_last_error_message().decode()
    assert bwd_gqa(lib, Hkv=Hkv) == mb.ERR_INVALID_ARG
    assert "H_kv" in lib.mha_last_error_message().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(lse=P + 2), mb.ERR_INVALID_ARG),
    (dict(dk=32, dv=32), mb.ERR_UNSUPPORTED),
    (dict(mask=1, Nk=6), mb.ERR_INVALID_ARG),
    (dict(k=None), mb.ERR_INVALID_ARG),
])
def test_forward_gqa_rejects(lib, kw, status):
    assert fwd_gqa(lib, **kw) == status
    assert lib.mha_last_error_message().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(dk=None), mb.ERR_INVALID_ARG),
    (dict(lse=None), mb.ERR_INVALID_ARG),
    (dict(d_k=32, d_v=32), mb.ERR_UNSUPPORTED),
    (dict(ws=None), mb.ERR_WORKSPACE),
    (dict(ws_bytes=255), mb.ERR_WORKSPACE),
])
def test_backward_gqa_rejects(lib, kw, status):
    assert bwd_gqa(lib, **kw) == status
    assert lib.mha_last_error_message().decode()


def test_gqa_empty_is_ok(lib):
    assert fwd_gqa(lib, Nq=0) == mb.OK
    assert fwd_gqa(lib, H=0, Hkv=0) == mb.OK
    assert bwd_gqa(lib, B=0) == mb.OK
    assert bwd_gqa(lib, H=0, Hkv=0) == mb.OK


def test_backward_gqa_workspace_bytes(lib):
    # D per row; plus, when the dK/dV pass splits each head group into runs,
    # two fp32 [runs][B*H_kv][Nk][64] buffers of the runs' sums.
    assert lib.mha_backward_gqa_workspace_bytes(32, 16, 8, 1024, 1024, 64, 64, mb.BF16) == 32 * 16 * 1024 * 4
    assert lib.mha_backward_gqa_workspace_bytes(32, 16, 4, 1024, 1024, 64, 64, mb.BF16) == (
        32 * 16 * 1024 * 4 + 2 * 2 * 32 * 4 * 1024 * 64 * 4)
    assert lib.mha_backward_gqa_workspace_bytes(2, 16, 4, 8192, 8192, 64, 64, mb.BF16) == (
        2 * 16 * 8192 * 4 + 2 * 4 * 2 * 4 * 8192 * 64 * 4)
    assert lib.mha_backward_gqa_workspace_bytes(2, 16, 16, 8192, 8192, 64, 64, mb.BF16) == \
        lib.mha_backward_workspace_bytes(2, 16, 8192, 8192, 64, 64, mb.BF16)
    # fp32 never splits; no queries: nothing to split
    assert lib.mha_backward_gqa_workspace_bytes(2, 16, 4, 8192, 8192, 64, 64, mb.F32) == 2 * 16 * 8192 * 4
    assert lib.mha_backward_gqa_workspace_bytes(2, 16, 4, 0, 8192, 64, 64, mb.BF16) == 0
    for Hkv in (0, 3, 17):
        assert lib.mha_backward_gqa_workspace_bytes(2, 16, Hkv, 64, 64, 64, 64, mb.BF16) == 0
    need = lib.mha_backward_gqa_workspace_bytes(2, 4, 2, 5, 7, 64, 64, mb.BF16)
    assert bwd_gqa(lib, ws_bytes=need - 1) == mb.ERR_WORKSPACE


def test_python_binding_checks_shared_head_shapes():
    """The binding rejects key/value head counts that do not divide the query
    heads, and mismatched k/v heads, before any device call."""
    torch = pytest.importorskip("torch")
    import transformer_head_scaled_softmax_amd as mha
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    k3 = torch.zeros(1, 3, 8, 64, dtype=torch.bfloat16)
    k2 = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    k1 = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    for fn in (mha.forward, mha.forward_lse):
        with pytest.raises(ValueError):
            fn(q, k3, k3)
        with pytest.raises(ValueError):
            fn(q, k2, k1)  # k and v must have the same heads
    lse = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError):
        mha.backward(q, k3, k3, q, q, lse)


def proj_gqa(lib, H=4, Hkv=2, ws_bytes=1 << 24, **kw):
    a = dict(B=2, Nq=4, Nk=6, D=64, d_k=64, d_v=64, mask=0, dtype=mb.BF16)
    a.update(kw)
    return lib.mha_proj_forward_gqa(P, P, P, P, P, P, None, None, None, None, P, a["B"], a["Nq"], a["Nk"], a["D"],
                                    H, Hkv, a["d_k"], a["d_v"], a["mask"], None, 0.125, a["dtype"], P, ws_bytes,
                                    None)


@pytest.mark.parametrize("Hkv", [0, -2, 3, 8])
def test_proj_gqa_head_counts_checked(lib, Hkv):
    assert proj_gqa(lib, Hkv=Hkv) == mb.ERR_INVALID_ARG
    assert "H_kv" in lib.mha_last_error_message().decode()
    assert lib.mha_proj_gqa_workspace_bytes(2, 4, 6, 64, 4, Hkv, 64, 64, mb.BF16) == 0


def test_proj_gqa_workspace(lib):
    # Q and O [B*Nq, H*64], K and V [B*Nk, H_kv*64], each rounded up to 256 bytes
    assert lib.mha_proj_gqa_workspace_bytes(64, 64, 64, 512, 8, 2, 64, 64, mb.BF16) == (
        2 * 64 * 64 * 8 * 64 * 2 + 2 * 64 * 64 * 2 * 64 * 2)
    need = lib.mha_proj_gqa_workspace_bytes(2, 4, 6, 64, 4, 2, 64, 64, mb.BF16)
    assert proj_gqa(lib, ws_bytes=need - 1) == mb.ERR_WORKSPACE
    assert proj_gqa(lib, d_k=32, d_v=32) == mb.ERR_UNSUPPORTED
    assert proj_gqa(lib, B=0) == mb.OK


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus above 1 exits with a message and status 2
    before touching a device."""
    res = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                         timeout=300, cwd=str(ROOT))
    assert res.returncode == 2, res.stderr
    assert "one GPU" in res.stdout


def test_backward_single_launch_rule(lib):
    """One launch for bf16/f16 problems of at most 64 queries and 64 keys with one
    key/value head per query head; two kernels otherwise."""
    assert lib.mha_backward_single_launch(64, 8, 8, 64, 64, 64, 64, mb.BF16) == 1
    assert lib.mha_backward_single_launch(2, 3, 3, 1, 64, 64, 64, mb.F16) == 1
    assert lib.mha_backward_single_launch(64, 8, 8, 65, 64, 64, 64, mb.BF16) == 0
    assert lib.mha_backward_single_launch(64, 8, 8, 64, 65, 64, 64, mb.BF16) == 0
    assert lib.mha_backward_single_launch(64, 8, 2, 64, 64, 64, 64, mb.BF16) == 0  # shared heads
    assert lib.mha_backward_single_launch(64, 8, 8, 0, 64, 64, 64, mb.BF16) == 0
    assert lib.mha_backward_single_launch(64, 8, 8, 64, 64, 64, 64, mb.F32) == 0
    # the non-square, padded gradient parity shapes run the single launch
    assert lib.mha_backward_single_launch(3, 2, 2, 37, 50, 64, 64, mb.BF16) == 1
    assert lib.mha_backward_single_launch(2, 2, 2, 50, 20, 64, 64, mb.F16) == 1


def test_decode_noalloc_rejects_steps_above_its_scratch(lib):
    """mha_decode_forward_noalloc takes its scratch from a 16 MiB array: a step
    whose decoding workspace is larger is refused before anything runs (no
    device needed), and the message names both sizes."""
    B, H, Hkv, Nq, S = 1000, 64, 1, 1, 1  # (1000 caches + 768 waves) x 64 rows x 272 B > 16 MiB
    need = lib.mha_decode_workspace_bytes(B, H, Hkv, Nq, S, 64, 64, mb.BF16)
    assert need > 16 << 20
    st = lib.mha_decode_forward_noalloc(P, P, P, P, B, H, Hkv, Nq, S, 64, 64, mb.MASK_CAUSAL, None, 0.125,
                                        mb.BF16, None)
    assert st == mb.ERR_UNSUPPORTED
    msg = lib.mha_last_error_message().decode()
    assert str(need) in msg and str(16 << 20) in msg
    # argument errors come first, as for mha_decode_forward
    assert lib.mha_decode_forward_noalloc(P, P, P, P, 2, 3, 2, 1, 8, 64, 64, 0, None, 0.125, mb.BF16,
                                          None) == mb.ERR_INVALID_ARG
