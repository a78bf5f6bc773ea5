"""MI355X-native multi-head scaled dot-product attention (forward and backward).

Thin PyTorch-facing wrappers over libmha's C ABI (include/mha.h).  PyTorch only
provides device memory and the current HIP stream; the computation is the
library's HIP kernels.  Functions raise ``MhaError`` on a non-zero status and
``RuntimeError`` if the library is not built.

    forward(q, k, v, mask_kind=MASK_NONE, key_lens=None, scale=None)
        q [B,H,Nq,d_k], k [B,H,Nk,d_k], v [B,H,Nk,d_v] -> out [B,H,Nq,d_v]
    proj_forward(x_q, x_kv, W_Q, W_K, W_V, W_O, H, ...)
        x_q [B,Nq,D], x_kv [B,Nk,D] or None -> out [B,Nq,D]
    proj_ln_forward(x_q, x_kv, W_Q, W_K, W_V, W_O, H, ln_gamma=None, ln_beta=None, ln_eps=1e-5, ...)
        LayerNorm(x_q + proj_forward(...)) -> out [B,Nq,D]
    decode_forward(q, k_cache, v_cache, cache_lens=None, mask_kind=MASK_CAUSAL, ...)
        q [B,H,Nq,d_k], k_cache [B,H_kv,S,d_k], v_cache [B,H_kv,S,d_v] -> out [B,H,Nq,d_v]
    forward_lse(q, k, v, ...) -> (out, lse [B,H,Nq] fp32)
    backward(q, k, v, out, dout, lse, ...) -> (dq, dk, dv)
"""
from __future__ import annotations

import math

from ._binding import (BF16, EXPORTS, F16, F32, MASK_CAUSAL, MASK_NONE, PLAN_AUTO, PLAN_FUSED, PLAN_UNFUSED,
                       MhaError, check, load)

__all__ = ["forward", "forward_lse", "backward", "backward_workspace_bytes", "proj_forward", "proj_ln_forward", "proj_workspace_bytes", "decode_forward",
           "decode_workspace_bytes",
           "decode_split", "MASK_NONE", "MASK_CAUSAL", "PLAN_AUTO", "PLAN_UNFUSED", "PLAN_FUSED", "MhaError",
           "load", "EXPORTS"]


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _dev_ptr(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _lens_ptr(key_lens, B):
    import torch
    if key_lens is None:
        return None
    if key_lens.dtype != torch.int32 or key_lens.shape != (B,):
        raise ValueError(f"key_lens must be an int32 tensor of shape ({B},)")
    return _dev_ptr(key_lens, "key_lens")


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _strides(t, name):
    """(device pointer, ctypes int64[3] of the batch, head, row strides) of a
    [B, H, N, d] view whose last dimension is contiguous."""
    import ctypes
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.stride(3) != 1 and t.shape[3] > 1:
        raise ValueError(f"{name} must be contiguous in its last dimension")
    return t.data_ptr(), (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def forward(q, k, v, mask_kind: int = MASK_NONE, key_lens=None, scale: float | None = None,
            out=None, stream=None):
    """Attention per head; see mha_forward in include/mha.h.  Views with other
    strides (e.g. [B, N, H, d] storage transposed to [B, H, N, d]) go through
    mha_forward_strided without a copy; k, v with H_kv < H heads (shared
    key/value heads) through mha_forward_gqa."""
    import torch
    B, H, Nq, dk = q.shape
    Hkv, Nk, dv = k.shape[1], k.shape[2], v.shape[3]
    if k.shape != (B, Hkv, Nk, dk) or v.shape != (B, Hkv, Nk, dv) or Hkv < 1 or H % Hkv:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    if out is None:
        out = torch.empty((B, H, Nq, dv), dtype=q.dtype, device=q.device)
    lib = load()
    if Hkv != H:
        st = lib.mha_forward_gqa(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(out, "out"), None,
                                 B, H, Hkv, Nq, Nk, dk, dv, int(mask_kind), _lens_ptr(key_lens, B), float(scale),
                                 _dtype_code(q), _stream(stream))
        check(lib, st)
        return out
    if not all(t.is_contiguous() for t in (q, k, v, out)):
        return _forward_strided(lib, q, k, v, out, None, mask_kind, key_lens, scale, stream)
    st = lib.mha_forward(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(out, "out"),
                         B, H, Nq, Nk, dk, dv, int(mask_kind), _lens_ptr(key_lens, B), float(scale),
                         _dtype_code(q), _stream(stream))
    check(lib, st)
    return out


def _forward_strided(lib, q, k, v, out, lse, mask_kind, key_lens, scale, stream):
    B, H, Nq, dk = q.shape
    Nk, dv = k.shape[2], v.shape[3]
    (qp, qs), (kp, ks), (vp, vs), (op, os_) = (_strides(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"),
                                                                           (out, "out")))
    st = lib.mha_forward_strided(qp, qs, kp, ks, vp, vs, op, os_, _dev_ptr(lse, "lse"), B, H, Nq, Nk, dk, dv,
                                 int(mask_kind), _lens_ptr(key_lens, B), float(scale), _dtype_code(q),
                                 _stream(stream))
    check(lib, st)
    return out


def proj_workspace_bytes(B, Nq, Nk, D, H, d_k, d_v, dtype_code: int = BF16) -> int:
    return int(load().mha_proj_workspace_bytes(B, Nq, Nk, D, H, d_k, d_v, dtype_code))


def proj_forward(x_q, x_kv, W_Q, W_K, W_V, W_O, H: int, b_Q=None, b_K=None, b_V=None, b_O=None,
                 mask_kind: int = MASK_NONE, key_lens=None, scale: float | None = None, out=None,
                 workspace=None, stream=None, plan: int | None = None, H_kv: int | None = None):
    """Multi-head attention with projections; see mha_proj_forward in include/mha.h.

    Weights are [out_features, in_features] (nn.Linear layout).  ``plan``
    (PLAN_UNFUSED / PLAN_FUSED) forces a kernel plan through
    mha_proj_forward_timed; None lets the library choose.  ``H_kv``: key/value
    heads shared by groups of query heads (W_K, W_V with H_kv*d rows), through
    mha_proj_forward_gqa."""
    import torch
    B, Nq, D = x_q.shape
    Nk = Nq if x_kv is None else x_kv.shape[1]
    dk = W_Q.shape[0] // H
    dv = W_O.shape[1] // H
    gqa = H_kv is not None and H_kv != H
    if H_kv is None:
        H_kv = H
    if H_kv < 1 or H % H_kv or W_K.shape[0] != H_kv * dk or W_V.shape[0] != H_kv * dv:
        raise ValueError(f"W_K {tuple(W_K.shape)}, W_V {tuple(W_V.shape)} do not fit H = {H}, H_kv = {H_kv}")
    if gqa and plan is not None:
        raise ValueError("plan: shared key/value heads take mha_proj_forward's plan for the sizes")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    code = _dtype_code(x_q)
    if out is None:
        out = torch.empty((B, Nq, D), dtype=x_q.dtype, device=x_q.device)
    lib = load()
    need = int(lib.mha_proj_gqa_workspace_bytes(B, Nq, Nk, D, H, H_kv, dk, dv, code))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x_q.device)
    ptrs = [_dev_ptr(t, n) for t, n in ((x_q, "x_q"), (x_kv, "x_kv"), (W_Q, "W_Q"), (W_K, "W_K"),
                                        (W_V, "W_V"), (W_O, "W_O"), (b_Q, "b_Q"), (b_K, "b_K"),
                                        (b_V, "b_V"), (b_O, "b_O"), (out, "out"))]
    args = (*ptrs, B, Nq, Nk, D, H, dk, dv, int(mask_kind), _lens_ptr(key_lens, B), float(scale), code,
            _dev_ptr(workspace, "workspace"), workspace.numel(), _stream(stream))
    if gqa:
        st = lib.mha_proj_forward_gqa(*ptrs, B, Nq, Nk, D, H, H_kv, *args[16:])
    elif plan is None:
        st = lib.mha_proj_forward(*args)
    else:
        st = lib.mha_proj_forward_timed(*args, None, int(plan))
    check(lib, st)
    return out


def proj_ln_forward(x_q, x_kv, W_Q, W_K, W_V, W_O, H: int, b_Q=None, b_K=None, b_V=None, b_O=None,
                    ln_gamma=None, ln_beta=None, ln_eps: float = 1e-5, mask_kind: int = MASK_NONE,
                    key_lens=None, scale: float | None = None, out=None, workspace=None, stream=None,
                    plan: int | None = None):
    """The sublayer with its residual connection and layer normalisation,
    LayerNorm(x_q + proj_forward(...)); see mha_proj_ln_forward in include/mha.h."""
    import torch
    B, Nq, D = x_q.shape
    Nk = Nq if x_kv is None else x_kv.shape[1]
    dk = W_Q.shape[0] // H
    dv = W_V.shape[0] // H
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    code = _dtype_code(x_q)
    if out is None:
        out = torch.empty((B, Nq, D), dtype=x_q.dtype, device=x_q.device)
    lib = load()
    need = int(lib.mha_proj_ln_workspace_bytes(B, Nq, Nk, D, H, dk, dv, code))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x_q.device)
    ptrs = [_dev_ptr(t, n) for t, n in ((x_q, "x_q"), (x_kv, "x_kv"), (W_Q, "W_Q"), (W_K, "W_K"),
                                        (W_V, "W_V"), (W_O, "W_O"), (b_Q, "b_Q"), (b_K, "b_K"),
                                        (b_V, "b_V"), (b_O, "b_O"), (ln_gamma, "ln_gamma"),
                                        (ln_beta, "ln_beta"))]
    args = (*ptrs, float(ln_eps), _dev_ptr(out, "out"), B, Nq, Nk, D, H, dk, dv, int(mask_kind),
            _lens_ptr(key_lens, B), float(scale), code, _dev_ptr(workspace, "workspace"), workspace.numel(),
            _stream(stream))
    if plan is None:
        st = lib.mha_proj_ln_forward(*args)
    else:
        st = lib.mha_proj_ln_forward_timed(*args, None, int(plan))
    check(lib, st)
    return out


def decode_workspace_bytes(B, H, H_kv, Nq, S, d_k, d_v, dtype_code: int = BF16) -> int:
    return int(load().mha_decode_workspace_bytes(B, H, H_kv, Nq, S, d_k, d_v, dtype_code))


def decode_split(B, H, H_kv, Nq, S, d_k, d_v, dtype_code: int = BF16) -> int:
    """Chunks per cache of the split decoding kernel (0: attention kernels)."""
    return int(load().mha_decode_split(B, H, H_kv, Nq, S, d_k, d_v, dtype_code))


def decode_forward(q, k_cache, v_cache, cache_lens=None, mask_kind: int = MASK_CAUSAL,
                   scale: float | None = None, out=None, workspace=None, stream=None, events=None):
    """One decoding step against a key/value cache; see mha_decode_forward in
    include/mha.h.  ``events``: None, or 4 hipEvent_t handles (ints) for
    mha_decode_forward_timed."""
    import torch
    B, H, Nq, dk = q.shape
    Hkv, S = k_cache.shape[1], k_cache.shape[2]
    dv = v_cache.shape[3]
    if k_cache.shape != (B, Hkv, S, dk) or v_cache.shape != (B, Hkv, S, dv):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k_cache {tuple(k_cache.shape)}, "
                         f"v_cache {tuple(v_cache.shape)}")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q, k_cache, v_cache must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    code = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, Nq, dv), dtype=q.dtype, device=q.device)
    lib = load()
    need = int(lib.mha_decode_workspace_bytes(B, H, Hkv, Nq, S, dk, dv, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    args = (_dev_ptr(q, "q"), _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"), _dev_ptr(out, "out"),
            B, H, Hkv, Nq, S, dk, dv, int(mask_kind), _lens_ptr(cache_lens, B), float(scale), code,
            _dev_ptr(workspace, "workspace"), 0 if workspace is None else workspace.numel(), _stream(stream))
    if events is None:
        st = lib.mha_decode_forward(*args)
    else:
        import ctypes
        arr = (ctypes.c_void_p * 4)(*events)
        st = lib.mha_decode_forward_timed(*args, arr)
    check(lib, st)
    return out


def forward_lse(q, k, v, mask_kind: int = MASK_NONE, key_lens=None, scale: float | None = None,
                out=None, lse=None, stream=None):
    """Attention per head plus the row statistic lse [B,H,Nq] (fp32) the backward
    pass needs; see mha_forward_lse in include/mha.h.  k, v may carry fewer
    heads H_kv dividing H (shared key/value heads, mha_forward_gqa).  Returns
    (out, lse)."""
    import torch
    B, H, Nq, dk = q.shape
    Hkv, Nk, dv = k.shape[1], k.shape[2], v.shape[3]
    if k.shape != (B, Hkv, Nk, dk) or v.shape != (B, Hkv, Nk, dv) or Hkv < 1 or H % Hkv:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    if out is None:
        out = torch.empty((B, H, Nq, dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or lse.shape != (B, H, Nq):
        raise ValueError(f"lse must be a float32 tensor of shape ({B}, {H}, {Nq})")
    lib = load()
    if Hkv != H:  # shared key/value heads: dense tensors only
        if not all(t.is_contiguous() for t in (q, k, v, out)):
            raise ValueError("shared key/value heads need contiguous q, k, v, out")
        st = lib.mha_forward_gqa(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(out, "out"),
                                 _dev_ptr(lse, "lse"), B, H, Hkv, Nq, Nk, dk, dv, int(mask_kind),
                                 _lens_ptr(key_lens, B), float(scale), _dtype_code(q), _stream(stream))
        check(lib, st)
        return out, lse
    if not all(t.is_contiguous() for t in (q, k, v, out)):
        return _forward_strided(lib, q, k, v, out, lse, mask_kind, key_lens, scale, stream), lse
    st = lib.mha_forward_lse(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(out, "out"),
                             _dev_ptr(lse, "lse"), B, H, Nq, Nk, dk, dv, int(mask_kind), _lens_ptr(key_lens, B),
                             float(scale), _dtype_code(q), _stream(stream))
    check(lib, st)
    return out, lse


def backward_workspace_bytes(B, H, Nq, Nk, d_k, d_v, dtype_code: int = BF16, H_kv=None) -> int:
    H_kv = H if H_kv is None else H_kv
    return int(load().mha_backward_gqa_workspace_bytes(B, H, H_kv, Nq, Nk, d_k, d_v, dtype_code))


def backward(q, k, v, out, dout, lse, mask_kind: int = MASK_NONE, key_lens=None, scale: float | None = None,
             dq=None, dk=None, dv=None, workspace=None, stream=None, events=None):
    """Gradients (dq, dk, dv) of attention for output gradient ``dout``; ``out`` and
    ``lse`` come from forward_lse with the same arguments.  See mha_backward in
    include/mha.h; k, v with H_kv < H heads go to mha_backward_gqa (dk, dv then
    sum over the query heads sharing each key/value head).  ``events``: None, or
    4 hipEvent_t handles (ints) for the timed variants."""
    import torch
    B, H, Nq, d_k = q.shape
    Hkv, Nk, d_v = k.shape[1], k.shape[2], v.shape[3]
    if k.shape != (B, Hkv, Nk, d_k) or v.shape != (B, Hkv, Nk, d_v) or Hkv < 1 or H % Hkv:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if out.shape != (B, H, Nq, d_v) or dout.shape != (B, H, Nq, d_v):
        raise ValueError("out and dout must have shape [B, H, Nq, d_v]")
    if lse.dtype != torch.float32 or lse.shape != (B, H, Nq):
        raise ValueError(f"lse must be a float32 tensor of shape ({B}, {H}, {Nq})")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise TypeError("q, k, v, out, dout must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    code = _dtype_code(q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    lib = load()
    need = int(lib.mha_backward_gqa_workspace_bytes(B, H, Hkv, Nq, Nk, d_k, d_v, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    args = (_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(out, "out"), _dev_ptr(dout, "dout"),
            _dev_ptr(lse, "lse"), _dev_ptr(dq, "dq"), _dev_ptr(dk, "dk"), _dev_ptr(dv, "dv"), B, H, Nq, Nk, d_k,
            d_v, int(mask_kind), _lens_ptr(key_lens, B), float(scale), code, _dev_ptr(workspace, "workspace"),
            0 if workspace is None else workspace.numel(), _stream(stream))
    if Hkv != H:
        gargs = args[:11] + (Hkv,) + args[11:]  # H_kv follows B, H
        if events is None:
            st = lib.mha_backward_gqa(*gargs)
        else:
            import ctypes
            st = lib.mha_backward_gqa_timed(*gargs, (ctypes.c_void_p * 4)(*events))
    elif events is None:
        st = lib.mha_backward(*args)
    else:
        import ctypes
        arr = (ctypes.c_void_p * 4)(*events)
        st = lib.mha_backward_timed(*args, arr)
    check(lib, st)
    return dq, dk, dv
