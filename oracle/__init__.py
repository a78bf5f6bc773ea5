"""fp64 CPU oracle for multi-head scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing but the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It is a plain
C library (``mha_oracle.c``, built with gcc, no HIP) behind a ctypes wrapper; it
shares no code with the GPU library.

Every function takes numpy arrays of any real dtype and converts them to float64
(bf16 and fp32 values convert exactly), and returns float64 results.  The method
and the readings taken where the pages are silent are described in the header of
``mha_oracle.c``.  Weights use the [out_features, in_features] layout of the
nn.Linear layers in the code listing on the aicassindra.com page ("A faithful layer
in code").
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1

_HERE = pathlib.Path(__file__).resolve().parent
SOURCE = _HERE / "mha_oracle.c"
DEFAULT_LIB = _HERE / "_build" / "liboracle.so"

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def default_threads() -> int:
    """Host threads for the oracle: all visible cores, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def build(source: pathlib.Path | str = SOURCE, out: pathlib.Path | str = DEFAULT_LIB) -> pathlib.Path:
    """Compile the oracle with gcc into a shared library and return its path."""
    out = pathlib.Path(out)
    out.parent.mkdir(parents=True, exist_ok=True)
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
           str(source), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class OracleError(RuntimeError):
    pass


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _lens(key_lens, B: int):
    if key_lens is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(key_lens, dtype=np.int32))
    if arr.shape != (B,):
        raise ValueError(f"key_lens must have shape ({B},), got {arr.shape}")
    return arr, arr.ctypes.data_as(_ip)


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, libpath: pathlib.Path | str):
        self.path = pathlib.Path(libpath)
        lib = ctypes.CDLL(str(self.path))
        i = ctypes.c_int
        lib.oracle_attention.argtypes = [_dp, _dp, _dp, _dp, i, i, i, i, i, i, i, _ip,
                                         ctypes.c_double, _dp, i]
        lib.oracle_scores.argtypes = [_dp, _dp, _dp, i, i, i, i, i, i, _ip, ctypes.c_double]
        lib.oracle_attention_rows.argtypes = [_dp, _dp, _dp, _dp, i, i, i, i, i, i, i, _ip,
                                              ctypes.c_double, i, _ip, i]
        lib.oracle_mha_proj.argtypes = [_dp] * 11 + [i] * 8 + [_ip, ctypes.c_double, i]
        lib.oracle_decode.argtypes = [_dp] * 4 + [i] * 8 + [_ip, ctypes.c_double, i]
        lib.oracle_mha_proj_ln.argtypes = ([_dp] * 12 + [ctypes.c_double, _dp] + [i] * 8
                                           + [_ip, ctypes.c_double, i])
        lib.oracle_attention_lse.argtypes = [_dp, _dp, _dp] + [i] * 6 + [_ip, ctypes.c_double, i]
        lib.oracle_attention_backward.argtypes = [_dp] * 7 + [i] * 7 + [_ip, ctypes.c_double, i]
        for f in (lib.oracle_attention, lib.oracle_scores, lib.oracle_attention_rows,
                  lib.oracle_mha_proj, lib.oracle_decode, lib.oracle_mha_proj_ln,
                  lib.oracle_attention_lse, lib.oracle_attention_backward):
            f.restype = ctypes.c_int
        self._lib = lib

    @staticmethod
    def _check(status: int, what: str) -> None:
        if status != 0:
            raise OracleError(f"{what} returned {status}")

    # -- attention on per-head tensors [B, H, N, d] ---------------------------
    def attention(self, q, k, v, mask_kind: int = MASK_NONE, key_lens=None, scale=None,
                  return_weights: bool = False, nthreads: int | None = None):
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, Nq, dk = q.shape
        Nk, dv = k.shape[2], v.shape[3]
        if k.shape != (B, H, Nk, dk) or v.shape != (B, H, Nk, dv):
            raise ValueError("q/k/v shapes disagree")
        if scale is None:
            scale = 1.0 / np.sqrt(dk)
        lens, lens_p = _lens(key_lens, B)
        out = np.empty((B, H, Nq, dv), np.float64)
        w = np.empty((B, H, Nq, Nk), np.float64) if return_weights else None
        st = self._lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Nq, Nk, dk, dv,
                                        int(mask_kind), lens_p, float(scale), _ptr(w),
                                        nthreads or default_threads())
        self._check(st, "oracle_attention")
        return (out, w) if return_weights else out

    def scores(self, q, k, mask_kind: int = MASK_NONE, key_lens=None, scale=None):
        q, k = _f64(q), _f64(k)
        B, H, Nq, dk = q.shape
        Nk = k.shape[2]
        if scale is None:
            scale = 1.0 / np.sqrt(dk)
        lens, lens_p = _lens(key_lens, B)
        s = np.empty((B, H, Nq, Nk), np.float64)
        st = self._lib.oracle_scores(_ptr(q), _ptr(k), _ptr(s), B, H, Nq, Nk, dk, int(mask_kind),
                                     lens_p, float(scale))
        self._check(st, "oracle_scores")
        return s

    def attention_rows(self, q, k, v, rows, mask_kind: int = MASK_NONE, key_lens=None,
                       scale=None, nthreads: int | None = None):
        """Output rows for the (b, h, i) triples in ``rows`` (shape [n, 3])."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, Nq, dk = q.shape
        Nk, dv = k.shape[2], v.shape[3]
        if scale is None:
            scale = 1.0 / np.sqrt(dk)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
        lens, lens_p = _lens(key_lens, B)
        out = np.empty((rows.shape[0], dv), np.float64)
        st = self._lib.oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Nq, Nk,
                                             dk, dv, int(mask_kind), lens_p, float(scale),
                                             rows.shape[0], rows.ctypes.data_as(_ip),
                                             nthreads or default_threads())
        self._check(st, "oracle_attention_rows")
        return out

    # -- training: row statistics and gradients ----------------------------------
    def attention_lse(self, q, k, mask_kind: int = MASK_NONE, key_lens=None, scale=None,
                      nthreads: int | None = None):
        """lse [B,H,Nq]: natural log of the softmax denominator of each row over its
        visible keys (-inf for a row with none)."""
        q, k = _f64(q), _f64(k)
        B, H, Nq, dk = q.shape
        Nk = k.shape[2]
        if scale is None:
            scale = 1.0 / np.sqrt(dk)
        lens, lens_p = _lens(key_lens, B)
        lse = np.empty((B, H, Nq), np.float64)
        st = self._lib.oracle_attention_lse(_ptr(q), _ptr(k), _ptr(lse), B, H, Nq, Nk, dk, int(mask_kind),
                                            lens_p, float(scale), nthreads or default_threads())
        self._check(st, "oracle_attention_lse")
        return lse

    def attention_backward(self, q, k, v, dout, mask_kind: int = MASK_NONE, key_lens=None, scale=None,
                           nthreads: int | None = None):
        """(dq, dk, dv): gradients of sum(dout * attention(q, k, v))."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, H, Nq, dk = q.shape
        Nk, dv = k.shape[2], v.shape[3]
        if dout.shape != (B, H, Nq, dv):
            raise ValueError("dout shape")
        if scale is None:
            scale = 1.0 / np.sqrt(dk)
        lens, lens_p = _lens(key_lens, B)
        gq = np.empty_like(q)
        gk = np.empty_like(k)
        gv = np.empty_like(v)
        st = self._lib.oracle_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(gq), _ptr(gk),
                                                 _ptr(gv), B, H, Nq, Nk, dk, dv, int(mask_kind), lens_p,
                                                 float(scale), nthreads or default_threads())
        self._check(st, "oracle_attention_backward")
        return gq, gk, gv

    # -- shared key/value heads (grouped-query attention) -----------------------
    # [TP] "Limitations of the Original Design" and [ZS] "Many heads, many
    # subspaces": the key/value heads are shared by groups of query heads.  Query
    # head h reads key/value head h // (H // H_kv).  The forward pass is
    # per-head attention on the key/value heads repeated to H; a shared head's
    # gradient is, by the chain rule, the sum of the gradients of its copies.
    @staticmethod
    def _group(H: int, Hkv: int) -> int:
        if Hkv < 1 or H % Hkv:
            raise ValueError(f"H_kv = {Hkv} does not divide H = {H}")
        return H // Hkv

    def attention_gqa(self, q, k, v, **kwargs):
        """q [B,H,Nq,dk]; k [B,H_kv,Nk,dk]; v [B,H_kv,Nk,dv]."""
        G = self._group(q.shape[1], k.shape[1])
        return self.attention(q, np.repeat(_f64(k), G, axis=1), np.repeat(_f64(v), G, axis=1), **kwargs)

    def attention_lse_gqa(self, q, k, **kwargs):
        G = self._group(q.shape[1], k.shape[1])
        return self.attention_lse(q, np.repeat(_f64(k), G, axis=1), **kwargs)

    def attention_backward_gqa(self, q, k, v, dout, **kwargs):
        """(dq, dk, dv) with dk, dv of the shared shape [B,H_kv,Nk,d]."""
        B, Hkv, Nk = k.shape[:3]
        G = self._group(q.shape[1], Hkv)
        gq, gk, gv = self.attention_backward(q, np.repeat(_f64(k), G, axis=1), np.repeat(_f64(v), G, axis=1),
                                             dout, **kwargs)
        return gq, gk.reshape(B, Hkv, G, Nk, -1).sum(axis=2), gv.reshape(B, Hkv, G, Nk, -1).sum(axis=2)

    # -- multi-head attention with projections ---------------------------------
    def mha_proj(self, x_q, x_kv, W_Q, W_K, W_V, W_O, H: int, b_Q=None, b_K=None, b_V=None,
                 b_O=None, mask_kind: int = MASK_NONE, key_lens=None, scale=None,
                 nthreads: int | None = None):
        """x_q [B,Nq,D]; x_kv [B,Nk,D] or None; W_Q/W_K [H*dk, D]; W_V [H*dv, D];
        W_O [D, H*dv]; biases [out_features] or None.  Returns out [B,Nq,D]."""
        x_q = _f64(x_q)
        B, Nq, D = x_q.shape
        x_kv = None if x_kv is None else _f64(x_kv)
        Nk = Nq if x_kv is None else x_kv.shape[1]
        W_Q, W_K, W_V, W_O = _f64(W_Q), _f64(W_K), _f64(W_V), _f64(W_O)
        dk = W_Q.shape[0] // H
        dv = W_V.shape[0] // H
        if scale is None:
            scale = 1.0 / np.sqrt(dk)
        biases = [None if b is None else _f64(b) for b in (b_Q, b_K, b_V, b_O)]
        lens, lens_p = _lens(key_lens, B)
        out = np.empty((B, Nq, D), np.float64)
        st = self._lib.oracle_mha_proj(_ptr(x_q), _ptr(x_kv), _ptr(W_Q), _ptr(W_K), _ptr(W_V),
                                       _ptr(W_O), *[_ptr(b) for b in biases], _ptr(out), B, Nq,
                                       Nk, D, H, dk, dv, int(mask_kind), lens_p, float(scale),
                                       nthreads or default_threads())
        self._check(st, "oracle_mha_proj")
        return out

    def mha_proj_gqa(self, x_q, x_kv, W_Q, W_K, W_V, W_O, H: int, H_kv: int, b_Q=None, b_K=None, b_V=None,
                     b_O=None, **kwargs):
        """mha_proj with the key and value projections shared by groups of query
        heads ([TP] "Limitations of the Original Design"): W_K [H_kv*dk, D],
        W_V [H_kv*dv, D], b_K, b_V [H_kv*d] or None; query head h uses key/value
        head h // (H // H_kv).  Computed as mha_proj with each shared block of
        rows repeated for its group, which is the same function."""
        G = self._group(H, H_kv)

        def rep(w):
            if w is None:
                return None
            w = _f64(w)
            rows = w.shape[0] // H_kv
            return np.repeat(w.reshape((H_kv, rows) + w.shape[1:]), G, axis=0).reshape((H * rows,) + w.shape[1:])

        return self.mha_proj(x_q, x_kv, W_Q, rep(W_K), rep(W_V), W_O, H, b_Q=b_Q, b_K=rep(b_K), b_V=rep(b_V),
                             b_O=b_O, **kwargs)

    def mha_proj_ln(self, x_q, x_kv, W_Q, W_K, W_V, W_O, H: int, b_Q=None, b_K=None, b_V=None,
                    b_O=None, gamma=None, beta=None, eps: float = 1e-5, mask_kind: int = MASK_NONE,
                    key_lens=None, scale=None, nthreads: int | None = None):
        """LayerNorm(x_q + MHA(x_q, x_kv)) per token over its D features; gamma, beta
        [D] or None (1 and 0).  Other arguments as mha_proj.  Returns [B,Nq,D]."""
        x_q = _f64(x_q)
        B, Nq, D = x_q.shape
        x_kv = None if x_kv is None else _f64(x_kv)
        Nk = Nq if x_kv is None else x_kv.shape[1]
        W_Q, W_K, W_V, W_O = _f64(W_Q), _f64(W_K), _f64(W_V), _f64(W_O)
        dk = W_Q.shape[0] // H
        dv = W_V.shape[0] // H
        if scale is None:
            scale = 1.0 / np.sqrt(dk)
        vecs = [None if b is None else _f64(b) for b in (b_Q, b_K, b_V, b_O, gamma, beta)]
        lens, lens_p = _lens(key_lens, B)
        out = np.empty((B, Nq, D), np.float64)
        st = self._lib.oracle_mha_proj_ln(_ptr(x_q), _ptr(x_kv), _ptr(W_Q), _ptr(W_K), _ptr(W_V),
                                          _ptr(W_O), *[_ptr(v) for v in vecs], float(eps), _ptr(out),
                                          B, Nq, Nk, D, H, dk, dv, int(mask_kind), lens_p,
                                          float(scale), nthreads or default_threads())
        self._check(st, "oracle_mha_proj_ln")
        return out

    # -- one decoding step against a key/value cache ----------------------------
    def decode(self, q, k_cache, v_cache, mask_kind: int = MASK_CAUSAL, cache_lens=None,
               scale=None, nthreads: int | None = None):
        """q [B,H,Nq,dk] (the Nq newest positions); k_cache [B,Hkv,S,dk] and
        v_cache [B,Hkv,S,dv] with cache_lens[b] filled slots (None: all S).
        CAUSAL: query i sits at position cache_lens[b] - Nq + i; NONE: every
        query sees the whole filled cache.  Query head h reads cache head
        h // (H // Hkv).  Returns out [B,H,Nq,dv]."""
        q, k, v = _f64(q), _f64(k_cache), _f64(v_cache)
        B, H, Nq, dk = q.shape
        Hkv, S = k.shape[1], k.shape[2]
        dv = v.shape[3]
        if k.shape != (B, Hkv, S, dk) or v.shape != (B, Hkv, S, dv):
            raise ValueError("q/k_cache/v_cache shapes disagree")
        if scale is None:
            scale = 1.0 / np.sqrt(dk)
        lens, lens_p = _lens(cache_lens, B)
        out = np.empty((B, H, Nq, dv), np.float64)
        st = self._lib.oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, Nq, S, dk,
                                     dv, int(mask_kind), lens_p, float(scale),
                                     nthreads or default_threads())
        self._check(st, "oracle_decode")
        return out


_DEFAULT: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``mha_oracle.c`` (compiled on first use if absent)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not DEFAULT_LIB.exists():
            build()
        _DEFAULT = Oracle(DEFAULT_LIB)
    return _DEFAULT


def attention(*args, **kwargs):
    return get().attention(*args, **kwargs)


def scores(*args, **kwargs):
    return get().scores(*args, **kwargs)


def attention_rows(*args, **kwargs):
    return get().attention_rows(*args, **kwargs)


def mha_proj(*args, **kwargs):
    return get().mha_proj(*args, **kwargs)


def decode(*args, **kwargs):
    return get().decode(*args, **kwargs)


def mha_proj_ln(*args, **kwargs):
    return get().mha_proj_ln(*args, **kwargs)


def attention_lse(*args, **kwargs):
    return get().attention_lse(*args, **kwargs)


def attention_backward(*args, **kwargs):
    return get().attention_backward(*args, **kwargs)


def attention_gqa(*args, **kwargs):
    return get().attention_gqa(*args, **kwargs)


def attention_lse_gqa(*args, **kwargs):
    return get().attention_lse_gqa(*args, **kwargs)


def attention_backward_gqa(*args, **kwargs):
    return get().attention_backward_gqa(*args, **kwargs)


def mha_proj_gqa(*args, **kwargs):
    return get().mha_proj_gqa(*args, **kwargs)
