"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the attention arithmetic, so both the GPU path and the fp64 oracle
can be fed from it.  Inputs are numpy float32 arrays whose values are exactly
representable in the workload's dtype (bf16 / fp16 / fp32), so the GPU receives
them bit-exactly and the oracle converts them to fp64 exactly.

Workload shapes follow the pages: d_model 512 with h = 8 and 1024 with h = 16,
d_k = d_v = 64 ([TP] "Multi-Head Attention"; the model sizes in [AC] "The training
recipe"), sentences of a few dozen tokens ([AC] "The problem the paper set out to
fix"), and long contexts where the n^2 term dominates ([TP] "The Trade-Off:
Quadratic Cost").  No dataset is read: the draws stand in for WMT 2014 batches.

Decoding workloads (one new token against long key/value caches) follow the
pages' generation loop ([AD] "Translation and summarization (encoder-decoder)":
keys and values of earlier positions are cached, only the new one is computed).

Recipe: ``numpy.random.Generator(PCG64(seed))``; fp32 N(0,1) draws in the order
(x_q | q), (x_kv | k | k_cache), (v | v_cache), dout, W_Q, W_K, W_V, W_O,
(key_lens | cache_lens); rounding to bf16 is
round-to-nearest-even; Xavier-uniform weights are U(-a, a) with
a = sqrt(6 / (fan_in + fan_out)); key lengths are i.i.d. discrete uniform over the
inclusive range.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str                 # "f32" | "bf16" | "f16"
    mask: int
    lens: tuple | None          # inclusive (lo, hi) of key lengths, or None
    proj: bool                  # with Q/K/V/O projections (d_model = H * d)
    cross: bool                 # keys/values from a second sequence
    seed: int
    description: str
    # Decoding against a key/value cache: Nq new positions per sequence, Nk the
    # cache capacity S, ``lens`` the filled slots, Hkv cache heads (None: H).
    decode: bool = False
    Hkv: int | None = None
    # The sublayer with its residual connection and layer normalisation.
    ln: bool = False
    # Training: the backward pass for an N(0,1) output gradient (after the
    # forward pass that leaves its row statistic).
    backward: bool = False

    @property
    def D(self) -> int:
        return self.H * self.d

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv is None else self.Hkv


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_encoder_f32", 1, 8, 16, 16, 64, "f32", MASK_NONE, None, False, False, 1,
                 "tiny encoder self-attention, no mask, fp32 (B=1, n=16, h=8, d=64)"),
        Workload("base_encoder_proj", 64, 8, 64, 64, 64, "bf16", MASK_NONE, (10, 64), True, False, 2,
                 "Transformer-base encoder self-attention with projections and key padding "
                 "(B=64, n=64, d_model=512, h=8, lengths U{10..64})"),
        Workload("base_encoder_proj_b384", 384, 8, 64, 64, 64, "bf16", MASK_NONE, (10, 64), True, False, 12,
                 "the base encoder layer at about the pages' batch of 25k tokens (B=384, n=64, d_model=512, "
                 "h=8, lengths U{10..64})"),
        Workload("base_decoder_causal", 64, 8, 64, 64, 64, "bf16", MASK_CAUSAL, (10, 64), False, False, 3,
                 "Transformer-base decoder masked self-attention with key padding "
                 "(B=64, n=64, h=8, d=64, lengths U{10..64})"),
        Workload("big_cross_proj", 32, 16, 64, 80, 64, "bf16", MASK_NONE, (20, 80), True, True, 4,
                 "Transformer-big encoder-decoder cross-attention with projections "
                 "(B=32, Nq=64, Nk=80, d_model=1024, h=16, source lengths U{20..80})"),
        Workload("long_causal", 2, 16, 8192, 8192, 64, "bf16", MASK_CAUSAL, None, False, False, 5,
                 "long-context causal self-attention (B=2, n=8192, h=16, d=64)"),
        Workload("base_encoder_proj_ln", 64, 8, 64, 64, 64, "bf16", MASK_NONE, (10, 64), True, False, 2,
                 "Transformer-base encoder self-attention sublayer with its residual connection and "
                 "layer normalisation (B=64, n=64, d_model=512, h=8, lengths U{10..64})", ln=True),
        Workload("big_cross_proj_ln", 32, 16, 64, 80, 64, "bf16", MASK_NONE, (20, 80), True, True, 4,
                 "Transformer-big encoder-decoder cross-attention sublayer with its residual connection "
                 "and layer normalisation (B=32, Nq=64, Nk=80, d_model=1024, h=16, source lengths "
                 "U{20..80})", ln=True),
        Workload("long_decode", 16, 16, 1, 8192, 64, "bf16", MASK_CAUSAL, (1024, 8192), False, False, 6,
                 "one decoding step against long key/value caches (B=16, h=16, d=64, one new token, "
                 "cache of 8192 slots filled U{1024..8192})", decode=True),
        Workload("long_decode_gqa", 16, 16, 1, 8192, 64, "bf16", MASK_CAUSAL, (1024, 8192), False, False, 7,
                 "one decoding step with grouped-query attention (B=16, h=16 query heads over 4 cache "
                 "heads, d=64, one new token, cache of 8192 slots filled U{1024..8192})", decode=True, Hkv=4),
        Workload("long_causal_bwd", 2, 16, 8192, 8192, 64, "bf16", MASK_CAUSAL, None, False, False, 5,
                 "backward pass of long-context causal self-attention (B=2, n=8192, h=16, d=64, "
                 "output gradient N(0,1))", backward=True),
        Workload("base_decoder_causal_bwd", 64, 8, 64, 64, 64, "bf16", MASK_CAUSAL, (10, 64), False, False, 3,
                 "backward pass of Transformer-base decoder masked self-attention with key padding "
                 "(B=64, n=64, h=8, d=64, lengths U{10..64}, output gradient N(0,1))", backward=True),
        Workload("base_encoder_proj_gqa", 64, 8, 64, 64, 64, "bf16", MASK_NONE, (10, 64), True, False, 8,
                 "Transformer-base encoder self-attention with grouped-query projections (B=64, n=64, "
                 "d_model=512, 8 query heads over 2 key/value heads, d=64, lengths U{10..64})", Hkv=2),
        Workload("translation_decoder_causal", 64, 8, 100, 100, 64, "bf16", MASK_CAUSAL, (10, 100), False, False,
                 13, "Transformer-base decoder masked self-attention at the translation length the pages give "
                 "(B=64, n=100, h=8, d=64, lengths U{10..100})"),
        Workload("mid_causal", 64, 16, 256, 256, 64, "bf16", MASK_CAUSAL, None, False, False, 14,
                 "causal self-attention over a few hundred tokens with many heads (B=64, n=256, h=16, d=64)"),
        Workload("long_causal_gqa_bwd", 2, 16, 8192, 8192, 64, "bf16", MASK_CAUSAL, None, False, False, 6,
                 "backward pass of long-context causal self-attention with grouped-query attention "
                 "(B=2, n=8192, h=16 query heads over 4 key/value heads, d=64, output gradient N(0,1))",
                 backward=True, Hkv=4),
    ]
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def generator(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(g: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return round_to(g.standard_normal(shape, dtype=np.float32), dtype)


def xavier_uniform(g: np.random.Generator, fan_out: int, fan_in: int, dtype: str) -> np.ndarray:
    """[fan_out, fan_in] weight (the nn.Linear layout), U(-a, a)."""
    a = math.sqrt(6.0 / (fan_in + fan_out))
    return round_to(g.uniform(-a, a, size=(fan_out, fan_in)).astype(np.float32), dtype)


def key_lengths(g: np.random.Generator, B: int, lo: int, hi: int) -> np.ndarray:
    return g.integers(lo, hi + 1, size=B).astype(np.int32)


def core_inputs(B, H, Nq, Nk, dk, dv, dtype, seed, lens=None):
    """q [B,H,Nq,dk], k [B,H,Nk,dk], v [B,H,Nk,dv] ~ N(0,1); key_lens drawn from
    ``lens`` = (lo, hi) if given."""
    g = generator(seed)
    q = normal(g, (B, H, Nq, dk), dtype)
    k = normal(g, (B, H, Nk, dk), dtype)
    v = normal(g, (B, H, Nk, dv), dtype)
    key_lens = key_lengths(g, B, *lens) if lens is not None else None
    return {"q": q, "k": k, "v": v, "key_lens": key_lens}


def train_inputs(B, H, Nq, Nk, dk, dv, dtype, seed, lens=None, Hkv=None):
    """core_inputs plus an output gradient dout [B,H,Nq,dv] ~ N(0,1), drawn after
    v and before the key lengths.  ``Hkv``: k and v carry that many (shared)
    heads instead of H."""
    g = generator(seed)
    Hkv = H if Hkv is None else Hkv
    q = normal(g, (B, H, Nq, dk), dtype)
    k = normal(g, (B, Hkv, Nk, dk), dtype)
    v = normal(g, (B, Hkv, Nk, dv), dtype)
    dout = normal(g, (B, H, Nq, dv), dtype)
    key_lens = key_lengths(g, B, *lens) if lens is not None else None
    return {"q": q, "k": k, "v": v, "dout": dout, "key_lens": key_lens}


def proj_inputs(B, Nq, Nk, D, H, dk, dv, dtype, seed, cross, lens=None, ln=False, Hkv=None):
    """x_q [B,Nq,D] (and x_kv [B,Nk,D] when ``cross``) ~ N(0,1); Xavier-uniform
    W_Q, W_K [H*dk, D], W_V [H*dv, D], W_O [D, H*dv]; key_lens from ``lens``;
    with ``ln`` the norm's scale ~ U(0.5, 1.5) and shift ~ N(0, 0.5^2), drawn
    last.  ``Hkv``: W_K and W_V have Hkv*d rows (shared key/value heads)."""
    g = generator(seed)
    Hkv = H if Hkv is None else Hkv
    x_q = normal(g, (B, Nq, D), dtype)
    x_kv = normal(g, (B, Nk, D), dtype) if cross else None
    W_Q = xavier_uniform(g, H * dk, D, dtype)
    W_K = xavier_uniform(g, Hkv * dk, D, dtype)
    W_V = xavier_uniform(g, Hkv * dv, D, dtype)
    W_O = xavier_uniform(g, D, H * dv, dtype)
    key_lens = key_lengths(g, B, *lens) if lens is not None else None
    out = {"x_q": x_q, "x_kv": x_kv, "W_Q": W_Q, "W_K": W_K, "W_V": W_V, "W_O": W_O, "key_lens": key_lens}
    if ln:
        out["ln_gamma"] = round_to(g.uniform(0.5, 1.5, size=D).astype(np.float32), dtype)
        out["ln_beta"] = round_to((g.standard_normal(D) * 0.5).astype(np.float32), dtype)
    return out


def decode_inputs(B, H, Hkv, Nq, S, dk, dv, dtype, seed, lens=None):
    """q [B,H,Nq,dk] (the new positions), k_cache [B,Hkv,S,dk], v_cache
    [B,Hkv,S,dv] ~ N(0,1) over every slot; cache_lens drawn from ``lens`` =
    (lo, hi) if given."""
    g = generator(seed)
    q = normal(g, (B, H, Nq, dk), dtype)
    k = normal(g, (B, Hkv, S, dk), dtype)
    v = normal(g, (B, Hkv, S, dv), dtype)
    cache_lens = key_lengths(g, B, *lens) if lens is not None else None
    return {"q": q, "k_cache": k, "v_cache": v, "cache_lens": cache_lens}


def workload_inputs(w: Workload, seed: int | None = None):
    seed = w.seed if seed is None else seed
    if w.decode:
        return decode_inputs(w.B, w.H, w.kv_heads, w.Nq, w.Nk, w.d, w.d, w.dtype, seed, w.lens)
    if w.proj:
        return proj_inputs(w.B, w.Nq, w.Nk, w.D, w.H, w.d, w.d, w.dtype, seed, w.cross, w.lens, w.ln, Hkv=w.Hkv)
    if w.backward:
        return train_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.d, w.dtype, seed, w.lens, Hkv=w.Hkv)
    return core_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.d, w.dtype, seed, w.lens)


def sample_rows(B: int, H: int, N: int, seed: int, n_random: int = 64):
    """(b, h, i) triples for checking long sequences row by row: the tile edges
    {0, 1, 63, 64, 65, 127, 128, N/2 - 1, N/2, N - 2, N - 1} of every (b, h) plus
    ``n_random`` seeded random rows per (b, h)."""
    g = generator(seed)
    fixed = sorted({i for i in (0, 1, 63, 64, 65, 127, 128, N // 2 - 1, N // 2, N - 2, N - 1)
                    if 0 <= i < N})
    rows = []
    for b in range(B):
        for h in range(H):
            extra = g.integers(0, N, size=n_random)
            for i in sorted(set(fixed) | set(int(x) for x in extra)):
                rows.append((b, h, i))
    return np.array(rows, dtype=np.int32)


def plant_score_outliers(q: np.ndarray, k: np.ndarray, slots, jump: float, scale: float, dtype: str,
                         seed: int) -> None:
    """Give later keys scores far above the earlier ones, in place.

    Every query row gets a common direction: q_i += a_i * sqrt(d) * u with u a
    seeded unit vector and a_i ~ U(0.5, 1.5), so t_i = q_i . u lies near
    a_i * sqrt(d) (mostly in [2, 14] for d = 64).  Key slot ``slots[m]`` (of
    every sequence and head; an index along axis 2 of k) becomes
    beta_m * u with beta_m = sign(scale) * jump * 2^m / (2 |scale|), so a query
    with t_i >= 2 sees the scaled score scale * q_i . k jump by at least
    ``jump`` (natural-log units) at each planted slot, over the previous
    planted slot and far over the unplanted keys.  The last slot is paired
    with the slot after it, given beta + sign(scale) / (8 |scale|), so the two
    largest scores of a row differ by about t_i / 8 and neither weight is 0 or
    1.  The arrays are rounded to ``dtype`` again afterwards.  Input
    construction only: nothing here evaluates attention.
    """
    g = generator(seed)
    d = q.shape[-1]
    u = g.standard_normal(d)
    u /= np.linalg.norm(u)
    a = g.uniform(0.5, 1.5, size=q.shape[:-1] + (1,))
    q[...] = round_to((q + a * math.sqrt(d) * u).astype(np.float32), dtype)
    sgn = 1.0 if scale >= 0 else -1.0
    beta0 = jump / (2.0 * abs(scale))
    slots = list(slots)
    for m, j in enumerate(slots):
        k[:, :, j, :] = round_to((sgn * beta0 * 2.0 ** m * u).astype(np.float32), dtype)
    last = slots[-1]
    if last + 1 < k.shape[2]:
        beta = beta0 * 2.0 ** (len(slots) - 1) + 1.0 / (8.0 * abs(scale))
        k[:, :, last + 1, :] = round_to((sgn * beta * u).astype(np.float32), dtype)
