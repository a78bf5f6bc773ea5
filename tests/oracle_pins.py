"""Pins that tie the fp64 oracle to what the pages and the mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` and returns a list of failure
messages (empty = pass).  ``test_oracle_pins.py`` runs them against the real
oracle; ``test_oracle_mutants.py`` runs them against deliberately broken builds
of the oracle and requires every broken build to fail at least one pin.

None of these re-types the oracle's own formula: each compares against a value
printed on a page, a closed form, a brute-force selection, an invariant, or a
reduction of one case to another.
"""
from __future__ import annotations

import json
import math
import pathlib

import numpy as np

import oracle as oracle_mod

GOLDEN = json.loads((pathlib.Path(__file__).parent / "golden" / "worked_example.json").read_text())
CAUSAL = oracle_mod.MASK_CAUSAL
NONE = oracle_mod.MASK_NONE


def _close(fails, what, got, want, tol):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if got.shape != want.shape:
        fails.append(f"{what}: shape {got.shape} != {want.shape}")
        return
    if not np.all(np.isfinite(got)):
        fails.append(f"{what}: non-finite values")
        return
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    if not err <= tol:
        fails.append(f"{what}: max err {err:.3g} > {tol:.3g}")


def _same(fails, what, got, want):
    if not np.array_equal(np.asarray(got), np.asarray(want)):
        fails.append(f"{what}: not bit-identical")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# Values printed on the pages.

def pin_worked_example(orc):
    """aicomputerinstitute.com chapter, 'Worked example: attention weights and outputs
    by hand' and 'Active recall' answers 2 and 3: weights, outputs and scaled scores
    printed to 6 decimals for the 3-token example (Q = K = V = X, d_k = 2)."""
    fails = []
    tol = GOLDEN["tolerance"]
    toks = GOLDEN["tokens"]
    for case in GOLDEN["cases"]:
        x = np.array(case["X"], np.float64)[None, None]
        out, w = orc.attention(x, x, x, scale=case["scale"], return_weights=True, nthreads=1)
        s = orc.scores(x, x, scale=case["scale"])
        for tok, vals in case["weights"].items():
            _close(fails, f"{case['name']} weights[{tok}]", w[0, 0, toks.index(tok)], vals, tol)
        for tok, vals in case["outputs"].items():
            _close(fails, f"{case['name']} out[{tok}]", out[0, 0, toks.index(tok)], vals, tol)
        for tok, vals in case.get("scaled_scores", {}).items():
            _close(fails, f"{case['name']} scores[{tok}]", s[0, 0, toks.index(tok)], vals, tol)
    return fails


def _case(name):
    return next(c for c in GOLDEN["cases"] if c["name"] == name)


def _printed_outputs(case):
    toks = GOLDEN["tokens"]
    return np.array([case["outputs"][t] for t in toks], np.float64)


def pin_worked_example_projection(orc):
    """The same example through the projection path.  The page uses identity
    projections, so with H = 1 and W_Q = W_K = W_V = W_O = I the printed outputs
    must come back.  With H = 2 and the two printed variants side by side in the
    two heads' feature blocks, head h's outputs land in column block h of the
    concatenation ([TP] "Multi-Head Attention"); a W_O that swaps the two blocks
    swaps them in the output ([TP] "The Output Projection W^O")."""
    fails = []
    tol = GOLDEN["tolerance"]
    base, dbl = _case("scaled"), _case("was_doubled")
    xb = np.array(base["X"], np.float64)
    xd = np.array(dbl["X"], np.float64)
    eye2 = np.eye(2)
    out = orc.mha_proj(xb[None], None, eye2, eye2, eye2, eye2, H=1, scale=base["scale"], nthreads=1)
    _close(fails, "H=1 identity projections", out[0], _printed_outputs(base), tol)

    x2 = np.concatenate([xb, xd], axis=1)[None]          # [1, 3, 4]
    eye4 = np.eye(4)
    out = orc.mha_proj(x2, None, eye4, eye4, eye4, eye4, H=2, scale=base["scale"], nthreads=1)
    _close(fails, "H=2 head 0 block", out[0, :, 0:2], _printed_outputs(base), tol)
    _close(fails, "H=2 head 1 block", out[0, :, 2:4], _printed_outputs(dbl), tol)
    swap = np.zeros((4, 4))
    for r in range(4):
        swap[r, (r + 2) % 4] = 1.0
    out = orc.mha_proj(x2, None, eye4, eye4, eye4, swap, H=2, scale=base["scale"], nthreads=1)
    _close(fails, "H=2 swapped W_O block 0", out[0, :, 0:2], _printed_outputs(dbl), tol)
    _close(fails, "H=2 swapped W_O block 1", out[0, :, 2:4], _printed_outputs(base), tol)
    return fails


# --------------------------------------------------------------------------
# Closed forms and invariants.

def _random_case(seed, B=3, H=2, Nq=21, Nk=21, dk=16, dv=12, lo=1):
    g = _rng(seed)
    q = g.standard_normal((B, H, Nq, dk))
    k = g.standard_normal((B, H, Nk, dk))
    v = g.standard_normal((B, H, Nk, dv))
    lens = g.integers(lo, Nk + 1, size=B).astype(np.int32)
    return q, k, v, lens


def pin_row_sums_and_zero_weights(orc):
    """Every softmax row sums to 1 ([TP] step 3; [AD] 'The attention mechanism');
    masked keys get weight exactly 0 and visible keys a positive weight ([TP] 'Why
    Masking Is Required': exp(-inf) = 0)."""
    fails = []
    for mask in (NONE, CAUSAL):
        q, k, v, lens = _random_case(11 + mask)
        lens[0] = q.shape[2]
        _, w = orc.attention(q, k, v, mask_kind=mask, key_lens=lens, return_weights=True, nthreads=2)
        B, H, Nq, Nk = w.shape
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        for b in range(B):
            vis = j < lens[b]
            if mask == CAUSAL:
                vis = vis & (j <= i)
            vis = np.broadcast_to(vis, (H, Nq, Nk))
            wb = w[b]
            if np.any(wb[~vis] != 0.0):
                fails.append(f"mask={mask} b={b}: masked weight not exactly 0")
            if np.any(wb[vis] <= 0.0):
                fails.append(f"mask={mask} b={b}: visible weight not positive")
            _close(fails, f"mask={mask} b={b} row sums", wb.sum(-1), np.ones((H, Nq)), 1e-14)
    return fails


def pin_zero_query_gives_mean(orc):
    """With Q = 0 every visible score is equal, so the weights are uniform and each
    output row is the mean of the visible V rows ([TP] steps 3-4)."""
    fails = []
    for mask, Nq, Nk in ((NONE, 13, 29), (CAUSAL, 17, 17)):
        q, k, v, lens = _random_case(21 + mask, Nq=Nq, Nk=Nk)
        q[:] = 0.0
        out = orc.attention(q, k, v, mask_kind=mask, key_lens=lens, nthreads=2)
        want = np.zeros_like(out)
        for b in range(q.shape[0]):
            for i in range(Nq):
                n = min(lens[b], i + 1) if mask == CAUSAL else lens[b]
                want[b, :, i] = v[b, :, :n].mean(axis=1)
        _close(fails, f"Q=0 mean (mask={mask})", out, want, 1e-13)
    return fails


def pin_causal_first_row(orc):
    """Under the causal mask query 0 sees only key 0, whose weight is then exactly
    1, so output row 0 equals V row 0 ([AD] 'Masked Multi-Head Attention')."""
    fails = []
    q, k, v, lens = _random_case(31)
    out = orc.attention(q, k, v, mask_kind=CAUSAL, key_lens=lens, nthreads=2)
    _same(fails, "causal row 0 == V row 0", out[:, :, 0], v[:, :, 0])
    return fails


def pin_one_hot_selection(orc):
    """One-hot keys k_j = c e_pi(j) and one-hot queries q_i = e_pi(t_i): the only
    large score in row i is at key t_i (scaled score 40 against 0), so the output is
    V row t_i up to e^-40 -- a brute-force selection, for cross-attention shapes
    (Nq != Nk, padded source) and for causal self-attention."""
    fails = []
    g = _rng(41)
    d = 64
    scale = 1.0 / math.sqrt(d)
    c = 40.0 / scale
    for mask, B, Nq, Nk in ((NONE, 3, 37, 50), (CAUSAL, 2, 45, 45)):
        H = 2
        q = np.zeros((B, H, Nq, d))
        k = np.zeros((B, H, Nk, d))
        v = g.standard_normal((B, H, Nk, 24))
        lens = g.integers(1, Nk + 1, size=B).astype(np.int32)
        want = np.zeros((B, H, Nq, 24))
        for b in range(B):
            for h in range(H):
                pi = g.permutation(d)[:Nk]
                k[b, h, np.arange(Nk), pi] = c
                for i in range(Nq):
                    hi = min(lens[b], i + 1) if mask == CAUSAL else lens[b]
                    t = int(g.integers(0, hi))
                    q[b, h, i, pi[t]] = 1.0
                    want[b, h, i] = v[b, h, t]
        out = orc.attention(q, k, v, mask_kind=mask, key_lens=lens, scale=scale, nthreads=2)
        _close(fails, f"one-hot selection (mask={mask})", out, want, 1e-12)
    return fails


def pin_large_logits(orc):
    """Scaled logits of about 1000 (far beyond exp's range) must still give the
    selected V row: softmax is shift-invariant, so a correct implementation never
    forms exp of a large positive number."""
    fails = []
    B, H, Nq, Nk, d = 1, 1, 5, 7, 8
    q = np.zeros((B, H, Nq, d))
    k = np.zeros((B, H, Nk, d))
    v = _rng(43).standard_normal((B, H, Nk, 3))
    for j in range(Nk):
        k[0, 0, j, j] = 1000.0 + j
    for i in range(Nq):
        q[0, 0, i, (3 * i + 1) % Nk] = 1.0
    out = orc.attention(q, k, v, scale=1.0, nthreads=1)
    want = v[0, 0, [(3 * i + 1) % Nk for i in range(Nq)]][None, None]
    _close(fails, "selection with logits ~1e3", out, want, 1e-12)
    return fails


def pin_two_key_logistic(orc):
    """With two visible keys the softmax is the logistic function of the score gap:
    w0 = 1 / (1 + exp(s1 - s0)).  q = (1, 2), k0 = (3, 0), k1 = (0, 1) give raw
    scores 3 and 2, so at scale 1/2 the gap is 1/2."""
    fails = []
    q = np.array([1.0, 2.0])[None, None, None]
    k = np.array([[3.0, 0.0], [0.0, 1.0]])[None, None]
    v = np.array([[1.0, -2.0, 5.0], [-4.0, 0.5, 7.0]])[None, None]
    out, w = orc.attention(q, k, v, scale=0.5, return_weights=True, nthreads=1)
    w0 = 1.0 / (1.0 + math.exp(-0.5))
    _close(fails, "two-key weights", w[0, 0, 0], [w0, 1.0 - w0], 1e-15)
    _close(fails, "two-key output", out[0, 0, 0], w0 * v[0, 0, 0] + (1.0 - w0) * v[0, 0, 1], 1e-14)
    return fails


def pin_sqrt_dk_statistics(orc):
    """For N(0,1) query and key components q.k has variance d_k, so over 4,000
    independent pairs std(q.k) is near sqrt(d_k) and near 1 after the 1/sqrt(d_k)
    scale ([TP] 'Why the sqrt(d_k) Scaling Exists'; [AC] 'Why the dot product is
    divided by the square root of d_k', which reports 1.99 / 7.89 / 22.54)."""
    fails = []
    g = _rng(51)
    for dk in (4, 64, 512):
        q = g.standard_normal((4000, 1, 1, dk))
        k = g.standard_normal((4000, 1, 1, dk))
        raw = orc.scores(q, k, scale=1.0).ravel()
        scaled = orc.scores(q, k, scale=1.0 / math.sqrt(dk)).ravel()
        r = raw.std() / math.sqrt(dk)
        if abs(r - 1.0) > 0.05:
            fails.append(f"d_k={dk}: std(q.k)/sqrt(d_k) = {r:.3f}")
        if abs(scaled.std() - 1.0) > 0.05:
            fails.append(f"d_k={dk}: std(scaled) = {scaled.std():.3f}")
    return fails


def pin_permutation_equivariance(orc):
    """Without a mask, permuting the query rows permutes the output rows, and
    permuting the key and value rows together leaves the output unchanged
    ([ACI] 'The problem attention creates...'; [ZS] 'Telling the positions apart')."""
    fails = []
    q, k, v, _ = _random_case(61, Nq=19, Nk=26)
    g = _rng(62)
    out = orc.attention(q, k, v, nthreads=2)
    pq = g.permutation(q.shape[2])
    _same(fails, "query permutation", orc.attention(q[:, :, pq], k, v, nthreads=2), out[:, :, pq])
    pk = g.permutation(k.shape[2])
    _close(fails, "joint key/value permutation",
           orc.attention(q, k[:, :, pk], v[:, :, pk], nthreads=2), out, 1e-13)
    return fails


def pin_future_tokens(orc):
    """Changing a future token never changes an earlier output under the causal
    mask ([AC] 'Pitfalls when reproducing the paper')."""
    fails = []
    q, k, v, lens = _random_case(71, Nq=24, Nk=24)
    lens[:] = 24
    out = orc.attention(q, k, v, mask_kind=CAUSAL, key_lens=lens, nthreads=2)
    g = _rng(72)
    for i0 in (0, 7, 22):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        for t in (q2, k2, v2):
            t[:, :, i0 + 1:] = g.standard_normal(t[:, :, i0 + 1:].shape) * 100.0
        out2 = orc.attention(q2, k2, v2, mask_kind=CAUSAL, key_lens=lens, nthreads=2)
        _same(fails, f"rows <= {i0} after changing later tokens", out2[:, :, :i0 + 1],
              out[:, :, :i0 + 1])
        if np.array_equal(out2[:, :, i0 + 1:], out[:, :, i0 + 1:]):
            fails.append(f"rows > {i0} did not react to changed tokens")
    return fails


def pin_padding_is_on_keys(orc):
    """Padding hides keys, not queries ([AC] 'Pitfalls'; [AD] 'Two masks, not one'):
    the result for a sequence of length L equals attention over its first L keys and
    values alone; padded query rows are ordinary rows; whatever sits in padded key
    and value slots (even inf or NaN) never reaches the output."""
    fails = []
    for mask in (NONE, CAUSAL):
        q, k, v, lens = _random_case(81 + mask, B=4, Nq=20, Nk=20)
        lens[:] = [20, 13, 1, 7]
        out = orc.attention(q, k, v, mask_kind=mask, key_lens=lens, nthreads=2)
        for b in range(4):
            L = int(lens[b])
            if mask == NONE:
                ref = orc.attention(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L], nthreads=1)
                _same(fails, f"mask={mask} b={b} truncated keys", out[b:b + 1], ref)
            else:
                ref = orc.attention(q[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L],
                                    mask_kind=CAUSAL, nthreads=1)
                _same(fails, f"mask={mask} b={b} truncated rows < L", out[b:b + 1, :, :L], ref)
                # rows i >= L see exactly the L visible keys, like an unmasked query
                tail = orc.attention(q[b:b + 1, :, L:], k[b:b + 1, :, :L], v[b:b + 1, :, :L],
                                     nthreads=1)
                _same(fails, f"mask={mask} b={b} padded query rows", out[b:b + 1, :, L:], tail)
        for poison in (np.inf, np.nan, 1e300):
            k2, v2 = k.copy(), v.copy()
            for b in range(4):
                k2[b, :, lens[b]:] = poison
                v2[b, :, lens[b]:] = -poison
            out2 = orc.attention(q, k2, v2, mask_kind=mask, key_lens=lens, nthreads=2)
            _same(fails, f"mask={mask} poison {poison} in padded slots", out2, out)
    return fails


def pin_empty_rows(orc):
    """A row with no visible key (key length 0) returns 0 -- the reading taken for
    the NaN case of [AC] 'Pitfalls' -- and has all-zero weights."""
    fails = []
    q, k, v, lens = _random_case(91, B=2)
    lens[:] = [0, 5]
    out, w = orc.attention(q, k, v, key_lens=lens, return_weights=True, nthreads=1)
    _same(fails, "empty row output", out[0], np.zeros_like(out[0]))
    _same(fails, "empty row weights", w[0], np.zeros_like(w[0]))
    if not np.all(np.abs(out[1]) > 0):
        fails.append("non-empty rows returned zeros")
    return fails


def pin_projection_uniform_closed_form(orc):
    """W_Q = W_K = 0 makes every score equal (b_Q . b_K times the scale), so each
    head averages its visible value rows: out = mean_{j<L}(x_kv_j W_V^T + b_V) W_O^T
    + b_O, a closed form checked here for cross-attention with padding."""
    fails = []
    g = _rng(101)
    B, Nq, Nk, D, H, dk, dv = 3, 6, 9, 12, 3, 4, 5
    x_q = g.standard_normal((B, Nq, D))
    x_kv = g.standard_normal((B, Nk, D))
    W_Q = np.zeros((H * dk, D))
    W_K = np.zeros((H * dk, D))
    W_V = g.standard_normal((H * dv, D))
    W_O = g.standard_normal((D, H * dv))
    b_Q, b_K = g.standard_normal(H * dk), g.standard_normal(H * dk)
    b_V, b_O = g.standard_normal(H * dv), g.standard_normal(D)
    lens = np.array([9, 4, 1], np.int32)
    out = orc.mha_proj(x_q, x_kv, W_Q, W_K, W_V, W_O, H=H, b_Q=b_Q, b_K=b_K, b_V=b_V, b_O=b_O,
                       key_lens=lens, nthreads=2)
    want = np.zeros_like(out)
    for b in range(B):
        mean_v = (x_kv[b, :lens[b]] @ W_V.T + b_V).mean(axis=0)
        want[b] = (mean_v @ W_O.T + b_O)[None, :]
    _close(fails, "uniform-attention closed form", out, want, 1e-12)
    return fails


def pin_projection_one_hot_cross(orc):
    """Cross-attention through the projection path: the decoder side x_q carries a
    one-hot query in its second feature half, the encoder side x_kv a one-hot key in
    its first half and a payload in its second half.  W_Q reads x_q's second half,
    W_K x_kv's first half, W_V x_kv's second half and W_O copies the head output to
    the first D/2 output features, so out[i] = payload of the key query i points
    at ([AD] 'Multi-Head Attention (middle) - cross-attention')."""
    fails = []
    g = _rng(111)
    B, Nq, Nk, m = 2, 7, 11, 16
    D = 2 * m
    scale = 0.25
    c = 40.0 / scale
    x_q = np.zeros((B, Nq, D))
    x_kv = np.zeros((B, Nk, D))
    x_kv[:, :, m:] = g.standard_normal((B, Nk, m))
    lens = np.array([11, 6], np.int32)
    want = np.zeros((B, Nq, D))
    for b in range(B):
        pi = g.permutation(m)[:Nk]
        x_kv[b, np.arange(Nk), pi] = c
        for i in range(Nq):
            t = int(g.integers(0, lens[b]))
            x_q[b, i, m + pi[t]] = 1.0
            want[b, i, :m] = x_kv[b, t, m:]
    first = np.concatenate([np.eye(m), np.zeros((m, m))], axis=1)     # reads features [0, m)
    second = np.concatenate([np.zeros((m, m)), np.eye(m)], axis=1)    # reads features [m, 2m)
    W_O = np.concatenate([np.eye(m), np.zeros((m, m))], axis=0)       # [D, m]
    out = orc.mha_proj(x_q, x_kv, second, first, second, W_O, H=1, key_lens=lens, scale=scale,
                       nthreads=2)
    _close(fails, "projected one-hot cross-attention", out, want, 1e-12)
    return fails


def pin_rejects_causal_cross(orc):
    """The causal mask is defined for self-attention only ([TP] 'Why Masking Is
    Required'); a causal call with Nq != Nk is rejected."""
    fails = []
    q, k, v, _ = _random_case(121, Nq=4, Nk=5)
    try:
        orc.attention(q, k, v, mask_kind=CAUSAL, nthreads=1)
        fails.append("causal with Nq != Nk accepted")
    except oracle_mod.OracleError:
        pass
    return fails


# --------------------------------------------------------------------------
# Decoding against a key/value cache.

def _decode_case(seed, B, H, Hkv, S, dk=16, dv=12):
    g = _rng(seed)
    return (g, g.standard_normal((B, H, S, dk)), g.standard_normal((B, Hkv, S, dk)),
            g.standard_normal((B, Hkv, S, dv)))


def _poison_tail(cache, lens):
    """Copy of ``cache`` [B, Hkv, S, d] with every slot >= clamp(len_b, 0, S) set
    to NaN: a correct decoder never reads them."""
    out = cache.copy()
    S = cache.shape[2]
    for b, L in enumerate(lens):
        out[b, :, min(max(int(L), 0), S):] = np.nan
    return out


def pin_decode_matches_full_recompute(orc):
    """A decoding step against the cache equals causal attention recomputed over
    the whole prefix: the cache only saves recomputing past keys and values
    ([AD] 'This parallelism is a training-time property'; [AD] 'Translation and
    summarization (encoder-decoder)': only the new position is computed).  The Nq
    new queries of sequence b are rows L_b - Nq .. L_b - 1 of the full causal
    result; a query whose position would be negative sees no key and gives 0.
    Cache slots past L_b hold NaN.  Both sides sum the same keys in the same
    order, so the match is exact."""
    fails = []
    B, H, S, Nq = 6, 3, 29, 3
    g, q, k, _ = _decode_case(131, B, H, H, S)
    v = g.standard_normal((B, H, S, 12))
    full = orc.attention(q, k, v, mask_kind=CAUSAL, nthreads=2)
    for lens in (np.array([S + 6, S, 17, 3, 1, 0], np.int32), None):
        Ls = [S] * B if lens is None else [min(max(int(L), 0), S) for L in lens]
        qd = np.zeros((B, H, Nq, q.shape[3]))
        want = np.zeros((B, H, Nq, 12))
        for b, L in enumerate(Ls):
            for i in range(Nq):
                p = L - Nq + i
                if p >= 0:
                    qd[b, :, i] = q[b, :, p]
                    want[b, :, i] = full[b, :, p]
                else:
                    qd[b, :, i] = g.standard_normal((H, q.shape[3]))
        kc = _poison_tail(k, Ls)
        vc = _poison_tail(v, Ls)
        out = orc.decode(qd, kc, vc, mask_kind=CAUSAL, cache_lens=lens, nthreads=2)
        _same(fails, f"decode == full causal rows (lens={'ragged' if lens is not None else 'none'})",
              out, want)
    return fails


def pin_decode_cross_is_padded_attention(orc):
    """Cross-attention against a source's cached keys and values (computed once,
    [AD] 'Translation and summarization (encoder-decoder)') is attention with the
    source padding mask: every new query sees the L_b filled slots and nothing
    else, so it equals the padded attention result exactly."""
    fails = []
    B, H, S, Nq = 5, 2, 23, 5
    g, _, k, v = _decode_case(141, B, H, H, S)
    q = g.standard_normal((B, H, Nq, k.shape[3]))
    lens = np.array([23, 0, 40, 7, 1], np.int32)
    want = orc.attention(q, k, v, mask_kind=NONE, key_lens=lens, nthreads=2)
    out = orc.decode(q, _poison_tail(k, lens), _poison_tail(v, lens), mask_kind=NONE,
                     cache_lens=lens, nthreads=2)
    _same(fails, "cross decode == padded attention", out, want)
    return fails


def pin_decode_shared_heads(orc):
    """Grouped-query and multi-query attention are multi-head attention whose
    key/value heads are shared ([ZS] 'Many heads, many subspaces'; [TP]
    'Limitations of the Original Design'): with Hkv cache heads, the result equals
    ordinary multi-head decoding with each cache head repeated for its run of
    H / Hkv consecutive query heads."""
    fails = []
    B, H, S, Nq = 3, 6, 19, 2
    lens = np.array([19, 11, 2], np.int32)
    for Hkv in (1, 2, 3):
        g, _, k, v = _decode_case(150 + Hkv, B, H, Hkv, S)
        q = g.standard_normal((B, H, Nq, k.shape[3]))
        G = H // Hkv
        for mask in (CAUSAL, NONE):
            out = orc.decode(q, k, v, mask_kind=mask, cache_lens=lens, nthreads=2)
            want = orc.decode(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), mask_kind=mask,
                              cache_lens=lens, nthreads=2)
            _same(fails, f"Hkv={Hkv} mask={mask} vs repeated heads", out, want)
    return fails


def pin_decode_short_caches(orc):
    """Closed forms on short caches.  One filled slot: the single visible key
    has weight 1, so the output is that value row exactly, whatever the query.
    No filled slot: output 0.  Q = 0 under the causal mask: equal scores, so
    query i returns the mean of the first L_b - Nq + i + 1 cached values."""
    fails = []
    B, H, S, Nq = 4, 2, 9, 3
    g, _, k, v = _decode_case(161, B, H, H, S)
    q = g.standard_normal((B, H, 1, k.shape[3])) * 10.0
    out = orc.decode(q, k, v, mask_kind=CAUSAL, cache_lens=np.array([1, 1, 0, 0], np.int32),
                     nthreads=2)
    _same(fails, "one cached key -> its value row", out[:2, :, 0], v[:2, :, 0])
    _same(fails, "empty cache -> 0", out[2:], np.zeros_like(out[2:]))
    lens = np.array([9, 5, 3, 2], np.int32)
    out = orc.decode(np.zeros((B, H, Nq, k.shape[3])), k, v, mask_kind=CAUSAL, cache_lens=lens,
                     nthreads=2)
    want = np.zeros_like(out)
    for b in range(B):
        for i in range(Nq):
            n = int(lens[b]) - Nq + i + 1
            if n > 0:
                want[b, :, i] = v[b, :, :n].mean(axis=1)
    _close(fails, "Q=0 causal decode -> mean of visible prefix", out, want, 1e-13)
    return fails


def pin_decode_rejects_bad_heads(orc):
    """The query heads must split evenly over the cache heads."""
    fails = []
    _, q, k, v = _decode_case(171, 1, 6, 4, 5)
    for Hkv in (4, 7):
        kk = np.zeros((1, Hkv, 5, 16))
        vv = np.zeros((1, Hkv, 5, 12))
        try:
            orc.decode(q[:, :, :1], kk, vv, nthreads=1)
            fails.append(f"H=6, Hkv={Hkv} accepted")
        except oracle_mod.OracleError:
            pass
    return fails


# --------------------------------------------------------------------------
# Residual connection and layer normalisation after the sublayer.

def _ln_case(seed, B=2, Nq=5, Nk=7, D=64, H=4, cross=True):
    g = _rng(seed)
    x_q = g.standard_normal((B, Nq, D))
    x_kv = g.standard_normal((B, Nk, D)) if cross else None
    W = [g.standard_normal((D, D)) * 0.2 for _ in range(4)]
    lens = g.integers(1, (Nk if cross else Nq) + 1, size=B).astype(np.int32)
    return g, x_q, x_kv, W, lens


def pin_ln_two_features(orc):
    """Two features and eps = 0: a normalised row is (-1, +1) or (+1, -1), by
    which feature is larger, then scaled and shifted per feature -- a closed form
    that holds only with the mean subtracted and the variance taken over the D
    features ([AD] 'Add & Norm': normalisation across each token's features).
    W_O = 0 makes the sublayer output exactly b_O, so the normalised row is that
    of x_q + b_O: the residual is the query-side input ([AC] listing).  With
    eps = 0.5 and z = (0, 2) the row becomes (-1, 1) / sqrt(1.5)."""
    fails = []
    g = _rng(181)
    B, Nq, Nk, D = 3, 4, 6, 2
    x_q = g.standard_normal((B, Nq, D))
    x_kv = g.standard_normal((B, Nk, D))
    W = [g.standard_normal((D, D)) for _ in range(3)] + [np.zeros((D, D))]
    b_O = np.array([0.25, -0.5])
    gamma, beta = np.array([2.0, -3.0]), np.array([0.5, 7.0])
    out = orc.mha_proj_ln(x_q, x_kv, *W, H=1, b_O=b_O, gamma=gamma, beta=beta, eps=0.0, nthreads=1)
    z = x_q + b_O
    sgn = np.sign(z[..., 1] - z[..., 0])
    want = np.stack([-sgn, sgn], axis=-1) * gamma + beta
    _close(fails, "two-feature rows", out, want, 1e-12)
    x0 = np.zeros((1, 1, 2))
    out = orc.mha_proj_ln(x0, None, *[np.zeros((2, 2))] * 4, H=1, b_O=np.array([0.0, 2.0]), eps=0.5,
                          nthreads=1)
    _close(fails, "eps inside the root", out[0, 0], np.array([-1.0, 1.0]) / math.sqrt(1.5), 1e-15)
    return fails


def pin_ln_rows_standardised(orc):
    """Without scale and shift every output row has mean 0 and mean square
    var / (var + eps): exactly 1 for eps = 0, just below 1 for eps > 0."""
    fails = []
    _, x_q, x_kv, W, lens = _ln_case(191)
    for eps in (0.0, 1e-3):
        out = orc.mha_proj_ln(x_q, x_kv, *W, H=4, eps=eps, key_lens=lens, nthreads=2)
        _close(fails, f"row means (eps={eps})", out.mean(-1), np.zeros(out.shape[:2]), 1e-12)
        ms = (out ** 2).mean(-1)
        if eps == 0.0:
            _close(fails, "row mean squares", ms, np.ones(out.shape[:2]), 1e-12)
        elif not (np.all(ms < 1.0 - 1e-6) and np.all(ms > 0.9)):
            fails.append("eps does not shrink the row scale")
    return fails


def pin_ln_affine(orc):
    """The per-feature scale and shift act last: out(gamma, beta) =
    gamma * out(1, 0) + beta, for self- and cross-attention."""
    fails = []
    for cross in (False, True):
        g, x_q, x_kv, W, lens = _ln_case(201 + cross, cross=cross, Nk=5)
        gamma = g.standard_normal(64)
        beta = g.standard_normal(64)
        base = orc.mha_proj_ln(x_q, x_kv, *W, H=4, key_lens=lens, mask_kind=NONE, nthreads=2)
        aff = orc.mha_proj_ln(x_q, x_kv, *W, H=4, gamma=gamma, beta=beta, key_lens=lens, nthreads=2)
        _close(fails, f"affine (cross={cross})", aff, gamma * base + beta, 1e-12)
    return fails


def pin_ln_shift_invariance(orc):
    """Adding the same amount to every feature of the sublayer output (a
    constant b_O) leaves the normalised rows unchanged; a non-constant b_O
    changes them."""
    fails = []
    g, x_q, x_kv, W, lens = _ln_case(211)
    base = orc.mha_proj_ln(x_q, x_kv, *W, H=4, key_lens=lens, nthreads=2)
    shifted = orc.mha_proj_ln(x_q, x_kv, *W, H=4, b_O=np.full(64, 3.75), key_lens=lens, nthreads=2)
    _close(fails, "constant shift", shifted, base, 1e-11)
    other = orc.mha_proj_ln(x_q, x_kv, *W, H=4, b_O=g.standard_normal(64), key_lens=lens, nthreads=2)
    if np.max(np.abs(other - base)) < 1e-3:
        fails.append("a non-constant b_O did not change the output")
    return fails


# --------------------------------------------------------------------------
# Training: row statistics and gradients.

def pin_lse_consistent_with_weights(orc):
    """exp(s_ij - lse_i) reproduces the softmax weights the forward pass uses, for
    padded and causal rows; one visible key gives lse = its score; a row with no
    visible key gives -inf."""
    fails = []
    for mask in (NONE, CAUSAL):
        q, k, v, lens = _random_case(221 + mask, Nq=12, Nk=12 if mask else 17, lo=0)
        _, w = orc.attention(q, k, v, mask_kind=mask, key_lens=lens, return_weights=True, nthreads=2)
        s = orc.scores(q, k, mask_kind=mask, key_lens=lens)
        lse = orc.attention_lse(q, k, mask_kind=mask, key_lens=lens, nthreads=2)
        with np.errstate(invalid="ignore"):
            p = np.where(np.isfinite(s), np.exp(s - lse[..., None]), 0.0)
        p = np.nan_to_num(p)
        _close(fails, f"exp(s - lse) == weights (mask={mask})", p, w, 1e-13)
        empty = lens == 0
        if np.any(empty) and not np.all(np.isneginf(lse[empty])):
            fails.append("empty rows not -inf")
    q, k, _, _ = _random_case(225, Nq=3, Nk=3)
    lse = orc.attention_lse(q, k, mask_kind=CAUSAL, nthreads=1)
    s = orc.scores(q, k, mask_kind=CAUSAL)
    _close(fails, "single visible key", lse[:, :, 0], s[:, :, 0, 0], 1e-14)
    return fails


def _fd_loss(orc, q, k, v, dout, mask, lens, scale):
    return float(np.sum(dout * orc.attention(q, k, v, mask_kind=mask, key_lens=lens, scale=scale, nthreads=1)))


def pin_backward_finite_differences(orc):
    """The gradients of L = sum(dout * out) match central finite differences of
    the forward oracle (step 1e-5, fp64) at sampled entries of q, k and v, for
    padded cross-shaped and causal inputs -- a check by a different method."""
    fails = []
    g = _rng(231)
    for mask, Nq, Nk in ((NONE, 5, 7), (CAUSAL, 6, 6)):
        B, H, d, dv = 2, 2, 4, 3
        q = g.standard_normal((B, H, Nq, d))
        k = g.standard_normal((B, H, Nk, d))
        v = g.standard_normal((B, H, Nk, dv))
        dout = g.standard_normal((B, H, Nq, dv))
        lens = np.array([Nk, Nk - 2], np.int32)
        scale = 0.7
        gq, gk, gv = orc.attention_backward(q, k, v, dout, mask_kind=mask, key_lens=lens, scale=scale, nthreads=1)
        h = 1e-5
        for name, arr, grad in (("q", q, gq), ("k", k, gk), ("v", v, gv)):
            for _ in range(12):
                idx = tuple(int(g.integers(0, n)) for n in arr.shape)
                a1, a2 = arr.copy(), arr.copy()
                a1[idx] += h
                a2[idx] -= h
                args1 = {"q": q, "k": k, "v": v}
                args2 = dict(args1)
                args1[name], args2[name] = a1, a2
                fd = (_fd_loss(orc, args1["q"], args1["k"], args1["v"], dout, mask, lens, scale)
                      - _fd_loss(orc, args2["q"], args2["k"], args2["v"], dout, mask, lens, scale)) / (2 * h)
                if abs(fd - grad[idx]) > 1e-7 * (1 + abs(fd)):
                    fails.append(f"d{name}{idx} (mask={mask}): analytic {grad[idx]:.9g} vs fd {fd:.9g}")
    return fails


def pin_backward_invariants(orc):
    """Softmax is unchanged by adding one vector to every key, so the key
    gradients of a row's visible keys sum to zero; padded keys get exactly zero
    gradient; the gradients are linear in dout."""
    fails = []
    for mask, Nq, Nk in ((NONE, 9, 13), (CAUSAL, 11, 11)):
        q, k, v, lens = _random_case(241 + mask, Nq=Nq, Nk=Nk)
        dout = _rng(242).standard_normal(v.shape[:2] + (Nq, v.shape[3]))
        gq, gk, gv = orc.attention_backward(q, k, v, dout, mask_kind=mask, key_lens=lens, nthreads=2)
        _close(fails, f"sum of key gradients (mask={mask})", gk.sum(axis=2), np.zeros(gk.sum(axis=2).shape), 1e-12)
        for b, L in enumerate(lens):
            if np.any(gk[b, :, L:] != 0.0) or np.any(gv[b, :, L:] != 0.0):
                fails.append(f"padded keys got gradient (mask={mask}, b={b})")
        g2 = orc.attention_backward(q, k, v, -2.5 * dout, mask_kind=mask, key_lens=lens, nthreads=2)
        for name, a, b2 in zip("qkv", (gq, gk, gv), g2):
            _close(fails, f"linearity d{name} (mask={mask})", b2, -2.5 * a, 1e-12)
    return fails


def pin_backward_selection(orc):
    """One-hot attention (each query selects one key with weight 1 up to e^-40):
    the value gradient is dout gathered onto the selected keys, and the query and
    key gradients vanish (the weights do not move)."""
    fails = []
    g = _rng(251)
    B, H, Nq, Nk, d = 1, 2, 6, 8, 16
    scale = 1.0
    q = np.zeros((B, H, Nq, d))
    k = np.zeros((B, H, Nk, d))
    v = g.standard_normal((B, H, Nk, 5))
    dout = g.standard_normal((B, H, Nq, 5))
    want_dv = np.zeros_like(v)
    for h in range(H):
        for j in range(Nk):
            k[0, h, j, j] = 40.0
        for i in range(Nq):
            t = (3 * i + h) % Nk
            q[0, h, i, t] = 1.0
            want_dv[0, h, t] += dout[0, h, i]
    gq, gk, gv = orc.attention_backward(q, k, v, dout, scale=scale, nthreads=1)
    _close(fails, "selection dv", gv, want_dv, 1e-12)
    _close(fails, "selection dq", gq, np.zeros_like(gq), 1e-12)
    _close(fails, "selection dk", gk, np.zeros_like(gk), 1e-12)
    return fails


def pin_backward_gqa_finite_differences(orc):
    """Shared key/value heads: the gradients of L = sum(dout * out) with respect to
    the shared k and v match central finite differences of the shared-head forward
    pass (each shared entry moves every query head of its group at once), and the
    forward pass and the query gradient equal those of explicitly copied heads
    computed head by head."""
    fails = []
    g = _rng(261)
    B, H, Hkv, Nq, Nk, d, dv = 2, 6, 2, 5, 7, 4, 3
    q = g.standard_normal((B, H, Nq, d))
    k = g.standard_normal((B, Hkv, Nk, d))
    v = g.standard_normal((B, Hkv, Nk, dv))
    dout = g.standard_normal((B, H, Nq, dv))
    lens = np.array([Nk, Nk - 3], np.int32)
    scale = 0.6

    def loss(kk, vv):
        return float(np.sum(dout * orc.attention_gqa(q, kk, vv, key_lens=lens, scale=scale, nthreads=1)))

    gq, gk, gv = orc.attention_backward_gqa(q, k, v, dout, key_lens=lens, scale=scale, nthreads=1)
    if gk.shape != k.shape or gv.shape != v.shape or gq.shape != q.shape:
        return [f"shapes {gq.shape} {gk.shape} {gv.shape}"]
    h = 1e-5
    for name, arr, grad in (("k", k, gk), ("v", v, gv)):
        for _ in range(16):
            idx = tuple(int(g.integers(0, n)) for n in arr.shape)
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            f1 = loss(a1, v) if name == "k" else loss(k, a1)
            f2 = loss(a2, v) if name == "k" else loss(k, a2)
            fd = (f1 - f2) / (2 * h)
            if abs(fd - grad[idx]) > 1e-7 * (1 + abs(fd)):
                fails.append(f"shared d{name}{idx}: analytic {grad[idx]:.9g} vs fd {fd:.9g}")
    # Head h reads key/value head h // 3: compare with single-head calls.
    out = orc.attention_gqa(q, k, v, key_lens=lens, scale=scale, nthreads=1)
    for hh in range(H):
        sl = slice(hh, hh + 1)
        kv = slice(hh // 3, hh // 3 + 1)
        one = orc.attention(q[:, sl], k[:, kv], v[:, kv], key_lens=lens, scale=scale, nthreads=1)
        _close(fails, f"shared-head forward, head {hh}", out[:, sl], one, 1e-14)
        dq1 = orc.attention_backward(q[:, sl], k[:, kv], v[:, kv], dout[:, sl], key_lens=lens, scale=scale,
                                     nthreads=1)[0]
        _close(fails, f"shared-head dq, head {hh}", gq[:, sl], dq1, 1e-14)
    return fails


def pin_projection_shared_heads(orc):
    """Shared key/value projections (H = 6 query heads over H_kv = 2, groups of
    three): with W_Q = W_K = 0 every query head averages the visible rows of its
    group's value head, out = sum_h mean_{j<L}(x_kv_j W_V[g(h)]^T + b_V[g(h)])
    W_O[:, h]^T + b_O with g(h) = h // 3 (closed form); and with random weights
    the result equals per-head projections by plain matrix products fed to the
    per-head attention oracle."""
    fails = []
    g = _rng(271)
    B, Nq, Nk, D, H, Hkv, dk, dv = 2, 5, 7, 12, 6, 2, 4, 3
    G = H // Hkv
    x_q = g.standard_normal((B, Nq, D))
    x_kv = g.standard_normal((B, Nk, D))
    W_V = g.standard_normal((Hkv * dv, D))
    W_O = g.standard_normal((D, H * dv))
    b_V, b_O = g.standard_normal(Hkv * dv), g.standard_normal(D)
    lens = np.array([7, 3], np.int32)
    out = orc.mha_proj_gqa(x_q, x_kv, np.zeros((H * dk, D)), np.zeros((Hkv * dk, D)), W_V, W_O, H=H, H_kv=Hkv,
                           b_Q=g.standard_normal(H * dk), b_K=g.standard_normal(Hkv * dk), b_V=b_V, b_O=b_O,
                           key_lens=lens, nthreads=1)
    want = np.tile(b_O, (B, Nq, 1))
    for b in range(B):
        for h in range(H):
            kv = h // G
            v = x_kv[b, :lens[b]] @ W_V[kv * dv:(kv + 1) * dv].T + b_V[kv * dv:(kv + 1) * dv]
            want[b] += (v.mean(axis=0) @ W_O[:, h * dv:(h + 1) * dv].T)[None, :]
    _close(fails, "shared-head uniform closed form", out, want, 1e-12)

    W_Q, W_K = g.standard_normal((H * dk, D)), g.standard_normal((Hkv * dk, D))
    out = orc.mha_proj_gqa(x_q, None, W_Q, W_K, W_V, W_O, H=H, H_kv=Hkv, mask_kind=CAUSAL, nthreads=1)
    q = np.stack([x_q @ W_Q[h * dk:(h + 1) * dk].T for h in range(H)], axis=1)
    k = np.stack([x_q @ W_K[(h // G) * dk:(h // G + 1) * dk].T for h in range(H)], axis=1)
    v = np.stack([x_q @ W_V[(h // G) * dv:(h // G + 1) * dv].T for h in range(H)], axis=1)
    heads = orc.attention(q, k, v, mask_kind=CAUSAL, nthreads=1)             # [B, H, Nq, dv]
    want = np.concatenate([heads[:, h] for h in range(H)], axis=-1) @ W_O.T  # head-major concatenation
    _close(fails, "shared-head projections through per-head attention", out, want, 1e-11)
    return fails


ALL_PINS = [
    pin_worked_example,
    pin_worked_example_projection,
    pin_row_sums_and_zero_weights,
    pin_zero_query_gives_mean,
    pin_causal_first_row,
    pin_one_hot_selection,
    pin_large_logits,
    pin_two_key_logistic,
    pin_sqrt_dk_statistics,
    pin_permutation_equivariance,
    pin_future_tokens,
    pin_padding_is_on_keys,
    pin_empty_rows,
    pin_projection_uniform_closed_form,
    pin_projection_one_hot_cross,
    pin_rejects_causal_cross,
    pin_decode_matches_full_recompute,
    pin_decode_cross_is_padded_attention,
    pin_decode_shared_heads,
    pin_decode_short_caches,
    pin_decode_rejects_bad_heads,
    pin_ln_two_features,
    pin_ln_rows_standardised,
    pin_ln_affine,
    pin_ln_shift_invariance,
    pin_lse_consistent_with_weights,
    pin_backward_finite_differences,
    pin_backward_invariants,
    pin_backward_selection,
    pin_backward_gqa_finite_differences,
    pin_projection_shared_heads,
]


def run_all(orc):
    """{pin name: failures} for every pin, catching crashes as failures."""
    res = {}
    for pin in ALL_PINS:
        try:
            res[pin.__name__] = pin(orc)
        except Exception as exc:  # a broken build may raise instead of returning
            res[pin.__name__] = [f"raised {type(exc).__name__}: {exc}"]
    return res
