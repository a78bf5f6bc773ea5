"""Plausible mistakes planted in copies of the oracle must each fail a pin.

Every mutant is the oracle's C source with one textual change (a dropped term, a
wrong sign, index or operand), compiled with gcc into a temporary directory on the
CPU.  Mutants run in this process, so none may read or write outside its arrays.  The pins of ``oracle_pins.py`` are run against it, and at least one must
fail.  This shows the pins constrain every step of the oracle, not just the ones a
particular example happens to touch.
"""
import pathlib

import pytest

import oracle
import oracle_pins

SRC = oracle.SOURCE.read_text()

# (name, text in the oracle, replacement)
MUTANTS = [
    ("dot product wrong index", "dot += q[c] * k[c];", "dot += q[c] * k[dk - 1 - c];"),
    ("dot product drops last term", "for (int c = 0; c < dk; ++c) dot", "for (int c = 0; c < dk - 1; ++c) dot"),
    ("scale dropped", "return dot * scale;", "return dot;"),
    ("scale inverted", "return dot * scale;", "return dot / scale;"),
    ("causal off by one", "j > i) return 0;", "j >= i) return 0;"),
    ("causal direction", "j > i) return 0;", "j < i) return 0;"),
    ("padding off by one", "if (j >= L) return 0;", "if (j > L) return 0;"),
    ("padding on queries", "if (j >= L) return 0;", "if (i >= L) return 0;"),
    ("key lengths ignored", "int L = key_lens[b];", "int L = Nk;"),
    ("row max is a min", "if (!any || w[j] > m) m = w[j];", "if (!any || w[j] < m) m = w[j];"),
    ("softmax exponent sign", "w[j] = exp(w[j] - m);", "w[j] = exp(m - w[j]);"),
    ("softmax not normalised", "if (key_visible(i, j, L, mask_kind)) w[j] /= z;", ";"),
    ("weighted sum uses wrong value row", "const double *vj = vbase + (long)j * ldv;",
     "const double *vj = vbase + (long)(Nk - 1 - j) * ldv;"),
    ("weighted sum uses wrong value column", "out[c] += w[j] * vj[c];", "out[c] += w[j] * vj[dv - 1 - c];"),
    ("empty row not zero", "if (!any) return;", "if (!any) { for (int c = 0; c < dv; ++c) out[c] = 1.0; return; }"),
    ("projection weight transposed", "acc += xm[d] * wr[d];", "acc += xm[d] * c->W[(long)d * c->R + r];"),
    ("projection bias dropped", "if (c->bias) acc += c->bias[r];", ";"),
    ("keys projected with W_Q", "linear(x_kv, W_K, b_K, K,", "linear(x_kv, W_Q, b_Q, K,"),
    ("values projected with W_K", "linear(x_kv, W_V, b_V, V,", "linear(x_kv, W_K, b_K, V,"),
    ("queries projected from x_kv", "linear(x_q, W_Q, b_Q, Q,", "linear(x_kv, W_Q, b_Q, Q,"),
    ("all heads read head 0 keys", "const double *kb = c->K + (long)b * c->Nk * ldq + (long)h * c->dk;",
     "const double *kb = c->K + (long)b * c->Nk * ldq;"),
    ("head outputs concatenated in reverse", "double *oi = c->O + ((long)b * c->Nq + i) * ldv + (long)h * c->dv;",
     "double *oi = c->O + ((long)b * c->Nq + i) * ldv + (long)(c->H - 1 - h) * c->dv;"),
    ("causal cross-attention accepted", "if (mask_kind == ORACLE_MASK_CAUSAL && Nq != Nk) return ORACLE_EINVAL;", ""),
    ("decode position one too early", "int p = L - Nq + i;", "int p = L - Nq + i - 1;"),
    ("decode position ignores the cache length", "int p = L - Nq + i;", "int p = i;"),
    ("decode causal mask ignored", "if (mask_kind != ORACLE_MASK_CAUSAL) return L;", "return L;"),
    ("decode cache head by modulo", "int g = h / (c->H / c->Hkv);", "int g = h % c->Hkv;"),
    ("decode cache length clamped one short", "int L = key_length(c->cache_lens, b, c->S);",
     "int L = key_length(c->cache_lens, b, c->S - 1);"),
    ("norm mean not subtracted", "y[c] = (z[c] - mean) * rstd * g + b;", "y[c] = z[c] * rstd * g + b;"),
    ("norm unbiased variance", "var /= D;", "var /= (D - 1);"),
    ("norm eps dropped", "1.0 / sqrt(var + eps);", "1.0 / sqrt(var);"),
    ("norm scale and shift swapped", "const double g = gamma ? gamma[c] : 1.0, b = beta ? beta[c] : 0.0;",
     "const double b = gamma ? gamma[c] : 1.0, g = beta ? beta[c] : 0.0;"),
    ("residual connection dropped", "z[c] = x_q[m * D + c] + out[m * D + c];", "z[c] = out[m * D + c];"),
    ("lse without the maximum", "c->lse[unit * c->Nq + i] = (m == -INFINITY) ? -INFINITY : m + log(z);",
     "c->lse[unit * c->Nq + i] = (m == -INFINITY) ? -INFINITY : log(z);"),
    ("backward softmax term dropped", "const double ds = p * (dp - D);", "const double ds = p * dp;"),
    ("backward softmax sign", "const double ds = p * (dp - D);", "const double ds = p * (D - dp);"),
    ("backward dq without the scale", "dq[(long)i * dkd + e] += c->scale * ds * k[(long)j * dkd + e];",
     "dq[(long)i * dkd + e] += ds * k[(long)j * dkd + e];"),
    ("backward dk from keys", "dk[(long)j * dkd + e] += c->scale * ds * q[(long)i * dkd + e];",
     "dk[(long)j * dkd + e] += c->scale * ds * k[(long)j * dkd + e];"),
    ("backward dv without the weight", "dv[(long)j * dvd + e] += p * dout[(long)i * dvd + e];",
     "dv[(long)j * dvd + e] += dout[(long)i * dvd + e];"),
    ("backward D from the values", "for (int e = 0; e < dvd; ++e) D += dout[(long)i * dvd + e] * out[e];",
     "for (int e = 0; e < dvd; ++e) D += dout[(long)i * dvd + e] * v[e];"),
]


def test_mutant_texts_are_present():
    for name, old, _ in MUTANTS:
        assert SRC.count(old) >= 1, f"{name}: text not found in the oracle source"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path: pathlib.Path, name, old, new):
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new, 1))
    lib = oracle.build(src, tmp_path / "libmutant.so")
    results = oracle_pins.run_all(oracle.Oracle(lib))
    caught = {pin: f for pin, f in results.items() if f}
    assert caught, f"mutant '{name}' passed every pin"
