"""Pins of the general-DPLR oracle (oracle.dplr_recurrent) against things other than itself (CPU only).

The general DPLR transition is Diag(alpha_t) - a_t b_t^T with independent vectors a
and b; KDA ties them to the key ("Kimi Linear" page, section "The constrained DPLR
form and the chunkwise algorithm"). The pins:

* the reduction the page states: a = beta k, b = alpha (.) k and write key beta k
  give KDA, here the separately pinned KDA oracle;
* explicit dense transition products (oracle.forms.dplr_attention_form);
* the chunked form derived from the recurrence (oracle.forms.dplr_chunkwise) at
  several chunk lengths;
* closed forms: a = 0 or b = 0 leaves a gated linear map whose state is a
  decayed sum of writes; alpha = 1, a = 2u, b = u (|u| = 1) is a Householder
  reflection and preserves the state's Frobenius norm; a = b = u with alpha = 1
  is a projection, so repeating a token changes nothing;
* varlen equals separate runs; bf16 inputs are read exactly.

The last test plants two mistakes in the oracle (compile-time mutants: b reading
the decayed state, a and b exchanged) and checks the pins catch both.
"""
import numpy as np
import pytest

import oracle
from oracle import forms
from synth import bf16_bits_to_f32, dplr_small


def _rand(seed, T, d, dv=None, gate=0.3, init=True):
    r = np.random.default_rng(seed)
    dv = dv or d
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = r.standard_normal((T, d))
    k = unit(r.standard_normal((T, d)))
    v = r.standard_normal((T, dv))
    a = unit(r.standard_normal((T, d))) * r.random((T, 1))
    b = unit(r.standard_normal((T, d)))
    la = -gate * r.random((T, d))
    S0 = 0.3 * r.standard_normal((d, dv)) if init else np.zeros((d, dv))
    f = lambda x: np.asarray(x, np.float32)
    return f(q), f(k), f(v), f(a), f(b), f(la), S0


def _run(q, k, v, a, b, la, S0, mutant=0):
    ex = lambda x: x[:, None, :]
    o, S = oracle.dplr_recurrent(ex(q), ex(k), ex(v), ex(a), ex(b), ex(la), np.asarray(S0)[None, None],
                                 threads=1, mutant=mutant)
    return o[:, 0], S[0, 0]


def _f64(*xs):
    return [np.asarray(x, np.float64) for x in xs]


def _close(x, ref, tol):
    return float(np.max(np.abs(x - ref))) <= tol * max(1.0, float(np.max(np.abs(ref))))


# ---- the reduction to KDA ---------------------------------------------------
def _reduction_ok(mutant=0):
    r = np.random.default_rng(11)
    T, d = 40, 8
    q, k, v, _, _, la, S0 = _rand(12, T, d, gate=0.4)
    beta = r.random(T).astype(np.float32)
    # fp64 KDA inputs equal to the fp32 numbers the DPLR oracle reads
    a = (beta[:, None].astype(np.float64) * k).astype(np.float32)       # beta k
    bb = (np.exp(la.astype(np.float64)) * k).astype(np.float32)         # alpha (.) k
    o, S = _run(q, k=a, v=v, a=a, b=bb, la=la, S0=S0, mutant=mutant)
    ex = lambda x: x[:, None, ...]
    ok, Sk = oracle.recurrent(ex(q.astype(np.float64)), ex(k.astype(np.float64)), ex(v.astype(np.float64)),
                              ex(la.astype(np.float64)), beta.astype(np.float64)[:, None], S0[None, None], threads=1)
    # a and b are rounded to fp32 on the DPLR side: agreement to that rounding
    return _close(o, ok[:, 0], 1e-6) and _close(S, Sk[0, 0], 1e-6)


def test_reduces_to_kda():
    assert _reduction_ok()


# ---- dense transitions and the chunked form --------------------------------
def _brute_ok(mutant=0, seed=3, T=17, d=5, dv=4):
    q, k, v, a, b, la, S0 = _rand(seed, T, d, dv)
    o, S = _run(q, k, v, a, b, la, S0, mutant)
    ob, Sb = forms.dplr_attention_form(*_f64(q, k, v, a, b, la), S0)
    return _close(o, ob, 1e-12) and _close(S, Sb, 1e-12)


def test_dense_transition_products():
    assert _brute_ok()
    assert _brute_ok(seed=4, T=9, d=3, dv=6)


@pytest.mark.parametrize("C", [1, 4, 7, 16, 64])
def test_chunked_form(C):
    q, k, v, a, b, la, S0 = _rand(5, 150, 12, 10, gate=0.8)
    o, S = _run(q, k, v, a, b, la, S0)
    oc, Sc = forms.dplr_chunkwise(*_f64(q, k, v, a, b, la), S0, C=C)
    assert _close(o, oc, 1e-11) and _close(S, Sc, 1e-11)


def test_chunked_form_strong_gates():
    # gates down to -30 per token: the chunked form's exponents stay <= 0
    q, k, v, a, b, la, S0 = _rand(6, 90, 6, 6, gate=30.0)
    o, S = _run(q, k, v, a, b, la, S0)
    oc, Sc = forms.dplr_chunkwise(*_f64(q, k, v, a, b, la), S0, C=64)
    assert _close(o, oc, 1e-11) and _close(S, Sc, 1e-11)


# ---- closed forms -------------------------------------------------------------
def _gla_closed(q, k, v, la, S0):
    """No rank-one term: S_t = e^{G_t} S0 + sum_{i<=t} e^{G_t - G_i} k_i v_i^T."""
    G = np.cumsum(la, axis=0)
    T = len(q)
    o = np.empty((T, v.shape[1]))
    for t in range(T):
        St = np.exp(G[t])[:, None] * S0
        for i in range(t + 1):
            St = St + np.exp(G[t] - G[i])[:, None] * np.outer(k[i], v[i])
        o[t] = St.T @ q[t]
    return o, St


@pytest.mark.parametrize("zero", ["a", "b"])
def test_no_rank_one_term(zero):
    q, k, v, a, b, la, S0 = _rand(7, 25, 6, 5)
    (a if zero == "a" else b)[:] = 0.0
    o, S = _run(q, k, v, a, b, la, S0)
    oc, Sc = _gla_closed(*_f64(q, k, v, la), S0)
    assert _close(o, oc, 1e-12) and _close(S, Sc, 1e-12)


def _householder_ok(mutant=0):
    r = np.random.default_rng(8)
    T, d = 30, 7
    u = r.standard_normal((T, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    u = u.astype(np.float32)
    z = np.zeros((T, d), np.float32)
    S0 = r.standard_normal((d, 5))
    _, S = _run(z, z, np.zeros((T, 5), np.float32), 2 * u, u, z, S0, mutant)
    # |u| = 1 only to fp32 rounding: the reflection preserves the norm to that order
    return abs(np.linalg.norm(S) - np.linalg.norm(S0)) <= 1e-5 * np.linalg.norm(S0)


def test_householder_preserves_norm():
    assert _householder_ok()


def test_projection_is_idempotent():
    r = np.random.default_rng(9)
    d = 6
    u = r.standard_normal(d)
    u = (u / np.linalg.norm(u)).astype(np.float32)
    S0 = r.standard_normal((d, 4))
    z = np.zeros((1, d), np.float32)
    one = [z, z, np.zeros((1, 4), np.float32), u[None], u[None], z]
    two = [np.repeat(x, 2, axis=0) for x in one]
    _, S1 = _run(*one, S0)
    _, S2 = _run(*two, S0)
    assert np.max(np.abs(S1 - S2)) <= 1e-6 * np.max(np.abs(S1))
    # and it removes the u direction: u^T S = 0 up to |u|'s fp32 rounding
    assert np.max(np.abs(u.astype(np.float64) @ S1)) <= 1e-6 * np.max(np.abs(S0))


# ---- layout invariants ----------------------------------------------------------
def test_varlen_equals_separate_runs():
    lens = [13, 0, 40, 7]
    d = dplr_small(21, 0, 3, 8, "f32", lens=lens, init_std=0.1)
    cu = d["cu_seqlens"]
    args = [d[x] for x in ("q", "k", "v", "a", "b", "log_alpha")]
    o, S = oracle.dplr_recurrent(*args, d["init"], cu, threads=2)
    for s in range(len(lens)):
        sl = slice(cu[s], cu[s + 1])
        os_, Ss = oracle.dplr_recurrent(*[x[sl] for x in args], d["init"][s:s + 1], threads=1)
        assert np.array_equal(o[sl], os_) and np.array_equal(S[s], Ss[0])


def test_bf16_read_exactly():
    d = dplr_small(22, 50, 2, 8, "bf16", init_std=0.1)
    args = [d[x] for x in ("q", "k", "v", "a", "b")]
    o, S = oracle.dplr_recurrent(*args, d["log_alpha"], d["init"])
    o2, S2 = oracle.dplr_recurrent(*[bf16_bits_to_f32(x) for x in args], d["log_alpha"], d["init"])
    assert np.array_equal(o, o2) and np.array_equal(S, S2)


# ---- planted mistakes -------------------------------------------------------------
@pytest.mark.parametrize("mutant", [8, 9])
def test_pins_catch_planted_mistakes(mutant):
    oracle.build(mutant)
    assert _brute_ok() and _reduction_ok()  # the correct oracle passes
    caught = [not _brute_ok(mutant), not _reduction_ok(mutant)]
    assert any(caught), f"mutant {mutant} slipped through every pin"
