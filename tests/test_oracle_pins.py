"""Pins of the fp64 oracle against things other than itself (CPU only).

Each pin checks the C recurrence (oracle/kda_oracle.c) against a fact fixed
by the "Kimi Linear" page or by the mathematics of the update rule:

* hand-derived golden examples (tests/golden/hand_examples.json);
* explicit dense transitions and the unrolled attention-like sum
  (section "Why channel-wise gating matters");
* the chunked WY/UT form (section "The constrained DPLR form and the
  chunkwise algorithm") and the forward substitution behind it;
* reductions: beta = 0, alpha = 1 (plain delta rule, section "Background:
  from the delta rule to gated DeltaNet"), one shared gate per head (gated
  delta rule), overwrite of a repeated key, the beta = 2 Householder
  reflection;
* invariants: linearity in (V, S0), value-column separability, split/handoff,
  varlen = separate runs, decode = one more prefill token, a contraction bound.

The last test plants mistakes in the oracle (compile-time mutants) and checks
that the pins catch every one.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import forms
from synth import as_f64, random_small

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rand(seed, T, dk, dv, gate=0.3, beta_hi=1.0, init=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, dk))
    k = r.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((T, dv))
    la = -gate * r.random((T, dk))
    b = beta_hi * r.random(T)
    S0 = 0.3 * r.standard_normal((dk, dv)) if init else np.zeros((dk, dv))
    # store as the operator's input dtypes (fp32) so both sides read identical numbers
    f = lambda x: np.asarray(x, np.float32)
    return f(q), f(k), f(v), f(la), f(b), S0


def _run(q, k, v, la, b, S0, mutant=0, cu=None):
    """Oracle on one head: inputs [T, d]; returns (o [T, dv], S [dk, dv])."""
    T, dk = q.shape
    dv = v.shape[1]
    ex = lambda x: x[:, None, ...]
    init = None if S0 is None else np.asarray(S0, np.float64)[None, None]
    o, S = oracle.recurrent(ex(q), ex(k), ex(v), ex(la), b[:, None], init, cu, threads=1,
                            mutant=mutant)
    return o[:, 0], S[0, 0] if cu is None else S[:, 0]


def _f64(*xs):
    return [np.asarray(x, np.float64) for x in xs]


def _close(a, b, tol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(1.0, float(np.abs(b).max()) if b.size else 1.0)
    return float(np.abs(a - b).max() if a.size else 0.0) <= tol * scale


# ----------------------------------------------------------------------------
# golden, hand-derived
# ----------------------------------------------------------------------------

def _golden_cases():
    return json.load(open(GOLDEN))["cases"]


def _golden_ok(case, mutant=0):
    q = np.array(case["q"], np.float32)
    k = np.array(case["k"], np.float32)
    v = np.array(case["v"], np.float32)
    if "log_alpha" in case:
        la = np.array(case["log_alpha"], np.float32)
    else:
        la = np.log(np.array(case["alpha"], np.float64)).astype(np.float32)
    b = np.array(case["beta"], np.float32)
    o, S = _run(q, k, v, la, b, np.array(case["init"], np.float64), mutant)
    eo, eS = np.array(case["out"], np.float64), np.array(case["final"], np.float64)
    if case["exact"]:
        return np.array_equal(o, eo) and np.array_equal(S, eS)
    return _close(o, eo, case["tol"]) and _close(S, eS, case["tol"])


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_hand_examples(oracle_lib, case):
    assert _golden_ok(case)


# ----------------------------------------------------------------------------
# P1: dense transitions; the unrolled attention-like sum
# ----------------------------------------------------------------------------

def _p1_ok(seed, T, dk, dv, mutant=0):
    q, k, v, la, b, S0 = _rand(seed, T, dk, dv)
    o, S = _run(q, k, v, la, b, S0, mutant)
    ob, Sb = forms.brute(*_f64(q, k, v, la, b), S0)
    return _close(o, ob, 1e-12) and _close(S, Sb, 1e-12)


@pytest.mark.parametrize("T,dk,dv", [(1, 1, 1), (5, 3, 2), (17, 5, 7), (40, 8, 8)])
def test_p1_dense_transitions(oracle_lib, T, dk, dv):
    assert _p1_ok(T * 31 + dk, T, dk, dv)


@pytest.mark.parametrize("T,dk,dv", [(1, 2, 2), (4, 3, 2), (8, 4, 3)])
def test_p1_attention_form(oracle_lib, T, dk, dv):
    q, k, v, la, b, S0 = _rand(7 + T, T, dk, dv)
    o, S = _run(q, k, v, la, b, S0)
    oa, Sa = forms.attention_form(*_f64(q, k, v, la, b), S0)
    assert _close(o, oa, 1e-12) and _close(S, Sa, 1e-12)


def test_tiny_hand_expanded_sum(oracle_lib):
    # T = 2, dk = dv = 1: everything is a scalar, expanded by hand:
    # s1 = a1 s0 + b1 (v1 - a1 s0 k1) k1 ; o1 = q1 s1
    # s2 = a2 s1 + b2 (v2 - a2 s1 k2) k2 ; o2 = q2 s2
    a1, a2 = np.exp(np.float64(np.float32(-0.25))), np.exp(np.float64(np.float32(-0.5)))
    q = np.array([[0.5], [-1.5]], np.float32)
    k = np.array([[1.0], [-1.0]], np.float32)
    v = np.array([[2.0], [3.0]], np.float32)
    b = np.array([0.75, 0.25], np.float32)
    s0 = 1.25
    s1 = a1 * s0 + 0.75 * (2.0 - a1 * s0 * 1.0) * 1.0
    s2 = a2 * s1 + 0.25 * (3.0 - a2 * s1 * -1.0) * -1.0
    la = np.array([[-0.25], [-0.5]], np.float32)
    o, S = _run(q, k, v, la, b, np.array([[s0]]))
    assert _close(o[:, 0], [0.5 * s1, -1.5 * s2], 1e-15) and _close(S[0, 0], s2, 1e-15)


# ----------------------------------------------------------------------------
# P2 / P3: chunked WY/UT form and forward substitution
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("C", [1, 7, 16, 64, 256])
def test_p2_chunkwise_matches_recurrence(oracle_lib, C):
    q, k, v, la, b, S0 = _rand(100 + C, 200, 16, 12, gate=1.0)
    o, S = _run(q, k, v, la, b, S0)
    oc, Sc = forms.chunkwise(*_f64(q, k, v, la, b), S0, C=C)
    assert _close(o, oc, 1e-12) and _close(S, Sc, 1e-12)


@settings(max_examples=25, deadline=None)
@given(T=st.integers(0, 150), dk=st.integers(1, 20), dv=st.integers(1, 20),
       C=st.sampled_from([1, 3, 16, 64]), gate=st.floats(0.0, 3.0), beta_hi=st.floats(0.0, 2.0),
       seed=st.integers(0, 2**31 - 1))
def test_p2_chunkwise_property(oracle_lib, T, dk, dv, C, gate, beta_hi, seed):
    q, k, v, la, b, S0 = _rand(seed, T, dk, dv, gate=gate, beta_hi=beta_hi)
    o, S = _run(q, k, v, la, b, S0)
    oc, Sc = forms.chunkwise(*_f64(q, k, v, la, b), S0, C=C)
    assert _close(o, oc, 1e-10) and _close(S, Sc, 1e-10)


def test_p3_forward_substitution_is_the_inverse():
    r = np.random.default_rng(3)
    for n in (1, 2, 16, 64):
        A = np.tril(r.standard_normal((n, n)) * 0.2, -1)
        T = forms.forward_substitution(A)
        assert np.abs(T - np.linalg.inv(np.eye(n) + A)).max() < 1e-13
        assert np.allclose(np.triu(T, 1), 0) and np.allclose(np.diag(T), 1)


def test_p2_substitution_vs_library_solve():
    q, k, v, la, b, S0 = _f64(*_rand(5, 130, 9, 6))
    o1, S1 = forms.chunkwise(q, k, v, la, b, S0, C=64)
    o2, S2 = forms.chunkwise(q, k, v, la, b, S0, C=64, solve="inverse")
    assert _close(o1, o2, 1e-13) and _close(S1, S2, 1e-13)


# ----------------------------------------------------------------------------
# P4-P9: reductions to known rules
# ----------------------------------------------------------------------------

def _p4_ok(mutant=0):
    q, k, v, la, b, S0 = _rand(11, 30, 6, 5)
    la[:] = 0
    b[:] = 0
    o, S = _run(q, k, v, la, b, S0, mutant)
    return np.array_equal(S, S0) and _close(o, q.astype(np.float64) @ S0, 1e-15)


def test_p4_beta0_alpha1_state_unchanged(oracle_lib):
    assert _p4_ok()


def _p5_ok(mutant=0):
    q, k, v, la, b, S0 = _rand(12, 40, 6, 5, gate=0.5)
    b[:] = 0
    o, S = _run(q, k, v, la, b, S0, mutant)
    G = np.cumsum(la.astype(np.float64), axis=0)
    ok = _close(S, np.exp(G[-1])[:, None] * S0, 1e-14)
    for t in (0, 17, 39):
        ok &= _close(o[t], (np.exp(G[t])[:, None] * S0).T @ q[t].astype(np.float64), 1e-14)
    return ok


def test_p5_beta0_pure_decay(oracle_lib):
    assert _p5_ok()


def _plain_delta(q, k, v, b, S0):
    S = S0.copy()
    o = []
    for t in range(len(q)):
        pred = S.T @ k[t]
        S = S + b[t] * np.outer(k[t], v[t] - pred)
        o.append(S.T @ q[t])
    return np.array(o), S


def _p6_ok(mutant=0):
    q, k, v, la, b, S0 = _rand(13, 50, 7, 4)
    la[:] = 0
    o, S = _run(q, k, v, la, b, S0, mutant)
    op, Sp = _plain_delta(*_f64(q, k, v, b), S0)
    return _close(o, op, 1e-13) and _close(S, Sp, 1e-13)


def test_p6_alpha1_is_plain_delta_rule(oracle_lib):
    assert _p6_ok()


def _gated_delta_scalar(q, k, v, a, b, S0):
    S = S0.copy()
    o = []
    for t in range(len(q)):
        S = a[t] * S
        S = S + b[t] * np.outer(k[t], v[t] - S.T @ k[t])
        o.append(S.T @ q[t])
    return np.array(o), S


def test_p7_shared_gate_is_gated_delta_rule(oracle_lib):
    q, k, v, la, b, S0 = _rand(14, 50, 7, 4, gate=0.4)
    la[:] = la[:, :1]  # every channel shares channel 0's gate
    o, S = _run(q, k, v, la, b, S0)
    og, Sg = _gated_delta_scalar(*_f64(q, k, v), np.exp(la[:, 0].astype(np.float64)),
                                 b.astype(np.float64), S0)
    assert _close(o, og, 1e-13) and _close(S, Sg, 1e-13)


def test_p7_per_head_gate_input(oracle_lib):
    """A [T, H] gate (one per head) is the scalar-gate gated delta rule, coded independently."""
    q, k, v, la, b, S0 = _rand(15, 50, 7, 4, gate=0.4)
    g = la[:, 0].copy()
    init = np.asarray(S0, np.float64)[None, None]
    ex = lambda x: x[:, None, ...]
    o, S = oracle.recurrent(ex(q), ex(k), ex(v), g[:, None], b[:, None], init, None, threads=1)
    og, Sg = _gated_delta_scalar(*_f64(q, k, v), np.exp(g.astype(np.float64)), b.astype(np.float64), S0)
    assert _close(o[:, 0], og, 1e-13) and _close(S[0, 0], Sg, 1e-13)


def test_p8_overwrite_repeated_key(oracle_lib):
    # one-hot keys, dyadic values: exact
    r = np.random.default_rng(15)
    dk, dv = 8, 5
    for trial in range(5):
        idx = r.integers(0, dk)
        k = np.zeros((2, dk), np.float32)
        k[:, idx] = 1
        v = (r.integers(-128, 128, (2, dv)) / 16).astype(np.float32)
        q = k.copy()
        la = np.zeros((2, dk), np.float32)
        b = np.ones(2, np.float32)
        o, S = _run(q, k, v, la, b, np.zeros((dk, dv)))
        assert np.array_equal(o[1], v[1].astype(np.float64))
    # orthonormal keys, random values: within a few ulps
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    kk = Qm[:, 0].astype(np.float32)
    other = Qm[:, 1].astype(np.float32)
    k = np.stack([kk, other, kk])
    v = r.standard_normal((3, dv)).astype(np.float32)
    o, S = _run(k.copy(), k, v, np.zeros((3, dk), np.float32), np.ones(3, np.float32),
                np.zeros((dk, dv)))
    # fp32 keys are unit to ~1e-7, so the overwrite is exact up to that
    assert np.abs(o[2] - v[2]).max() < 1e-6


def test_p9_beta2_householder_preserves_norm(oracle_lib):
    q, k, v, la, b, S0 = _rand(16, 60, 6, 6)
    k = (k.astype(np.float64) / np.linalg.norm(k.astype(np.float64), axis=1, keepdims=True))
    la[:] = 0
    b[:] = 2
    v[:] = 0
    # keys exactly unit in fp64 are not exactly unit in fp32: compare with the norm drift allowed
    o, S = _run(q, k.astype(np.float32), v, la, b, S0)
    kn = np.linalg.norm(k.astype(np.float32).astype(np.float64), axis=1)
    drift = np.prod(np.maximum(1.0, np.abs(1 - 2 * (kn**2 - 1)))) - 1
    assert abs(np.linalg.norm(S) - np.linalg.norm(S0)) <= (drift + 1e-13) * np.linalg.norm(S0) * 4


# ----------------------------------------------------------------------------
# P10-P15: invariants
# ----------------------------------------------------------------------------

def test_p10_linear_in_values_and_initial_state(oracle_lib):
    q, k, v1, la, b, S1 = _rand(17, 40, 5, 4)
    _, _, v2, _, _, S2 = _rand(18, 40, 5, 4)
    a, c = 0.75, -1.25
    o1, F1 = _run(q, k, v1, la, b, S1)
    o2, F2 = _run(q, k, v2, la, b, S2)
    v12 = (a * v1.astype(np.float64) + c * v2.astype(np.float64)).astype(np.float32)
    # v12 is rounded to fp32; use the rounded values on the left side too
    o3, F3 = _run(q, k, v12, la, b, a * S1 + c * S2)
    lhs_err = np.abs(v12.astype(np.float64) - (a * v1.astype(np.float64) + c * v2)).max()
    assert _close(o3, a * o1 + c * o2, 1e-12 + 50 * lhs_err)
    assert _close(F3, a * F1 + c * F2, 1e-12 + 50 * lhs_err)


def test_p11_value_columns_are_separable(oracle_lib):
    q, k, v, la, b, S0 = _rand(19, 45, 6, 7)
    o, S = _run(q, k, v, la, b, S0)
    oa, Sa = _run(q, k, np.ascontiguousarray(v[:, :3]), la, b, S0[:, :3])
    ob, Sb = _run(q, k, np.ascontiguousarray(v[:, 3:]), la, b, S0[:, 3:])
    assert np.array_equal(o, np.concatenate([oa, ob], 1))
    assert np.array_equal(S, np.concatenate([Sa, Sb], 1))
    perm = np.array([4, 0, 6, 2, 1, 5, 3])
    op, Sp = _run(q, k, np.ascontiguousarray(v[:, perm]), la, b, S0[:, perm])
    assert np.array_equal(op, o[:, perm]) and np.array_equal(Sp, S[:, perm])


def _p12_ok(mutant=0):
    q, k, v, la, b, S0 = _rand(20, 100, 6, 5)
    o, S = _run(q, k, v, la, b, S0, mutant)
    ok = True
    for T1 in (0, 1, 37, 64, 99, 100):
        oa, Sa = _run(q[:T1], k[:T1], v[:T1], la[:T1], b[:T1], S0, mutant)
        ob, Sb = _run(q[T1:], k[T1:], v[T1:], la[T1:], b[T1:], Sa, mutant)
        ok &= np.array_equal(np.concatenate([oa, ob]), o) and np.array_equal(Sb, S)
    return ok


def test_p12_split_and_handoff(oracle_lib):
    assert _p12_ok()


def test_p13_varlen_equals_separate_runs(oracle_lib):
    lens = [0, 5, 64, 1, 33, 0, 70]
    d = random_small(21, 0, 3, 6, 5, lens=lens)
    cu = d["cu_seqlens"]
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["init"], cu)
    for s in range(len(lens)):
        t0, t1 = cu[s], cu[s + 1]
        os_, Ss = oracle.recurrent(d["q"][t0:t1], d["k"][t0:t1], d["v"][t0:t1],
                                   d["log_alpha"][t0:t1], d["beta"][t0:t1], d["init"][s:s + 1])
        assert np.array_equal(o[t0:t1], os_) and np.array_equal(S[s], Ss[0])
        if t1 == t0:
            assert np.array_equal(S[s], d["init"][s].astype(np.float64))  # R9


def test_p14_decode_continues_prefill(oracle_lib):
    d = random_small(22, 41, 2, 8, 6, dtype="bf16")
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["init"])
    oa, Sa = oracle.recurrent(d["q"][:40], d["k"][:40], d["v"][:40], d["log_alpha"][:40],
                              d["beta"][:40], d["init"])
    step = {x: d[x][40:41] for x in ("q", "k", "v", "log_alpha", "beta")}
    outs, Sd = oracle.decode_steps(Sa, [step])
    assert np.array_equal(outs[0], o[40:41]) and np.array_equal(Sd, S)


def test_p15_contraction_bound(oracle_lib):
    q, k, v, la, b, S0 = _rand(23, 80, 6, 5, gate=0.7, beta_hi=1.0)
    S = S0
    for t in range(80):
        _, Sn = _run(q[t:t + 1], k[t:t + 1], v[t:t + 1], la[t:t + 1], b[t:t + 1], S)
        kn = np.linalg.norm(k[t].astype(np.float64))
        bound = np.linalg.norm(S, 2) * max(1.0, kn * kn) + b[t] * kn * np.linalg.norm(
            v[t].astype(np.float64))
        assert np.linalg.norm(Sn, 2) <= bound * (1 + 1e-12)
        S = Sn


def test_bf16_inputs_are_read_exactly(oracle_lib):
    d = random_small(24, 20, 2, 4, 3, dtype="bf16")
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["init"])
    f = {x: as_f64(d[x]).astype(np.float32) for x in ("q", "k", "v")}
    o2, S2 = oracle.recurrent(f["q"], f["k"], f["v"], d["log_alpha"], d["beta"], d["init"])
    assert np.array_equal(o, o2) and np.array_equal(S, S2)


# ----------------------------------------------------------------------------
# planted mistakes: every mutant must fail at least one pin
# ----------------------------------------------------------------------------

MUTANTS = {1: "decay after write", 2: "output before write", 3: "wrong prediction sign",
           4: "transposed state", 5: "beta dropped", 6: "gate without exp",
           7: "initial state ignored"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_pins_catch_planted_mistakes(oracle_lib, mutant):
    oracle.build(mutant, force=False)
    checks = [
        lambda: all(_golden_ok(c, mutant) for c in _golden_cases()),
        lambda: _p1_ok(5, 12, 4, 4, mutant),
        lambda: _p4_ok(mutant),
        lambda: _p5_ok(mutant),
        lambda: _p6_ok(mutant),
    ]
    assert not all(chk() for chk in checks), f"mutant {mutant} ({MUTANTS[mutant]}) went undetected"
    # the correct oracle passes the same battery
    assert all(chk() for chk in [lambda: all(_golden_ok(c) for c in _golden_cases()),
                                 lambda: _p1_ok(5, 12, 4, 4), _p4_ok, _p5_ok, _p6_ok])
