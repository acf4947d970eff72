"""Pins of the layer oracle (oracle/layer.py) against facts outside it (CPU only).

The layer wraps the pinned recurrence with the prologue and epilogue the
"Kimi Linear" page lists for a KDA head ("Kimi Delta Attention" section): L2
normalisation of q and k, the per-channel decay from a projection output, and
a head-wise RMSNorm with a sigmoid output gate.  Each pin below fails for a
plausible mistake in one of those steps:

* bf16 widening: exact values of known bit patterns;
* the gate map: closed forms of -softplus and its identity with log sigmoid;
* normalisation: unit rows, and invariance of the whole layer to positive
  per-(token, head) rescaling of q and k (fails for a norm over the wrong axis
  or a missing norm);
* reduction to the recurrence: already-unit q, k with g = log(expm1(-log_alpha))
  reproduce ``oracle.recurrent`` on log_alpha (fails for a sign or inversion
  error in the gate, or a normalisation that is not the identity on unit rows);
* the epilogue: with eps = 0, y / (w sigmoid(z)) has unit RMS per row and the
  direction of o (fails for a mean over the wrong axis, a missing weight or a
  missing gate);
* decode steps equal the prefill form token by token.
"""
import numpy as np
import pytest

import oracle
from oracle import layer


def _inputs(seed, T, H, d, per_head=False, scale=1.0):
    r = np.random.default_rng(seed)
    q = scale * r.standard_normal((T, H, d))
    k = scale * r.standard_normal((T, H, d))
    v = r.standard_normal((T, H, d))
    g = r.normal(-2.0, 1.0, (T, H) if per_head else (T, H, d))
    b = r.random((T, H))
    z = r.standard_normal((T, H, d))
    w = 1.0 + 0.1 * r.standard_normal(d)
    S0 = 0.2 * r.standard_normal((1, H, d, d))
    return q, k, v, g, b, z, w, S0


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x8000, 0x4049], np.uint16)
    got = layer.widen(bits)
    assert got.tolist() == [1.0, -2.0, 0.25, 0.0, -0.0, 3.140625]


def test_gate_map_closed_forms():
    g = np.array([0.0, 30.0, -30.0, 2.0, -700.0, 700.0])
    la = layer.log_alpha_from_gate(g)
    assert la[0] == pytest.approx(-np.log(2.0), rel=1e-15)
    assert la[1] == pytest.approx(-30.0 - np.exp(-30.0), rel=1e-15)
    assert la[2] == pytest.approx(-np.exp(-30.0), rel=1e-12)
    # alpha = sigmoid(-g), computed here as 1 / (1 + e^g)
    assert np.exp(la[3]) == pytest.approx(1.0 / (1.0 + np.exp(2.0)), rel=1e-15)
    assert la[4] == 0.0 or abs(la[4]) < 1e-300
    assert la[5] == pytest.approx(-700.0, rel=1e-15)
    assert np.all(la <= 0.0)


def test_l2_rows_are_unit():
    x = np.random.default_rng(1).standard_normal((7, 3, 16)) * 5.0
    n = layer.l2_normalize(x, 0.0)
    assert np.allclose(np.linalg.norm(n, axis=-1), 1.0, atol=1e-15)
    assert np.allclose(n * np.linalg.norm(x, axis=-1, keepdims=True), x, atol=1e-13)


def test_layer_invariant_to_qk_row_scaling():
    q, k, v, g, b, z, w, S0 = _inputs(2, 40, 2, 16)
    r = np.random.default_rng(3)
    cq = np.exp(r.normal(0.0, 1.0, (40, 2, 1)))
    ck = np.exp(r.normal(0.0, 1.0, (40, 2, 1)))
    y1, S1, _ = layer.forward(q, k, v, g, b, S0, None, z, w, True, 0.0)
    y2, S2, _ = layer.forward(q * cq, k * ck, v, g, b, S0, None, z, w, True, 0.0)
    assert np.abs(y1 - y2).max() < 1e-12 and np.abs(S1 - S2).max() < 1e-12
    # without the normalisation the same rescaling does change the result
    y3, _, _ = layer.forward(q * cq, k * ck, v, g, b, S0, None, z, w, False, 0.0)
    y4, _, _ = layer.forward(q, k, v, g, b, S0, None, z, w, False, 0.0)
    assert np.abs(y3 - y4).max() > 1e-3


@pytest.mark.parametrize("per_head", [False, True])
def test_layer_reduces_to_recurrence(per_head):
    T, H, d = 60, 2, 16
    r = np.random.default_rng(4)
    q = r.standard_normal((T, H, d))
    k = r.standard_normal((T, H, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, H, d))
    la = -r.uniform(0.01, 2.0, (T, H) if per_head else (T, H, d))
    g = np.log(np.expm1(-la))  # the projection output whose gate is exactly log_alpha
    b = r.random((T, H))
    S0 = 0.2 * r.standard_normal((1, H, d, d))
    y, S, o = layer.forward(q, k, v, g, b, S0, None, None, None, True, 0.0)
    o_ref, S_ref = oracle.recurrent(q, k, v, la, b, S0)
    assert np.array_equal(y, o)
    assert np.abs(o - o_ref).max() < 1e-12 and np.abs(S - S_ref).max() < 1e-12


def test_epilogue_unit_rms_and_direction():
    q, k, v, g, b, z, w, S0 = _inputs(5, 30, 3, 16)
    y, _, o = layer.forward(q, k, v, g, b, S0, None, z, w, True, 1e-6, 0.0)
    gate = 1.0 / (1.0 + np.exp(-z))  # sigmoid(z), computed here independently
    n = y / (w * gate)
    assert np.allclose(np.sqrt(np.mean(n * n, axis=-1)), 1.0, atol=1e-13)
    cos = np.sum(n * o, axis=-1) / (np.linalg.norm(n, axis=-1) * np.linalg.norm(o, axis=-1))
    assert np.allclose(cos, 1.0, atol=1e-13)


def test_decode_steps_match_prefill():
    N, H, d, steps = 3, 2, 16, 5
    r = np.random.default_rng(6)
    S0 = 0.2 * r.standard_normal((N, H, d, d))
    seq = [dict(q=r.standard_normal((N, H, d)), k=r.standard_normal((N, H, d)),
                v=r.standard_normal((N, H, d)), g=r.normal(-1.0, 1.0, (N, H, d)),
                beta=r.random((N, H)), out_gate=r.standard_normal((N, H, d))) for _ in range(steps)]
    w = 1.0 + 0.1 * r.standard_normal(d)
    outs, S = layer.decode_steps(S0, seq, w)
    # the same tokens as N sequences of length `steps`, packed sequence-major
    cat = lambda key: np.concatenate([np.stack([st[key][n] for st in seq]) for n in range(N)])
    cu = np.arange(N + 1) * steps
    y, S2, _ = layer.forward(cat("q"), cat("k"), cat("v"), cat("g"), cat("beta"), S0, cu,
                             cat("out_gate"), w)
    for s in range(steps):
        for n in range(N):
            assert np.abs(outs[s][n] - y[n * steps + s]).max() < 1e-12
    assert np.abs(S - S2).max() < 1e-12
