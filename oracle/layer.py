"""fp64 oracle of the KDA layer's prologue and epilogue -- TEST INFRASTRUCTURE ONLY.

The "Kimi Linear" page ("Kimi Delta Attention" section) wraps the recurrence
of every KDA head in a prologue and an epilogue: queries and keys are scaled to
unit L2 norm, the per-channel decay comes out of a small low-rank projection,
and the head's output is normalised by its RMS and multiplied by a sigmoid
gate.  The page fixes neither the
squashing of the projection into a decay nor the constants, so this module
takes the plainest readings:

* L2 normalisation over a head's key channels, per token:
  x / sqrt(sum_c x_c^2 + l2_eps)
* the gate: the projection output g (one value per key channel, or one per
  head for the scalar-gate variant) enters as log alpha = -softplus(g), the
  standard map of a real pre-activation onto a log-decay <= 0
  (alpha = sigmoid(-g))
* the epilogue: y = o / sqrt(mean_j o_j^2 + rms_eps) * w * sigmoid(z), with the
  mean over a head's dv value channels, w [dv] a weight shared by the heads and
  z [.., H, dv] the output-gate pre-activation.

Every step is computed in fp64 and the recurrence itself is ``oracle.recurrent``
fed in fp64, so nothing here is rounded below fp64.
"""
from __future__ import annotations

import numpy as np

from . import recurrent


def widen(x):
    """bf16 bit patterns (uint16) or any float array -> fp64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def l2_normalize(x, eps):
    """Per-token, per-head L2 normalisation over the last axis ("Kimi Delta Attention")."""
    x = widen(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def log_alpha_from_gate(g):
    """log alpha = -softplus(g), evaluated without overflow: -(max(g, 0) + log1p(exp(-|g|)))."""
    g = widen(g)
    return -(np.maximum(g, 0.0) + np.log1p(np.exp(-np.abs(g))))


def sigmoid(z):
    z = widen(z)
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def rms_gate(o, z, w, eps):
    """Head-wise RMSNorm of o over its last axis, scaled by w and by sigmoid(z)."""
    o = np.asarray(o, np.float64)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    wt = np.ones(o.shape[-1]) if w is None else widen(w)
    return o * r * wt * sigmoid(z)


def prologue(q, k, g, qk_l2norm, l2_eps):
    """fp64 (q, k, log_alpha) the recurrence sees."""
    if qk_l2norm:
        qn, kn = l2_normalize(q, l2_eps), l2_normalize(k, l2_eps)
    else:
        qn, kn = widen(q), widen(k)
    return qn, kn, log_alpha_from_gate(g)


def forward(q, k, v, g, beta, init_state=None, cu_seqlens=None, out_gate=None, norm_weight=None,
            qk_l2norm=True, l2_eps=1e-6, rms_eps=1e-6, threads=None):
    """The layer around the recurrence, fp64 throughout.

    q, k [T, H, dk], v [T, H, dv] (fp32 or bf16 bits, or fp64); g [T, H, dk] or
    [T, H] (gate pre-activation); beta [T, H]; init_state [N, H, dk, dv] or None;
    out_gate [T, H, dv] or None (no epilogue: y = o); norm_weight [dv] or None
    (ones).  A leading batch axis is accepted when cu_seqlens is None.
    Returns (y, final_state, o), all fp64.
    """
    qn, kn, la = prologue(q, k, g, qk_l2norm, l2_eps)
    o, S = recurrent(qn, kn, widen(v), la, widen(beta), init_state, cu_seqlens, threads)
    y = o if out_gate is None else rms_gate(o, out_gate, norm_weight, rms_eps)
    return y, S, o


def decode_steps(state, steps, norm_weight=None, epilogue=True, qk_l2norm=True, l2_eps=1e-6,
                 rms_eps=1e-6, threads=None):
    """Consecutive one-token layer steps of N sequences (state carried in fp64).

    ``steps``: dicts with q, k [N, H, dk], v [N, H, dv], g [N, H, dk] or [N, H],
    beta [N, H] and, when ``epilogue`` is on, out_gate [N, H, dv].
    Returns (list of fp64 outputs [N, H, dv], fp64 final state).
    """
    S = np.asarray(state, np.float64)
    cu = np.arange(S.shape[0] + 1, dtype=np.int64)
    outs = []
    for st in steps:
        z = st["out_gate"] if epilogue else None
        y, S, _ = forward(st["q"], st["k"], st["v"], st["g"], st["beta"], S, cu, z, norm_weight,
                          qk_l2norm, l2_eps, rms_eps, threads)
        outs.append(y)
    return outs, S
