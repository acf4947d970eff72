"""Pins of the oracle's reverse mode (kda_oracle_backward) against facts outside it (CPU only).

The gradients are those of L = sum(dO * O) + sum(dS_T * S_T) through the KDA
recurrence ("Kimi Linear" page, "Kimi Delta Attention").  Pins:

* central finite differences of L, in fp64, for every element of every input
  (q, k, v, log_alpha, beta, the initial state) on a small varlen problem --
  the gradient's definition, independent of the adjoint code;
* the closed form of one token from a zero state (every term of the adjoint,
  including the initial-state gradient Diag(alpha)(q - beta (q.k) k) dO^T);
* a per-head gate receives the sum of the per-channel gradients;
* a segment boundary of the checkpointed recomputation (70 tokens) changes
  nothing: the gradients equal those of the same problem solved in one piece
  by finite differences;
* PyTorch's fp64 reverse mode through a plain token loop, on sequences that
  span several checkpoint segments.
"""
import numpy as np
import pytest

import oracle


def _problem(seed, lens, H, dk, dv, gate=0.3, per_head=False):
    r = np.random.default_rng(seed)
    T = int(sum(lens))
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, H, dv))
    la = -gate * r.random((T, H) if per_head else (T, H, dk))
    b = r.random((T, H))
    N = len(lens)
    S0 = 0.3 * r.standard_normal((N, H, dk, dv))
    dO = r.standard_normal((T, H, dv))
    dF = r.standard_normal((N, H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return dict(q=q, k=k, v=v, la=la, b=b, S0=S0, dO=dO, dF=dF, cu=cu)


def _loss(p, **over):
    x = dict(p, **over)
    o, S = oracle.recurrent(x["q"], x["k"], x["v"], x["la"], x["b"], x["S0"], x["cu"], threads=1)
    return float(np.sum(x["dO"] * o) + np.sum(x["dF"] * S))


def _fd(p, name, eps=1e-6):
    base = p[name]
    g = np.zeros_like(base)
    it = np.nditer(base, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp = base.copy(); xp[i] += eps
        xm = base.copy(); xm[i] -= eps
        g[i] = (_loss(p, **{name: xp}) - _loss(p, **{name: xm})) / (2 * eps)
    return g


def _grads(p):
    return oracle.backward(p["q"], p["k"], p["v"], p["la"], p["b"], p["dO"], p["S0"], p["dF"], p["cu"], threads=1)


@pytest.mark.parametrize("per_head", [False, True])
def test_backward_matches_finite_differences(per_head):
    p = _problem(1, [5, 0, 4], H=2, dk=4, dv=3, per_head=per_head)
    g = _grads(p)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("la", "dlog_alpha"), ("b", "dbeta"),
                      ("S0", "dinit")):
        fd = _fd(p, name)
        err = np.abs(g[key] - fd).max()
        assert err < 1e-7 * max(1.0, np.abs(fd).max()), (name, err)


def test_backward_single_token_closed_form():
    r = np.random.default_rng(2)
    dk, dv = 5, 4
    q = r.standard_normal((1, 1, dk)); k = r.standard_normal((1, 1, dk)); v = r.standard_normal((1, 1, dv))
    la = -r.random((1, 1, dk)); b = np.array([[0.7]]); dO = r.standard_normal((1, 1, dv))
    g = oracle.backward(q, k, v, la, b, dO, np.zeros((1, 1, dk, dv)), None, threads=1)
    qv, kv, vv, ov, a = q[0, 0], k[0, 0], v[0, 0], dO[0, 0], np.exp(la[0, 0])
    qk, dov = qv @ kv, ov @ vv
    assert np.allclose(g["dq"][0, 0], 0.7 * dov * kv, atol=1e-14)
    assert np.allclose(g["dk"][0, 0], 0.7 * dov * qv, atol=1e-14)
    assert np.allclose(g["dv"][0, 0], 0.7 * qk * ov, atol=1e-14)
    assert g["dbeta"][0, 0] == pytest.approx(qk * dov, abs=1e-14)
    assert np.allclose(g["dlog_alpha"], 0.0, atol=1e-15)
    dS0 = a[:, None] * np.outer(qv - 0.7 * qk * kv, ov)
    assert np.allclose(g["dinit"][0, 0], dS0, atol=1e-14)


def test_backward_across_checkpoint_segments():
    """70 tokens cross the 64-token checkpoint boundary of the recomputation."""
    p = _problem(3, [70], H=1, dk=3, dv=2, gate=0.05)
    g = _grads(p)
    for name, key in (("la", "dlog_alpha"), ("S0", "dinit"), ("b", "dbeta")):
        fd = _fd(p, name)
        assert np.abs(g[key] - fd).max() < 1e-7 * max(1.0, np.abs(fd).max()), name


@pytest.mark.parametrize("per_head", [False, True])
def test_backward_matches_autograd(per_head):
    """Reverse mode of PyTorch (fp64, CPU) through a plain token loop of the recurrence, on a
    problem long enough to span several checkpoint segments (200 and 70 tokens, an empty
    sequence between them): shares nothing with the oracle's adjoint but the definition."""
    torch = pytest.importorskip("torch")
    p = _problem(4, [200, 0, 70], H=2, dk=8, dv=6, gate=0.2, per_head=per_head)
    t = {x: torch.tensor(p[x], dtype=torch.float64, requires_grad=True) for x in ("q", "k", "v", "la", "b", "S0")}
    loss = torch.zeros((), dtype=torch.float64)
    cu = p["cu"]
    for n in range(len(cu) - 1):
        for h in range(2):
            S = t["S0"][n, h]
            for i in range(int(cu[n]), int(cu[n + 1])):
                kk, qq, vv, bb = t["k"][i, h], t["q"][i, h], t["v"][i, h], t["b"][i, h]
                a = torch.exp(t["la"][i, h]) * torch.ones_like(kk)  # one gate per head broadcasts
                S = a[:, None] * S                                   # Diag(alpha) S
                S = S - bb * torch.outer(kk, kk @ S) + bb * torch.outer(kk, vv)
                loss = loss + torch.dot(torch.as_tensor(p["dO"][i, h]), S.t() @ qq)
            loss = loss + torch.sum(torch.as_tensor(p["dF"][n, h]) * S)
    loss.backward()
    g = _grads(p)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("la", "dlog_alpha"), ("b", "dbeta"),
                      ("S0", "dinit")):
        ref = t[name].grad.numpy()
        assert np.abs(g[key] - ref).max() < 1e-10 * max(1.0, np.abs(ref).max()), name
