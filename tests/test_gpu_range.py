"""bf16 inputs with values past the fp16 matrix-core operands' range, through the C ABI (needs an MI355X).

With KDA_CHECK=1 the prefill, the fused layer and the backward measure max|v| and
max|initial state| on the device; past 1024 they run with fp32 matrix-core operands
and records, and match the fp64 oracle at the bf16 bar (2e-2) for |v| up to about 4e5
(v ~ 1e5 N(0, 1)).  Without KDA_CHECK the fp16 operands overflow, and the result is
non-finite rather than wrong.  With KDA_CHECK=1 and ordinary values the fp16 path
runs unchanged (bit-identical results).
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import layer as olayer
from synth import random_small

from kda_testlib import TOL, assert_close, run_chunk, to_dev, nan_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCALE = 1.0e5


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd as m
    m._lib.lib()
    return m


def _large(d):
    """v scaled by 1e5 (rounded to bf16) and the initial state by 1e5."""
    d = dict(d)
    d["v"] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(d["v"]) * np.float32(SCALE))
    if d.get("init") is not None:
        d["init"] = (d["init"] * SCALE).astype(np.float32)
    return d


@pytest.mark.parametrize("T,H,D,lens", [(300, 2, 128, None), (0, 2, 64, [70, 0, 130, 64])])
def test_prefill_large_values_under_check(kda, monkeypatch, T, H, D, lens):
    monkeypatch.setenv("KDA_CHECK", "1")
    d = _large(random_small(61, T, H, D, D, "bf16", init_std=0.02, lens=lens))
    assert np.abs(synth.bf16_bits_to_f32(d["v"])).max() > 6.5e4
    o, S = run_chunk(kda, torch, d)
    ro, rS = oracle.recurrent(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["init"], d["cu_seqlens"])
    assert_close("out", o, ro, TOL["bf16"])
    assert_close("final_state", S, rS, TOL["bf16"])


def test_prefill_large_values_without_check_not_silent(kda, monkeypatch):
    """No KDA_CHECK: the fp16 operands overflow; some output or state entry is non-finite
    (or, if nothing overflowed, the result passes the bar)."""
    monkeypatch.delenv("KDA_CHECK", raising=False)
    d = _large(random_small(62, 300, 2, 128, 128, "bf16", init_std=0.02))
    o, S = run_chunk(kda, torch, d)
    if np.isfinite(o).all() and np.isfinite(S).all():
        ro, rS = oracle.recurrent(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["init"])
        assert_close("out", o, ro, TOL["bf16"])
        assert_close("final_state", S, rS, TOL["bf16"])


def test_check_keeps_fp16_path_for_ordinary_values(kda, monkeypatch):
    d = random_small(63, 300, 2, 128, 128, "bf16", init_std=0.02)
    monkeypatch.delenv("KDA_CHECK", raising=False)
    o1, S1 = run_chunk(kda, torch, d)
    monkeypatch.setenv("KDA_CHECK", "1")
    o2, S2 = run_chunk(kda, torch, d)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_layer_large_values_under_check(kda, monkeypatch):
    monkeypatch.setenv("KDA_CHECK", "1")
    d = synth.layer_small(64, 260, 2, 128, 128, "bf16")
    d["v"] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(d["v"]) * np.float32(SCALE))
    q, k, v, g, b = (to_dev(d[x], torch).unsqueeze(0) for x in ("q", "k", "v", "g", "beta"))
    og = to_dev(d["out_gate"], torch).unsqueeze(0)
    w = to_dev(d["norm_weight"], torch)
    init = None if d.get("init") is None else to_dev(d["init"], torch)
    y = nan_tensor(torch, v.shape)
    fin = nan_tensor(torch, (1, 2, 128, 128))
    y, fin = kda.layer_fwd(q, k, v, g, b, init, None, out_gate=og, norm_weight=w, out=y, final_state=fin)
    torch.cuda.synchronize()
    ry, rS, _ = olayer.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d.get("init"), None, d["out_gate"],
                               d["norm_weight"], True)
    assert_close("y", y[0].cpu().numpy(), ry, TOL["bf16"])
    assert_close("final_state", fin.cpu().numpy(), rS, TOL["bf16"])
    # bf16 y with the epilogue: o would pass through fp16 in the output buffer, refused
    with pytest.raises(kda.KdaError):
        kda.layer_fwd(q, k, v, g, b, init, None, out_gate=og, norm_weight=w, out_dtype=torch.bfloat16)


def test_backward_large_values_under_check(kda, monkeypatch):
    monkeypatch.setenv("KDA_CHECK", "1")
    d = _large(random_small(65, 200, 2, 128, 128, "bf16", init_std=0.02))
    r = np.random.default_rng(65)
    dO = r.standard_normal((200, 2, 128)).astype(np.float32)
    dF = r.standard_normal((1, 2, 128, 128)).astype(np.float32)
    q, k, v, la, b = (to_dev(d[x], torch).unsqueeze(0) for x in ("q", "k", "v", "log_alpha", "beta"))
    init = to_dev(d["init"], torch)
    bufs = {"dq": q.shape, "dk": q.shape, "dv": v.shape, "dlog_alpha": la.shape, "dbeta": b.shape,
            "d_init": (1, 2, 128, 128)}
    out = {x: nan_tensor(torch, shp) for x, shp in bufs.items()}
    g = kda.chunk_bwd(q, k, v, la, b, to_dev(dO, torch).unsqueeze(0), init, to_dev(dF, torch), None, out=out)
    torch.cuda.synchronize()
    ref = oracle.backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], synth.as_f64(dO), d["init"], dF,
                          d["cu_seqlens"])
    for gk, rk in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dlog_alpha", "dlog_alpha"), ("dbeta", "dbeta"),
                   ("d_init", "dinit")):
        got = g[gk].cpu().numpy()
        assert_close(gk, got[0] if gk != "d_init" else got, ref[rk], TOL["bf16"])
