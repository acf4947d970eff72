"""HIP reverse mode of the chunked prefill vs the fp64 oracle's (``oracle.backward``), through the C ABI.

Gradients of L = sum(dO * out) + sum(dS_T * final_state) with respect to q, k,
v, log_alpha, beta and the initial state.  Each gradient tensor is compared
element by element at the forward's bars: max|gpu - oracle| / RMS(oracle)
<= 1e-4 with fp32 inputs, 2e-2 with bf16 inputs (the recomputed states come
from the same fp16-operand state pass as the forward's).
"""
import numpy as np
import pytest

import oracle
import synth
from synth import WORKLOADS, random_small

from kda_testlib import TOL, assert_close, assert_metrics, to_dev, nan_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

KEYS = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dlog_alpha", "dlog_alpha"), ("dbeta", "dbeta"),
        ("d_init", "dinit"))


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd as m
    m._lib.lib()
    return m


def _grads(seed, d, d_out_bf16=False, with_final=True):
    r = np.random.default_rng(seed)
    T, H, dv = d["v"].shape
    N = len(d["cu_seqlens"]) - 1
    dO = r.standard_normal((T, H, dv)).astype(np.float32)
    if d_out_bf16:
        dO = synth.f32_to_bf16_bits(dO)
    dF = r.standard_normal((N, H, dv, dv)).astype(np.float32) if with_final else None
    return dO, dF


def run_bwd(kda, d, dO, dF, max_seqlen=None):
    q, k, v, la, b = (to_dev(d[x], torch).unsqueeze(0) for x in ("q", "k", "v", "log_alpha", "beta"))
    cu = d["cu_seqlens"]
    varlen = len(cu) != 2
    cu_t = torch.from_numpy(np.asarray(cu, np.int32)).cuda() if varlen else None
    init = None if d.get("init") is None else to_dev(d["init"], torch)
    N, (H, dk), dv = len(cu) - 1, q.shape[2:], v.shape[3]
    # NaN-filled gradient buffers: an element the kernels never write fails the comparison
    bufs = {"dq": q.shape, "dk": q.shape, "dv": v.shape, "dlog_alpha": la.shape, "dbeta": b.shape,
            "d_init": (N, H, dk, dv)}
    out = {x: nan_tensor(torch, shp) for x, shp in bufs.items()}
    g = kda.chunk_bwd(q, k, v, la, b, to_dev(dO, torch).unsqueeze(0), init,
                      None if dF is None else to_dev(dF, torch), cu_t, max_seqlen=max_seqlen, out=out)
    torch.cuda.synchronize()
    return {x: t.cpu().numpy() for x, t in g.items()}


def oracle_bwd(d, dO, dF):
    N = len(d["cu_seqlens"]) - 1
    H, dk = d["q"].shape[1], d["q"].shape[2]
    init = d.get("init")
    if init is None:
        init = np.zeros((N, H, dk, d["v"].shape[2]))
    return oracle.backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], synth.as_f64(dO), init,
                           None if dF is None else dF, d["cu_seqlens"])


def check(g, ref, tol):
    for gk, rk in KEYS:
        got = g[gk][0] if gk not in ("d_init",) else g[gk]
        assert_close(gk, got, ref[rk], tol)


def check_terms_scale(g, ref, d, dF, tol, bf16):
    """check() for gates past any floor, with two gradients measured against the terms they
    are formed from rather than their own RMS, which the strong gates make vanish:

    * dlog_alpha is a reverse cumulative sum of q o dq and k o dk terms that cancel where the
      gates are strong (at log alpha = -30 per token its RMS is ~1e-14 against terms of order
      1), so its max error is taken over max(RMS(dlog_alpha), RMS(q o dq), RMS(k o dk));
    * with bf16 inputs the reverse chain takes fp16 operands, which cannot hold contributions
      below fp16's smallest subnormal (2^-24) of their scale: d_init, which strong gates
      shrink to ~1e-13, is measured against max(RMS(d_init), 2^-20 RMS(d_final)).

    Every other gradient keeps the plain bar (oracle values throughout)."""
    rms = lambda x: float(np.sqrt(np.mean(np.square(x)))) if np.size(x) else 0.0

    def bounded(name, got, ref_x, scale):
        got = np.asarray(got, np.float64)
        assert np.isfinite(got).all(), f"{name}: non-finite values"
        err = float(np.max(np.abs(got - ref_x))) if got.size else 0.0
        assert err <= tol * scale, f"{name}: max|err| {err:.3e} > {tol:.1e} x {scale:.3e}"

    for gk, rk in KEYS:
        got = g[gk][0] if gk not in ("d_init",) else g[gk]
        if gk == "dlog_alpha":
            q, k = synth.as_f64(d["q"]), synth.as_f64(d["k"])
            if ref[rk].ndim == 2:  # one gate per head: the sums over the key channels
                terms = max(rms((q * ref["dq"]).sum(-1)), rms((k * ref["dk"]).sum(-1)))
            else:
                terms = max(rms(q * ref["dq"]), rms(k * ref["dk"]))
            bounded(gk, got, ref[rk], max(rms(ref[rk]), terms))
        elif gk == "d_init" and bf16:
            bounded(gk, got, ref[rk], max(rms(ref[rk]), 2.0 ** -20 * rms(dF)))
        else:
            assert_close(gk, got, ref[rk], tol)


@pytest.mark.parametrize("T,H,D,dtype,lens,gate", [
    (130, 2, 64, "f32", None, "channel"),
    (200, 2, 128, "bf16", None, "channel"),
    (0, 3, 64, "f32", [1, 0, 64, 70], "channel"),
    (0, 2, 128, "bf16", [65, 0, 190, 3], "channel"),
    (150, 2, 64, "f32", None, "head"),
    (0, 2, 128, "bf16", [100, 37], "head"),
])
def test_backward_small(kda, T, H, D, dtype, lens, gate):
    d = random_small(T * 7 + D + H, T, H, D, D, dtype=dtype, lens=lens, gate=gate)
    dO, dF = _grads(5 + T, d)
    g = run_bwd(kda, d, dO, dF)
    check(g, oracle_bwd(d, dO, dF), TOL[dtype])


def test_backward_bf16_dout_zero_init(kda):
    """d_out in bf16 (the dtype out had), no initial state, no final-state gradient."""
    d = random_small(61, 300, 2, 128, 128, dtype="bf16", init_std=None)
    dO, dF = _grads(62, d, d_out_bf16=True, with_final=False)
    g = run_bwd(kda, d, dO, dF)
    check(g, oracle_bwd(d, dO, dF), TOL["bf16"])


def test_backward_strong_decay(kda):
    """Gates down to about -10 per token: the anchored decay factors at their range."""
    d = random_small(71, 256, 2, 128, 128, dtype="bf16", gate_scale=4.0)
    dO, dF = _grads(72, d)
    g = run_bwd(kda, d, dO, dF)
    check(g, oracle_bwd(d, dO, dF), TOL["bf16"])


def _wide_gates(kind, shape, rng):
    """log alpha past any floor: uniform -30, channels split between -0.01 and -60, a draw
    uniform in [-20, 0] per token, and the more extreme draws of the precision test below."""
    if kind == "uniform30":
        return np.full(shape, -30.0, np.float32)
    if kind == "mixed":
        la = np.full(shape, -0.01, np.float32)
        la[..., 1::2] = -60.0
        return la
    if kind == "wild20":
        return (-20.0 * rng.random(shape)).astype(np.float32)
    if kind == "wild200":
        return (-200.0 * rng.random(shape)).astype(np.float32)
    la = (-0.05 * rng.random(shape)).astype(np.float32)  # "spikes"
    la[5::64] = -1.0e4
    la[37::64, :, ::3] = -80.0
    return la


def chunk_decay_max(d, chunk=64):
    """G*: the largest |sum of log alpha| over the tokens of one 64-token chunk (per sequence,
    head and channel) -- the magnitude of the backward's prefix sums G inside a chunk."""
    la = np.asarray(d["log_alpha"], np.float64)
    cu = d["cu_seqlens"]
    best = 0.0
    for s0, s1 in zip(cu[:-1], cu[1:]):
        for c0 in range(int(s0), int(s1), chunk):
            best = max(best, float(np.max(np.abs(la[c0:min(c0 + chunk, int(s1))].sum(axis=0)))))
    return best


def fp32_bar(d):
    """The backward's bar with fp32 inputs: its decay factors are exponentials of differences of
    fp32 prefix sums G, so each exponent carries up to about ulp(G*) ~ 2^-23 G*, and the sums a
    gradient is formed from cancel by a few times more; the bar is max(1e-4, 2^-20 G*) -- the
    plain bar up to G* of about 100 (a chunk-local decay of e^-100), in proportion beyond it."""
    return max(TOL["f32"], 2.0 ** -20 * chunk_decay_max(d))


def _run_wide(kda, kind, dtype, seed):
    d = random_small(seed, 0, 2, 128, 128, dtype=dtype, init_std=0.5, lens=[200, 64, 1, 135])
    d["log_alpha"] = _wide_gates(kind, d["log_alpha"].shape, np.random.default_rng(9))
    dO, dF = _grads(seed + 50, d)
    return d, dF, run_bwd(kda, d, dO, dF), oracle_bwd(d, dO, dF)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["uniform30", "mixed", "wild20", "wild200", "spikes"])
def test_backward_full_gate_domain(kda, kind, dtype):
    """Every gradient with gates past any floor (uniform -30; channels at -0.01 and -60; uniform
    in [-20, 0] and [-200, 0] per token; one token per chunk at -1e4): the diagonal blocks whose
    single-anchor exponents pass the limit are formed level by level (every exponent <= 0).
    Bars: 2e-2 with bf16 inputs; with fp32 inputs fp32_bar (1e-4 up to a chunk-local cumulative
    decay of about 100, then in proportion to it)."""
    seed = {"uniform30": 601, "mixed": 603, "wild20": 605, "wild200": 621, "spikes": 623}[kind] + (dtype == "bf16")
    d, dF, g, ref = _run_wide(kda, kind, dtype, seed)
    check_terms_scale(g, ref, d, dF, TOL["bf16"] if dtype == "bf16" else fp32_bar(d), dtype == "bf16")


def test_backward_full_gate_domain_d64_head_gate(kda):
    """The same at d = 64 and with one gate per head, gates uniform in [-20, 0] per token."""
    for gate, dtype in (("channel", "f32"), ("head", "bf16"), ("head", "f32")):
        d = random_small(411, 0, 3, 64, 64, dtype=dtype, init_std=0.5, lens=[130, 77], gate=gate)
        d["log_alpha"] = (-20.0 * np.random.default_rng(4).random(d["log_alpha"].shape)).astype(np.float32)
        dO, dF = _grads(412, d)
        g = run_bwd(kda, d, dO, dF)
        check_terms_scale(g, oracle_bwd(d, dO, dF), d, dF, TOL["bf16"] if dtype == "bf16" else fp32_bar(d),
                          dtype == "bf16")


def test_backward_workload1(kda):
    """4K tokens x 32 heads (bf16): every gradient element."""
    w = WORKLOADS[1]
    d = synth.make_prefill(w)
    dO, dF = _grads(81, d)
    g = run_bwd(kda, d, dO, dF)
    check(g, oracle_bwd(d, dO, dF), TOL["bf16"])


def test_backward_workload2_every_head(kda):
    """64K tokens x 32 heads (bf16), the benchmark's launch: every element of every gradient.
    Heads are independent, so the oracle runs on 16 heads at a time and the figures
    accumulate over the two groups (no fp64 copy of all 32 heads is held)."""
    w = WORKLOADS[2]
    d = synth.make_prefill(w)
    dO, dF = _grads(91, d)
    g = run_bwd(kda, d, dO, dF)
    acc = {gk: oracle.Metrics() for gk, _ in KEYS}
    for h0 in (0, 16):
        heads = list(range(h0, h0 + 16))
        print(f"  oracle backward, heads {h0}..{h0 + 15}", flush=True)
        sub = {x: d[x][:, heads] for x in ("q", "k", "v", "log_alpha", "beta")}
        sub.update(cu_seqlens=d["cu_seqlens"], init=d["init"][:, heads])
        ref = oracle_bwd(sub, dO[:, heads], dF[:, heads])
        for gk, rk in KEYS:
            got = g[gk][:, heads] if gk == "d_init" else g[gk][0][:, heads]
            assert np.isfinite(got).all(), f"{gk}: non-finite values"
            acc[gk].add(got, ref[rk])
        del ref
    for gk, _ in KEYS:
        assert_metrics(gk, acc[gk], TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_d64_long(kda, dtype):
    """Head dimension 64 at length: 8,192 tokens x 8 heads (128-chunk reverse chain), every
    gradient element."""
    d = random_small(131, 8192, 8, 64, 64, dtype=dtype, init_std=0.02)
    dO, dF = _grads(132, d)
    g = run_bwd(kda, d, dO, dF)
    check(g, oracle_bwd(d, dO, dF), TOL[dtype])


@pytest.mark.parametrize("B,T,D,dtype", [(3, 130, 64, "f32"), (2, 100, 128, "bf16")])
def test_backward_dense_batch(kda, B, T, D, dtype):
    """A dense batch [B, T, H, d] (no cu_seqlens): the same gradients as the B sequences packed."""
    H = 2
    d = random_small(B * 31 + D, 0, H, D, D, dtype=dtype, lens=[T] * B)
    dO, dF = _grads(97, d)
    dense = lambda x: to_dev(x, torch).reshape((B, T) + x.shape[1:])
    q, k, v, la, b = (dense(d[x]) for x in ("q", "k", "v", "log_alpha", "beta"))
    g = kda.chunk_bwd(q, k, v, la, b, dense(dO), to_dev(d["init"], torch), to_dev(dF, torch))
    torch.cuda.synchronize()
    ref = oracle_bwd(d, dO, dF)
    for gk, rk in KEYS:
        got = g[gk].cpu().numpy()
        if gk != "d_init":
            got = got.reshape((B * T,) + got.shape[2:])
        assert_close(gk, got, ref[rk], TOL[dtype])


def test_backward_varlen_windows(kda):
    """32 heads (bf16), sequences of 8,192 and 5,000 tokens: the forward recompute runs in
    three record windows and the shorter sequence ends inside the second; two heads checked."""
    H = 32
    d = random_small(123, 0, H, 128, 128, dtype="bf16", lens=[8192, 5000])
    dO, dF = _grads(124, d)
    g = run_bwd(kda, d, dO, dF)
    heads = [5, 30]
    sub = {x: d[x][:, heads] for x in ("q", "k", "v", "log_alpha", "beta")}
    sub.update(cu_seqlens=d["cu_seqlens"], init=d["init"][:, heads])
    ref = oracle_bwd(sub, dO[:, heads], dF[:, heads])
    for gk, rk in KEYS:
        got = g[gk][:, heads] if gk == "d_init" else g[gk][0][:, heads]
        assert_close(gk, got, ref[rk], TOL["bf16"])


@pytest.mark.parametrize("D,dtype,window", [(128, "bf16", "2"), (64, "f32", "3"), (128, "bf16", "5")])
def test_backward_windows_same_bits(kda, monkeypatch, D, dtype, window):
    """Backward windows of a few chunks (state checkpoints, carried dL/dS, per-window recompute)
    give the same bits as one window; sequences end inside, at the edge of and before a window."""
    d = random_small(D + int(window), 0, 3, D, D, dtype=dtype, lens=[700, 0, 130, 64, 1000, 1])
    dO, dF = _grads(131, d)
    monkeypatch.delenv("KDA_BWD_WINDOW", raising=False)
    one = run_bwd(kda, d, dO, dF)
    monkeypatch.setenv("KDA_BWD_WINDOW", window)
    win = run_bwd(kda, d, dO, dF)
    for gk, _ in KEYS:
        assert np.array_equal(one[gk], win[gk]), gk
    check(win, oracle_bwd(d, dO, dF), TOL[dtype])


def test_backward_windows_span_record_windows(kda, monkeypatch):
    """32 heads, sequences of 8,192 and 5,000 tokens: a record window holds 48 chunks of both
    sequences, so a request for 100-chunk backward windows gets 96, two record windows each; the
    shorter sequence ends inside the first backward window.  Same bits as one window."""
    H = 32
    d = random_small(123, 0, H, 128, 128, dtype="bf16", lens=[8192, 5000])
    dO, dF = _grads(124, d)
    monkeypatch.delenv("KDA_BWD_WINDOW", raising=False)
    one = run_bwd(kda, d, dO, dF, max_seqlen=8192)
    monkeypatch.setenv("KDA_BWD_WINDOW", "100")
    win = run_bwd(kda, d, dO, dF, max_seqlen=8192)
    for gk, _ in KEYS:
        assert np.array_equal(one[gk], win[gk]), gk


def test_backward_workload4_varlen_1m(kda):
    """1M packed tokens in 16 Dirichlet-length sequences, four of the 32 heads (heads are
    independent; the generator reproduces a head subset exactly): every gradient element against
    the oracle.  Holding every chunk at once would take about 105 GB here, so the backward runs in
    five windows of 960 chunks with a state checkpoint entering each."""
    w = WORKLOADS[4]
    heads = (0, 11, 22, 31)
    d = synth.make_prefill(w, heads=heads)
    lens = np.diff(d["cu_seqlens"])
    assert len(lens) == 16 and int(lens.sum()) == w.seqlen
    dO, dF = _grads(141, d)
    n_ws = kda.bwd_workspace_size(1, w.seqlen, len(heads), w.dk, w.dv, torch.bfloat16, torch.float32,
                                  num_seqs=16, max_seqlen=int(lens.max()))
    assert n_ws < 30 * (1 << 30)
    g = run_bwd(kda, d, dO, dF, max_seqlen=int(lens.max()))
    check(g, oracle_bwd(d, dO, dF), TOL["bf16"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_beta_up_to_two(kda, dtype):
    """beta uniform in [0, 2]: gradients against the oracle's adjoint."""
    d = random_small(151 if dtype == "f32" else 152, 200, 2, 128, 128, dtype=dtype)
    d["beta"] = np.random.default_rng(6).uniform(0.0, 2.0, d["beta"].shape).astype(np.float32)
    dO, dF = _grads(153, d)
    g = run_bwd(kda, d, dO, dF)
    check(g, oracle_bwd(d, dO, dF), TOL[dtype])
