"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Small cases span several 64-token chunks, partial chunks and empty
sequences; the workload cases run the exact shapes and launch configuration
the benchmark times.  Every output and final state is compared element by
element with max|gpu - oracle| / RMS(oracle) <= 1e-4 (fp32 inputs) or 2e-2
(bf16 inputs); decode, which is fp32 arithmetic throughout, must meet 1e-4.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import WORKLOADS, random_small

from kda_testlib import (DECODE_TOL, TOL, assert_close, assert_metrics, nan_tensor, oracle_chunk, run_chunk,
                         to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd as m
    m._lib.lib()
    return m


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("N,H,D,dtype", [(1, 1, 64, "f32"), (5, 3, 64, "bf16"), (4, 2, 128, "f32"),
                                         (16, 4, 128, "bf16")])
def test_decode_small(kda, N, H, D, dtype):
    st = synth.gen_tokens(11 + N, N, H, D, D, dtype, 0.05)
    S0 = synth.gen_states(11 + N, N, H, D, D, 0.5)
    args = [to_dev(st[x], torch) for x in ("q", "k", "v", "log_alpha", "beta")]
    state = to_dev(S0, torch)
    outs, ref_outs = [], []
    S = S0
    for step in range(3):
        outs.append(kda.decode_step(*args, state, out=nan_tensor(torch, args[2].shape)).cpu().numpy())
        o, S = oracle.decode_steps(S, [st])
        ref_outs.append(o[0])
    torch.cuda.synchronize()
    for i in range(3):
        assert_close(f"out{i}", outs[i], ref_outs[i], DECODE_TOL)
    assert_close("state", state.cpu().numpy(), S, DECODE_TOL)


def test_decode_workload_100_steps(kda):
    """256 sequences x 32 heads, 100 distinct steps, state in place: every output of every step
    and every state element (all 8,192 units) against the oracle.  The oracle runs 32 sequences
    at a time and the figures accumulate piece by piece, so no full fp64 copy is held."""
    w = WORKLOADS[3]
    S0 = synth.make_decode_state(w)
    state = to_dev(S0, torch)
    steps = [synth.make_decode_step(w, s) for s in range(w.steps)]
    outs = []
    for st in steps:
        args = [to_dev(st[x], torch) for x in ("q", "k", "v", "log_alpha", "beta")]
        outs.append(kda.decode_step(*args, state, out=nan_tensor(torch, args[2].shape)))
    torch.cuda.synchronize()
    S_gpu = state.cpu().numpy()
    mo, ms = oracle.Metrics(), oracle.Metrics()
    for s0 in range(0, w.batch, 32):
        sl = slice(s0, s0 + 32)
        S = S0[sl]
        for i, st in enumerate(steps):
            o, S = oracle.decode_steps(S, [{x: y[sl] for x, y in st.items()}])
            mo.add(outs[i][sl].cpu().numpy(), o[0])
        ms.add(S_gpu[sl], S)
    assert mo.count == w.steps * w.batch * w.heads * w.dv and ms.count == S0.size
    assert_metrics("outputs x100", mo, DECODE_TOL)
    assert_metrics("state", ms, DECODE_TOL)


# ----------------------------------------------------------------------------
# chunked prefill: small and edge cases
# ----------------------------------------------------------------------------

CASES = [
    # (T, H, D, dtype, init, lens)
    (1, 1, 64, "f32", False, None), (63, 2, 64, "f32", True, None), (64, 1, 128, "f32", True, None),
    (65, 2, 128, "f32", False, None), (129, 1, 64, "bf16", True, None), (127, 2, 128, "bf16", True, None),
    (300, 3, 128, "bf16", True, None), (513, 2, 64, "bf16", False, None),
    (0, 2, 64, "f32", True, [0, 5, 64, 1, 65, 130]), (0, 3, 128, "bf16", True, [1, 0, 64, 200, 63, 129, 0]),
]


@pytest.mark.parametrize("T,H,D,dtype,init,lens", CASES)
def test_chunk_small(kda, T, H, D, dtype, init, lens):
    d = random_small(T * 7 + D + H, T, H, D, D, dtype=dtype, init_std=0.02 if init else None, lens=lens)
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    if o_ref.size:
        assert_close("out", o, o_ref, TOL[dtype])
    assert_close("state", S, S_ref, TOL[dtype])
    if lens is not None and d["init"] is not None:
        for s, L in enumerate(lens):
            if L == 0:  # an empty sequence hands its initial state through unchanged
                assert np.array_equal(S[s], d["init"][s])


def test_chunk_strong_decay(kda):
    """Strong gates (log_alpha down to about -10 per token): diagonal sub-blocks near the
    single-anchor form's range limit and past it."""
    d = random_small(5, 256, 2, 128, 128, dtype="bf16", gate_scale=4.0)
    assert d["log_alpha"].min() < -8
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


@pytest.mark.parametrize("la", [-50.0, -20.0, -11.0, -10.0, -1.5, -1.2, -0.8, -0.6, -0.05])
def test_chunk_diagonal_operand_range(kda, la):
    """Uniform gates across the range of the diagonal-block factors (up to e^{8|la|} over
    eight rows): from -0.8 on they exceed what fp16 operands carry accurately (at -1.2
    and -1.5 the small partner operands fall into the fp16 subnormals) and every
    workgroup takes fp32 diagonal operands; at -0.6 and -0.05 fp16 operands suffice."""
    d = random_small(21, 200, 2, 128, 128, dtype="bf16", lens=[137, 63])
    d["log_alpha"] = np.full_like(d["log_alpha"], la)
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


def _gates(kind, shape, rng):
    """Gate layouts past any floor on log alpha: uniform -30, channels split between -0.01 and
    -60, a draw up to -200 per token, and mild gates with one token per chunk near zero alpha."""
    if kind == "uniform30":
        return np.full(shape, -30.0, np.float32)
    if kind == "mixed":
        la = np.full(shape, -0.01, np.float32)
        la[..., 1::2] = -60.0
        return la
    if kind == "wild":
        return (-200.0 * rng.random(shape)).astype(np.float32)
    la = (-0.05 * rng.random(shape)).astype(np.float32)  # "spikes"
    la[5::64] = -1.0e4
    la[37::64, :, ::3] = -80.0
    return la


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["uniform30", "mixed", "wild", "spikes"])
def test_chunk_full_gate_domain(kda, kind, dtype):
    """Any finite log alpha <= 0: chunks whose single-anchor factors leave range are formed in
    the multi-level form (every factor a product of gates, at most 1) and match the oracle."""
    seed = {"uniform30": 501, "mixed": 503, "wild": 505, "spikes": 507}[kind] + (dtype == "bf16")
    d = random_small(seed, 0, 2, 128, 128, dtype=dtype, init_std=0.5, lens=[200, 64, 1, 135])
    d["log_alpha"] = _gates(kind, d["log_alpha"].shape, np.random.default_rng(7))
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL[dtype])
    assert_close("state", S, S_ref, TOL[dtype])


def test_chunk_full_gate_domain_d64_head_gate(kda):
    """The same at d = 64 and with one gate per head (Gated DeltaNet), down to -40 per token."""
    for gate, dtype in (("channel", "f32"), ("head", "bf16"), ("head", "f32")):
        d = random_small(401, 0, 3, 64, 64, dtype=dtype, init_std=0.5, lens=[130, 77], gate=gate)
        d["log_alpha"] = (-40.0 * np.random.default_rng(3).random(d["log_alpha"].shape)).astype(np.float32)
        o, S = run_chunk(kda, torch, d)
        o_ref, S_ref = oracle_chunk(d)
        assert_close(f"out {gate} {dtype}", o, o_ref, TOL[dtype])
        assert_close(f"state {gate} {dtype}", S, S_ref, TOL[dtype])


def test_chunk_workspace_windows(kda):
    """The smallest workspace (one chunk per window) gives the same bits as the default one."""
    d = random_small(8, 400, 2, 128, 128, dtype="bf16")
    o1, S1 = run_chunk(kda, torch, d)
    # a one-chunk problem with the same sequences and heads needs exactly one record per window
    need = kda.workspace_size(1, 64, 2, 128, 128, torch.bfloat16, torch.float32)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o2, S2 = run_chunk(kda, torch, d, workspace=ws)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    # a workspace of four chunk records: windows of four chunks
    state = 2 * 128 * 128 * 4
    per_chunk = need - state
    ws2 = torch.empty(state + 4 * per_chunk, dtype=torch.uint8, device="cuda")
    o3, S3 = run_chunk(kda, torch, d, workspace=ws2)
    assert np.array_equal(o1, o3) and np.array_equal(S1, S3)


def test_value_slice_widths_same_bits(kda, monkeypatch):
    """Every state-pass slice width gives the same bits: value columns never interact."""
    for dtype, D in (("bf16", 128), ("f32", 64)):
        d = random_small(41 + D, 0, 3, D, D, dtype=dtype, init_std=0.02, lens=[70, 0, 130, 64])
        ref = None
        for bv in ("16", "32", "64"):
            monkeypatch.setenv("KDA_VALUE_SLICE", bv)
            o, S = run_chunk(kda, torch, d)
            if ref is None:
                ref = (o, S)
            else:
                assert np.array_equal(o, ref[0]) and np.array_equal(S, ref[1]), (dtype, D, bv)
        monkeypatch.delenv("KDA_VALUE_SLICE")
        o_ref, S_ref = oracle_chunk(d)
        assert_close("out", ref[0], o_ref, TOL[dtype])
        assert_close("state", ref[1], S_ref, TOL[dtype])


@pytest.mark.parametrize("nseq,H", [(24, 4), (80, 4)])
def test_many_units(kda, nseq, H):
    """Enough (sequence, head) pairs for the wider default slices (32 and 64 columns)."""
    lens = [int(x) for x in np.random.default_rng(nseq).integers(0, 150, nseq)]
    d = random_small(nseq, 0, H, 128, 128, dtype="bf16", init_std=0.02, lens=lens)
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


def test_check_mode_rejects_bad_cu_seqlens(kda, monkeypatch):
    """KDA_CHECK=1 verifies cu_seqlens on the host; good inputs give the same bits."""
    d = random_small(12, 0, 2, 64, 64, dtype="f32", lens=[70, 5, 130])
    o1, S1 = run_chunk(kda, torch, d)
    monkeypatch.setenv("KDA_CHECK", "1")
    o2, S2 = run_chunk(kda, torch, d, max_seqlen=130)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    with pytest.raises(kda.KdaError, match="invalid argument"):
        run_chunk(kda, torch, d, max_seqlen=100)          # a sequence longer than max_seqlen
    bad = dict(d, cu_seqlens=np.array([0, 75, 70, 205]))  # decreasing
    with pytest.raises(kda.KdaError, match="invalid argument"):
        run_chunk(kda, torch, bad, max_seqlen=200)
    bad = dict(d, cu_seqlens=np.array([0, 70, 75, 200]))  # does not end at the token count
    with pytest.raises(kda.KdaError, match="invalid argument"):
        run_chunk(kda, torch, bad, max_seqlen=200)


def test_chunk_deterministic(kda):
    d = random_small(9, 333, 4, 128, 128, dtype="bf16")
    o1, S1 = run_chunk(kda, torch, d)
    o2, S2 = run_chunk(kda, torch, d)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_chunk_bf16_output(kda):
    d = random_small(10, 200, 2, 128, 128, dtype="bf16")
    o, S = run_chunk(kda, torch, d, out_dtype=torch.bfloat16)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out(bf16)", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


# ----------------------------------------------------------------------------
# state handoff, aliasing, varlen and decode continuation
# ----------------------------------------------------------------------------

def test_split_handoff_and_alias(kda):
    """[0, T1) then [T1, T) from the returned state equals [0, T); final may alias init."""
    T, T1 = 500, 190
    d = random_small(12, T, 2, 128, 128, dtype="bf16")
    o_ref, S_ref = oracle_chunk(d)
    a = {x: d[x][:T1] for x in ("q", "k", "v", "log_alpha", "beta")}
    a["init"] = d["init"]
    oa, Sa = run_chunk(kda, torch, a)
    b = {x: d[x][T1:] for x in ("q", "k", "v", "log_alpha", "beta")}
    b["init"] = Sa
    ob, Sb = run_chunk(kda, torch, b)
    assert_close("out", np.concatenate([oa, ob]), o_ref, TOL["bf16"])
    assert_close("state", Sb, S_ref, TOL["bf16"])
    # in-place continuation: final_state is the init_state tensor
    q, k, v, la, be = (to_dev(b[x], torch).unsqueeze(0) for x in ("q", "k", "v", "log_alpha", "beta"))
    st = to_dev(Sa, torch)
    _, fin = kda.chunk_fwd(q, k, v, la, be, st, None, out_dtype=torch.float32, final_state=st)
    torch.cuda.synchronize()
    assert fin.data_ptr() == st.data_ptr()
    assert np.array_equal(st.cpu().numpy(), Sb)


def test_varlen_matches_separate_runs(kda):
    lens = [70, 1, 128, 0, 257]
    d = random_small(13, 0, 2, 128, 128, dtype="bf16", lens=lens)
    o, S = run_chunk(kda, torch, d)
    cu = d["cu_seqlens"]
    for s in range(len(lens)):
        t0, t1 = cu[s], cu[s + 1]
        part = {x: d[x][t0:t1] for x in ("q", "k", "v", "log_alpha", "beta")}
        part["init"] = d["init"][s:s + 1]
        if t1 > t0:
            os_, Ss = run_chunk(kda, torch, part)
            np.testing.assert_allclose(o[t0:t1], os_, rtol=0, atol=1e-6 * max(1.0, np.abs(os_).max()))
            np.testing.assert_allclose(S[s], Ss[0], rtol=0, atol=1e-6 * max(1.0, np.abs(Ss).max()))


def test_prefill_then_decode(kda):
    """Decode from the prefill's final state equals prefill over one more token."""
    T = 200
    d = random_small(14, T + 1, 4, 128, 128, dtype="bf16")
    o_ref, S_ref = oracle_chunk(d)
    a = {x: d[x][:T] for x in ("q", "k", "v", "log_alpha", "beta")}
    a["init"] = d["init"]
    _, Sa = run_chunk(kda, torch, a)
    state = to_dev(Sa, torch)
    args = [to_dev(d[x][T:T + 1], torch) for x in ("q", "k", "v", "log_alpha", "beta")]
    o = kda.decode_step(*args, state, out=nan_tensor(torch, args[2].shape))
    torch.cuda.synchronize()
    assert_close("decoded token", o.cpu().numpy(), o_ref[T:T + 1], TOL["bf16"])
    assert_close("state", state.cpu().numpy(), S_ref, TOL["bf16"])


def test_pins_on_gpu(kda):
    """beta = 0 with alpha = 1 leaves the state exactly unchanged; a rewritten key returns its new value."""
    d = random_small(15, 150, 2, 128, 128, dtype="bf16")
    d["beta"][:] = 0
    d["log_alpha"][:] = 0
    _, S = run_chunk(kda, torch, d)
    assert np.array_equal(S, d["init"])
    # overwrite: one-hot key written twice (beta = 1, alpha = 1), then queried
    D = 128
    T = 70
    q = np.zeros((T, 1, D), np.float32)
    k = np.zeros((T, 1, D), np.float32)
    v = np.random.default_rng(0).standard_normal((T, 1, D)).astype(np.float32)
    for t in range(T):
        k[t, 0, t % D] = 1.0
    k[66, 0, :] = 0
    k[66, 0, 3] = 1.0    # key e3 again, in a later chunk
    q[69, 0, 3] = 1.0    # query e3 at the end
    one = {"q": q, "k": k, "v": v, "log_alpha": np.zeros((T, 1, D), np.float32),
           "beta": np.ones((T, 1), np.float32), "init": None}
    o, _ = run_chunk(kda, torch, one)
    np.testing.assert_allclose(o[69, 0], v[66, 0], atol=1e-5)


# ----------------------------------------------------------------------------
# the benchmark workloads at full size
# ----------------------------------------------------------------------------

def test_workload0_f32(kda):
    w = WORKLOADS[0]
    d = synth.make_prefill(w)
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["f32"])
    assert_close("state", S, S_ref, TOL["f32"])


def test_workload1_bf16(kda):
    w = WORKLOADS[1]
    d = synth.make_prefill(w)
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


def test_workload2_long(kda):
    """64K tokens x 32 heads with a random initial state: every output and state element."""
    w = WORKLOADS[2]
    d = synth.make_prefill(w)
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


def test_workload4_varlen_1m(kda):
    """1M packed tokens in 16 Dirichlet-length sequences with per-sequence initial states.

    Runs every token and every sequence on four of the 32 heads (each head is an
    independent unit, and the generator reproduces a head subset exactly), and
    compares every output and final-state element with the oracle.
    """
    w = WORKLOADS[4]
    heads = (0, 11, 22, 31)
    d = synth.make_prefill(w, heads=heads)
    lens = np.diff(d["cu_seqlens"])
    assert len(lens) == 16 and int(lens.sum()) == w.seqlen and lens.min() >= w.min_len
    o, S = run_chunk(kda, torch, d, max_seqlen=int(lens.max()))
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


def test_long_d64(kda):
    """Head dimension 64 at length: 65,536 tokens x 8 heads, bf16, long-memory gates and a
    random initial state (1,024-step chain in 32-column value slices), every element."""
    w = synth.Workload("kda_prefill_bf16_h8_t65536_d64", "prefill", "bf16", heads=8, dk=64, dv=64,
                       seqlen=65536, batch=1, gate_scale=0.01, init_std=0.02, seed=6)
    d = synth.make_prefill(w)
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


def test_long_single_sequence_1m(kda):
    """One sequence of 1,048,576 tokens (the context length the pages give the released model)
    on 4 heads, with the long-memory gate draw (log_alpha = -0.01 softplus(N(0,1))) and a
    random initial state: every output and final-state element against the oracle.  With
    four (sequence, head) pairs the state pass runs sequence-parallel; the 16,384-chunk chain
    bounds how far the fp16 matrix-core operands let the state drift."""
    w = synth.Workload("kda_long_bf16_h4_t1048576_d128", "prefill", "bf16", heads=4, dk=128, dv=128,
                       seqlen=1 << 20, batch=1, gate_scale=0.01, init_std=0.02, seed=5)
    d = synth.make_prefill(w)
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


# ----------------------------------------------------------------------------
# scalar (per-head) gate: the Gated DeltaNet special case on the same kernels
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,H,D,dtype,lens", [(300, 3, 128, "bf16", None), (130, 2, 64, "f32", None),
                                             (0, 3, 128, "bf16", [1, 0, 64, 200, 63, 129]),
                                             (0, 2, 64, "f32", [0, 5, 64, 65, 130])])
def test_scalar_gate_chunk(kda, T, H, D, dtype, lens):
    d = random_small(T * 3 + D + 17, T, H, D, D, dtype=dtype, lens=lens, gate="head")
    assert d["log_alpha"].ndim == 2
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL[dtype])
    assert_close("state", S, S_ref, TOL[dtype])


@pytest.mark.parametrize("N,H,D,dtype", [(5, 3, 64, "f32"), (16, 4, 128, "bf16")])
def test_scalar_gate_decode(kda, N, H, D, dtype):
    st = synth.gen_tokens(23 + N, N, H, D, D, dtype, 0.05, gate="head")
    S0 = synth.gen_states(23 + N, N, H, D, D, 0.5)
    args = [to_dev(st[x], torch) for x in ("q", "k", "v", "log_alpha", "beta")]
    state = to_dev(S0, torch)
    out = kda.decode_step(*args, state, out=nan_tensor(torch, args[2].shape)).cpu().numpy()
    o, S = oracle.decode_steps(S0, [st])
    assert_close("out", out, o[0], DECODE_TOL)
    assert_close("state", state.cpu().numpy(), S, DECODE_TOL)


def test_scalar_gate_prefill_workload(kda):
    """The 4K-token, 32-head bf16 prefill with one gate per (token, head)."""
    d = synth.make_prefill(WORKLOADS[1], gate="head")
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


# ----------------------------------------------------------------------------
# sequence-parallel state pass (few sequence-head pairs)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D,G", [("bf16", 128, "2"), ("bf16", 128, "5"), ("f32", 64, "3"),
                                       ("f32", 128, "4")])
def test_segments_forced(kda, monkeypatch, dtype, D, G):
    """KDA_SEGMENTS=G splits every sequence into G segments; ragged lengths leave some empty."""
    d = random_small(60 + D + int(G), 0, 2, D, D, dtype=dtype, init_std=0.02, lens=[0, 70, 300, 640, 129])
    monkeypatch.setenv("KDA_SEGMENTS", G)
    o, S = run_chunk(kda, torch, d, max_seqlen=640)
    monkeypatch.setenv("KDA_SEGMENTS", "0")
    o_w, S_w = run_chunk(kda, torch, d, max_seqlen=640)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL[dtype])
    assert_close("state", S, S_ref, TOL[dtype])
    assert_close("out vs windows", o, o_w, TOL[dtype])


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_segments_natural(kda, gate):
    """Two heads x 4,096 tokens: few enough pairs that the sequence-parallel pass is chosen."""
    d = random_small(77, 4096, 2, 128, 128, dtype="bf16", init_std=0.02, gate=gate, gate_scale=0.01)
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])


@pytest.mark.parametrize("B,T,H,D,dtype", [(3, 200, 2, 128, "bf16"), (2, 129, 3, 64, "f32")])
def test_dense_batch(kda, B, T, H, D, dtype):
    """A dense batch [B, T, H, d] without cu_seqlens: B independent sequences of T tokens."""
    d = random_small(90 + B + T, T, H, D, D, dtype=dtype, init_std=0.02, batch=B)
    q, k, v, la = (to_dev(d[x].reshape((B, T) + d[x].shape[1:]), torch) for x in ("q", "k", "v", "log_alpha"))
    b = to_dev(d["beta"].reshape(B, T, H), torch)
    init = to_dev(d["init"], torch)
    out, fin = kda.chunk_fwd(q, k, v, la, b, init, None, out=nan_tensor(torch, v.shape),
                             final_state=nan_tensor(torch, (B, H, D, D)))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", out.cpu().numpy().reshape(B * T, H, D), o_ref, TOL[dtype])
    assert_close("state", fin.cpu().numpy(), S_ref, TOL[dtype])


def test_many_sequences_grid_rows(kda):
    """1,100 sequences with one of 64 chunks: 1,100 x 64 rows exceed the 65,535 a launch can
    hold, so even with a workspace for every chunk the prefill runs in windows of 59 chunks."""
    lens = [4096] + [1 + (i % 3) for i in range(1099)]
    d = random_small(1100, 0, 2, 64, 64, dtype="bf16", lens=lens)
    T = int(d["cu_seqlens"][-1])
    # room for every chunk's record (41,216 bytes per chunk and head at d = 64) and the states
    ws = torch.empty(1100 * 64 * 2 * 41216 + (64 << 20), dtype=torch.uint8, device="cuda")
    o, S = run_chunk(kda, torch, d, workspace=ws, max_seqlen=4096)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["bf16"])
    assert_close("state", S, S_ref, TOL["bf16"])
    assert T == 4096 + sum(lens[1:])



def test_most_sequences_one_launch_holds(kda):
    """65,535 sequences of 0 to 3 tokens (the most a launch's grid rows hold: one chunk index
    per window), one head, d = 64, fp32: every output and final state."""
    lens = [int(x) for x in np.random.default_rng(65535).integers(0, 4, 65535)]
    d = random_small(77, 0, 1, 64, 64, dtype="f32", init_std=0.02, lens=lens)
    o, S = run_chunk(kda, torch, d, max_seqlen=3)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL["f32"])
    assert_close("state", S, S_ref, TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_beta_up_to_two(kda, dtype):
    """beta uniform in [0, 2] (the method allows any finite beta; 2 is a reflection): parity with
    the oracle, where the corrections of the WY form are twice as large as with beta <= 1."""
    d = random_small(27 if dtype == "f32" else 28, 300, 2, 128, 128, dtype=dtype)
    d["beta"] = np.random.default_rng(5).uniform(0.0, 2.0, d["beta"].shape).astype(np.float32)
    o, S = run_chunk(kda, torch, d)
    o_ref, S_ref = oracle_chunk(d)
    assert_close("out", o, o_ref, TOL[dtype])
    assert_close("state", S, S_ref, TOL[dtype])


def test_householder_keeps_state_norm(kda):
    """beta = 2, alpha = 1, v = 0: every step applies I - 2 k k^T to the state (unit k), an
    orthogonal map, so the Frobenius norm of each head's state is unchanged (fp32 inputs)."""
    d = random_small(31, 200, 2, 64, 64, dtype="f32")
    d["beta"][:] = 2.0
    d["log_alpha"][:] = 0.0
    d["v"][:] = 0.0
    _, S = run_chunk(kda, torch, d)
    n0 = np.linalg.norm(d["init"].reshape(2, -1), axis=1)
    n1 = np.linalg.norm(S.reshape(2, -1), axis=1)
    np.testing.assert_allclose(n1, n0, rtol=1e-4)
