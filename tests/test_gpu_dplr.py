"""General DPLR variant (kda_dplr_chunk_fwd) vs its fp64 oracle, through the C ABI (needs an MI355X).

S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T with independent a and b ("Kimi
Linear" page, "The constrained DPLR form and the chunkwise algorithm").  Cases: several
chunks with ragged tails, a dense batch, varlen with empty and one-token sequences, bf16 output, the
reduction to KDA, gates strong enough that the diagonal blocks take the form whose
factors are all at most 1 (every chunk, and single chunks among ordinary ones), a
workspace small enough for several windows, and the benchmark's shape (1 x 65,536
tokens x 16 heads, bf16), every head.  Bar: max|gpu - oracle| / RMS(oracle) <= 1e-4
(fp32 inputs) or 2e-2 (bf16 inputs) for every output and final state.
"""
import numpy as np
import pytest

import oracle
import synth

from kda_testlib import TOL, assert_close, nan_tensor, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd as m
    m._lib.lib()
    return m


def run_dplr(kda, d, out_dtype=None, final=True, workspace=None):
    q, k, v, a, b, la = (to_dev(d[x], torch).unsqueeze(0) for x in ("q", "k", "v", "a", "b", "log_alpha"))
    cu = d.get("cu_seqlens")
    varlen = cu is not None and len(cu) != 2
    cu_t = torch.from_numpy(np.asarray(cu, np.int32)).cuda() if varlen else None
    init = None if d.get("init") is None else to_dev(d["init"], torch)
    N = len(cu) - 1 if varlen else 1
    H = q.shape[2]
    out = nan_tensor(torch, v.shape, out_dtype or torch.float32)
    fin = nan_tensor(torch, (N, H, D, D)) if final else False
    out, fin = kda.dplr_chunk_fwd(q, k, v, a, b, la, init, cu_t, out=out, final_state=fin, workspace=workspace)
    torch.cuda.synchronize()
    return out[0].float().cpu().numpy(), (None if fin is None else fin.cpu().numpy())


def oracle_dplr(d):
    return oracle.dplr_recurrent(d["q"], d["k"], d["v"], d["a"], d["b"], d["log_alpha"], d.get("init"),
                                 d.get("cu_seqlens"))


def check(d, o, S, dtype):
    ro, rS = oracle_dplr(d)
    m = assert_close("out", o, ro, TOL[dtype])
    ms = assert_close("final_state", S, rS, TOL[dtype])
    print(f"  parity: out {m['max_over_rms']:.2e}, final state {ms['max_over_rms']:.2e}", flush=True)


@pytest.mark.parametrize("T,H,dtype,init", [(64, 1, "f32", False), (300, 2, "f32", True), (37, 1, "f32", True),
                                            (200, 3, "bf16", True), (1000, 2, "bf16", False)])
def test_dplr_small(kda, T, H, dtype, init):
    print(f"dplr small T={T} H={H} {dtype}", flush=True)
    d = synth.dplr_small(100 + T, T, H, D, dtype, init_std=0.02 if init else None)
    o, S = run_dplr(kda, d)
    check(d, o, S, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dplr_varlen(kda, dtype):
    lens = [1, 0, 64, 130, 63, 200, 65]
    d = synth.dplr_small(31, 0, 2, D, dtype, lens=lens, init_std=0.05)
    o, S = run_dplr(kda, d)
    check(d, o, S, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dplr_dense_batch(kda, dtype):
    """A dense batch of three 150-token sequences ([B, T, H, d], no cu_seqlens), against the
    oracle run over the same rows as three sequences; the final state once returned and once
    not requested (the output must not change)."""
    B, T, H = 3, 150, 2
    d = synth.dplr_small(37, T, H, D, dtype, init_std=0.02, batch=B)
    q, k, v, a, b, la = (to_dev(d[x], torch).reshape(B, T, H, -1) for x in ("q", "k", "v", "a", "b", "log_alpha"))
    init = to_dev(d["init"], torch)
    out = nan_tensor(torch, (B, T, H, D), torch.float32)
    fin = nan_tensor(torch, (B, H, D, D))
    out, fin = kda.dplr_chunk_fwd(q, k, v, a, b, la, init, out=out, final_state=fin)
    out2 = nan_tensor(torch, (B, T, H, D), torch.float32)
    out2, fin2 = kda.dplr_chunk_fwd(q, k, v, a, b, la, init, out=out2, final_state=None)
    torch.cuda.synchronize()
    assert fin2 is None
    o = out.reshape(B * T, H, D).cpu().numpy()
    assert np.array_equal(o, out2.reshape(B * T, H, D).cpu().numpy())
    check(d, o, fin.cpu().numpy(), dtype)


def test_dplr_bf16_output(kda):
    """bf16 output: the fp32 output rounded to nearest even, bit for bit (everything before
    the store is shared), and the fp32 output within the bar.  The rounding alone reaches
    2^-9 of the largest outputs, so the bar is not applied to the rounded values."""
    d = synth.dplr_small(32, 260, 2, D, "bf16", init_std=0.02)
    o32, S32 = run_dplr(kda, d)
    o16, S16 = run_dplr(kda, d, out_dtype=torch.bfloat16)
    assert np.array_equal(synth.f32_to_bf16_bits(o32), synth.f32_to_bf16_bits(o16))
    assert np.array_equal(S32, S16)
    check(d, o32, S32, "bf16")


def test_dplr_reduces_to_kda(kda):
    """a = beta k, b = alpha (.) k and write key beta k (formed in fp32) against the KDA oracle."""
    d = synth.random_small(33, 257, 2, D, D, "f32", init_std=0.02)
    beta = d["beta"][..., None].astype(np.float64)
    k = d["k"].astype(np.float64)
    dd = {"q": d["q"], "v": d["v"], "log_alpha": d["log_alpha"], "init": d["init"],
          "k": (beta * k).astype(np.float32), "a": (beta * k).astype(np.float32),
          "b": (np.exp(d["log_alpha"].astype(np.float64)) * k).astype(np.float32)}
    o, S = run_dplr(kda, dd)
    ro, rS = oracle.recurrent(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["init"])
    assert_close("out", o, ro, TOL["f32"])
    assert_close("final_state", S, rS, TOL["f32"])


@pytest.mark.parametrize("dtype,scale", [("f32", 15.0), ("bf16", 3.0), ("bf16", 40.0)])
def test_dplr_strong_gates(kda, dtype, scale):
    """Gates whose eight-token decays leave the single-anchor range (fp16 factors past 256,
    fp32 past 2^64): every diagonal block in the form with all factors <= 1."""
    d = synth.dplr_small(34, 200, 2, D, dtype, gate_scale=scale, init_std=0.02)
    o, S = run_dplr(kda, d)
    check(d, o, S, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dplr_strong_gates_in_some_chunks(kda, dtype):
    """Ordinary gates except a few tokens of -30 in some channels: chunks of both forms in one launch."""
    d = synth.dplr_small(35, 400, 2, D, dtype, init_std=0.02)
    la = d["log_alpha"].copy()
    la[70:74, 0, :40] = -30.0
    la[300, 1, 64:] = -30.0
    d["log_alpha"] = la
    o, S = run_dplr(kda, d)
    check(d, o, S, dtype)


def test_dplr_windows(kda):
    """A workspace that holds 3 chunks of records: 14 windows, same results as one window."""
    d = synth.dplr_small(36, 64 * 40 + 17, 2, D, "bf16", init_std=0.02)
    o1, S1 = run_dplr(kda, d)
    rec = (kda.lib().kda_dplr_chunk_fwd_workspace_size(
        kda._lib.shape(1, 64, 0, 2, D, D, 1, 0)) - 2 * D * D * 4)
    ws = torch.empty(2 * D * D * 4 + 3 * rec, dtype=torch.uint8, device="cuda")
    o2, S2 = run_dplr(kda, d, workspace=ws)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    check(d, o2, S2, "bf16")


def test_dplr_bench_shape_every_head(kda):
    """1 x 65,536 tokens x 16 heads, bf16, the benchmark's launch: every head against the oracle
    (one oracle thread per head)."""
    T, H = 65536, 16
    print("dplr bench shape: generating inputs", flush=True)
    d = synth.gen_dplr_tokens(53, T, H, D, "bf16", 0.01)
    init = synth.gen_states(53, 1, H, D, D, 0.02)
    d["init"] = init
    d["cu_seqlens"] = np.array([0, T], np.int64)
    print("dplr bench shape: GPU", flush=True)
    o, S = run_dplr(kda, d)
    print("dplr bench shape: oracle, all heads", flush=True)
    ro, rS = oracle.dplr_recurrent(*[d[x] for x in ("q", "k", "v", "a", "b", "log_alpha")], init)
    m = assert_close("out", o, ro, TOL["bf16"])
    ms = assert_close("final_state", S, rS, TOL["bf16"])
    print(f"dplr bench shape: out {m['max_over_rms']:.2e}, final state {ms['max_over_rms']:.2e}", flush=True)


# ----------------------------------------------------------------------------
# decode: one token per sequence, state in place (kda_dplr_decode_step)
# ----------------------------------------------------------------------------

DECODE_TOL = 1e-4  # fp32 arithmetic from the inputs to the state, whatever the input dtype


def oracle_dplr_step(S, st):
    """One step for N sequences: the oracle's DPLR recurrence over N one-token sequences."""
    N = st["q"].shape[0]
    return oracle.dplr_recurrent(st["q"], st["k"], st["v"], st["a"], st["b"], st["log_alpha"], S,
                                 np.arange(N + 1, dtype=np.int64))


@pytest.mark.parametrize("N,H,dtype,D", [(5, 3, "f32", 64), (16, 4, "bf16", 128), (7, 2, "f32", 128),
                                         (9, 2, "bf16", 64)])
def test_dplr_decode_steps(kda, N, H, dtype, D):
    """Three steps from a random state, every output and the final state against the oracle."""
    S0 = synth.gen_states(81 + N, N, H, D, D, 0.3)
    steps = [synth.gen_dplr_tokens(82 + N + i, N, H, D, dtype, 0.05) for i in range(3)]
    names = ("q", "k", "v", "a", "b", "log_alpha")
    state = to_dev(S0, torch)
    outs = [kda.dplr_decode_step(*[to_dev(st[x], torch) for x in names], state,
                                 out=nan_tensor(torch, (N, H, D))).cpu().numpy() for st in steps]
    torch.cuda.synchronize()
    S = S0
    for i, st in enumerate(steps):
        o, S = oracle_dplr_step(S, st)
        assert_close(f"out{i}", outs[i], o, DECODE_TOL)
    assert_close("state", state.cpu().numpy(), S, DECODE_TOL)


def test_dplr_decode_continues_prefill(kda):
    """A prefill of 200 tokens (2 sequences of 120 and 80, bf16) then one decode step from its
    final state: the oracle over the same 121 and 81 tokens at once."""
    lens = [120, 80]
    d = synth.dplr_small(91, 0, 2, D, "bf16", lens=lens, init_std=0.02)
    o, S = run_dplr(kda, d)
    st = synth.gen_dplr_tokens(92, 2, 2, D, "bf16", 0.05)
    state = torch.from_numpy(S).cuda()
    y = kda.dplr_decode_step(*[to_dev(st[x], torch) for x in ("q", "k", "v", "a", "b", "log_alpha")], state,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the oracle over each sequence with its decode token appended
    cu = np.asarray(d["cu_seqlens"], np.int64)
    joined = {x: np.concatenate([d[x][cu[0]:cu[1]], st[x][0:1], d[x][cu[1]:cu[2]], st[x][1:2]])
              for x in ("q", "k", "v", "a", "b", "log_alpha")}
    cu2 = np.array([0, lens[0] + 1, lens[0] + lens[1] + 2], np.int64)
    ro, rS = oracle.dplr_recurrent(*[joined[x] for x in ("q", "k", "v", "a", "b", "log_alpha")], d["init"], cu2)
    assert_close("decode out", y.cpu().numpy(), ro[[cu2[1] - 1, cu2[2] - 1]], TOL["bf16"])
    assert_close("state", state.cpu().numpy(), rS, TOL["bf16"])
