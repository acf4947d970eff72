"""Rows a1-a3 at their own boundary: the per-chunk record of the chunk-local pass against
the fp64 chunk-local quantities (``oracle.forms.chunk_local``, the state-free part of the
pinned chunkwise form; "Kimi Linear" page, "The constrained DPLR form and the chunkwise
algorithm"), and the same for the general DPLR variant's records
(``oracle.forms.dplr_chunk_local``).  Needs an MI355X.

A white-box test: after a prefill whose chunks all fit one window, the workspace still
holds every chunk's record, and this file decodes it with the layout the kernels write.
The workspace starts with the fp32 state buffer [N, H, dk, dv] (rounded up to 256 bytes);
then one record per (sequence, chunk, head) slot, slot = (s * chunks + j) * H + h, each
holding, at 256-byte aligned offsets:

* W = T diag(beta) K e^G, 64 x dk, and Q e^G, 64 x dk: matrix-core fragment order;
* K e^{G_last - G} transposed, dk x 64: fragment order;
* P (inclusive lower), 64 x 64: fragment order;
* Util = T diag(beta) V as [4 row tiles][dv][16 rows];
* gamma = e^{G_last}, dk fp32.

Fragment order stores a matrix of NC columns as 16-row tiles of KS-column fragments,
each fragment as 64 lanes of KE consecutive elements (KE = 8 fp16, 1 fp32; KS = 4 KE):
element (r, c) sits at (((r/16) (NC/KS) + c/KS) 64 + ((c mod KS)/KE) 16 + r mod 16) KE + c mod KE.

Operands are fp16 for bf16 inputs and fp32 for fp32 inputs.  Each quantity is compared
over every chunk and head at the operator's own bars, max|gpu - oracle| / RMS(oracle)
<= 2e-2 (bf16 inputs, fp16 records) or 1e-4 (fp32).  Measured: about 3-7e-3 for the
fp16 records with ordinary gates; with gates strong enough for the multi-level form,
1.2e-2 for W and 1.6e-2 for Q e^G (rows deep in a strongly decaying chunk hold values
in fp16's subnormal range, whose absolute spacing 2^-24 is what the state pass sees);
about 1e-6 to 1e-5 for the fp32 records.  Rows of the
last chunk past the sequence end must be exactly zero (gamma there is the decay of the
valid rows only); a decay gamma below fp32's normal range (2^-126) is only required
to stay below it.
"""
import numpy as np
import pytest

import oracle
from oracle import forms
import synth

from kda_testlib import TOL, run_chunk

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CH = 64
BAR = TOL


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd as m
    m._lib.lib()
    return m


def a256(x):
    return (x + 255) // 256 * 256


def layout(D, osz):
    off = {"W": 0}
    off["QG"] = a256(off["W"] + CH * D * osz)
    off["KHT"] = a256(off["QG"] + CH * D * osz)
    off["P"] = a256(off["KHT"] + CH * D * osz)
    off["UT"] = a256(off["P"] + CH * CH * osz)
    off["GAM"] = a256(off["UT"] + CH * D * osz)
    off["BYTES"] = a256(off["GAM"] + D * 4)
    return off


def frag_index(R, NC, ke):
    ks = 4 * ke
    r = np.arange(R)[:, None]
    c = np.arange(NC)[None, :]
    return ((((r >> 4) * (NC // ks) + c // ks) * 64 + ((c % ks) // ke) * 16 + (r & 15)) * ke + (c % ke))


def decode(rec, D, osz):
    """One record (uint8 bytes) -> dict of fp64 matrices."""
    off = layout(D, osz)
    ke = 8 if osz == 2 else 1
    dt = np.float16 if osz == 2 else np.float32
    mat = lambda key, n: rec[off[key]:off[key] + n * osz].view(dt).astype(np.float64)
    W = mat("W", CH * D)[frag_index(CH, D, ke)]
    Qg = mat("QG", CH * D)[frag_index(CH, D, ke)]
    Kh = mat("KHT", CH * D)[frag_index(D, CH, ke)].T
    P = mat("P", CH * CH)[frag_index(CH, CH, ke)]
    r = np.arange(CH)[:, None]
    c = np.arange(D)[None, :]
    Ut = mat("UT", CH * D)[((r >> 4) * D + c) * 16 + (r & 15)]
    gamma = rec[off["GAM"]:off["GAM"] + 4 * D].view(np.float32).astype(np.float64)
    return {"W": W, "Qg": Qg, "Kh": Kh, "P": P, "Ut": Ut, "gamma": gamma}


def check_records(kda, d, dtype, D):
    cu = np.asarray(d["cu_seqlens"], np.int64)
    N, H = len(cu) - 1, d["q"].shape[1]
    lens = np.diff(cu)
    chunks = int((lens.max() + CH - 1) // CH)
    osz = 2 if dtype == "bf16" else 4
    off = layout(D, osz)
    T = int(cu[-1])
    need = kda.workspace_size(1, T, H, D, D, torch.bfloat16 if dtype == "bf16" else torch.float32,
                              num_seqs=N if N > 1 else 0, max_seqlen=int(lens.max()) if N > 1 else 0)
    state = a256(N * H * D * D * 4)
    assert need >= state + N * chunks * H * off["BYTES"], "the test needs every chunk in one window"
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    run_chunk(kda, torch, d, workspace=ws)
    wsh = ws.cpu().numpy()
    q, k, v = (synth.as_f64(d[x]) for x in ("q", "k", "v"))
    la = np.asarray(d["log_alpha"], np.float64)
    if la.ndim == 2:  # one gate per (token, head): the same for every key channel
        la = np.repeat(la[:, :, None], D, axis=2)
    beta = np.asarray(d["beta"], np.float64)
    acc = {key: oracle.Metrics() for key in ("W", "Ut", "Qg", "Kh", "P", "gamma")}
    for s in range(N):
        for j in range((int(lens[s]) + CH - 1) // CH):
            t0 = int(cu[s]) + j * CH
            n = min(CH, int(cu[s + 1]) - t0)
            for h in range(H):
                slot = (s * chunks + j) * H + h
                rec = wsh[state + slot * off["BYTES"]: state + (slot + 1) * off["BYTES"]]
                g = decode(rec, D, osz)
                with np.errstate(over="ignore", invalid="ignore"):  # exp of the unused upper triangle
                    ref = forms.chunk_local(q[t0:t0 + n, h], k[t0:t0 + n, h], v[t0:t0 + n, h],
                                            la[t0:t0 + n, h], beta[t0:t0 + n, h])
                for key in ("W", "Ut", "Qg", "Kh"):
                    acc[key].add(g[key][:n], ref[key])
                    assert not g[key][n:].any(), f"{key}: rows past the sequence end are not zero"
                acc["P"].add(g["P"][:n, :n], ref["P"])
                assert not g["P"][n:].any() and not g["P"][:, n:].any()
                # a chunk's decay below fp32's normal range is 0 or a subnormal on the GPU and
                # no longer compares relative to the others: only its size is checked
                tiny = ref["gamma"] < 2.0 ** -126
                assert (g["gamma"][tiny] < 2.0 ** -126).all(), "gamma: a vanishing decay came out normal"
                acc["gamma"].add(g["gamma"][~tiny], ref["gamma"][~tiny])
    for key, m in acc.items():
        r = m.result()
        print(f"  {key}: max|err|/rms {r['max_over_rms']:.2e} (bar {BAR[dtype]:.0e})", flush=True)
        assert r["max_over_rms"] <= BAR[dtype], f"{key}: {r['max_over_rms']:.3e} > {BAR[dtype]:.0e}"


@pytest.mark.parametrize("T,H,D,dtype", [(300, 2, 128, "bf16"), (200, 3, 64, "f32"), (129, 2, 64, "bf16"),
                                         (64, 1, 128, "f32")])
def test_records_dense(kda, T, H, D, dtype):
    d = synth.random_small(500 + T, T, H, D, D, dtype=dtype)
    check_records(kda, d, dtype, D)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_records_head_gate(kda, dtype):
    """One gate per (token, head) (the scalar gate of Gated DeltaNet) on the same kernels."""
    d = synth.random_small(505, 230, 2, 128, 128, dtype=dtype, gate="head")
    check_records(kda, d, dtype, 128)


def test_records_varlen(kda):
    """Three sequences (one shorter than a chunk): the slot of each (sequence, chunk, head)."""
    d = synth.random_small(510, 0, 2, 128, 128, dtype="bf16", lens=[130, 40, 200])
    check_records(kda, d, "bf16", 128)


@pytest.mark.parametrize("dtype,scale", [("bf16", 3.0), ("f32", 40.0)])
def test_records_strong_gates(kda, dtype, scale):
    """Gates strong enough that the diagonal blocks take the multi-level form (its records are
    written by the second chunk-local kernel)."""
    d = synth.random_small(520, 200, 2, 128, 128, dtype=dtype, gate_scale=scale)
    check_records(kda, d, dtype, 128)


# ----------------------------------------------------------------------------
# the general DPLR variant's records (kda_dplr_chunk_fwd, d = 128): Y = T B e^{Gx} and
# Q e^G in fragment order, K e^{G_last - G} and -A e^{G_last - G} transposed, Mqk and
# -Mqa (64 x 64) in fragment order, Z = (T Mbk) V and V as [4 row tiles][dv][16 rows],
# gamma fp32; against oracle.forms.dplr_chunk_local
# ----------------------------------------------------------------------------

def dplr_layout(osz, D=128):
    tile, sq = CH * D * osz, CH * CH * osz
    off = {"Y": 0}
    off["QG"] = a256(off["Y"] + tile)
    off["KHT"] = a256(off["QG"] + tile)
    off["ANT"] = a256(off["KHT"] + tile)
    off["MQK"] = a256(off["ANT"] + tile)
    off["NQA"] = a256(off["MQK"] + sq)
    off["Z"] = a256(off["NQA"] + sq)
    off["V"] = a256(off["Z"] + tile)
    off["GAM"] = a256(off["V"] + tile)
    off["BYTES"] = a256(off["GAM"] + D * 4)
    return off


def decode_dplr(rec, osz, D=128):
    off = dplr_layout(osz, D)
    ke = 8 if osz == 2 else 1
    dt = np.float16 if osz == 2 else np.float32
    mat = lambda key, n: rec[off[key]:off[key] + n * osz].view(dt).astype(np.float64)
    r = np.arange(CH)[:, None]
    c = np.arange(D)[None, :]
    tiles = ((r >> 4) * D + c) * 16 + (r & 15)
    return {"Y": mat("Y", CH * D)[frag_index(CH, D, ke)], "Qg": mat("QG", CH * D)[frag_index(CH, D, ke)],
            "Kh": mat("KHT", CH * D)[frag_index(D, CH, ke)].T, "Ah": -mat("ANT", CH * D)[frag_index(D, CH, ke)].T,
            "Mqk": mat("MQK", CH * CH)[frag_index(CH, CH, ke)], "Mqa": -mat("NQA", CH * CH)[frag_index(CH, CH, ke)],
            "Z": mat("Z", CH * D)[tiles], "V": mat("V", CH * D)[tiles],
            "gamma": rec[off["GAM"]:off["GAM"] + 4 * D].view(np.float32).astype(np.float64)}


def check_dplr_records(kda, d, dtype):
    D = 128
    cu = np.asarray(d["cu_seqlens"], np.int64)
    N, H = len(cu) - 1, d["q"].shape[1]
    lens = np.diff(cu)
    chunks = int((lens.max() + CH - 1) // CH)
    osz = 2 if dtype == "bf16" else 4
    off = dplr_layout(osz)
    T = int(cu[-1])
    varlen = N > 1
    need = kda.dplr_workspace_size(1, T, H, D, D, torch.bfloat16 if dtype == "bf16" else torch.float32,
                                   num_seqs=N if varlen else 0, max_seqlen=int(lens.max()) if varlen else 0)
    state = a256(N * H * D * D * 4)
    assert need >= state + N * chunks * H * off["BYTES"], "the test needs every chunk in one window"
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    dev = lambda x: (torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16) if x.dtype == np.uint16
                     else torch.from_numpy(np.ascontiguousarray(x))).cuda().unsqueeze(0)
    args = [dev(d[x]) for x in ("q", "k", "v", "a", "b", "log_alpha")]
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda() if varlen else None
    init = None if d.get("init") is None else torch.from_numpy(d["init"]).cuda()
    kda.dplr_chunk_fwd(*args, init, cu_t, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    wsh = ws.cpu().numpy()
    q, k, v, a, b = (synth.as_f64(d[x]) for x in ("q", "k", "v", "a", "b"))
    la = np.asarray(d["log_alpha"], np.float64)
    keys = ("Y", "Z", "Qg", "Kh", "Ah", "V", "Mqk", "Mqa", "gamma")
    acc = {key: oracle.Metrics() for key in keys}
    for s in range(N):
        for j in range((int(lens[s]) + CH - 1) // CH):
            t0 = int(cu[s]) + j * CH
            n = min(CH, int(cu[s + 1]) - t0)
            for h in range(H):
                slot = (s * chunks + j) * H + h
                g = decode_dplr(wsh[state + slot * off["BYTES"]: state + (slot + 1) * off["BYTES"]], osz)
                sl = slice(t0, t0 + n)
                ref = forms.dplr_chunk_local(q[sl, h], k[sl, h], v[sl, h], a[sl, h], b[sl, h], la[sl, h])
                ref["V"] = v[sl, h]
                for key in ("Y", "Z", "Qg", "Kh", "Ah", "V"):
                    acc[key].add(g[key][:n], ref[key])
                    assert not g[key][n:].any(), f"{key}: rows past the sequence end are not zero"
                for key in ("Mqk", "Mqa"):
                    acc[key].add(g[key][:n, :n], ref[key])
                    assert not g[key][n:].any() and not g[key][:, n:].any()
                tiny = ref["gamma"] < 2.0 ** -126
                assert (g["gamma"][tiny] < 2.0 ** -126).all()
                acc["gamma"].add(g["gamma"][~tiny], ref["gamma"][~tiny])
    for key, m in acc.items():
        r = m.result()
        print(f"  dplr {key}: max|err|/rms {r['max_over_rms']:.2e} (bar {BAR[dtype]:.0e})", flush=True)
        assert r["max_over_rms"] <= BAR[dtype], f"dplr {key}: {r['max_over_rms']:.3e} > {BAR[dtype]:.0e}"


@pytest.mark.parametrize("T,H,dtype,scale", [(300, 2, "bf16", 0.05), (200, 2, "f32", 0.05),
                                             (200, 2, "bf16", 3.0), (150, 1, "f32", 15.0)])
def test_dplr_records(kda, T, H, dtype, scale):
    """Ordinary gates, and gates strong enough for the form whose factors are all <= 1."""
    d = synth.dplr_small(530 + T, T, H, 128, dtype, gate_scale=scale)
    check_dplr_records(kda, d, dtype)


def test_dplr_records_varlen(kda):
    d = synth.dplr_small(540, 0, 2, 128, "bf16", lens=[130, 40, 200])
    check_dplr_records(kda, d, "bf16")
