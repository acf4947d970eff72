"""The C ABI without a GPU: exports, status strings, workspace sizing, argument validation.

Every call here fails validation (or has nothing to do) before any HIP call,
so no kernel is ever launched; the fake device addresses are never touched.
"""
import ctypes
import os
import re

import pytest

from gated_delta_rule_53_amd import _lib
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16 = 0, 1
A = 1 << 20  # a 16-byte-aligned fake device address; never dereferenced


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for st in range(5):
        s = _lib.status_string(st)
        assert isinstance(s, str) and s
    assert _lib.status_string(99) == "unknown status"


def _shape(B=1, T=256, N=0, maxT=0, H=2, dk=64, dv=64, i=F32, o=F32, gph=0):
    return _lib.shape(B, T, N, H, dk, dv, i, o, maxT, gph)


def test_workspace_size(L):
    for idx in (0, 1, 2):
        w = WORKLOADS[idx]
        s = _shape(1, w.seqlen, 0, 0, w.heads, w.dk, w.dv, BF16 if w.dtype == "bf16" else F32, F32)
        n = L.kda_chunk_fwd_workspace_size(s)
        state = w.heads * w.dk * w.dv * 4
        assert n > state
        assert n < (1 << 31)
    # varlen: grows with the number of sequences
    s1 = _shape(1, 1 << 20, 16, 1 << 17, 32, 128, 128, BF16, F32)
    s2 = _shape(1, 1 << 20, 1, 1 << 20, 32, 128, 128, BF16, F32)
    assert L.kda_chunk_fwd_workspace_size(s1) > 0 and L.kda_chunk_fwd_workspace_size(s2) > 0
    # invalid shapes: 0
    assert L.kda_chunk_fwd_workspace_size(_shape(dk=96, dv=96)) == 0
    assert L.kda_chunk_fwd_workspace_size(_shape(dk=64, dv=128)) == 0
    assert L.kda_chunk_fwd_workspace_size(_shape(H=0)) == 0
    assert L.kda_chunk_fwd_workspace_size(None) == 0


def _fwd(L, s, q=A, k=2 * A, v=3 * A, la=4 * A, b=5 * A, init=None, cu=None, out=6 * A, fin=None,
         ws=None, wsb=0):
    return L.kda_chunk_fwd(s, q, k, v, la, b, init, cu, out, fin, ws, wsb, None)


def test_chunk_fwd_validation(L):
    s = _shape()
    assert L.kda_chunk_fwd(None, A, A, A, A, A, None, None, A, None, A, 1 << 30, None) == INVALID
    assert _fwd(L, _shape(dk=96, dv=96)) == UNSUPPORTED
    assert _fwd(L, _shape(dk=64, dv=128)) == UNSUPPORTED
    assert _fwd(L, _shape(i=7)) == UNSUPPORTED
    assert _fwd(L, _shape(o=3)) == UNSUPPORTED
    assert _fwd(L, _shape(H=0)) == INVALID
    assert _fwd(L, _shape(T=-1)) == INVALID
    assert _fwd(L, s, q=None) == INVALID
    assert _fwd(L, s, q=A + 4) == INVALID                       # misaligned
    assert _fwd(L, s, out=A + 100) == INVALID                   # out overlaps q
    assert _fwd(L, s, init=7 * A, fin=7 * A + 64) == INVALID    # partial state overlap
    assert _fwd(L, s, cu=9 * A, ws=10 * A, wsb=1 << 30) == OK       # varlen with zero sequences: no work
    assert _fwd(L, _shape(B=2), cu=9 * A) == INVALID            # varlen needs batch 1
    assert _fwd(L, s, ws=None) == WORKSPACE
    assert _fwd(L, s, ws=10 * A, wsb=1024) == WORKSPACE
    assert _fwd(L, s, ws=10 * A + 8, wsb=1 << 30) == WORKSPACE  # misaligned workspace
    assert _fwd(L, _shape(gph=2)) == INVALID                    # gate layout flag is 0 or 1
    # one launch holds at most 65535 / N chunks of every sequence: N > 65535 is refused
    F = 1 << 40  # pointers far enough apart that the large tensors do not overlap
    assert _fwd(L, _shape(B=70000, T=64), q=F, k=2 * F, v=3 * F, la=4 * F, b=5 * F, out=6 * F,
                ws=7 * F, wsb=1 << 39) == UNSUPPORTED
    # out right after log_alpha: overlaps a per-channel gate [T,H,dk] but not a per-head one [T,H]
    la_head = 256 * 2 * 4
    assert _fwd(L, s, la=4 * A, out=4 * A + la_head) == INVALID
    assert _fwd(L, _shape(gph=1), la=4 * A, out=4 * A + la_head) == WORKSPACE  # passes validation


def _bwd(L, s, q=A, k=2 * A, v=3 * A, la=4 * A, b=5 * A, init=None, cu=None, dout=6 * A, dfin=None,
         dq=7 * A, dk=8 * A, dv=9 * A, dla=10 * A, db=11 * A, dinit=None, ws=None, wsb=0):
    return L.kda_chunk_bwd(s, q, k, v, la, b, init, cu, dout, dfin, dq, dk, dv, dla, db, dinit, ws, wsb, None)


def test_chunk_bwd_validation(L):
    s = _shape()
    assert _bwd(L, None) == INVALID
    assert _bwd(L, _shape(dk=96, dv=96)) == UNSUPPORTED
    assert _bwd(L, _shape(H=0)) == INVALID
    assert _bwd(L, _shape(gph=2)) == INVALID
    assert _bwd(L, s, dq=None) == INVALID
    assert _bwd(L, s, dout=None) == INVALID
    assert _bwd(L, s, dk=8 * A + 4) == INVALID                   # misaligned
    assert _bwd(L, s, dv=A + 64) == INVALID                      # a gradient over q
    assert _bwd(L, s, db=7 * A + 128) == INVALID                 # two gradients overlap
    assert _bwd(L, s, init=12 * A, dinit=12 * A + 256) == INVALID  # d_init over init
    assert _bwd(L, _shape(B=2), cu=13 * A) == INVALID           # varlen needs batch 1
    assert _bwd(L, s, cu=13 * A, ws=14 * A, wsb=1 << 30) == OK   # varlen with zero sequences: no work
    assert _bwd(L, s, ws=None) == WORKSPACE
    assert _bwd(L, s, ws=14 * A, wsb=1024) == WORKSPACE
    assert _bwd(L, s, ws=14 * A + 8, wsb=1 << 30) == WORKSPACE   # misaligned workspace
    # dlog_alpha right after dv: overlaps a per-channel gate gradient only when it is per channel
    la_head = 256 * 2 * 4
    assert _bwd(L, s, dla=9 * A - la_head) == INVALID
    assert _bwd(L, _shape(gph=1), dla=9 * A - la_head) == WORKSPACE  # passes validation
    n = L.kda_chunk_bwd_workspace_size(s)
    assert n > L.kda_chunk_fwd_workspace_size(s) > 0
    assert L.kda_chunk_bwd_workspace_size(None) == 0
    # a backward window holds at most 65535 // N chunks per sequence, so only N > 65535 is refused
    assert L.kda_chunk_bwd_workspace_size(_shape(B=1100, T=4096)) > 0
    assert L.kda_chunk_bwd_workspace_size(_shape(B=70000, T=64)) == 0
    assert _bwd(L, _shape(B=70000, T=64)) == UNSUPPORTED


def test_backward_workspace_windows(L, monkeypatch):
    """The backward holds one window of chunks: its workspace stays bounded for the 1M-token
    varlen batch, and forcing short windows shrinks it further."""
    w = WORKLOADS[4]
    # every length is at least w.min_len, so no sequence is longer than the rest of the tokens
    longest = w.seqlen - (w.num_seqs - 1) * w.min_len
    s = _shape(1, w.seqlen, w.num_seqs, longest, w.heads, w.dk, w.dv, BF16, F32)
    n = L.kda_chunk_bwd_workspace_size(s)
    # 24 GiB of per-chunk arrays, one record window, and the state entering each of ~128 windows
    assert 0 < n < 32 * (1 << 30)
    full = _shape(1, 65536, 0, 0, 32, 128, 128, BF16, F32)
    one = L.kda_chunk_bwd_workspace_size(full)        # 64K x 32 heads: one window, every chunk at once
    assert 11 * (1 << 30) < one < 13 * (1 << 30)
    monkeypatch.setenv("KDA_BWD_WINDOW", "128")
    part = L.kda_chunk_bwd_workspace_size(full)
    assert part < one / 4                             # 128 of 1,024 chunks per window, plus 7 checkpoints


def test_decode_validation(L):
    for f in (L.kda_decode_step, L.kda_decode_step_head_gate):
        assert f(0, 2, 64, 64, F32, F32, A, A, A, A, A, A, A, None) == OK  # empty batch: nothing to do
        assert f(-1, 2, 64, 64, F32, F32, A, A, A, A, A, A, A, None) == INVALID
        assert f(2, 2, 96, 96, F32, F32, A, A, A, A, A, A, A, None) == UNSUPPORTED
        assert f(2, 2, 64, 128, F32, F32, A, A, A, A, A, A, A, None) == UNSUPPORTED
        assert f(2, 2, 64, 64, 5, F32, A, A, A, A, A, A, A, None) == UNSUPPORTED
        assert f(2, 2, 64, 64, F32, F32, None, A, A, A, A, A, A, None) == INVALID
        st, out = 8 * A, 12 * A
        assert f(2, 2, 64, 64, F32, F32, A, 2 * A, 3 * A, 4 * A, 5 * A, st + 4, out, None) == INVALID  # misaligned
        assert f(2, 2, 64, 64, F32, F32, A, 2 * A, 3 * A, 4 * A, 5 * A, st, st + 256, None) == INVALID  # out in state
        assert f(2, 2, 64, 64, F32, F32, st + 512, 2 * A, 3 * A, 4 * A, 5 * A, st, out, None) == INVALID  # q in state
        assert f(2, 2, 64, 64, F32, F32, A, 2 * A, 3 * A, 4 * A, st + 64, st, out, None) == INVALID  # beta in state
    # the state right after log_alpha: overlaps a per-channel gate [N,H,dk] only
    la_head = 2 * 2 * 4
    st = 8 * A
    assert L.kda_decode_step(2, 2, 64, 64, F32, F32, A, 2 * A, 3 * A, st - la_head, 5 * A, st, 12 * A,
                             None) == INVALID


def test_dplr_decode_validation(L):
    """kda_dplr_decode_step: the decode checks, with a and b counted among the inputs."""
    f = L.kda_dplr_decode_step
    assert f(0, 2, 64, 64, F32, F32, A, A, A, A, A, A, A, A, None) == OK  # empty batch: nothing to do
    assert f(-1, 2, 64, 64, F32, F32, A, A, A, A, A, A, A, A, None) == INVALID
    assert f(2, 2, 96, 96, F32, F32, A, A, A, A, A, A, A, A, None) == UNSUPPORTED
    assert f(2, 2, 64, 128, F32, F32, A, A, A, A, A, A, A, A, None) == UNSUPPORTED
    assert f(2, 2, 64, 64, F32, 7, A, A, A, A, A, A, A, A, None) == UNSUPPORTED
    for i in range(8):  # each of q, k, v, a, b, log_alpha, state, out missing
        ptrs = [j * A for j in range(1, 7)] + [8 * A, 12 * A]
        ptrs[i] = None
        assert f(2, 2, 64, 64, F32, F32, *ptrs, None) == INVALID
    st, out = 8 * A, 12 * A
    assert f(2, 2, 64, 64, F32, F32, A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, st + 4, out, None) == INVALID  # misaligned
    assert f(2, 2, 64, 64, F32, F32, A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, st, st + 256, None) == INVALID  # out in state
    assert f(2, 2, 64, 64, F32, F32, A, 2 * A, 3 * A, st + 64, 5 * A, 6 * A, st, out, None) == INVALID  # a in state
    assert f(2, 2, 64, 64, F32, F32, A, 2 * A, 3 * A, 4 * A, out + 16, 6 * A, st, out, None) == INVALID  # b in out


def test_shape_struct_layout_matches_the_boundary():
    """kda_shape_t starts with the fields batch, seqlen, num_seqs, heads, dk, dv, in_dtype,
    out_dtype at the offsets a C compiler gives them, then max_seqlen and gate_per_head;
    the ctypes mirror has the same offsets.  Compiled from include/kda.h with gcc as C11."""
    import shutil
    import subprocess
    import tempfile
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    names = ("batch", "seqlen", "num_seqs", "heads", "dk", "dv", "in_dtype", "out_dtype", "max_seqlen",
             "gate_per_head")
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"kda.h\"\nint main(void) {\n"
    src += "".join(f'  printf("%zu\\n", offsetof(kda_shape_t, {n}));\n' for n in names)
    src += '  printf("%zu\\n", sizeof(kda_shape_t));\n  return 0;\n}\n'
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I" + os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()]
    # int32 batch | pad | int64 seqlen | int32 num_seqs, heads, dk, dv, in, out | int64 max_seqlen | int32 gph
    assert got == [0, 8, 16, 20, 24, 28, 32, 36, 40, 48, 56]
    assert [getattr(_lib.Shape, n).offset for n in names] + [ctypes.sizeof(_lib.Shape)] == got


def test_chunk_fwd_aliasing_of_final_state_and_workspace(L):
    """final_state and the workspace are written by the kernels: overlapping any argument is
    rejected before any launch."""
    s = _shape()  # T = 256, H = 2, dk = dv = 64, fp32: token tensors 128 KiB, states 32 KiB
    fin, ws = 20 * A, 30 * A
    ok = dict(fin=fin, ws=ws, wsb=1 << 20)
    assert _fwd(L, s, **dict(ok, fin=4 * A + 4096)) == INVALID              # final state over log_alpha
    assert _fwd(L, s, **dict(ok, fin=5 * A)) == INVALID                     # over beta
    sv = _shape(N=1, maxT=256)  # one packed sequence: cu_seqlens [2] is read
    assert _fwd(L, sv, cu=fin + 16, **ok) == INVALID                        # over cu_seqlens
    assert _fwd(L, s, **dict(ok, ws=A + 64)) == INVALID                     # workspace over q
    assert _fwd(L, s, **dict(ok, ws=6 * A - 4096)) == INVALID               # over out
    assert _fwd(L, s, init=ws + 1024, **ok) == INVALID                      # over init
    assert _fwd(L, s, **dict(ok, ws=fin - (1 << 20) + 1024)) == INVALID     # over final state
    assert _fwd(L, sv, cu=ws + 4096, **ok) == INVALID                       # over cu_seqlens


def test_layer_fwd_aliasing_of_final_state(L):
    s = _shape(1, 256, 0, 0, 2, 64, 64, BF16, BF16)
    q, k, v, b, out, ws = (i * A for i in (2, 4, 6, 8, 10, 12))
    lay = _layer()  # gate at 40 A, out_gate at 41 A, weight at 42 A
    assert L.kda_layer_fwd(s, lay, q, k, v, b, None, None, out, 41 * A + 64, ws, 1 << 20, None) == INVALID
    assert L.kda_layer_fwd(s, lay, q, k, v, b, None, None, out, 42 * A, ws, 1 << 20, None) == INVALID
    assert L.kda_layer_fwd(s, lay, q, k, v, b, None, None, out, None, 41 * A - 64, 1 << 20, None) == INVALID


def test_chunk_bwd_workspace_aliasing(L):
    s = _shape()
    n = L.kda_chunk_bwd_workspace_size(s)
    ws = 20 * A
    for over in (A + 64, 6 * A, 7 * A, 11 * A):  # q, d_out, dq, dbeta inside the workspace
        assert _bwd(L, s, ws=over - 64, wsb=n) == INVALID
    sv = _shape(N=1, maxT=256)
    nv = L.kda_chunk_bwd_workspace_size(sv)
    assert _bwd(L, sv, cu=ws + 256, ws=ws, wsb=nv) == INVALID
    assert _bwd(L, s, init=ws + 512, ws=ws, wsb=n) == INVALID


def test_missing_library_fails_loudly(monkeypatch):
    """Without libkda.so the binding raises: there is no CPU or PyTorch fallback."""
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libkda.so"))
    with pytest.raises(ImportError, match="no fallback"):
        _lib.lib()


def test_workspace_size_sequence_parallel(L, monkeypatch):
    """Few (sequence, head) pairs: the workspace holds every record plus three per-segment state arrays."""
    s = _shape(1, 65536, 0, 0, 2, 128, 128, BF16, F32)
    state, rec = 2 * 128 * 128 * 4, 74240
    records = 1024 * 2 * rec
    n = L.kda_chunk_fwd_workspace_size(s)
    assert n >= state + records + 3 * 2 * 16 * 128 * 128 * 4  # 16 segments
    monkeypatch.setenv("KDA_SEGMENTS", "0")                   # windows only
    n0 = L.kda_chunk_fwd_workspace_size(s)
    assert state < n0 < n and n0 <= state + (220 << 20)


def test_workspace_size_windows(L):
    """Record windows stay within the 220 MiB record budget unless that leaves fewer than 32 chunks
    per window; then windows of 32 chunks (or every chunk), with at most 4 GiB of records."""
    rec = 74240
    # one 65,536-token sequence, 32 heads: 96-chunk windows (2 x 48 chunk indices)
    s = _shape(1, 65536, 0, 0, 32, 128, 128, BF16, F32)
    state = 32 * 128 * 128 * 4
    n = L.kda_chunk_fwd_workspace_size(s)
    assert n == state + 96 * 32 * rec and n - state <= (220 << 20)
    # 64 sequences of 1,024 tokens: one chunk index of every (sequence, head) pair is 152 MB, so
    # the budget would hold a single index; the window holds all 16 chunks instead (2.4 GB)
    s = _shape(1, 65536, 64, 1024, 32, 128, 128, BF16, F32)
    state = 64 * 32 * 128 * 128 * 4
    assert L.kda_chunk_fwd_workspace_size(s) == state + 16 * 64 * 32 * rec
    # the 1M-token batch of 16 sequences (longest 250,811 tokens): 32-chunk windows, 1.2 GB
    s = _shape(1, 1 << 20, 16, 250811, 32, 128, 128, BF16, F32)
    state = 16 * 32 * 128 * 128 * 4
    assert L.kda_chunk_fwd_workspace_size(s) == state + 32 * 16 * 32 * rec
    # 200 sequences of 4,096 tokens: 32 chunks would exceed 4 GiB of records, so 9 chunks
    s = _shape(1, 200 * 4096, 200, 4096, 32, 128, 128, BF16, F32)
    state = 200 * 32 * 128 * 128 * 4
    assert L.kda_chunk_fwd_workspace_size(s) == state + ((4 << 30) // (200 * 32 * rec)) * 200 * 32 * rec


def _layer(norm=1, l2=1e-6, gate=True, og=True, w=True, rms=1e-6, base=40):
    addr = lambda i: (base + i) * A
    return _lib.Layer(norm, l2, addr(0) if gate else None, addr(1) if og else None, addr(2) if w else None, rms)


def _layer_fwd(L, layer, ws_bytes=0):
    s = _shape(1, 256, 0, 0, 2, 64, 64, BF16, BF16)
    q, k, v, b, out, ws = (i * A for i in (2, 4, 6, 8, 10, 12))
    return L.kda_layer_fwd(s, layer, q, k, v, b, None, None, out, None, ws, ws_bytes, None)


def test_layer_fwd_validation(L):
    """Valid layer options reach the workspace check; bad ones stop before it."""
    assert _layer_fwd(L, _layer()) == WORKSPACE
    assert _layer_fwd(L, _layer(og=False, w=False)) == WORKSPACE  # no epilogue
    assert _layer_fwd(L, _layer(norm=0)) == WORKSPACE
    assert _layer_fwd(L, None) == INVALID
    assert _layer_fwd(L, _layer(norm=2)) == INVALID
    assert _layer_fwd(L, _layer(l2=-1.0)) == INVALID
    assert _layer_fwd(L, _layer(rms=float("nan"))) == INVALID
    assert _layer_fwd(L, _layer(rms=float("inf"))) == INVALID
    assert _layer_fwd(L, _layer(gate=False)) == INVALID  # the gate pre-activation is required
    # output overlapping the output gate or the weight
    s = _shape(1, 256, 0, 0, 2, 64, 64, BF16, BF16)
    lay = _lib.Layer(1, 1e-6, 40 * A, 10 * A + 64, 42 * A, 1e-6)
    q, k, v, b, out, ws = (i * A for i in (2, 4, 6, 8, 10, 12))
    assert L.kda_layer_fwd(s, lay, q, k, v, b, None, None, out, None, ws, 0, None) == INVALID


def test_layer_decode_validation(L):
    """Rejections of kda_layer_decode_step, all before any launch."""
    q, k, v, b, st, out = (i * A for i in (2, 4, 6, 8, 10, 14))
    call = lambda lay, gph=0: L.kda_layer_decode_step(4, 2, 64, 64, BF16, F32, gph, lay, q, k, v, b, st, out,
                                                      None)
    assert call(None) == INVALID
    assert call(_layer(norm=3)) == INVALID
    assert call(_layer(l2=float("nan"))) == INVALID
    assert call(_layer(rms=-1e-3)) == INVALID
    assert call(_layer(gate=False)) == INVALID
    assert call(_layer(), gph=2) == INVALID
    assert L.kda_layer_decode_step(4, 2, 96, 96, BF16, F32, 0, _layer(), q, k, v, b, st, out, None) == UNSUPPORTED


def test_binding_argument_counts_match_header(L):
    """Each ctypes prototype has exactly the parameters include/kda.h declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name in _lib.EXPORTS:
        m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(getattr(L, name).argtypes) == len(params), name


def test_noalloc_validation(L):
    """kda_chunk_fwd_noalloc: the kda_chunk_fwd argument checks, and shapes whose least workspace
    exceeds the static scratch rejected with KDA_ERR_WORKSPACE, all before any device call."""
    call = lambda s, q=A, out=6 * A: L.kda_chunk_fwd_noalloc(s, q, 2 * A, 3 * A, 4 * A, 5 * A, None, None, out,
                                                             None, None)
    assert call(None) == INVALID
    assert call(_shape(dk=96, dv=96)) == UNSUPPORTED
    assert call(_shape(H=0)) == INVALID
    assert call(_shape(), q=A + 4) == INVALID       # misaligned
    assert call(_shape(), out=A + 64) == INVALID    # out over q
    assert _lib.NOALLOC_SCRATCH_BYTES == 256 << 20
    # 4,096 heads: one chunk of records per head is 4,096 x 74,240 bytes > 256 MiB
    F = 1 << 40
    big = _shape(1, 64, 0, 0, 4096, 128, 128, BF16, F32)
    assert L.kda_chunk_fwd_noalloc(big, F, 2 * F, 3 * F, 4 * F, 5 * F, None, None, 6 * F, None, None) == WORKSPACE


def _dplr(L, s, q=A, k=2 * A, v=3 * A, a=4 * A, b=5 * A, la=6 * A, init=None, cu=None, out=7 * A, fin=None,
          ws=None, wsb=0):
    return L.kda_dplr_chunk_fwd(s, q, k, v, a, b, la, init, cu, out, fin, ws, wsb, None)


def test_dplr_chunk_fwd_validation(L):
    """kda_dplr_chunk_fwd: dk = dv = 128 and per-channel gates only; the kda_chunk_fwd checks
    with a and b counted among the inputs."""
    s = _shape(T=128, dk=128, dv=128)
    assert L.kda_dplr_chunk_fwd_workspace_size(s) > 2 * 128 * 128 * 4
    assert L.kda_dplr_chunk_fwd_workspace_size(_shape()) == 0                     # dk = 64
    assert L.kda_dplr_chunk_fwd_workspace_size(_shape(T=128, dk=128, dv=128, gph=1)) == 0
    assert _dplr(L, None) == INVALID
    assert _dplr(L, _shape()) == UNSUPPORTED                                      # dk = 64
    assert _dplr(L, _shape(T=128, dk=128, dv=128, gph=1)) == UNSUPPORTED          # one gate per head
    assert _dplr(L, _shape(T=128, dk=128, dv=128, i=7)) == UNSUPPORTED
    assert _dplr(L, s, a=None) == INVALID
    assert _dplr(L, s, b=5 * A + 4) == INVALID                                   # misaligned
    assert _dplr(L, s, out=4 * A + 64) == INVALID                                # out over a
    assert _dplr(L, s, out=5 * A + 64) == INVALID                                # out over b
    assert _dplr(L, s, fin=5 * A) == INVALID                                     # final state over b
    assert _dplr(L, s, init=9 * A, fin=9 * A + 64) == INVALID                    # partial state overlap
    assert _dplr(L, s, ws=None) == WORKSPACE
    assert _dplr(L, s, ws=10 * A, wsb=1024) == WORKSPACE
    assert _dplr(L, s, ws=4 * A, wsb=1 << 30) == INVALID                         # workspace over a
    assert _dplr(L, s, cu=9 * A, ws=10 * A, wsb=1 << 30) == OK                   # varlen, zero sequences
    assert _dplr(L, _shape(B=2, T=128, dk=128, dv=128), cu=9 * A) == INVALID     # varlen needs batch 1
    # the record is larger than KDA's: the workspace of the same shape is larger at a single window
    s1 = _shape(T=4096, H=4, dk=128, dv=128, i=BF16)
    assert L.kda_dplr_chunk_fwd_workspace_size(s1) > L.kda_chunk_fwd_workspace_size(s1)
