"""fp64 CPU oracle of the KDA operator -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
this package never imports the product library: the two share no code.

Three independent forms of the same operator (the "Kimi Linear" page,
sections "Background: from the delta rule to gated DeltaNet", "Kimi Delta
Attention", "Why channel-wise gating matters" and "The constrained DPLR form
and the chunkwise algorithm"):

* ``recurrent``   -- plain C, fp64, token by token (kda_oracle.c); the oracle.
* ``metrics`` / ``Metrics`` -- the parity figure max|x - ref| / RMS(ref), whole
  or accumulated over pieces; pinned by hand-computed cases.
* ``backward``    -- its reverse mode: the adjoint of each token step, fp64,
  in the same C file; pinned by finite differences and a closed form.
* ``forms.brute`` -- explicit dk x dk transition matrices, and the output
  expanded as a sum over earlier tokens in which each key reaches the query
  through the product of the transitions between them; numpy fp64, tiny
  sizes only.
* ``forms.chunkwise`` -- the chunked WY/UT form, fp64, written from the
  algebra of the recurrence; used to pin the recurrent form.
* ``dplr_recurrent`` -- the general DPLR transition KDA constrains (section
  "The constrained DPLR form and the chunkwise algorithm": independent a and
  b), plain C fp64 token by token; pinned by its reduction to KDA and by
  ``forms.dplr_brute`` / ``forms.dplr_chunkwise``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD = os.path.join(_HERE, "_build")
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIBS: dict = {}


# KDA_ORACLE_SANITIZE=1 builds and loads the oracle with AddressSanitizer and
# UndefinedBehaviorSanitizer (a separate library; the Python process must then
# preload gcc's libasan and libubsan, as tests/test_sanitizers.py does).
_SANITIZE = os.environ.get("KDA_ORACLE_SANITIZE") == "1"
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def lib_path(mutant: int = 0) -> str:
    name = "libkda_oracle" + ("" if mutant == 0 else f"_m{mutant}") + ("_san" if _SANITIZE else "") + ".so"
    return os.path.join(_BUILD, name)


def build(mutant: int = 0, force: bool = True) -> str:
    """Compile the C oracle with gcc (no GPU code involved)."""
    os.makedirs(_BUILD, exist_ok=True)
    out = lib_path(mutant)
    if force or not os.path.exists(out):
        tmp = out + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", *(_SAN_FLAGS if _SANITIZE else []),
               f"-DKDA_ORACLE_MUTANT={mutant}", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _lib(mutant: int = 0):
    if mutant in _LIBS:
        return _LIBS[mutant]
    path = lib_path(mutant)
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        build(mutant)
    lib = ctypes.CDLL(path)
    f = lib.kda_oracle_forward
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    b = lib.kda_oracle_backward
    b.restype = ctypes.c_int
    b.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int] + \
        [ctypes.c_void_p] * 14 + [ctypes.c_int]
    d = lib.dplr_oracle_forward
    d.restype = ctypes.c_int
    d.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int] + \
        [ctypes.c_void_p] * 9 + [ctypes.c_int]
    _LIBS[mutant] = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def recurrent(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, threads=None,
              mutant: int = 0):
    """fp64 token-by-token KDA forward.

    Inputs (numpy): q, k [T, H, dk] and v [T, H, dv] as float32 or uint16
    (bf16 bits), or float64 (then log_alpha and beta are taken in fp64 too);
    log_alpha float32 [T, H, dk], or [T, H] for one gate per head
    shared by every key channel (the scalar gate of Gated DeltaNet: it is the
    same recurrence with the gate broadcast over dk); beta float32 [T, H];
    init_state [N, H, dk, dv] (widened to fp64) or None; cu_seqlens int [N+1] or None
    (one sequence).  A leading batch axis [B, T, H, d] is accepted when
    cu_seqlens is None and is treated as B sequences of length T.

    Returns (out fp64 with the shape of v, final_state fp64 [N, H, dk, dv]).
    """
    vshape = v.shape
    if q.ndim == 4:
        assert cu_seqlens is None
        B, T = q.shape[:2]
        q, k, v = (x.reshape((B * T,) + x.shape[2:]) for x in (q, k, v))
        log_alpha = log_alpha.reshape((B * T,) + log_alpha.shape[2:])
        beta = beta.reshape(B * T, -1)
        cu_seqlens = np.arange(B + 1, dtype=np.int64) * T
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], np.int64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    assert int(cu[-1]) == T, "cu_seqlens must cover every token"
    bf16 = q.dtype == np.uint16
    f64 = q.dtype == np.float64  # every per-token input then enters in fp64
    kind = 2 if f64 else int(bf16)
    want = np.float64 if f64 else (np.uint16 if bf16 else np.float32)
    fwant = np.float64 if f64 else np.float32
    q, k, v = (np.ascontiguousarray(x, dtype=want) for x in (q, k, v))
    la = np.ascontiguousarray(log_alpha, dtype=fwant)
    if la.ndim == 2:
        la = np.ascontiguousarray(np.broadcast_to(la[:, :, None], (T, H, dk)))
    be = np.ascontiguousarray(beta, dtype=fwant).reshape(T, H)
    init = None if init_state is None else np.ascontiguousarray(init_state, dtype=np.float64)
    if init is not None:
        assert init.shape == (N, H, dk, dv)
    out = np.zeros((T, H, dv), np.float64)
    fin = np.zeros((N, H, dk, dv), np.float64)
    nt = threads or max(1, min(64, os.cpu_count() or 1))
    rc = _lib(mutant).kda_oracle_forward(N, cu.ctypes.data, H, dk, dv, kind, _ptr(q), _ptr(k),
                                         _ptr(v), _ptr(la), _ptr(be), _ptr(init), _ptr(out),
                                         _ptr(fin), nt)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward failed ({rc})")
    return out.reshape(vshape), fin


def dplr_recurrent(q, k, v, a, b, log_alpha, init_state=None, cu_seqlens=None, threads=None, mutant: int = 0):
    """fp64 token-by-token general DPLR forward:
    S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t.

    q, k, a, b [T, H, dk] and v [T, H, dv] as float32 or uint16 (bf16 bits), all
    the same dtype; log_alpha float32 [T, H, dk]; init_state [N, H, dk, dv] or None;
    cu_seqlens int [N+1] or None.  A leading batch axis [B, T, H, d] is accepted
    without cu_seqlens.  Returns (out fp64 [.., H, dv], final_state fp64 [N, H, dk, dv]).
    """
    vshape = v.shape
    if q.ndim == 4:
        assert cu_seqlens is None
        B, T = q.shape[:2]
        q, k, v, a, b, log_alpha = (x.reshape((B * T,) + x.shape[2:]) for x in (q, k, v, a, b, log_alpha))
        cu_seqlens = np.arange(B + 1, dtype=np.int64) * T
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], np.int64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    assert int(cu[-1]) == T, "cu_seqlens must cover every token"
    bf16 = q.dtype == np.uint16
    want = np.uint16 if bf16 else np.float32
    q, k, v, a, b = (np.ascontiguousarray(x, dtype=want) for x in (q, k, v, a, b))
    la = np.ascontiguousarray(log_alpha, dtype=np.float32)
    assert la.shape == (T, H, dk) and a.shape == b.shape == (T, H, dk)
    init = None if init_state is None else np.ascontiguousarray(init_state, dtype=np.float64)
    if init is not None:
        assert init.shape == (N, H, dk, dv)
    out = np.zeros((T, H, dv), np.float64)
    fin = np.zeros((N, H, dk, dv), np.float64)
    nt = threads or max(1, min(64, os.cpu_count() or 1))
    rc = _lib(mutant).dplr_oracle_forward(N, cu.ctypes.data, H, dk, dv, int(bf16), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(a), _ptr(b), _ptr(la), _ptr(init), _ptr(out), _ptr(fin), nt)
    if rc != 0:
        raise RuntimeError(f"dplr_oracle_forward failed ({rc})")
    return out.reshape(vshape), fin


def backward(q, k, v, log_alpha, beta, d_out, init_state=None, d_final=None, cu_seqlens=None, threads=None):
    """fp64 gradients of L = sum(d_out * out) + sum(d_final * final_state) through the recurrence.

    Inputs as for ``recurrent`` (packed [T, H, d]; float32, bf16 bits or float64);
    d_out [T, H, dv] and d_final [N, H, dk, dv] (or None) any float dtype.  The
    reverse mode is the hand-derived adjoint of each token step
    (kda_oracle_backward in kda_oracle.c).  A per-head log_alpha [T, H] gets the
    sum over key channels of the per-channel gradient.
    Returns dict dq, dk [T, H, dk], dv [T, H, dv], dlog_alpha (shape of
    log_alpha), dbeta [T, H], dinit [N, H, dk, dv], all fp64.
    """
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], np.int64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    assert int(cu[-1]) == T
    bf16 = q.dtype == np.uint16
    f64 = q.dtype == np.float64
    kind = 2 if f64 else int(bf16)
    want = np.float64 if f64 else (np.uint16 if bf16 else np.float32)
    fwant = np.float64 if f64 else np.float32
    q, k, v = (np.ascontiguousarray(x, dtype=want) for x in (q, k, v))
    per_head = np.asarray(log_alpha).ndim == 2
    la = np.ascontiguousarray(log_alpha, dtype=fwant)
    if per_head:
        la = np.ascontiguousarray(np.broadcast_to(la[:, :, None], (T, H, dk)))
    be = np.ascontiguousarray(beta, dtype=fwant).reshape(T, H)
    init = None if init_state is None else np.ascontiguousarray(init_state, dtype=np.float64)
    dO = np.ascontiguousarray(d_out, dtype=np.float64)
    dF = None if d_final is None else np.ascontiguousarray(d_final, dtype=np.float64)
    g = {"dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
         "dlog_alpha": np.zeros((T, H, dk)), "dbeta": np.zeros((T, H)), "dinit": np.zeros((N, H, dk, dv))}
    nt = threads or max(1, min(64, os.cpu_count() or 1))
    rc = _lib(0).kda_oracle_backward(N, cu.ctypes.data, H, dk, dv, kind, _ptr(q), _ptr(k), _ptr(v), _ptr(la),
                                     _ptr(be), _ptr(init), _ptr(dO), _ptr(dF), _ptr(g["dq"]), _ptr(g["dk"]),
                                     _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["dbeta"]), _ptr(g["dinit"]), nt)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_backward failed ({rc})")
    if per_head:
        g["dlog_alpha"] = g["dlog_alpha"].sum(axis=2)
    return g


def decode_steps(state, steps, threads=None, mutant: int = 0):
    """Consecutive one-token updates of N independent sequences.

    ``state`` [N, H, dk, dv] (any float dtype); ``steps`` a list of dicts with
    q, k [N, H, dk], v [N, H, dv], beta [N, H], log_alpha [N, H, dk] or [N, H].  Each
    step is the recurrence over N one-token sequences starting from the
    current state, which is carried in fp64 between steps.  Returns (list of
    fp64 outputs [N, H, dv], fp64 final state).
    """
    S = np.asarray(state, np.float64)
    cu = np.arange(S.shape[0] + 1, dtype=np.int64)
    outs = []
    for st in steps:
        o, S = recurrent(st["q"], st["k"], st["v"], st["log_alpha"], st["beta"], S, cu,
                         threads, mutant)
        outs.append(o)
    return outs, S


class Metrics:
    """Parity figures over a tensor fed in pieces (so no full fp64 copy of a large
    output is ever held): the largest |x - ref|, the sum of ref^2, the sum of
    (x - ref)^2 and the element count, from which

        max_over_rms = max_i |x_i - ref_i| / sqrt(mean_i ref_i^2)   (the parity figure)
        max_abs      = max_i |x_i - ref_i|
        rms_err      = sqrt(mean_i (x_i - ref_i)^2)
        rms_ref      = sqrt(mean_i ref_i^2)

    With RMS(ref) = 0 the figure is 0 when every error is 0, else infinite; an
    empty tensor has no error.  A non-finite x gives a non-finite error (NaN
    propagates through the maximum)."""

    def __init__(self):
        self.max_err = 0.0
        self.sum_ref2 = 0.0
        self.sum_err2 = 0.0
        self.count = 0

    def add(self, x, ref):
        x = np.asarray(x, np.float64)
        ref = np.asarray(ref, np.float64)
        if x.shape != ref.shape:
            raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
        if ref.size == 0:
            return self
        err = np.abs(x - ref)
        m = float(np.max(err))
        # NaN in x must not vanish in a max with an earlier finite value
        self.max_err = m if (np.isnan(m) or m > self.max_err) else self.max_err
        self.sum_ref2 += float(np.sum(ref * ref))
        self.sum_err2 += float(np.sum(err * err))
        self.count += ref.size
        return self

    def result(self):
        if self.count == 0:
            return {"max_over_rms": 0.0, "max_abs": 0.0, "rms_err": 0.0, "rms_ref": 0.0}
        rms = float(np.sqrt(self.sum_ref2 / self.count))
        mx = self.max_err
        if rms > 0:
            ratio = mx / rms
        else:
            ratio = 0.0 if mx == 0 else float("inf")
        return {"max_over_rms": ratio, "max_abs": mx, "rms_err": float(np.sqrt(self.sum_err2 / self.count)),
                "rms_ref": rms}


def metrics(x, ref):
    """max|x - ref| / RMS(ref) plus the absolute max and RMS errors (see ``Metrics``)."""
    return Metrics().add(x, ref).result()
