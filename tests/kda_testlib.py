"""Shared helpers for the GPU parity tests: device transfer, oracle comparison, tolerances.

Tolerances (max|gpu - oracle| / RMS(oracle), per output tensor):
  * 1e-4 for fp32 q/k/v, 2e-2 for bf16 q/k/v -- the bars set for the KDA
    operator on this hardware;
  * decode runs entirely in fp32 arithmetic, so its tests use 1e-4 whatever
    the input dtype.
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}
DECODE_TOL = 1e-4


def to_dev(x, torch, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def _report(name, m, tol):
    """One line per comparison (shown with pytest -s), then the bar."""
    print(f"  {name}: max|err|/rms {m['max_over_rms']:.2e} (bar {tol:.0e}), max abs {m['max_abs']:.2e}, "
          f"rms ref {m['rms_ref']:.2e}", flush=True)
    assert m["max_over_rms"] <= tol, (f"{name}: max|err|/rms = {m['max_over_rms']:.3e} > {tol:.1e} "
                                      f"(max abs {m['max_abs']:.3e}, rms ref {m['rms_ref']:.3e})")
    return m


def assert_close(name, got, ref, tol):
    m = oracle.metrics(got, ref)
    assert np.isfinite(np.asarray(got, np.float64)).all(), f"{name}: non-finite values"
    return _report(name, m, tol)


def assert_close_bf16_storage(name, got, ref, tol):
    """Parity of a bf16-stored output: each element may differ from the reference by the
    rounding of its storage, up to 2^-8 of its magnitude (round to nearest even at 8
    significant bits), on top of tol x RMS(ref).  Over many elements the largest ones reach
    several times RMS(ref), where that rounding alone can exceed an RMS-relative bar."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    excess = np.abs(got - ref) - 2.0 ** -8 * np.maximum(np.abs(got), np.abs(ref))
    worst = max(float(excess.max()), 0.0) if ref.size else 0.0
    fig = worst / rms if rms > 0 else (0.0 if worst == 0 else float("inf"))
    print(f"  {name}: beyond bf16 storage rounding, max|err|/rms {fig:.2e} (bar {tol:.0e})", flush=True)
    assert fig <= tol, f"{name}: {fig:.3e} beyond the bf16 storage rounding > {tol:.1e}"


def assert_metrics(name, acc, tol):
    """assert_close for a figure accumulated over pieces (oracle.Metrics)."""
    return _report(name, acc.result(), tol)


def nan_tensor(torch, shape, dtype=None, device="cuda"):
    """An output buffer filled with NaN: an element the kernels never write stays NaN and fails
    the comparison, whatever an earlier run left in that memory."""
    return torch.full(tuple(shape), float("nan"), dtype=dtype or torch.float32, device=device)


def run_chunk(kda, torch, d, out_dtype=None, final=True, workspace=None, max_seqlen=None):
    """Run kda.chunk_fwd on a synth dict (packed [T, H, d] arrays), into NaN-filled output
    and final-state buffers; returns numpy (out [T,H,dv], final)."""
    q, k, v, la, b = (to_dev(d[x], torch).unsqueeze(0) for x in ("q", "k", "v", "log_alpha", "beta"))
    cu = d.get("cu_seqlens")
    varlen = cu is not None and len(cu) != 2
    cu_t = torch.from_numpy(np.asarray(cu, np.int32)).cuda() if varlen else None
    init = None if d.get("init") is None else to_dev(d["init"], torch)
    N = len(cu) - 1 if varlen else 1
    H, dk, dv = q.shape[2], q.shape[3], v.shape[3]
    out = nan_tensor(torch, v.shape, out_dtype or torch.float32)
    fin = nan_tensor(torch, (N, H, dk, dv)) if final else False
    out, fin = kda.chunk_fwd(q, k, v, la, b, init, cu_t, out=out, final_state=fin, workspace=workspace,
                             max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    o = out[0].float().cpu().numpy()
    return o, (None if fin is None else fin.cpu().numpy())


def oracle_chunk(d):
    return oracle.recurrent(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d.get("init"),
                            d.get("cu_seqlens"))
