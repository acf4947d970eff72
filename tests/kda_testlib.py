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


def assert_close(name, got, ref, tol):
    m = oracle.metrics(got, ref)
    assert np.isfinite(np.asarray(got, np.float64)).all(), f"{name}: non-finite values"
    assert m["max_over_rms"] <= tol, (f"{name}: max|err|/rms = {m['max_over_rms']:.3e} > {tol:.1e} "
                                      f"(max abs {m['max_abs']:.3e}, rms ref {m['rms_ref']:.3e})")
    return m


def run_chunk(kda, torch, d, out_dtype=None, final=True, workspace=None, max_seqlen=None):
    """Run kda.chunk_fwd on a synth dict (packed [T, H, d] arrays); returns numpy (out [T,H,dv], final)."""
    q, k, v, la, b = (to_dev(d[x], torch).unsqueeze(0) for x in ("q", "k", "v", "log_alpha", "beta"))
    cu = d.get("cu_seqlens")
    varlen = cu is not None and len(cu) != 2
    cu_t = torch.from_numpy(np.asarray(cu, np.int32)).cuda() if varlen else None
    init = None if d.get("init") is None else to_dev(d["init"], torch)
    out, fin = kda.chunk_fwd(q, k, v, la, b, init, cu_t, out_dtype=out_dtype or torch.float32,
                             final_state=final, workspace=workspace, max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    o = out[0].float().cpu().numpy()
    return o, (None if fin is None else fin.cpu().numpy())


def oracle_chunk(d):
    return oracle.recurrent(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d.get("init"),
                            d.get("cu_seqlens"))
