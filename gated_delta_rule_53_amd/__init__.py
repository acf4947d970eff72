"""MI355X (gfx950) Kimi Delta Attention operator: chunked prefill and recurrent decode,
and the general DPLR transition it constrains (chunked prefill).

A thin binding over ``libkda.so`` (see ``include/kda.h``).  Every step of the
computation runs in the library's HIP kernels; this module only checks
shapes, allocates outputs and workspace through PyTorch, and passes device
pointers and the current HIP stream across the C ABI.  If the library has
not been built the calls raise; there is no CPU fallback.
"""
from __future__ import annotations

from . import _lib
from ._lib import KdaError, lib, status_string  # noqa: F401

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "dplr_chunk_fwd", "dplr_decode_step", "chunk_bwd", "decode_step",
           "layer_fwd", "layer_decode_step",
           "workspace_size", "dplr_workspace_size", "bwd_workspace_size", "KdaError"]


def _torch():
    import torch
    return torch


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.float32:
        return _lib.DTYPE_F32
    if dt == torch.bfloat16:
        return _lib.DTYPE_BF16
    raise TypeError(f"unsupported dtype {dt}; use torch.float32 or torch.bfloat16")


def _stream_handle(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _check_dev(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def workspace_size(batch, seqlen, heads, dk, dv, in_dtype, out_dtype=None, num_seqs=0, max_seqlen=0):
    """Bytes of device workspace ``chunk_fwd`` needs (varlen iff num_seqs > 0)."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    shape = _lib.shape(batch, seqlen, num_seqs, heads, dk, dv, _dtype_code(in_dtype), _dtype_code(out_dtype),
                       max_seqlen)
    return int(lib().kda_chunk_fwd_workspace_size(shape))


def dplr_workspace_size(batch, seqlen, heads, dk, dv, in_dtype, out_dtype=None, num_seqs=0, max_seqlen=0):
    """Bytes of device workspace ``dplr_chunk_fwd`` needs (varlen iff num_seqs > 0)."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    shape = _lib.shape(batch, seqlen, num_seqs, heads, dk, dv, _dtype_code(in_dtype), _dtype_code(out_dtype),
                       max_seqlen)
    return int(lib().kda_dplr_chunk_fwd_workspace_size(shape))


def bwd_workspace_size(batch, seqlen, heads, dk, dv, in_dtype, dout_dtype=None, num_seqs=0, max_seqlen=0):
    """Bytes of device workspace ``chunk_bwd`` needs (varlen iff num_seqs > 0)."""
    torch = _torch()
    dout_dtype = torch.float32 if dout_dtype is None else dout_dtype
    shape = _lib.shape(batch, seqlen, num_seqs, heads, dk, dv, _dtype_code(in_dtype), _dtype_code(dout_dtype),
                       max_seqlen)
    return int(lib().kda_chunk_bwd_workspace_size(shape))


def _prefill_args(q, k, v, log_alpha, beta, init_state, cu_seqlens, out, out_dtype, final_state, max_seqlen):
    """Check the prefill's tensors, allocate out / final_state if asked; returns (shape, out, final)."""
    torch = _torch()
    _check_dev(q, "q")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _check_dev(k, "k", q.dtype, q.shape)
    _check_dev(v, "v", q.dtype, (B, T, H, dv))
    gate_per_head = log_alpha.dim() == 3
    _check_dev(log_alpha, "log_alpha", torch.float32, (B, T, H) if gate_per_head else (B, T, H, dk))
    if beta is not None:  # the general DPLR variant has none
        _check_dev(beta, "beta", torch.float32, (B, T, H))
    if cu_seqlens is not None:
        _check_dev(cu_seqlens, "cu_seqlens", torch.int32)
        if B != 1:
            raise ValueError("varlen inputs must have batch 1")
        N = cu_seqlens.numel() - 1
        if max_seqlen is None:
            max_seqlen = T  # safe upper bound without a device sync
    else:
        N = B
    if init_state is not None:
        _check_dev(init_state, "init_state", torch.float32, (N, H, dk, dv))
    out_dtype = q.dtype if out_dtype is None and out is None else (out.dtype if out is not None else out_dtype)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    _check_dev(out, "out", out_dtype, (B, T, H, dv))
    if final_state is True:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is False:
        final_state = None
    if final_state is not None:
        _check_dev(final_state, "final_state", torch.float32, (N, H, dk, dv))
    shape = _lib.shape(B, T, N if cu_seqlens is not None else 0, H, dk, dv, _dtype_code(q.dtype),
                       _dtype_code(out_dtype), int(max_seqlen or 0), int(gate_per_head))
    return shape, out, final_state


def chunk_fwd(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, *, out=None,
              out_dtype=None, final_state=True, max_seqlen=None, workspace=None):
    """Chunked KDA prefill.

    q, k [B,T,H,dk], v [B,T,H,dv] (fp32 or bf16), log_alpha [B,T,H,dk] fp32
    (or [B,T,H]: one gate per head shared by the key channels, the scalar gate
    of Gated DeltaNet), beta [B,T,H] fp32; init_state [N,H,dk,dv] fp32 or None; cu_seqlens int32
    [N+1] (GPU) or None.  ``final_state`` may be True (allocate), False/None
    (skip) or a tensor to write into (may be ``init_state`` itself).
    Returns (out, final_state or None).
    """
    torch = _torch()
    shape, out, final_state = _prefill_args(q, k, v, log_alpha, beta, init_state, cu_seqlens, out, out_dtype,
                                            final_state, max_seqlen)
    L = lib()
    need = int(L.kda_chunk_fwd_workspace_size(shape))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_dev(workspace, "workspace", torch.uint8)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = L.kda_chunk_fwd(shape, ptr(q), ptr(k), ptr(v), ptr(log_alpha), ptr(beta), ptr(init_state),
                         ptr(cu_seqlens), ptr(out), ptr(final_state), ptr(workspace), workspace.numel(),
                         _stream_handle(q.device))
    _lib.check(st, "kda_chunk_fwd")
    return out, final_state



def dplr_chunk_fwd(q, k, v, a, b, log_alpha, init_state=None, cu_seqlens=None, *, out=None, out_dtype=None,
                   final_state=True, max_seqlen=None, workspace=None):
    """Chunked prefill of the general DPLR transition (kda_dplr_chunk_fwd):
    S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t.

    q, k, a, b [B,T,H,128] and v [B,T,H,128] (all fp32 or all bf16); log_alpha
    [B,T,H,128] fp32; no beta.  init_state, cu_seqlens, out, final_state,
    max_seqlen and workspace as for ``chunk_fwd``.  Returns (out, final_state or None).
    """
    torch = _torch()
    _check_dev(a, "a", q.dtype, q.shape)
    _check_dev(b, "b", q.dtype, q.shape)
    if log_alpha.dim() != 4:
        raise ValueError("the general DPLR variant takes a per-channel log_alpha [B,T,H,dk]")
    shape, out, final_state = _prefill_args(q, k, v, log_alpha, None, init_state, cu_seqlens, out, out_dtype,
                                            final_state, max_seqlen)
    L = lib()
    need = int(L.kda_dplr_chunk_fwd_workspace_size(shape))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_dev(workspace, "workspace", torch.uint8)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = L.kda_dplr_chunk_fwd(shape, ptr(q), ptr(k), ptr(v), ptr(a), ptr(b), ptr(log_alpha), ptr(init_state),
                              ptr(cu_seqlens), ptr(out), ptr(final_state), ptr(workspace), workspace.numel(),
                              _stream_handle(q.device))
    _lib.check(st, "kda_dplr_chunk_fwd")
    return out, final_state

def chunk_fwd_noalloc(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, *, out, final_state=None,
                      max_seqlen=None):
    """``chunk_fwd`` without a workspace: the library's static per-device scratch of
    ``_lib.NOALLOC_SCRATCH_BYTES`` serves instead, and nothing is allocated -- the caller
    passes ``out`` and, if wanted, ``final_state`` (a tensor, or None to skip it).  Calls
    overlapping in time on one device race on that scratch."""
    if final_state is True or final_state is False:
        raise TypeError("chunk_fwd_noalloc allocates nothing: pass final_state as a tensor or None")
    shape, out, final_state = _prefill_args(q, k, v, log_alpha, beta, init_state, cu_seqlens, out, None,
                                            final_state, max_seqlen)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib().kda_chunk_fwd_noalloc(shape, ptr(q), ptr(k), ptr(v), ptr(log_alpha), ptr(beta), ptr(init_state),
                                     ptr(cu_seqlens), ptr(out), ptr(final_state), _stream_handle(q.device))
    _lib.check(st, "kda_chunk_fwd_noalloc")
    return out, final_state


def decode_step(q, k, v, log_alpha, beta, state, *, out=None, out_dtype=None):
    """One recurrent KDA step for N sequences; updates ``state`` [N,H,dk,dv] in place.

    q, k [N,H,dk], v [N,H,dv] (fp32 or bf16), log_alpha [N,H,dk] fp32 (or [N,H]:
    one gate per head), beta [N,H] fp32.  Returns out [N,H,dv].
    """
    torch = _torch()
    _check_dev(q, "q")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _check_dev(k, "k", q.dtype, q.shape)
    _check_dev(v, "v", q.dtype, (N, H, dv))
    gate_per_head = log_alpha.dim() == 2
    _check_dev(log_alpha, "log_alpha", torch.float32, (N, H) if gate_per_head else (N, H, dk))
    _check_dev(beta, "beta", torch.float32, (N, H))
    _check_dev(state, "state", torch.float32, (N, H, dk, dv))
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    _check_dev(out, "out", None, (N, H, dv))
    name = "kda_decode_step_head_gate" if gate_per_head else "kda_decode_step"
    st = getattr(lib(), name)(N, H, dk, dv, _dtype_code(q.dtype), _dtype_code(out.dtype), q.data_ptr(),
                              k.data_ptr(), v.data_ptr(), log_alpha.data_ptr(), beta.data_ptr(), state.data_ptr(),
                              out.data_ptr(), _stream_handle(q.device))
    _lib.check(st, name)
    return out


def dplr_decode_step(q, k, v, a, b, log_alpha, state, *, out=None, out_dtype=None):
    """One recurrent step of the general DPLR transition (kda_dplr_decode_step) for N
    sequences: S <- Diag(alpha) S - a (b^T S) + k v^T, o = S^T q; updates ``state``
    [N,H,dk,dv] in place.  q, k, a, b [N,H,dk], v [N,H,dv] (all fp32 or all bf16),
    log_alpha [N,H,dk] fp32.  Returns out [N,H,dv]."""
    torch = _torch()
    _check_dev(q, "q")
    N, H, dk = q.shape
    dv = v.shape[-1]
    for t, name in ((k, "k"), (a, "a"), (b, "b")):
        _check_dev(t, name, q.dtype, q.shape)
    _check_dev(v, "v", q.dtype, (N, H, dv))
    _check_dev(log_alpha, "log_alpha", torch.float32, (N, H, dk))
    _check_dev(state, "state", torch.float32, (N, H, dk, dv))
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    _check_dev(out, "out", None, (N, H, dv))
    st = lib().kda_dplr_decode_step(N, H, dk, dv, _dtype_code(q.dtype), _dtype_code(out.dtype), q.data_ptr(),
                                    k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(), log_alpha.data_ptr(),
                                    state.data_ptr(), out.data_ptr(), _stream_handle(q.device))
    _lib.check(st, "kda_dplr_decode_step")
    return out


def _layer(gate, out_gate, norm_weight, qk_l2norm, l2_eps, rms_eps, dv):
    torch = _torch()
    if gate.dtype != torch.bfloat16:
        raise TypeError("gate must be bf16 (the gate pre-activation)")
    if out_gate is not None and out_gate.dtype != torch.bfloat16:
        raise TypeError("out_gate must be bf16")
    if norm_weight is not None:
        _check_dev(norm_weight, "norm_weight", torch.float32, (dv,))
    ptr = lambda t: None if t is None else t.data_ptr()
    return _lib.Layer(int(bool(qk_l2norm)), float(l2_eps), ptr(gate), ptr(out_gate), ptr(norm_weight),
                      float(rms_eps))


def layer_fwd(q, k, v, gate, beta, init_state=None, cu_seqlens=None, *, out_gate=None, norm_weight=None,
              qk_l2norm=True, l2_eps=1e-6, rms_eps=1e-6, out=None, out_dtype=None, final_state=True,
              max_seqlen=None, workspace=None):
    """Chunked prefill of the KDA layer: q/k L2 normalisation, log alpha = -softplus(gate),
    the recurrence, then y = RMSNorm(o) * norm_weight * sigmoid(out_gate) (skipped when
    out_gate is None).

    q, k [B,T,H,dk], v [B,T,H,dv] (fp32 or bf16); gate bf16 [B,T,H,dk] (or [B,T,H]: one
    gate per head); beta [B,T,H] fp32; out_gate bf16 [B,T,H,dv] or None; norm_weight
    fp32 [dv] or None (ones).  Other arguments as ``chunk_fwd``.  Returns (y, final_state).
    """
    torch = _torch()
    _check_dev(q, "q")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _check_dev(k, "k", q.dtype, q.shape)
    _check_dev(v, "v", q.dtype, (B, T, H, dv))
    gate_per_head = gate.dim() == 3
    _check_dev(gate, "gate", torch.bfloat16, (B, T, H) if gate_per_head else (B, T, H, dk))
    _check_dev(beta, "beta", torch.float32, (B, T, H))
    if out_gate is not None:
        _check_dev(out_gate, "out_gate", torch.bfloat16, (B, T, H, dv))
    if cu_seqlens is not None:
        _check_dev(cu_seqlens, "cu_seqlens", torch.int32)
        if B != 1:
            raise ValueError("varlen inputs must have batch 1")
        N = cu_seqlens.numel() - 1
        if max_seqlen is None:
            max_seqlen = T
    else:
        N = B
    if init_state is not None:
        _check_dev(init_state, "init_state", torch.float32, (N, H, dk, dv))
    out_dtype = q.dtype if out_dtype is None and out is None else (out.dtype if out is not None else out_dtype)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    _check_dev(out, "out", out_dtype, (B, T, H, dv))
    if final_state is True:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is False:
        final_state = None
    if final_state is not None:
        _check_dev(final_state, "final_state", torch.float32, (N, H, dk, dv))
    shape = _lib.shape(B, T, N if cu_seqlens is not None else 0, H, dk, dv, _dtype_code(q.dtype),
                       _dtype_code(out_dtype), int(max_seqlen or 0), int(gate_per_head))
    layer = _layer(gate, out_gate, norm_weight, qk_l2norm, l2_eps, rms_eps, dv)
    L = lib()
    need = int(L.kda_chunk_fwd_workspace_size(shape))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_dev(workspace, "workspace", torch.uint8)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = L.kda_layer_fwd(shape, layer, ptr(q), ptr(k), ptr(v), ptr(beta), ptr(init_state), ptr(cu_seqlens),
                         ptr(out), ptr(final_state), ptr(workspace), workspace.numel(), _stream_handle(q.device))
    _lib.check(st, "kda_layer_fwd")
    return out, final_state


def layer_decode_step(q, k, v, gate, beta, state, *, out_gate=None, norm_weight=None, qk_l2norm=True,
                      l2_eps=1e-6, rms_eps=1e-6, out=None, out_dtype=None):
    """One decode step of the KDA layer (see ``layer_fwd``); updates ``state`` in place.

    q, k [N,H,dk], v [N,H,dv]; gate bf16 [N,H,dk] or [N,H]; beta [N,H] fp32; out_gate
    bf16 [N,H,dv] or None.  Returns y [N,H,dv].
    """
    torch = _torch()
    _check_dev(q, "q")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _check_dev(k, "k", q.dtype, q.shape)
    _check_dev(v, "v", q.dtype, (N, H, dv))
    gate_per_head = gate.dim() == 2
    _check_dev(gate, "gate", torch.bfloat16, (N, H) if gate_per_head else (N, H, dk))
    _check_dev(beta, "beta", torch.float32, (N, H))
    _check_dev(state, "state", torch.float32, (N, H, dk, dv))
    if out_gate is not None:
        _check_dev(out_gate, "out_gate", torch.bfloat16, (N, H, dv))
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    _check_dev(out, "out", None, (N, H, dv))
    layer = _layer(gate, out_gate, norm_weight, qk_l2norm, l2_eps, rms_eps, dv)
    st = lib().kda_layer_decode_step(N, H, dk, dv, _dtype_code(q.dtype), _dtype_code(out.dtype),
                                     int(gate_per_head), layer, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     beta.data_ptr(), state.data_ptr(), out.data_ptr(), _stream_handle(q.device))
    _lib.check(st, "kda_layer_decode_step")
    return out


def chunk_bwd(q, k, v, log_alpha, beta, d_out, init_state=None, d_final=None, cu_seqlens=None, *,
              max_seqlen=None, want_d_init=True, workspace=None, out=None):
    """Gradients of sum(d_out * out) + sum(d_final * final_state) through the chunked prefill.

    Inputs as for ``chunk_fwd``; d_out [B,T,H,dv] (the dtype ``out`` had), d_final
    [N,H,dk,dv] fp32 or None.  Returns a dict of fp32 tensors dq, dk, dv, dlog_alpha
    (the shape of log_alpha), dbeta and, with ``want_d_init``, d_init.  ``out`` may hold
    any of those tensors, preallocated; the rest are allocated here.
    """
    torch = _torch()
    _check_dev(q, "q")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _check_dev(k, "k", q.dtype, q.shape)
    _check_dev(v, "v", q.dtype, (B, T, H, dv))
    gate_per_head = log_alpha.dim() == 3
    _check_dev(log_alpha, "log_alpha", torch.float32, (B, T, H) if gate_per_head else (B, T, H, dk))
    _check_dev(beta, "beta", torch.float32, (B, T, H))
    _check_dev(d_out, "d_out", None, (B, T, H, dv))
    if cu_seqlens is not None:
        _check_dev(cu_seqlens, "cu_seqlens", torch.int32)
        if B != 1:
            raise ValueError("varlen inputs must have batch 1")
        N = cu_seqlens.numel() - 1
        if max_seqlen is None:
            max_seqlen = T
    else:
        N = B
    if init_state is not None:
        _check_dev(init_state, "init_state", torch.float32, (N, H, dk, dv))
    if d_final is not None:
        _check_dev(d_final, "d_final", torch.float32, (N, H, dk, dv))
    shape = _lib.shape(B, T, N if cu_seqlens is not None else 0, H, dk, dv, _dtype_code(q.dtype),
                       _dtype_code(d_out.dtype), int(max_seqlen or 0), int(gate_per_head))
    f32 = dict(dtype=torch.float32, device=q.device)
    shapes = {"dq": (B, T, H, dk), "dk": (B, T, H, dk), "dv": (B, T, H, dv), "dlog_alpha": tuple(log_alpha.shape),
              "dbeta": (B, T, H)}
    if want_d_init:
        shapes["d_init"] = (N, H, dk, dv)
    out = {} if out is None else out
    g = {}
    for name, shp in shapes.items():
        g[name] = out[name] if name in out else torch.empty(shp, **f32)
        _check_dev(g[name], name, torch.float32, shp)
    L = lib()
    need = int(L.kda_chunk_bwd_workspace_size(shape))
    if need == 0:
        raise KdaError(2, "kda_chunk_bwd_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check_dev(workspace, "workspace", torch.uint8)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = L.kda_chunk_bwd(shape, ptr(q), ptr(k), ptr(v), ptr(log_alpha), ptr(beta), ptr(init_state),
                         ptr(cu_seqlens), ptr(d_out), ptr(d_final), ptr(g["dq"]), ptr(g["dk"]), ptr(g["dv"]),
                         ptr(g["dlog_alpha"]), ptr(g["dbeta"]), ptr(g.get("d_init")), ptr(workspace),
                         workspace.numel(), _stream_handle(q.device))
    _lib.check(st, "kda_chunk_bwd")
    return g
