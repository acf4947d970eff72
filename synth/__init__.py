"""Seeded synthetic inputs for the KDA operator (prefill and decode).

This module only draws and shapes random inputs. It holds none of the
operator's arithmetic, so both the fp64 oracle and the HIP library can be
fed from it without sharing any code with each other.

Workloads follow the head geometry of one Kimi-Linear-48B-A3B KDA layer
("Kimi Linear" page, section "The constrained DPLR form and the chunkwise
algorithm": key and value head dimensions 128, chunks of 64; the context
window of 1,048,576 tokens is in the page's infobox).

Recipe (every tensor is drawn block-wise so any subset can be regenerated):

* Each (tensor, head, token block of ``BLOCK`` tokens) gets its own
  ``numpy.random.SeedSequence(seed, spawn_key=(tensor_id, head, block))``
  feeding a PCG64 generator; the draw order inside a block is token-major.
* q, k ~ N(0, 1), L2-normalised per (token, head) in fp64, then rounded to
  fp32 and, for bf16 workloads, from fp32 to bf16 by round-to-nearest-even.
* v ~ N(0, 1), rounded the same way.
* beta = sigmoid(N(0, 1)) in fp32.
* log_alpha = -s * softplus(N(0, 1)) in fp32 with s = 0.05 (0.01 for the
  long-memory 64K-token workload).
* Initial states ~ N(0, 0.02^2) fp32, one per (sequence, head).
* Varlen lengths: Dirichlet(1, ..., 1) shares of the tokens above a floor of
  4,096 per sequence, floored, with the remainder handed to the largest
  fractional parts (ties to the lower index).

Layer inputs (the prologue and epilogue around the operator, ``gen_layer_tokens``):

* q, k ~ N(0, 1) per element, not normalised (the layer normalises them);
  v and beta as above.
* the gate pre-activation g ~ N(mu, 1) per (token, head, key channel), or per
  (token, head), rounded to bf16, with mu = log(0.69 s) so that the median
  decay -softplus(g) ~ -e^g matches the -s * softplus(N(0, 1)) draw above.
* the output-gate pre-activation z ~ N(0, 1), bf16; the RMSNorm weight
  1 + 0.1 N(0, 1) fp32 [dv].

General-DPLR inputs (``gen_dplr_tokens``; the baseline with independent low-rank
vectors that KDA constrains): q, k, v and log_alpha as above (k is the write key,
unit length); a = rate * (unit row), rate = sigmoid(N(0, 1)) per (token, head);
b = an independent unit row; a and b rounded like q and k.

bf16 tensors are returned as ``numpy.uint16`` arrays holding the bf16 bit
patterns; fp32 tensors as ``numpy.float32``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK = 16384  # tokens per independently seeded block

# tensor ids used in the spawn keys
_TID = {"q": 0, "k": 1, "v": 2, "beta": 3, "log_alpha": 4, "init": 5, "lengths": 6, "log_alpha_head": 7,
        "q_raw": 8, "k_raw": 9, "gate_pre": 10, "gate_pre_head": 11, "out_gate": 12, "norm_weight": 13,
        "dplr_a": 14, "dplr_rate": 15, "dplr_b": 16}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload. ``kind`` is "prefill", "varlen" or "decode"."""
    name: str
    kind: str
    dtype: str            # "f32" or "bf16": dtype of q, k, v
    heads: int
    dk: int
    dv: int
    seqlen: int = 0       # tokens per sequence (prefill) or total tokens (varlen)
    batch: int = 1        # dense batch (prefill) or number of sequences (decode)
    num_seqs: int = 1     # varlen: number of packed sequences
    min_len: int = 0      # varlen: floor on every sequence length
    steps: int = 1        # decode: consecutive steps
    gate_scale: float = 0.05
    init_std: float | None = None   # None: zero initial state
    seed: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    0: Workload("kda_fwd_f32_h2_t256_d64", "prefill", "f32", heads=2, dk=64, dv=64,
                seqlen=256, batch=1, gate_scale=0.05, init_std=None, seed=0),
    1: Workload("kda_prefill_bf16_h32_t4096_d128", "prefill", "bf16", heads=32, dk=128, dv=128,
                seqlen=4096, batch=1, gate_scale=0.05, init_std=None, seed=1),
    2: Workload("kda_prefill_bf16_h32_t65536_d128", "prefill", "bf16", heads=32, dk=128, dv=128,
                seqlen=65536, batch=1, gate_scale=0.01, init_std=0.02, seed=2),
    3: Workload("kda_decode_bf16_n256_h32_d128_x100", "decode", "bf16", heads=32, dk=128, dv=128,
                batch=256, steps=100, gate_scale=0.05, init_std=0.02, seed=3),
    4: Workload("kda_varlen_bf16_n16_h32_t1048576_d128", "varlen", "bf16", heads=32, dk=128, dv=128,
                seqlen=1048576, num_seqs=16, min_len=4096, gate_scale=0.05, init_std=0.02, seed=4),
}


# ----------------------------------------------------------------------------
# bf16 helpers (bit patterns in uint16)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); finite inputs."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(x: np.ndarray) -> np.ndarray:
    """The real numbers an input array stands for, in fp64 (bf16 bits widened exactly)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# block-wise generation
# ----------------------------------------------------------------------------

def _rng(seed: int, tensor: str, head: int, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(_TID[tensor], head, block))
    return np.random.Generator(np.random.PCG64(ss))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_blocks(seed, tensor, T, heads, width, fn, out, threads):
    """out[t, h, :width] for t in [0, T): fill block (h, b) with fn(rng, ntok)."""
    nb = (T + BLOCK - 1) // BLOCK
    jobs = [(h, b) for h in heads for b in range(nb)]

    def work(job):
        h, b = job
        t0 = b * BLOCK
        t1 = min(T, t0 + BLOCK)
        vals = fn(_rng(seed, tensor, h, b), t1 - t0)
        hi = heads.index(h)
        if width is None:
            out[t0:t1, hi] = vals
        else:
            out[t0:t1, hi, :] = vals

    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            work(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, jobs))


def _unit_rows(dtype):
    def fn(rng, n, d):
        x = rng.standard_normal((n, d))
        x /= np.sqrt(np.sum(x * x, axis=1, keepdims=True))
        x = x.astype(np.float32)
        return f32_to_bf16_bits(x) if dtype == "bf16" else x
    return fn


def gen_tokens(seed: int, T: int, H: int, dk: int, dv: int, dtype: str, gate_scale: float,
               heads=None, threads=None, gate: str = "channel") -> dict:
    """Token inputs for T packed tokens: q, k [T,Hs,dk], v [T,Hs,dv], beta [T,Hs], log_alpha [T,Hs,dk].

    ``heads`` selects a subset of heads (Hs = len(heads)); values are identical
    to the same heads of the full draw.  ``gate="head"`` draws one gate per
    (token, head) instead, log_alpha [T,Hs] (the scalar gate of Gated
    DeltaNet), from its own stream with the same distribution.
    """
    heads = list(range(H)) if heads is None else list(heads)
    Hs = len(heads)
    threads = _threads() if threads is None else threads
    qk_dt = np.uint16 if dtype == "bf16" else np.float32
    unit = _unit_rows(dtype)
    out = {
        "q": np.empty((T, Hs, dk), qk_dt),
        "k": np.empty((T, Hs, dk), qk_dt),
        "v": np.empty((T, Hs, dv), qk_dt),
        "beta": np.empty((T, Hs), np.float32),
        "log_alpha": np.empty((T, Hs, dk) if gate == "channel" else (T, Hs), np.float32),
    }
    assert gate in ("channel", "head"), gate
    _fill_blocks(seed, "q", T, heads, dk, lambda r, n: unit(r, n, dk), out["q"], threads)
    _fill_blocks(seed, "k", T, heads, dk, lambda r, n: unit(r, n, dk), out["k"], threads)

    def vfn(r, n):
        x = r.standard_normal((n, dv), dtype=np.float32)
        return f32_to_bf16_bits(x) if dtype == "bf16" else x
    _fill_blocks(seed, "v", T, heads, dv, vfn, out["v"], threads)

    def bfn(r, n):
        z = r.standard_normal(n)
        return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    _fill_blocks(seed, "beta", T, heads, None, bfn, out["beta"], threads)

    def afn(r, n):
        z = r.standard_normal((n, dk) if gate == "channel" else n)
        sp = np.logaddexp(0.0, z)  # softplus
        return (-gate_scale * sp).astype(np.float32)
    if gate == "channel":
        _fill_blocks(seed, "log_alpha", T, heads, dk, afn, out["log_alpha"], threads)
    else:
        _fill_blocks(seed, "log_alpha_head", T, heads, None, afn, out["log_alpha"], threads)
    return out


def gen_dplr_tokens(seed: int, T: int, H: int, d: int, dtype: str, gate_scale: float, heads=None,
                    threads=None) -> dict:
    """General-DPLR token inputs: q, k, v, a, b [T, Hs, d] and log_alpha [T, Hs, d]
    (q, k, v, log_alpha identical to ``gen_tokens``'s draw of the same seed)."""
    heads = list(range(H)) if heads is None else list(heads)
    threads = _threads() if threads is None else threads
    out = gen_tokens(seed, T, H, d, d, dtype, gate_scale, heads=heads, threads=threads)
    del out["beta"]
    dt = np.uint16 if dtype == "bf16" else np.float32
    Hs = len(heads)

    def afn(r, n):
        x = r.standard_normal((n, d))
        x /= np.sqrt(np.sum(x * x, axis=1, keepdims=True))
        rate = 1.0 / (1.0 + np.exp(-r.standard_normal(n)))
        x = (x * rate[:, None]).astype(np.float32)
        return f32_to_bf16_bits(x) if dtype == "bf16" else x
    out["a"] = np.empty((T, Hs, d), dt)
    out["b"] = np.empty((T, Hs, d), dt)
    _fill_blocks(seed, "dplr_a", T, heads, d, afn, out["a"], threads)
    unit = _unit_rows(dtype)
    _fill_blocks(seed, "dplr_b", T, heads, d, lambda r, n: unit(r, n, d), out["b"], threads)
    return out


def dplr_small(seed: int, T: int, H: int, d: int, dtype: str = "f32", gate_scale: float = 0.05,
               init_std: float | None = 0.02, batch: int = 1, lens=None) -> dict:
    """Small general-DPLR workload (tests): q, k, v, a, b, log_alpha, cu_seqlens, init."""
    lens = np.full(batch, T, np.int64) if lens is None else np.asarray(lens, np.int64)
    cu = cu_from_lengths(lens)
    out = gen_dplr_tokens(seed, int(cu[-1]), H, d, dtype, gate_scale, threads=1)
    out["cu_seqlens"] = cu
    out["init"] = None if init_std is None else gen_states(seed, len(lens), H, d, d, init_std)
    return out


def layer_gate_mu(gate_scale: float) -> float:
    """Mean of the gate pre-activation draw for a workload's gate scale."""
    return float(np.log(0.69 * gate_scale))


def gen_layer_tokens(seed: int, T: int, H: int, dk: int, dv: int, dtype: str, gate_mu: float,
                     heads=None, threads=None, gate: str = "channel") -> dict:
    """Layer inputs for T packed tokens: q, k [T,Hs,dk] (not normalised), v [T,Hs,dv],
    beta [T,Hs], g bf16 [T,Hs,dk] (or [T,Hs] for ``gate="head"``), out_gate bf16 [T,Hs,dv]."""
    heads = list(range(H)) if heads is None else list(heads)
    Hs = len(heads)
    threads = _threads() if threads is None else threads
    dt = np.uint16 if dtype == "bf16" else np.float32
    assert gate in ("channel", "head"), gate
    out = {
        "q": np.empty((T, Hs, dk), dt),
        "k": np.empty((T, Hs, dk), dt),
        "v": np.empty((T, Hs, dv), dt),
        "beta": np.empty((T, Hs), np.float32),
        "g": np.empty((T, Hs, dk) if gate == "channel" else (T, Hs), np.uint16),
        "out_gate": np.empty((T, Hs, dv), np.uint16),
    }

    def normal(width, dtype_out, mu=0.0):
        def fn(r, n):
            x = (mu + r.standard_normal((n, width) if width else n)).astype(np.float32)
            return f32_to_bf16_bits(x) if dtype_out == "bf16" else x
        return fn
    _fill_blocks(seed, "q_raw", T, heads, dk, normal(dk, dtype), out["q"], threads)
    _fill_blocks(seed, "k_raw", T, heads, dk, normal(dk, dtype), out["k"], threads)
    _fill_blocks(seed, "v", T, heads, dv, normal(dv, dtype), out["v"], threads)

    def bfn(r, n):
        z = r.standard_normal(n)
        return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    _fill_blocks(seed, "beta", T, heads, None, bfn, out["beta"], threads)
    if gate == "channel":
        _fill_blocks(seed, "gate_pre", T, heads, dk, normal(dk, "bf16", gate_mu), out["g"], threads)
    else:
        _fill_blocks(seed, "gate_pre_head", T, heads, None, normal(None, "bf16", gate_mu), out["g"], threads)
    _fill_blocks(seed, "out_gate", T, heads, dv, normal(dv, "bf16"), out["out_gate"], threads)
    return out


def gen_norm_weight(seed: int, dv: int) -> np.ndarray:
    """RMSNorm weight [dv] fp32 ~ 1 + 0.1 N(0, 1)."""
    return (1.0 + 0.1 * _rng(seed, "norm_weight", 0, 0).standard_normal(dv)).astype(np.float32)


def gen_states(seed: int, N: int, H: int, dk: int, dv: int, std: float, heads=None,
               seqs=None, tag: int = 0) -> np.ndarray:
    """Initial states [Ns, Hs, dk, dv] fp32 ~ N(0, std^2); one stream per (sequence, head)."""
    heads = list(range(H)) if heads is None else list(heads)
    seqs = list(range(N)) if seqs is None else list(seqs)
    st = np.empty((len(seqs), len(heads), dk, dv), np.float32)
    for si, s in enumerate(seqs):
        for hi, h in enumerate(heads):
            r = _rng(seed, "init", h, (tag << 32) | s)
            st[si, hi] = (std * r.standard_normal((dk, dv))).astype(np.float32)
    return st


def dirichlet_lengths(seed: int, total: int, n: int, floor: int) -> np.ndarray:
    """Sequence lengths: floor + Dirichlet(1,...,1) share of the rest; sums to ``total``."""
    rest = total - n * floor
    assert rest >= 0
    p = _rng(seed, "lengths", 0, 0).dirichlet(np.ones(n))
    raw = p * rest
    base = np.floor(raw).astype(np.int64)
    rem = int(rest - base.sum())
    frac = raw - base
    order = sorted(range(n), key=lambda i: (-frac[i], i))
    for i in order[:rem]:
        base[i] += 1
    lens = base + floor
    assert int(lens.sum()) == total and lens.min() >= floor
    return lens


def cu_from_lengths(lens) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    return cu


# ----------------------------------------------------------------------------
# whole workloads
# ----------------------------------------------------------------------------

def make_prefill(w: Workload, heads=None, threads=None, gate: str = "channel") -> dict:
    """Inputs for a "prefill" or "varlen" workload in packed token layout [T_total, H, d].

    Returns q, k, v, beta, log_alpha, cu_seqlens (int64 [N+1]) and init (or None).
    A dense batch B of length T is packed as B sequences of length T.
    """
    if w.kind == "varlen":
        lens = dirichlet_lengths(w.seed, w.seqlen, w.num_seqs, w.min_len)
    elif w.kind == "prefill":
        lens = np.full(w.batch, w.seqlen, np.int64)
    else:
        raise ValueError(w.kind)
    cu = cu_from_lengths(lens)
    T = int(cu[-1])
    d = gen_tokens(w.seed, T, w.heads, w.dk, w.dv, w.dtype, w.gate_scale, heads=heads, threads=threads, gate=gate)
    d["cu_seqlens"] = cu
    d["init"] = None if w.init_std is None else gen_states(
        w.seed, len(lens), w.heads, w.dk, w.dv, w.init_std, heads=heads)
    return d


def make_decode_step(w: Workload, step: int, heads=None, gate: str = "channel") -> dict:
    """Inputs of one decode step: q, k [N,H,dk], v [N,H,dv], beta [N,H], log_alpha [N,H,dk].

    Step s draws token index s of each of the N sequences, laid out as a packed
    batch of N one-token sequences.
    """
    assert w.kind == "decode"
    # each step is its own seed family so steps can be regenerated alone
    d = gen_tokens(w.seed * 1000003 + 7919 * (step + 1), w.batch, w.heads, w.dk, w.dv, w.dtype,
                   w.gate_scale, heads=heads, gate=gate)
    return d


def make_decode_state(w: Workload, heads=None) -> np.ndarray:
    return gen_states(w.seed, w.batch, w.heads, w.dk, w.dv, w.init_std, heads=heads)


def random_small(seed: int, T: int, H: int, dk: int, dv: int, dtype: str = "f32",
                 gate_scale: float = 0.05, init_std: float | None = 0.02, batch: int = 1,
                 lens=None, gate: str = "channel") -> dict:
    """Small ad-hoc workload (tests): same recipe, arbitrary shape; ``lens`` gives varlen."""
    lens = np.full(batch, T, np.int64) if lens is None else np.asarray(lens, np.int64)
    cu = cu_from_lengths(lens)
    d = gen_tokens(seed, int(cu[-1]), H, dk, dv, dtype, gate_scale, threads=1, gate=gate)
    d["cu_seqlens"] = cu
    d["init"] = None if init_std is None else gen_states(seed, len(lens), H, dk, dv, init_std)
    return d


def make_layer_prefill(w: Workload, heads=None, threads=None, gate: str = "channel") -> dict:
    """Layer inputs for a "prefill" or "varlen" workload (same lengths, seed and initial states)."""
    if w.kind == "varlen":
        lens = dirichlet_lengths(w.seed, w.seqlen, w.num_seqs, w.min_len)
    elif w.kind == "prefill":
        lens = np.full(w.batch, w.seqlen, np.int64)
    else:
        raise ValueError(w.kind)
    cu = cu_from_lengths(lens)
    d = gen_layer_tokens(w.seed, int(cu[-1]), w.heads, w.dk, w.dv, w.dtype, layer_gate_mu(w.gate_scale),
                         heads=heads, threads=threads, gate=gate)
    d["cu_seqlens"] = cu
    d["init"] = None if w.init_std is None else gen_states(
        w.seed, len(lens), w.heads, w.dk, w.dv, w.init_std, heads=heads)
    d["norm_weight"] = gen_norm_weight(w.seed, w.dv)
    return d


def make_layer_decode_step(w: Workload, step: int, heads=None, gate: str = "channel") -> dict:
    """Layer inputs of one decode step (see ``make_decode_step``)."""
    assert w.kind == "decode"
    return gen_layer_tokens(w.seed * 1000003 + 7919 * (step + 1), w.batch, w.heads, w.dk, w.dv, w.dtype,
                            layer_gate_mu(w.gate_scale), heads=heads, gate=gate)


def layer_small(seed: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16", gate_mu: float = -3.0,
                init_std: float | None = 0.02, batch: int = 1, lens=None, gate: str = "channel") -> dict:
    """Small ad-hoc layer workload (tests); ``lens`` gives varlen."""
    lens = np.full(batch, T, np.int64) if lens is None else np.asarray(lens, np.int64)
    cu = cu_from_lengths(lens)
    d = gen_layer_tokens(seed, int(cu[-1]), H, dk, dv, dtype, gate_mu, threads=1, gate=gate)
    d["cu_seqlens"] = cu
    d["init"] = None if init_std is None else gen_states(seed, len(lens), H, dk, dv, init_std)
    d["norm_weight"] = gen_norm_weight(seed, dv)
    return d
