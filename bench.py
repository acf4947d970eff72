#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one chunked prefill of a 64K-token, 32-head, d=128 KDA layer
(bf16 q/k/v, fp32 gates, fp32 state in and out, fp32 output) followed by 100
consecutive decode steps of 256 sequences x 32 heads (bf16 inputs, fp32
state updated in place, 512 MiB).  Inputs are synthetic, seeded, resident in
HBM before timing starts; a 512 MiB buffer is rewritten before every timed
prefill (outside its events) so no input is served from L2 or the MALL.

Prints one JSON line.  ``value`` is prefill tokens/s; the decode HBM
bandwidth is in ``decode``.  ``roofline`` describes the dominant kernel of a
step (the decode kernel: 100 launches per step); ``prefill_roofline`` the
prefill call.  ``layer`` times the fused layer (q/k L2 norm, gate from its
projection output, RMSNorm with sigmoid output gate, bf16 y) on the same
shapes; ``backward`` the gradients of the 64K prefill; ``prefill_configs`` the other prefill
workloads (4K x 32 heads, the 1M-token varlen batch, and the 64K workload with one gate per head).
``cpu_baseline`` times the fp64 oracle (test infrastructure) on the 64K prefill (all of it, a few
seconds on the host's cores), ``cpu_baseline_other_workloads`` on bounded samples of the others.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16/fp16 matrix peak
PAGE_FLOP_PER_TOKEN_HEAD = lambda d, C=64: 6 * d * d + 3 * C * d + C * C  # cost per head, per token
METRIC = "KDA prefill tokens/s (H32,d128,T64K) + decode-step HBM GB/s, 1 MI355X"
# sources each traffic measurement depends on (profiles/traffic.json is ignored once they change)
KERNEL_SOURCES = {
    "decode": ["gated_delta_rule_53_amd/csrc/kda_decode.hip", "gated_delta_rule_53_amd/csrc/kda_device.h"],
    "prefill": ["gated_delta_rule_53_amd/csrc/kda_chunk.hip", "gated_delta_rule_53_amd/csrc/kda_chunk_common.h",
                "gated_delta_rule_53_amd/csrc/kda_device.h", "gated_delta_rule_53_amd/csrc/kda_internal.h",
                "gated_delta_rule_53_amd/csrc/kda_api.hip"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_bytes(tokens, heads, d, in_b=2, out_b=4, states=1, gate_per_head=False):
    """Algorithmic HBM bytes: q,k,v + fp32 log_alpha + fp32 beta + out, plus state in/out."""
    per_th = 3 * d * in_b + 4 * (1 if gate_per_head else d) + 4 + d * out_b
    return tokens * heads * per_th + 2 * states * heads * d * d * 4


def decode_bytes(units, d, in_b=2, out_b=4, gate_per_head=False):
    """State read + write, plus q,k,v, log_alpha, beta and out, per (sequence, head)."""
    return units * (2 * d * d * 4 + 3 * d * in_b + 4 * (1 if gate_per_head else d) + 4 + d * out_b)


def layer_prefill_bytes(tokens, heads, d, states=1):
    """Algorithmic HBM bytes of the fused layer prefill: bf16 q,k,v, gate pre-activation, output
    gate and y, fp32 beta, plus state in/out and the RMSNorm weight."""
    return tokens * heads * (3 * d * 2 + d * 2 + 4 + d * 2 + d * 2) + 2 * states * heads * d * d * 4 + d * 4


def layer_decode_bytes(units, d):
    """State read + write plus the layer's per-(sequence, head) inputs and bf16 y."""
    return units * (2 * d * d * 4 + 3 * d * 2 + d * 2 + 4 + d * 2 + d * 2) + d * 4


def backward_bytes(tokens, heads, d, states=1):
    """Algorithmic HBM bytes of the backward: bf16 q,k,v, fp32 log_alpha, beta and d_out read,
    fp32 dq, dk, dv, dlog_alpha, dbeta written, plus the initial state and the final-state
    gradient read and the initial-state gradient written."""
    return tokens * heads * (3 * d * 2 + d * 4 + 4 + d * 4 + 4 * d * 4 + 4) + 3 * states * heads * d * d * 4


def backward_matrix_flops(tokens, heads, d, c=64):
    """Matrix-core FLOPs of the three backward kernels per call, as (fp32, fp16): with bf16
    inputs the chain's products take fp16 operands, prep and local stay fp32 (2 m n k per product, over
    the 16x16 blocks each product needs: lower blocks of triangular results, and for a
    lower-triangular T or dT operand only its nonzero 16-row blocks).  Per chunk and head:
    prep A0 and P (10 lower blocks each over d) and W = T Bk; the chain
    dU = P^T dO + Kh dS and dS = Qg^T dO - W^T dU; the local pass dQg, dKh and dW (c x d by
    d x d each; U = Ut - W S_j comes from the recompute's state pass), dP, dT and its
    second term (10 lower blocks over d), dBk = T^T dW and
    dBv = T^T dU, T^T dT and the strictly lower dAtil = -X T^T, and the four decay-weighted
    products (per 16-column block, 160 reduction steps over the four row blocks)."""
    chunks = -(-tokens // c) * heads
    nb = c // 16
    tri = 16 * nb * (nb + 1) // 2                                    # K summed over row blocks, T or T^T
    t_prod = 2 * 16 * tri * d                                        # T (c x c) by a c x d operand
    x_k = sum((2 * m + 1) * (c - 16 * m) for m in range(nb))         # T^T dT: K = c - 16 max(mt, nt)
    a_k = sum(16 * (m + 1) * (m + 2) // 2 for m in range(nb))        # X T^T, lower blocks: K = 16 (nt + 1)
    prep = 20 * (2 * 16 * 16 * d) + t_prod
    chain = 2 * c * d * (c + d) + 2 * d * d * 2 * c
    local = (3 * 2 * c * d * d + 3 * 10 * (2 * 16 * 16 * d) + 2 * t_prod + 2 * 16 * 16 * (x_k + a_k)
             + 4 * (d // 16) * 160 * 2 * 16 * 16)
    return chunks * (prep + local), chunks * chain


def to_dev(x, torch):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def kernel_hash(kernel):
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, key):
    """Calibrated HBM bytes from committed counter summaries, if they match the current source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("source_hash") != kernel_hash(kernel):
        return None
    return ent.get(key)


def oracle_threads(units):
    """Host threads for the oracle: one per (sequence, head) unit, at most the 16 cores of the GPU
    box's host share (and at most os.cpu_count())."""
    return max(1, min(16, os.cpu_count() or 1, units))


def cpu_baseline(w, d, sample_tokens):
    """Time the fp64 oracle on the first ``sample_tokens`` tokens of every head of workload w.

    ``d`` holds the workload's host inputs (the same arrays the GPU ran on).
    """
    import oracle
    n = min(sample_tokens, w.seqlen)
    threads = oracle_threads(w.heads)
    oracle.build(force=False)
    t = time.perf_counter()
    oracle.recurrent(d["q"][:n], d["k"][:n], d["v"][:n], d["log_alpha"][:n], d["beta"][:n], d["init"],
                     threads=threads)
    dt = time.perf_counter() - t
    what = "all" if n == w.seqlen else f"the first {n} of the"
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} {w.seqlen} tokens x {w.heads} heads of the {w.name} workload, "
                      f"fp64 token-by-token recurrence, {dt:.1f} s"}


def cpu_baselines_other(synth, d1):
    """The oracle on the other workloads, each on a bounded sample (seconds of host time):
    the whole 4K x 32-head prefill; 100 decode steps of 32 of the 256 sequences (all 32 heads);
    the 1M-token varlen batch on one of its 32 heads (all 16 sequences)."""
    import oracle
    from synth import WORKLOADS
    oracle.build(force=False)
    out = {}
    w1 = WORKLOADS[1]
    th = oracle_threads(w1.heads)
    t = time.perf_counter()
    oracle.recurrent(d1["q"], d1["k"], d1["v"], d1["log_alpha"], d1["beta"], d1["init"], threads=th)
    dt = time.perf_counter() - t
    out[w1.name] = {"value": w1.seqlen / dt, "unit": "tokens/s", "cores": th, "kind": "oracle",
                    "sample": f"all {w1.seqlen} tokens x {w1.heads} heads, {dt:.2f} s"}
    w3 = WORKLOADS[3]
    nseq = 32
    S = synth.make_decode_state(w3)[:nseq]
    steps = [{x: y[:nseq] for x, y in synth.make_decode_step(w3, s).items()} for s in range(w3.steps)]
    th = oracle_threads(nseq * w3.heads)
    t = time.perf_counter()
    for st in steps:
        _, S = oracle.recurrent(st["q"], st["k"], st["v"], st["log_alpha"], st["beta"], S,
                                np.arange(nseq + 1), threads=th)
    dt = time.perf_counter() - t
    updates = nseq * w3.heads * w3.steps
    out[w3.name] = {"value": updates / dt, "unit": "sequence-head updates/s", "cores": th, "kind": "oracle",
                    "full_step_ms": dt / w3.steps * (w3.batch / nseq) * 1e3,
                    "sample": f"{w3.steps} steps of {nseq} of the {w3.batch} sequences x {w3.heads} heads, "
                              f"{dt:.2f} s (full_step_ms scales it to all {w3.batch} sequences)"}
    w4 = WORKLOADS[4]
    d4 = synth.make_prefill(w4, heads=(0,))
    th = oracle_threads(w4.num_seqs)
    t = time.perf_counter()
    oracle.recurrent(d4["q"], d4["k"], d4["v"], d4["log_alpha"], d4["beta"], d4["init"], d4["cu_seqlens"],
                     threads=th)
    dt = time.perf_counter() - t
    out[w4.name] = {"value": w4.seqlen / dt, "unit": "token-heads/s", "cores": th, "kind": "oracle",
                    "sample": f"all {w4.seqlen} tokens (16 sequences) of head 0 of {w4.heads}, {dt:.2f} s "
                              f"(the longest sequence, {int(np.max(np.diff(d4['cu_seqlens'])))} tokens, "
                              f"bounds the time)"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--cpu-sample", type=int, default=65536, help="tokens per head for the oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time only the prefill (tuning runs)")
    ap.add_argument("--gate", choices=("channel", "head"), default="channel",
                    help="channel: KDA (log_alpha [.., H, dk]); head: one gate per head (Gated DeltaNet)")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the fused layer (q/k L2 norm, gate from its projection, RMSNorm-sigmoid epilogue)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward pass of the prefill")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other prefill workloads (4K x 32, 1M varlen, one gate per head)")
    ap.add_argument("--no-varlen", action="store_true", help="skip the 1M-token varlen prefill")
    ap.add_argument("--no-dplr", action="store_true", help="skip the KDA vs general-DPLR prefill comparison")
    ap.add_argument("--dplr-only", action="store_true",
                    help="only the KDA vs general-DPLR prefill comparison (profiling runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 10 device-to-device copies of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; pass --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_53_amd as kda
    import synth
    from synth import WORKLOADS

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    kda._lib.lib()  # fail loudly if the library is missing
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        ms = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        med = float(np.median(ms[2:]))
        print(json.dumps({"copy_probe_bytes": n, "launches": 10, "ms_median": med,
                          "read_plus_write_tb_s": 2 * n / med / 1e9}), flush=True)
        return

    if args.dplr_only:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        print(json.dumps({"dplr_vs_kda": bench_dplr(kda, torch, synth, args, flush, torch.cuda.current_stream())}),
              flush=True)
        return
    wp, wd = WORKLOADS[2], WORKLOADS[3]
    # ---- prefill inputs (64K tokens, 32 heads) ----
    t0 = time.time()
    gph = args.gate == "head"
    d = synth.make_prefill(wp, gate=args.gate)
    log(f"prefill inputs generated in {time.time() - t0:.1f}s")
    T, H, D = wp.seqlen, wp.heads, wp.dk
    q, k, v = (to_dev(d[x], torch).unsqueeze(0) for x in ("q", "k", "v"))
    la = to_dev(d["log_alpha"], torch).unsqueeze(0)
    be = to_dev(d["beta"], torch).unsqueeze(0)
    init = to_dev(d["init"], torch)
    if args.no_cpu_baseline:
        del d
    out = torch.empty((1, T, H, D), dtype=torch.float32, device="cuda")
    fin = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.workspace_size(1, T, H, D, D, torch.bfloat16, torch.float32), dtype=torch.uint8,
                     device="cuda")

    # ---- decode inputs (256 x 32, 100 distinct steps) ----
    t0 = time.time()
    state0 = to_dev(synth.make_decode_state(wd), torch)
    steps = []
    for s in range(0 if args.prefill_only else args.decode_steps):
        st = synth.make_decode_step(wd, s, gate=args.gate)
        steps.append(tuple(to_dev(st[x], torch) for x in ("q", "k", "v", "log_alpha", "beta")))
    log(f"decode inputs generated in {time.time() - t0:.1f}s")
    state = state0.clone()
    dout = torch.empty((wd.batch, wd.heads, wd.dv), dtype=torch.float32, device="cuda")

    stream = torch.cuda.current_stream()
    # written before every timed prefill so that no input is left in L2 or the 256 MB MALL
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def prefill():
        kda.chunk_fwd(q, k, v, la, be, init, None, out=out, final_state=fin, workspace=ws)

    def decode_all():
        for (sq, sk, sv, sla, sb) in steps:
            kda.decode_step(sq, sk, sv, sla, sb, state, out=dout)

    for _ in range(args.warmup):
        prefill()
        decode_all()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        flush.fill_(i & 0xFF)
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
        decode_all()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    pre_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)])
    dec_ms = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)])

    pre_s = float(np.median(pre_ms)) / 1e3
    tok_s = T / pre_s
    pbytes = prefill_bytes(T, H, D, gate_per_head=gph)
    pflops = PAGE_FLOP_PER_TOKEN_HEAD(D) * T * H
    dec_launch_s = float(np.median(dec_ms)) / 1e3 / max(1, len(steps))
    units = wd.batch * wd.heads
    dbytes = decode_bytes(units, D, gate_per_head=gph)
    dec_gbs = dbytes / dec_launch_s / 1e9

    res = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "precision": "bf16 q/k/v in; fp16 matrix-core operands; fp32 gates, accumulation, state and output",
        "data": "synthetic (seeded; q,k L2-normalised, beta=sigmoid(N), log_alpha=-s*softplus(N))",
        "config": {"workload": f"{wp.name} + {wd.name}" + ("" if not gph else " (one gate per head)"),
                   "gate": "per key channel (KDA)" if not gph else "per head (Gated DeltaNet)",
                   "prefill": {"batch": 1, "seq_len": T, "heads": H, "dk": D, "dv": D, "chunk": 64,
                               "in": "bf16", "out": "fp32", "init_state": "fp32 N(0,0.02^2)"},
                   "decode": {"batch": wd.batch, "heads": wd.heads, "dk": D, "dv": D,
                              "steps": args.decode_steps, "in": "bf16", "out": "fp32", "state": "fp32 in place"}},
        "prefill": {"ms": pre_s * 1e3, "ms_min": float(pre_ms.min()), "tokens_per_s": tok_s,
                    "hbm_gbs": pbytes / pre_s / 1e9},
        "decode": {"value": dec_gbs, "unit": "GB/s", "us_per_step": dec_launch_s * 1e6,
                   "ms_per_100_steps": dec_launch_s * 1e5},
        "roofline": {"kernel": "decode_kernel<128,bf16,fp32>", "bound": "hbm", "achieved": dec_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                     "traffic": None if gph else traffic_from_profiles("decode", "bytes_per_launch"),
                     "algorithmic_bytes_per_launch": dbytes, "launch_us": dec_launch_s * 1e6},
        "prefill_roofline": {"bound": "hbm", "achieved": pbytes / pre_s / 1e9, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": pbytes / pre_s / 1e9 / HBM_PEAK_GBS,
                             "algorithmic_bytes_per_call": pbytes,
                             "mfma_frac_page_flops": pflops / pre_s / 1e12 / BF16_DENSE_TFLOPS,
                             "traffic": None if gph else traffic_from_profiles("prefill", "bytes_per_call")},
        "context": "pages quote up to 75% KV cache reduction and up to 6x decoding throughput at 1M context "
                   "(model level, hardware not stated)",
    }
    d1 = None
    if not (args.no_configs or args.prefill_only or gph):
        del out, fin, ws
        res["prefill_configs"], d1 = bench_prefill_configs(kda, torch, synth, args, flush, stream, q, k, v, be, init)
        log("other prefill workloads timed")
    if not (args.no_dplr or args.prefill_only or gph):
        res["dplr_vs_kda"] = bench_dplr(kda, torch, synth, args, flush, stream)
        log("KDA vs general DPLR timed")
    if not (args.no_backward or args.prefill_only or gph):
        res["backward"] = bench_backward(kda, torch, wp, q, k, v, la, be, init, args, flush, stream)
        log("backward timed")
    if not (args.no_layer or args.prefill_only or gph):
        res["layer"] = bench_layer(kda, torch, synth, wp, wd, args, flush, stream)
        log("layer timed")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wp, d, args.cpu_sample)
        if d1 is not None:
            res["cpu_baseline_other_workloads"] = cpu_baselines_other(synth, d1)
        log("oracle timed")
    print(json.dumps(res), flush=True)


def time_calls(torch, call, n, warmup, flush, stream):
    """Median and minimum HIP-event time (ms) of n calls on ``stream``, the 512 MiB buffer
    rewritten before each so no input is left in L2 or the MALL."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ms = []
    for i in range(n):
        flush.fill_(i & 0xFF)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return float(np.median(ms)), float(np.min(ms))


def prefill_entry(name, ms, ms_min, tokens, heads, d, gate_per_head=False, states=1, extra=None):
    b = prefill_bytes(tokens, heads, d, gate_per_head=gate_per_head, states=states)
    e = {"workload": name, "ms": ms, "ms_min": ms_min, "tokens_per_s": tokens / (ms / 1e3),
         "algorithmic_bytes": b, "hbm_gbs": b / (ms / 1e3) / 1e9, "hbm_frac": b / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}
    if extra:
        e.update(extra)
    return e


def gpu_varlen_inputs(torch, synth, w):
    """The 1M-token varlen workload drawn on the GPU (43 GB of inputs would take minutes on the
    host): the synth recipe -- q, k ~ N(0,1) L2-normalised per (token, head) then bf16; v ~ N(0,1)
    bf16; beta = sigmoid(N(0,1)); log_alpha = -s softplus(N(0,1)), s = 0.05; initial states
    N(0, 0.02^2) -- from torch's seeded generator; the sequence lengths are synth's exactly."""
    lens = synth.dirichlet_lengths(w.seed, w.seqlen, w.num_seqs, w.min_len)
    cu = torch.from_numpy(synth.cu_from_lengths(lens).astype(np.int32)).cuda()
    g = torch.Generator(device="cuda").manual_seed(1000 + w.seed)
    T, H, D = w.seqlen, w.heads, w.dk
    blk = 1 << 16
    q, k, v = (torch.empty((1, T, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    la = torch.empty((1, T, H, D), dtype=torch.float32, device="cuda")
    for t0 in range(0, T, blk):
        t1 = min(T, t0 + blk)
        for x in (q, k):
            r = torch.randn((t1 - t0, H, D), generator=g, device="cuda")
            x[0, t0:t1] = (r / r.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        v[0, t0:t1] = torch.randn((t1 - t0, H, D), generator=g, device="cuda").to(torch.bfloat16)
        la[0, t0:t1] = -w.gate_scale * torch.nn.functional.softplus(
            torch.randn((t1 - t0, H, D), generator=g, device="cuda"))
    be = torch.sigmoid(torch.randn((1, T, H), generator=g, device="cuda"))
    init = w.init_std * torch.randn((w.num_seqs, H, D, D), generator=g, device="cuda")
    return q, k, v, la, be, init, cu, int(lens.max())


def bench_prefill_configs(kda, torch, synth, args, flush, stream, q2, k2, v2, be2, init2):
    """The other prefill workloads, as fields of the same line: 4K x 32 heads; the 1M-token
    varlen batch; and the 64K x 32-head prefill with one gate per head (Gated DeltaNet)."""
    from synth import WORKLOADS
    out = {}
    w1 = WORKLOADS[1]
    d1 = synth.make_prefill(w1)
    T, H, D = w1.seqlen, w1.heads, w1.dk
    a = [to_dev(d1[x], torch).unsqueeze(0) for x in ("q", "k", "v", "log_alpha", "beta")]
    o = torch.empty((1, T, H, D), dtype=torch.float32, device="cuda")
    f = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.workspace_size(1, T, H, D, D, torch.bfloat16, torch.float32), dtype=torch.uint8,
                     device="cuda")
    ms, mn = time_calls(torch, lambda: kda.chunk_fwd(*a, None, None, out=o, final_state=f, workspace=ws),
                        max(10, args.steps), args.warmup, flush, stream)
    out[w1.name] = prefill_entry(w1.name, ms, mn, T, H, D, states=0)
    del a, o, f, ws
    w2 = WORKLOADS[2]
    T, H, D = w2.seqlen, w2.heads, w2.dk
    la_h = to_dev(synth.make_prefill(w2, gate="head")["log_alpha"], torch).unsqueeze(0)
    o = torch.empty((1, T, H, D), dtype=torch.float32, device="cuda")
    f = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.workspace_size(1, T, H, D, D, torch.bfloat16, torch.float32), dtype=torch.uint8,
                     device="cuda")
    ms, mn = time_calls(torch, lambda: kda.chunk_fwd(q2, k2, v2, la_h, be2, init2, None, out=o, final_state=f,
                                                     workspace=ws), max(10, args.steps), args.warmup, flush, stream)
    out[w2.name + " (one gate per head)"] = prefill_entry(w2.name + " (one gate per head)", ms, mn, T, H, D,
                                                          gate_per_head=True)
    del la_h, o, f, ws
    if not args.no_varlen:
        w4 = WORKLOADS[4]
        q, k, v, la, be, init, cu, longest = gpu_varlen_inputs(torch, synth, w4)
        T, H, D = w4.seqlen, w4.heads, w4.dk
        o = torch.empty((1, T, H, D), dtype=torch.float32, device="cuda")
        f = torch.empty((w4.num_seqs, H, D, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(kda.workspace_size(1, T, H, D, D, torch.bfloat16, torch.float32, num_seqs=w4.num_seqs,
                                            max_seqlen=longest), dtype=torch.uint8, device="cuda")
        ms, mn = time_calls(torch, lambda: kda.chunk_fwd(q, k, v, la, be, init, cu, out=o, final_state=f,
                                                         max_seqlen=longest, workspace=ws),
                            5, 1, flush, stream)
        out[w4.name] = prefill_entry(w4.name, ms, mn, T, H, D, states=w4.num_seqs,
                                     extra={"inputs": "drawn on the GPU with the synth recipe (torch generator)",
                                            "longest_sequence": longest})
        del q, k, v, la, be, init, cu, o, f, ws
    torch.cuda.empty_cache()
    return out, d1


def bench_dplr(kda, torch, synth, args, flush, stream):
    """KDA against the general DPLR transition it constrains, at the pages' comparison shape
    (batch 1, 16 heads, inputs up to 64K tokens): the same synthetic q, k, v and gates; KDA with
    beta, the DPLR kernel with independent a and b (synth's general-DPLR recipe)."""
    H, D = 16, 128
    res = {"heads": H, "dk": D, "dv": D, "in": "bf16", "out": "fp32", "init_state": "fp32 N(0,0.02^2)",
           "pages": "KDA kernel close to twice the speed of a general DPLR kernel for inputs up to 64K tokens "
                    "at batch 1 with 16 heads (hardware not stated)", "lengths": {}}
    for T in (4096, 16384, 65536):
        dd = synth.gen_dplr_tokens(5, T, H, D, "bf16", 0.01)
        be = to_dev(synth.gen_tokens(5, T, H, D, D, "bf16", 0.01)["beta"], torch).unsqueeze(0)
        q, k, v, a, b, la = (to_dev(dd[x], torch).unsqueeze(0) for x in ("q", "k", "v", "a", "b", "log_alpha"))
        del dd
        init = to_dev(synth.gen_states(5, 1, H, D, D, 0.02), torch)
        o = torch.empty((1, T, H, D), dtype=torch.float32, device="cuda")
        f = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
        wk = torch.empty(kda.workspace_size(1, T, H, D, D, torch.bfloat16, torch.float32), dtype=torch.uint8,
                         device="cuda")
        wd = torch.empty(kda.dplr_workspace_size(1, T, H, D, D, torch.bfloat16, torch.float32), dtype=torch.uint8,
                         device="cuda")
        n = max(10, args.steps)
        km, kmin = time_calls(torch, lambda: kda.chunk_fwd(q, k, v, la, be, init, None, out=o, final_state=f,
                                                           workspace=wk), n, args.warmup, flush, stream)
        dm, dmin = time_calls(torch, lambda: kda.dplr_chunk_fwd(q, k, v, a, b, la, init, None, out=o,
                                                                final_state=f, workspace=wd),
                              n, args.warmup, flush, stream)
        res["lengths"][str(T)] = {"kda_ms": km, "dplr_ms": dm, "kda_ms_min": kmin, "dplr_ms_min": dmin,
                                  "kda_tokens_per_s": T / (km / 1e3), "dplr_tokens_per_s": T / (dm / 1e3),
                                  "dplr_over_kda_time": dm / km}
        del q, k, v, a, b, la, be, init, o, f, wk, wd
    torch.cuda.empty_cache()
    res["decode"] = bench_dplr_decode(kda, torch, synth, args, stream)
    return res


def bench_dplr_decode(kda, torch, synth, args, stream):
    """One decode step of KDA and of the general DPLR transition at the decode workload's shape
    (256 sequences x 32 heads, d = 128, bf16 inputs, fp32 state in place, fp32 out): time per
    step over 20 consecutive steps, the two kernels alternating over 5 rounds (medians), each
    updating the same state buffer in place."""
    N, H, D = 256, 32, 128
    dd = synth.gen_dplr_tokens(7, N, H, D, "bf16", 0.05)
    be = to_dev(synth.gen_tokens(7, N, H, D, D, "bf16", 0.05)["beta"], torch)
    q, k, v, a, b, la = (to_dev(dd[x], torch) for x in ("q", "k", "v", "a", "b", "log_alpha"))
    del dd
    gen = torch.Generator(device="cuda").manual_seed(7)
    state = torch.randn((N, H, D, D), dtype=torch.float32, device="cuda", generator=gen).mul_(0.02)
    out = torch.empty((N, H, D), dtype=torch.float32, device="cuda")
    steps, rounds = 20, 5

    def per_step(call):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps  # us

    kda_call = lambda: kda.decode_step(q, k, v, la, be, state, out=out)
    dplr_call = lambda: kda.dplr_decode_step(q, k, v, a, b, la, state, out=out)
    for _ in range(3):
        kda_call()
        dplr_call()
    torch.cuda.synchronize()
    # the two kernels alternate, so neither is timed only while the clocks settle
    kt, dt = [], []
    for _ in range(rounds):
        kt.append(per_step(kda_call))
        dt.append(per_step(dplr_call))
    kda_us, dplr_us = float(np.median(kt)), float(np.median(dt))
    kda_b = decode_bytes(N * H, D)
    dplr_b = N * H * (2 * D * D * 4 + 5 * D * 2 + D * 4 + D * 4)  # state twice; q, k, v, a, b; log_alpha; out
    del q, k, v, a, b, la, be, state, out
    torch.cuda.empty_cache()
    return {"units": N * H, "steps": steps, "rounds": rounds, "kda_us_per_step": kda_us, "dplr_us_per_step": dplr_us,
            "kda_hbm_gbs": kda_b / (kda_us * 1e3), "dplr_hbm_gbs": dplr_b / (dplr_us * 1e3),
            "dplr_algorithmic_bytes": dplr_b, "dplr_over_kda_time": dplr_us / kda_us}


def bench_backward(kda, torch, wp, q, k, v, la, be, init, args, flush, stream):
    """Gradients of the 64K-token prefill (fp32 d_out and final-state gradient), timed after
    the main steps: one call recomputes the forward's records and states, then runs the
    reverse chain and the per-chunk gradients."""
    T, H, D = wp.seqlen, wp.heads, wp.dk
    gen = torch.Generator(device="cuda").manual_seed(wp.seed)
    d_out = torch.randn((1, T, H, D), dtype=torch.float32, device="cuda", generator=gen)
    d_fin = torch.randn((1, H, D, D), dtype=torch.float32, device="cuda", generator=gen)

    def call():
        return kda.chunk_bwd(q, k, v, la, be, d_out, init, d_fin)

    for _ in range(min(args.warmup, 2)):
        call()
    torch.cuda.synchronize()
    ms = []
    for i in range(max(3, args.steps // 4)):
        flush.fill_(i & 0xFF)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    s = float(np.median(ms)) / 1e3
    b = backward_bytes(T, H, D)
    f32, f16 = backward_matrix_flops(T, H, D)
    at_peak = f32 / (FP32_MFMA_PEAK_TFLOPS * 1e12) + f16 / (BF16_DENSE_TFLOPS * 1e12)
    return {"what": "dq, dk, dv, dlog_alpha, dbeta, d_init of the 64K x 32-head prefill (bf16 in, fp32 d_out "
                    "and gradients), forward recompute included",
            "ms": s * 1e3, "tokens_per_s": T / s, "algorithmic_bytes": b, "hbm_gbs": b / s / 1e9,
            "frac": b / s / 1e9 / HBM_PEAK_GBS,
            "matrix": {"fp32_flop_per_call": f32, "fp16_flop_per_call": f16,
                       "fp32_tflops": f32 / s / 1e12, "fp16_tflops": f16 / s / 1e12,
                       "peaks_tflops": {"fp32": FP32_MFMA_PEAK_TFLOPS, "fp16": BF16_DENSE_TFLOPS},
                       "ms_at_peaks": at_peak * 1e3, "frac": at_peak / s}}


def bench_layer(kda, torch, synth, wp, wd, args, flush, stream):
    """The fused layer on the same shapes: prefill (bf16 y) and 100 decode steps (bf16 y), timed
    after the main steps with their own warm-up."""
    t0 = time.time()
    d = synth.make_layer_prefill(wp)
    T, H, D = wp.seqlen, wp.heads, wp.dk
    q, k, v, g, be, z = (to_dev(d[x], torch).unsqueeze(0) for x in ("q", "k", "v", "g", "beta", "out_gate"))
    init, wt = to_dev(d["init"], torch), to_dev(d["norm_weight"], torch)
    del d
    y = torch.empty((1, T, H, D), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.workspace_size(1, T, H, D, D, torch.bfloat16, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    state = to_dev(synth.make_decode_state(wd), torch)
    steps = []
    for s in range(args.decode_steps):
        st = synth.make_layer_decode_step(wd, s)
        steps.append(tuple(to_dev(st[x], torch) for x in ("q", "k", "v", "g", "beta", "out_gate")))
    dy = torch.empty((wd.batch, wd.heads, wd.dv), dtype=torch.bfloat16, device="cuda")
    log(f"layer inputs generated in {time.time() - t0:.1f}s")

    def prefill():
        kda.layer_fwd(q, k, v, g, be, init, None, out_gate=z, norm_weight=wt, out=y, final_state=fin,
                      workspace=ws)

    def decode_all():
        for (sq, sk, sv, sg, sb, sz) in steps:
            kda.layer_decode_step(sq, sk, sv, sg, sb, state, out_gate=sz, norm_weight=wt, out=dy)

    for _ in range(args.warmup):
        prefill()
        decode_all()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        flush.fill_(i & 0xFF)
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
        decode_all()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    pre_s = float(np.median([ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)])) / 1e3
    dec_s = float(np.median([ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)])) / 1e3 / len(steps)
    pb, db = layer_prefill_bytes(T, H, D), layer_decode_bytes(wd.batch * wd.heads, D)
    return {"what": "q/k L2 norm + log alpha = -softplus(bf16 gate) + recurrence + RMSNorm * sigmoid(bf16 gate), "
                    "bf16 y",
            "prefill": {"ms": pre_s * 1e3, "tokens_per_s": T / pre_s, "algorithmic_bytes": pb,
                        "hbm_gbs": pb / pre_s / 1e9, "frac": pb / pre_s / 1e9 / HBM_PEAK_GBS},
            "decode": {"us_per_step": dec_s * 1e6, "algorithmic_bytes": db, "hbm_gbs": db / dec_s / 1e9,
                       "frac": db / dec_s / 1e9 / HBM_PEAK_GBS}}


if __name__ == "__main__":
    main()
