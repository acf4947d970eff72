"""The seeded input generator: determinism, distributions, bf16 rounding, varlen lengths."""
import numpy as np

import synth
from synth import WORKLOADS, bf16_bits_to_f32, dirichlet_lengths, f32_to_bf16_bits


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, 1.0078125 + 2**-8 + 2**-10, -3.140625, 0.0, 1e-30,
                  3.0e38], np.float32)
    b = f32_to_bf16_bits(x)
    y = bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa -> 1.0
    assert y[1] == 1.0
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even -> 1 + 2^-6
    assert y[2] == np.float32(1.015625)
    # above the tie rounds up
    assert y[3] == np.float32(1.015625)
    assert y[4] == np.float32(-3.140625)
    assert y[0] == 1.0 and y[5] == 0.0
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    e = np.abs(bf16_bits_to_f32(f32_to_bf16_bits(r)) - r) / np.abs(r)
    assert e.max() <= 2.0**-8


def test_determinism_and_head_subsets():
    a = synth.gen_tokens(5, 300, 4, 16, 8, "bf16", 0.05)
    b = synth.gen_tokens(5, 300, 4, 16, 8, "bf16", 0.05)
    for x in a:
        assert np.array_equal(a[x], b[x])
    sub = synth.gen_tokens(5, 300, 4, 16, 8, "bf16", 0.05, heads=[2])
    for x in a:
        assert np.array_equal(a[x][:, 2:3], sub[x])
    c = synth.gen_tokens(6, 300, 4, 16, 8, "bf16", 0.05)
    assert not np.array_equal(a["q"], c["q"])


def test_distributions():
    d = synth.gen_tokens(1, 4000, 2, 128, 128, "f32", 0.05)
    n = np.linalg.norm(d["q"].astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 1e-6
    assert 0 < d["beta"].min() and d["beta"].max() < 1
    assert abs(float(d["beta"].mean()) - 0.5) < 0.01
    la = d["log_alpha"].astype(np.float64)
    assert la.max() <= 0
    # E[softplus(N(0,1))] = 0.806...
    assert abs(-la.mean() / 0.05 - 0.806) < 0.01
    assert abs(float(d["v"].std()) - 1) < 0.01


def test_dirichlet_lengths():
    w = WORKLOADS[4]
    lens = dirichlet_lengths(w.seed, w.seqlen, w.num_seqs, w.min_len)
    assert len(lens) == 16 and lens.sum() == 1048576 and lens.min() >= 4096
    assert np.array_equal(lens, dirichlet_lengths(w.seed, w.seqlen, w.num_seqs, w.min_len))
    for seed in range(20):
        l2 = dirichlet_lengths(seed, 10000, 7, 100)
        assert l2.sum() == 10000 and l2.min() >= 100


def test_workload_table():
    assert WORKLOADS[0].dtype == "f32" and WORKLOADS[0].dk == 64 and WORKLOADS[0].seqlen == 256
    assert WORKLOADS[2].gate_scale == 0.01 and WORKLOADS[2].init_std == 0.02
    assert WORKLOADS[3].kind == "decode" and WORKLOADS[3].batch == 256 and WORKLOADS[3].steps == 100
    assert WORKLOADS[4].kind == "varlen" and WORKLOADS[4].num_seqs == 16
    d = synth.make_prefill(WORKLOADS[0])
    assert d["q"].shape == (256, 2, 64) and d["q"].dtype == np.float32 and d["init"] is None


def test_per_head_gate_draw():
    """gate="head" draws log_alpha [T, H] from its own stream with the KDA gate's distribution."""
    import synth
    d = synth.gen_tokens(3, 5000, 3, 16, 16, "f32", 0.05, threads=1, gate="head")
    la = d["log_alpha"]
    assert la.shape == (5000, 3) and la.dtype == np.float32
    assert (la <= 0).all() and np.isfinite(la).all()
    # -0.05 * softplus(N(0,1)) has mean -0.05 * 0.8066 (E softplus(Z) for Z ~ N(0,1))
    assert abs(la.mean() / -0.05 - 0.8066) < 0.02
    # q, k, v and beta are the same draws as with per-channel gates
    d2 = synth.gen_tokens(3, 5000, 3, 16, 16, "f32", 0.05, threads=1)
    for x in ("q", "k", "v", "beta"):
        assert np.array_equal(d[x], d2[x])
