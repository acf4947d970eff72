"""The entry points under HIP graph capture (needs an MI355X).

kda_chunk_fwd_noalloc exists for callers that cannot allocate, code under graph capture
among them; kda_chunk_fwd with a preallocated workspace and kda_decode_step allocate
nothing either.  Without KDA_CHECK none of them issues a memset, a copy or a
synchronisation, so each can be captured into a graph and replayed.  Each test captures
a call with torch.cuda.graph on torch's capture stream, replays it several times with
eager work of the library in between (other calls on the same static scratch or
workspace, and new contents in the captured input buffers), and requires every replay to
match the eager result bit for bit: the kernels are deterministic and no call relies on
what an earlier one left in its scratch.
"""
import numpy as np
import pytest

import synth

from kda_testlib import nan_tensor, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd as m
    m._lib.lib()
    return m


def prefill_inputs(seed, T, H, lens=None):
    d = synth.random_small(seed, T, H, 128, 128, dtype="bf16", lens=lens)
    args = [to_dev(d[x], torch).unsqueeze(0) for x in ("q", "k", "v", "log_alpha", "beta")]
    cu = d["cu_seqlens"]
    cu_t = torch.from_numpy(np.asarray(cu, np.int32)).cuda() if len(cu) != 2 else None
    return args, to_dev(d["init"], torch), cu_t, len(cu) - 1


@pytest.mark.parametrize("mode", ["noalloc", "workspace", "windows"])
def test_prefill_graph_replay(kda, mode):
    """A varlen prefill (3 sequences of 700, 64 and 1,300 tokens, 4 heads) captured once: the
    allocation-free entry point, kda_chunk_fwd with its workspace, and kda_chunk_fwd with a
    workspace of four chunk indices of records (six windows, each carrying the state to the
    next through the state buffer)."""
    args, init, cu, N = prefill_inputs(61, 0, 4, lens=[700, 64, 1300])
    H = 4
    noalloc = mode == "noalloc"
    if mode == "workspace":
        ws_bytes = kda.workspace_size(1, 2064, H, 128, 128, torch.bfloat16, num_seqs=N, max_seqlen=1300)
    else:
        state = N * H * 128 * 128 * 4
        per_index = N * H * 74240  # one chunk index of fp16 records for every (sequence, head)
        ws_bytes = state + 4 * per_index
    ws = None if noalloc else torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    def call(a, i0, out, fin):
        if noalloc:
            kda.chunk_fwd_noalloc(*a, i0, cu, out=out, final_state=fin, max_seqlen=1300)
        else:
            kda.chunk_fwd(*a, i0, cu, out=out, final_state=fin, workspace=ws, max_seqlen=1300)

    ref_o = nan_tensor(torch, args[2].shape)
    ref_s = nan_tensor(torch, (N, H, 128, 128))
    call(args, init, ref_o, ref_s)
    torch.cuda.synchronize()
    # other inputs of the same shape, for eager calls between the replays
    other, other_init, _, _ = prefill_inputs(62, 0, 4, lens=[700, 64, 1300])
    o_g = nan_tensor(torch, args[2].shape)
    s_g = nan_tensor(torch, (N, H, 128, 128))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(args, init, o_g, s_g)
    torch.cuda.synchronize()
    for rep in range(3):
        o_g.fill_(float("nan"))
        s_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, ref_o) and torch.equal(s_g, ref_s), f"replay {rep} differs from the eager call"
        # eager work on the same scratch between replays
        scratch_o = nan_tensor(torch, args[2].shape)
        call(other, other_init, scratch_o, nan_tensor(torch, (N, H, 128, 128)))
        torch.cuda.synchronize()
        assert torch.isfinite(scratch_o).all()


def test_decode_graph_replay(kda):
    """One decode step (32 sequences x 8 heads, state in place) captured once and replayed as a
    loop of 4 steps with each step's inputs copied into the captured buffers, against 4
    eager steps from the same state."""
    N, H, D = 32, 8, 128
    S0 = synth.gen_states(71, N, H, D, D, 0.3)
    steps = [synth.gen_tokens(72 + i, N, H, D, D, "bf16", 0.05) for i in range(4)]
    names = ("q", "k", "v", "log_alpha", "beta")
    # eager
    state = to_dev(S0, torch)
    outs = []
    for st in steps:
        outs.append(kda.decode_step(*[to_dev(st[x], torch) for x in names], state,
                                    out=nan_tensor(torch, (N, H, D))))
    torch.cuda.synchronize()
    # captured: static input buffers, state updated in place
    bufs = [to_dev(steps[0][x], torch) for x in names]
    state_g = to_dev(S0, torch)
    out_g = nan_tensor(torch, (N, H, D))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kda.decode_step(*bufs, state_g, out=out_g)
    torch.cuda.synchronize()
    state_g.copy_(to_dev(S0, torch))  # capture did not run the step; start from S0 regardless
    for i, st in enumerate(steps):
        for b, x in zip(bufs, names):
            b.copy_(to_dev(st[x], torch))
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, outs[i]), f"step {i}: output differs from the eager step"
    assert torch.equal(state_g, state), "final state differs from the eager steps"
