"""kda_chunk_fwd_noalloc (static per-device scratch, no allocation) against kda_chunk_fwd.

Two calls in a row on one device, the second with a smaller input: each must give the
same bits as kda_chunk_fwd with a workspace of the same size (the same windows of
chunks), and match the fp64 oracle at the operator's bar.  Collected last, so a
failure here hides no other test.
"""
import numpy as np
import pytest

import synth
from synth import WORKLOADS, random_small

from kda_testlib import TOL, assert_close, nan_tensor, oracle_chunk, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd as m
    m._lib.lib()
    return m


def _inputs(d):
    q, k, v, la, b = (to_dev(d[x], torch).unsqueeze(0) for x in ("q", "k", "v", "log_alpha", "beta"))
    cu = d["cu_seqlens"]
    varlen = len(cu) != 2
    cu_t = torch.from_numpy(np.asarray(cu, np.int32)).cuda() if varlen else None
    init = None if d.get("init") is None else to_dev(d["init"], torch)
    N = len(cu) - 1
    return (q, k, v, la, b, init, cu_t), N, int(np.max(np.diff(cu)))


def test_noalloc_matches_workspace_entry_point(kda):
    cases = [synth.make_prefill(WORKLOADS[1]),  # 4,096 tokens x 32 heads, bf16
             random_small(77, 0, 2, 128, 128, dtype="bf16", init_std=0.02, lens=[300, 0, 65, 1000])]
    ws = torch.empty(kda._lib.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    for d in cases:
        args, N, maxlen = _inputs(d)
        q, v = args[0], args[2]
        H, D = q.shape[2], q.shape[3]
        out_a, fin_a = nan_tensor(torch, v.shape), nan_tensor(torch, (N, H, D, D))
        kda.chunk_fwd_noalloc(*args, out=out_a, final_state=fin_a, max_seqlen=maxlen)
        out_b, fin_b = nan_tensor(torch, v.shape), nan_tensor(torch, (N, H, D, D))
        kda.chunk_fwd(*args, out=out_b, final_state=fin_b, workspace=ws, max_seqlen=maxlen)
        torch.cuda.synchronize()
        oa, sa = out_a[0].cpu().numpy(), fin_a.cpu().numpy()
        assert np.array_equal(oa, out_b[0].cpu().numpy()) and np.array_equal(sa, fin_b.cpu().numpy())
        o_ref, S_ref = oracle_chunk(d)
        assert_close("out", oa, o_ref, TOL["bf16"])
        assert_close("state", sa, S_ref, TOL["bf16"])
