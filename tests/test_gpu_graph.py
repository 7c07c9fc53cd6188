"""HIP-graph capture of the encode (GPU).

hstu_encode with a caller-owned workspace, and hstu_encode_static (the entry point for
callers that cannot allocate), are captured into a graph on torch's capture stream and
replayed. The plan travels in the captured kernel arguments, so a replay runs the same
batch shape; it reads the input buffers as they are at replay time. Each replay is
checked bit for bit against an eager call, with eager work of the program (clearing the
outputs, writing new inputs) and synchronizations between the replays."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import workloads
from gpu_util import BF16_TOL, make_model, normwise_per_user, oracle_encode, say, to_dev, to_np, torch_cuda

pytestmark = pytest.mark.gpu


def _inputs(torch, wl, seed):
    rng = np.random.default_rng(seed)
    u = workloads.to_bf16_values(rng.standard_normal(wl.uih.shape).astype(np.float32))
    c = workloads.to_bf16_values(rng.standard_normal(wl.cand.shape).astype(np.float32))
    return to_dev(torch, u, "bf16"), to_dev(torch, c, "bf16")


@pytest.mark.parametrize("static", [False, True])
def test_encode_replays_from_a_graph(static):
    torch = torch_cuda()
    # dh = 128, two users with ragged histories and candidates, one with candidates only
    wl = workloads.make_custom(seed=1401, dtype="bf16", layers=2, d_model=256, heads=2, max_len=1200,
                               uih_lengths=[700, 131, 0], cand_lengths=[150, 33, 9])
    model = make_model(torch, wl)
    uo, co = workloads.lengths_to_offsets(wl.uih_lengths), workloads.lengths_to_offsets(wl.cand_lengths)
    du, dc = to_dev(torch, wl.uih, "bf16"), to_dev(torch, wl.cand, "bf16")
    out = (torch.empty_like(du), torch.empty_like(dc))
    ws = None if static else torch.empty(hsa.workspace_bytes(model, uo, co), dtype=torch.uint8, device="cuda")

    def call(u, c, o, stream=None):
        if static:
            return hsa.encode_static(model, u, uo, c, co, out=o, stream=stream)
        return hsa.encode(model, u, uo, c, co, out=o, workspace=ws, stream=stream)

    def eager(u, c):
        o = (torch.empty_like(u), torch.empty_like(c))
        call(u, c, o)
        torch.cuda.synchronize()
        return o

    ref = eager(du, dc)                      # also the first call (the static scratch's set-up)
    eu = normwise_per_user(to_np(ref[0]), oracle_encode(wl, "bf16")[0], wl.uih_lengths)
    assert eu <= BF16_TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(du, dc, out, stream=torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        out[0].fill_(7.0)
        out[1].fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[0], ref[0]) and torch.equal(out[1], ref[1]), f"replay {rep}"
    # new values in the same input buffers: the replay computes them
    nu, nc = _inputs(torch, wl, 1402)
    du.copy_(nu)
    dc.copy_(nc)
    ref2 = eager(du, dc)
    assert not torch.equal(ref2[0], ref[0])
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[0], ref2[0]) and torch.equal(out[1], ref2[1]), f"replay {rep} on new inputs"
        out[0].zero_()
    say(f"  graph ({'static entry' if static else 'workspace'}): 5 replays bit-identical to eager calls")
