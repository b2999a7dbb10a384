"""The whole forward (routing plan, activation quantization, fused experts and combine) captured
once in a HIP graph and replayed with new contents in the same input buffers: every replay
equals the eager call on the same inputs, bit for bit.

The library allocates nothing on this path, never synchronizes and clears its counters with
kernels (no memset nodes), and its grids are sized by the plan capacity, so one captured graph
serves any routing of the same shape.  Replays alternate with eager work and synchronizations.
"""

import numpy as np
import pytest
import torch

from synth import WORKLOADS, make_activations, make_routing
from synth.workloads import Workload

from gpu_common import Problem, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_scaled_fp4_plan_amd import runner

# several tiles of 1 to 8 token fragments and K not a multiple of the prefetch depth
SKEWED = Workload("graph_skewed", M=384, H=1280, I=640, E=6, top_k=3, block_m=128,
                  routing="zipf")

CASES = [("tiny", 8, True), ("tiny", 128, True), ("tiny", 128, False), ("decode_ll", 8, True),
         ("graph_skewed", 128, True)]


def _inputs(wl, seed, M):
    x_bits = make_activations(wl, seed, M)
    ids, w = make_routing(wl, seed, M)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    return x, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("name,bm,fin", CASES,
                         ids=["%s-bm%d-%s" % (n, b, "fin" if f else "unfin") for n, b, f in CASES])
def test_graph_replay_matches_eager(name, bm, fin):
    wl = SKEWED if name == "graph_skewed" else WORKLOADS[name]
    say("graph replay", name, "block_m", bm, "finalize", fin)
    p = Problem(wl)
    pw = runner.prepare_weights(p.w1, p.w2, gated=wl.gated)
    fwd_e = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm, wl.local_offset, fin)
    fwd_g = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm, wl.local_offset, fin)
    x, ids, w = p.x.clone(), p.ids_d.clone(), p.w_d.clone()      # the graph's input buffers
    out_g = torch.zeros((p.M, wl.H), dtype=torch.bfloat16, device="cuda")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd_g(x, ids, w, out=out_g)                  # first call outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res_g = fwd_g(x, ids, w, out=out_g)

    for seed in (1, 2, 0, 3, 1):
        xs, idss, ws = _inputs(wl, seed, p.M)
        x.copy_(xs)
        ids.copy_(idss)
        w.copy_(ws)
        out_g.zero_()
        graph.replay()
        res_e = fwd_e(xs, idss, ws)
        torch.cuda.synchronize()
        if fin:
            assert torch.equal(_bits(out_g), _bits(res_e)), seed
        else:
            (y_g, w_g, ttr_g), (y_e, w_e, ttr_e) = res_g, res_e
            assert torch.equal(ttr_g, ttr_e), seed
            assert torch.equal(w_g, ws) and torch.equal(w_e, ws)
            rows = ttr_e.reshape(-1)
            rows = rows[rows >= 0].long()
            assert rows.numel() > 0
            assert torch.equal(_bits(y_g[rows]), _bits(y_e[rows])), seed
