"""The fused call without a workspace argument (bfp4_fused_moe_nvfp4_noalloc, for callers that
cannot allocate): through the C ABI, its output equals the workspace entry point's bit for bit
(the same kernels run on the library's static scratch array), on two calls in a row, the second
with a smaller input, for the decode (block_m 8) and the tiled (block_m 128) kernels, finalized
and unfinalized; a call whose workspace would exceed the array is refused on the host."""

import dataclasses

import numpy as np
import pytest
import torch

from synth import WORKLOADS

from gpu_common import Problem, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_scaled_fp4_plan_amd as bf
    from block_scaled_fp4_plan_amd import runner


def _bits(t):
    return t.view(torch.int16)


def _pair(wl, bm, fin, M):
    """(no-alloc result, workspace result) of one forward of workload wl with M tokens."""
    p = Problem(wl, M=M)
    pw = runner.prepare_weights(p.w1, p.w2, gated=wl.gated)
    res = []
    for noalloc in (True, False):
        f = runner.MoeForward(pw, M, wl.top_k, wl.E, bm, wl.local_offset, do_finalize=fin,
                              noalloc=noalloc)
        o0 = torch.full((M, wl.H), 0.5, dtype=torch.bfloat16, device="cuda")
        r = f(p.x, p.ids_d, p.w_d, out=o0 if fin else None)
        torch.cuda.synchronize()
        if fin:
            res.append(r.clone())
        else:
            y, _, ttr = r
            rows = ttr.reshape(-1)
            rows = rows[rows >= 0].long()
            res.append(y[rows].clone())
    return res


CASES = [  # (workload, block_m, finalize, M of the first call, M of the second, smaller call)
    ("decode", 8, True, 8, 3),
    ("decode", 8, False, 8, 5),
    ("tiny", 128, True, 16, 7),
    ("tiny", 128, False, 16, 9),
]


@pytest.mark.parametrize("name,bm,fin,m1,m2", CASES,
                         ids=["%s-bm%d-%s-M%d-M%d" % (c[0], c[1], "fin" if c[2] else "unfin",
                                                      c[3], c[4]) for c in CASES])
def test_noalloc_matches_workspace_call(name, bm, fin, m1, m2):
    wl = WORKLOADS[name]
    for M in (m1, m2):                      # two calls in a row, the second smaller
        say("noalloc", name, "block_m", bm, "finalize", fin, "M", M)
        assert bf.bfp4_workspace_size(M, wl.H, wl.I, wl.top_k, wl.n_local, bm, int(fin)) \
            <= bf.NOALLOC_SCRATCH_BYTES
        got, want = _pair(wl, bm, fin, M)
        assert torch.equal(_bits(got), _bits(want)), (name, bm, fin, M)
        assert torch.any(_bits(want) != 0)


def test_noalloc_refuses_oversized_call():
    """The prefill shape needs far more workspace than the static array holds: refused with
    BFP4_ERR_WORKSPACE on the host, before anything is launched."""
    wl = WORKLOADS["prefill"]
    say("noalloc oversized")
    need = bf.bfp4_workspace_size(wl.M, wl.H, wl.I, wl.top_k, wl.n_local, wl.block_m, 1)
    assert need > bf.NOALLOC_SCRATCH_BYTES
    A = 1 << 20                              # never dereferenced: the size check comes first
    with pytest.raises(bf.Bfp4Error) as ei:
        bf.bfp4_fused_moe_nvfp4_noalloc(A, A, A, A, 1 << 40, A, A, A, 1.0, A, A, A, A,
                                        bf.bfp4_plan_capacity(wl.M, wl.top_k, wl.n_local,
                                                              wl.block_m),
                                        A, 0, wl.M, wl.H, wl.I, wl.n_local, wl.top_k,
                                        wl.block_m, 0, 1.0, 1, A, None, None)
    assert bf.STATUS[ei.value.status] == "BFP4_ERR_WORKSPACE"
