"""GPU parity of the debug validators (bfp4_check_topk_ids, bfp4_check_plan) with the oracle's
routing_violations and plan_violations: every count and the first offending token equal the
oracle's exactly, on the workloads' own routings and plans (clean) and on planted breaches; the
validators leave what they read unchanged."""

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_routing

from gpu_common import say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_scaled_fp4_plan_amd as bf
    from block_scaled_fp4_plan_amd import runner


def _gpu_topk(ids, E):
    d = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    before = d.clone()
    res = runner.check_topk_ids(d, E)
    assert torch.equal(d, before)
    return res


def test_check_topk_ids_matches_oracle():
    for name in ("tiny", "decode_ll", "decode", "prefill", "skewed_relu2"):
        wl = WORKLOADS[name]
        say("check_topk_ids", name)
        ids, _ = make_routing(wl, 0)
        assert _gpu_topk(ids, wl.E) == oracle.routing_violations(ids, wl.E) == (0, 0, None)
    rng = np.random.default_rng(7)
    # dense breaches over ragged sizes (not multiples of the 256-thread block)
    for M, k, E in ((1, 1, 1), (300, 4, 6), (1000, 8, 16), (5000, 10, 128), (0, 3, 4)):
        say("check_topk_ids random", M, k, E)
        ids = rng.integers(-3, E + 3, size=(M, k)).astype(np.int32)
        assert _gpu_topk(ids, E) == oracle.routing_violations(ids, E)
    # a few planted breaches in a clean decode routing
    wl = WORKLOADS["decode"]
    ids, _ = make_routing(wl, 1)
    ids[6, 2] = wl.E                  # out of range
    ids[3, 5] = ids[3, 0]             # repeated expert
    ids[7, 1] = -2                    # out of range
    ids[7, 4] = ids[7, 3]             # and a repeat in the same token
    ids[2, 0] = -1                    # an empty slot is allowed
    exp = oracle.routing_violations(ids, wl.E)
    assert exp == (2, 2, 3)
    assert _gpu_topk(ids, wl.E) == exp


PLAN_CASES = [("tiny", 8), ("tiny", 128), ("decode", 8), ("prefill", 128), ("skewed_relu2", 128)]


@pytest.mark.parametrize("name,bm", PLAN_CASES, ids=["%s-bm%d" % c for c in PLAN_CASES])
def test_check_plan_matches_oracle(name, bm):
    wl = WORKLOADS[name]
    say("check_plan", name, "block_m", bm)
    M, k, nloc = wl.M, wl.top_k, wl.n_local
    ids, _ = make_routing(wl, 0)
    pb = runner.MoePlanBuffers(M, k, nloc, bm, "cuda")
    pb.build(torch.from_numpy(ids).cuda(), wl.E, wl.local_offset)
    cap = pb.capacity
    srt0 = pb.sorted_token_ids.cpu().numpy()
    eids0 = pb.expert_ids.cpu().numpy()
    P = int(pb.num_tokens_post_padded.item())
    assert pb.check() == oracle.plan_violations(srt0, eids0, P, cap, M, k, nloc, bm) == (0, 0, 0)
    assert np.array_equal(pb.sorted_token_ids.cpu().numpy(), srt0)
    assert np.array_equal(pb.expert_ids.cpu().numpy(), eids0)

    srt, eids = srt0.copy(), eids0.copy()
    srt[0] = -1
    srt[P - 1] = M * k + 1
    if P < cap:
        srt[P] = -5                   # past the extent: not a breach
    eids[(P // bm) // 2] = nloc
    pb.sorted_token_ids.copy_(torch.from_numpy(srt))
    pb.expert_ids.copy_(torch.from_numpy(eids))
    for ext in (P, P + 3, cap + bm, -bm, cap):
        pb.num_tokens_post_padded.fill_(ext)
        exp = oracle.plan_violations(srt, eids, ext, cap, M, k, nloc, bm)
        got = pb.check()
        say("extent", ext, "expected", exp, "got", got)
        assert got == exp, ext
    assert oracle.plan_violations(srt, eids, P, cap, M, k, nloc, bm)[:2] == (2, 1)


@pytest.mark.parametrize("nbytes", [16, 16 * 1000003, 64 << 20])
def test_xor_checksum_matches_numpy(nbytes):
    """bfp4_xor_checksum (the benchmark's read-stream diagnostic): the XOR of its partial words
    equals numpy's XOR of every 32-bit word of the buffer, for sizes that do and do not divide
    evenly over its reading waves."""
    say("xor checksum", nbytes)
    rng = np.random.default_rng(nbytes % 1000)
    host = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    partial = torch.zeros(bf.XOR_PARTIALS, dtype=torch.int32, device="cuda")
    bf.bfp4_xor_checksum(buf, nbytes, partial)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(partial.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)

