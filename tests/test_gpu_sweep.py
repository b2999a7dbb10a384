"""Seeded sweep of random small shapes through the whole path on the GPU against the oracle:
hidden and intermediate sizes, expert counts, top_k, block_m (decode and tiled kernels), local
expert windows, routing kinds and activations drawn per case.  Same bars as the per-workload
parity tests: plan and activation quantization bit-exact, pre-activation within 1e-5, BF16
intermediate within 2e-3, output within 2e-2, the combine of the GPU's own expert outputs
bit-exact."""

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import bf16_bits_to_f32
from synth import ACT_NAMES
from synth.workloads import Workload

from gpu_common import Problem, np_bits, np_u8, rel_fro, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_scaled_fp4_plan_amd import runner


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.integers(2, 40))
    top_k = int(rng.integers(1, min(E, 12) + 1))
    nloc = int(rng.integers(1, E + 1))
    off = int(rng.integers(0, E - nloc + 1))
    bm = int(rng.choice([8, 16, 24, 32, 40, 64, 128, 136, 256]))
    wl = Workload("sweep%d" % seed, M=int(rng.integers(1, 160)), H=256 * int(rng.integers(1, 5)),
                  I=128 * int(rng.integers(1, 5)), E=E, top_k=top_k, block_m=bm,
                  act=ACT_NAMES[int(rng.integers(0, len(ACT_NAMES)))],
                  routing=str(rng.choice(["softmax", "zipf"])), local_offset=off, num_local=nloc)
    return wl


CASES = list(range(24))


@pytest.mark.parametrize("seed", CASES)
def test_random_shape_matches_oracle(seed):
    wl = _case(seed)
    bm = wl.block_m
    say("sweep", seed, wl)
    p = Problem(wl)
    pw = runner.prepare_weights(p.w1, p.w2, gated=wl.gated)
    fwd = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm, wl.local_offset, act=wl.act_code)
    cap = fwd.plan.capacity
    dbg = dict(preact=torch.full((cap, wl.N1), float("nan"), device="cuda"),
               inter=torch.zeros((cap, wl.I), dtype=torch.bfloat16, device="cuda"),
               inter_q=torch.zeros((cap, wl.I // 2), dtype=torch.uint8, device="cuda"),
               inter_sf=torch.zeros((cap, wl.I // 16), dtype=torch.uint8, device="cuda"))
    out = fwd(p.x, p.ids_d, p.w_d, debug=dbg)
    torch.cuda.synchronize()
    out_bits = np_bits(out)
    oq, osf, odec = p.oracle_activations()
    assert np.array_equal(np_u8(fwd.a_q), oq) and np.array_equal(np_u8(fwd.a_sf), osf)
    srt, eids, P, ttr = p.oracle_plan(bm)
    assert int(fwd.plan.num_tokens_post_padded.item()) == P
    assert np.array_equal(fwd.plan.sorted_token_ids.cpu().numpy()[:len(srt)], srt)
    assert np.array_equal(fwd.plan.token_to_row.cpu().numpy(), ttr)
    experts = sorted(set(int(e) for e in eids[:P // bm]))
    a1, a2 = p.oracle_alphas(experts)
    res = oracle.fused_moe_nvfp4(oq, osf, odec, lambda e: p.oracle_expert(e)[0], a1, a1, a2, 1.0,
                                 srt, eids, P, ttr, p.w, wl.top_k, bm, wl.act_code)
    out_ref = bf16_bits_to_f32(res["out"]).astype(np.float64)
    e_out = rel_fro(bf16_bits_to_f32(out_bits), out_ref)
    rows = sorted(res["pre"].keys())
    if rows:
        e_pre = rel_fro(dbg["preact"].cpu().numpy()[rows], np.stack([res["pre"][r] for r in rows]))
        e_h = rel_fro(bf16_bits_to_f32(np_bits(dbg["inter"])[rows]),
                      np.stack([res["h"][r] for r in rows]))
        say("pre %.3e  h %.3e  out %.3e" % (e_pre, e_h, e_out))
        assert e_pre <= 1e-5
        assert e_h <= 2e-3
    else:
        assert np.array_equal(out_bits, np.zeros_like(out_bits))
    assert e_out <= 2e-2
    # the combine of the GPU's own expert outputs is the oracle's combine, bit for bit
    fwd_u = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm, wl.local_offset, do_finalize=False,
                              act=wl.act_code)
    y, wts, ttr_d = fwd_u(p.x, p.ids_d, p.w_d)
    torch.cuda.synchronize()
    ttr_np = ttr_d.cpu().numpy()
    ybits = np_bits(y)
    ydict = {int(r): bf16_bits_to_f32(ybits[r]).astype(np.float64)
             for r in ttr_np.reshape(-1) if r >= 0}
    comb = oracle.combine(np.zeros((p.M, wl.H), np.uint16), ydict, p.w, ttr_np)
    assert np.array_equal(comb, out_bits)
