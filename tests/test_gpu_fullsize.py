"""Full-size GPU parity, in the launch configuration bench.py times.

For the decode (M=8), prefill (M=4096) and skewed squared-ReLU (M=16384, 144 of 288 experts
local) workloads: the whole plan, the activation quantization, the combine of the GPU's own
expert outputs and finalize(unfinalized) are checked over every element; the expert
computation is checked on a sampled token against the oracle, which quantizes that token's
experts itself (all W1 rows, sampled W2 rows):  pre-activation within 1e-5, requantization of
the GPU's BF16 intermediate bit-exact, final output within 2e-2 (relative Frobenius).

The standalone permutation is checked over every element at the prefill and skewed sizes.
The weight-only mode (BF16 activations, NVFP4 or MXFP4 weights) is checked the same way at the
decode shape: pre-activation within 1e-5, BF16 intermediate within 2e-3, sampled output within
2e-2, the combine and finalize(unfinalized) over every element.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import bf16_bits_to_f32
from synth import WORKLOADS

from gpu_common import Problem, np_bits, np_u8, rel_fro, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_scaled_fp4_plan_amd as bf
    from block_scaled_fp4_plan_amd import runner


def _check(name, token, n_hidden=512):
    wl = WORKLOADS[name]
    say("full-size", name, "token", token)
    p = Problem(wl)
    M, k, H, I, N1 = wl.M, wl.top_k, wl.H, wl.I, wl.N1
    act = wl.act_code
    pw, lin = runner.prepare_weights(p.w1, p.w2, gated=wl.gated, keep_linear=True)
    fwd = runner.MoeForward(pw, M, k, wl.E, wl.block_m, wl.local_offset)
    cap = fwd.plan.capacity
    dbg = dict(preact=torch.empty((cap, N1), dtype=torch.float32, device="cuda"),
               inter=torch.empty((cap, I), dtype=torch.bfloat16, device="cuda"),
               inter_q=torch.empty((cap, I // 2), dtype=torch.uint8, device="cuda"),
               inter_sf=torch.empty((cap, I // 16), dtype=torch.uint8, device="cuda"))
    out = fwd(p.x, p.ids_d, p.w_d, debug=dbg)
    fwd_u = runner.MoeForward(pw, M, k, wl.E, wl.block_m, wl.local_offset, do_finalize=False)
    y, wts, ttr_d = fwd_u(p.x, p.ids_d, p.w_d)
    out_u = torch.zeros_like(out)
    bf.bfp4_moe_finalize(y, wts, runner.weights_dtype(wts), ttr_d, M, H, k, 1.0, out_u)
    torch.cuda.synchronize()
    out_bits = np_bits(out)

    say(name, "plan + activation quantization (all elements)")
    srt, eids, P, ttr = p.oracle_plan(wl.block_m)
    assert int(fwd.plan.num_tokens_post_padded.item()) == P
    assert np.array_equal(fwd.plan.sorted_token_ids.cpu().numpy(), srt)
    assert np.array_equal(fwd.plan.expert_ids.cpu().numpy(), eids)
    assert np.array_equal(fwd.plan.token_to_row.cpu().numpy(), ttr)
    aq, asf, adec = p.oracle_activations()
    assert np.array_equal(np_u8(fwd.a_q), aq) and np.array_equal(np_u8(fwd.a_sf), asf)
    assert np.array_equal(fwd.a_dec.cpu().numpy().view(np.uint32), adec.view(np.uint32))

    say(name, "finalize(unfinalized) and the ordered combine (all elements)")
    assert np.array_equal(np_bits(out_u), out_bits)
    ybits = np_bits(y)
    ydict = {int(r): bf16_bits_to_f32(ybits[r]).astype(np.float64) for r in ttr.reshape(-1) if r >= 0}
    assert np.array_equal(oracle.combine(np.zeros((M, H), np.uint16), ydict, p.w, ttr), out_bits)

    say(name, "expert computation of token", token)
    rng = np.random.default_rng(token)
    hs = np.sort(rng.choice(H, n_hidden, replace=False))
    rows_t = [int(r) for r in ttr[token] if r >= 0]
    assert rows_t, "sampled token has no routed slot"
    inter_bits = np_bits(dbg["inter"][rows_t])
    pre_gpu = dbg["preact"][rows_t].cpu().numpy()
    pre_ref, ys = [], {}
    for j in range(k):
        r = int(ttr[token, j])
        if r < 0:
            continue
        e = int(eids[r // wl.block_m])
        b1, b2 = (np_bits(p.w1[e]), np_bits(p.w2[e]))
        q1, s1, a1 = oracle.quantize_expert_rows(b1, np.arange(N1))
        q2, s2, a2 = oracle.quantize_expert_rows(b2, hs)
        # the GPU's weight quantization is the oracle's, bit for bit, on these rows
        assert np.array_equal(np_u8(lin[0][e]), q1) and np.array_equal(np_u8(lin[1][e]), s1)
        assert np.array_equal(np_u8(lin[2][e][torch.from_numpy(hs).cuda()]), q2)
        assert pw.alpha1_gate[e].item() == float(a1) and pw.alpha2[e].item() == float(a2)
        o = oracle.expert_rows_forward(aq[token:token + 1], asf[token:token + 1],
                                       adec[token:token + 1], q1, s1, q2, s2, a1, a1, a2, 1.0, act)
        pre_ref.append(o["pre"][0])
        ys[r] = o["y"][0]
    e_pre = rel_fro(pre_gpu, np.stack(pre_ref))
    rq, rsf, _ = oracle.quantize_nvfp4(bf16_bits_to_f32(inter_bits), oracle.SCALE_FIXED, None, 1.0)
    assert np.array_equal(np_u8(dbg["inter_q"][rows_t]), rq)
    assert np.array_equal(np_u8(dbg["inter_sf"][rows_t]), rsf)
    ref = oracle.combine(np.zeros((1, len(hs)), np.uint16), ys, p.w[token:token + 1],
                         ttr[token:token + 1])
    e_out = rel_fro(bf16_bits_to_f32(out_bits[token, hs]), bf16_bits_to_f32(ref[0]))
    say("%s: pre %.3e  out(sampled) %.3e" % (name, e_pre, e_out))
    assert e_pre <= 1e-5
    assert e_out <= 2e-2


def test_fullsize_decode_m8():
    _check("decode", token=3)


def test_fullsize_prefill_m4096():
    _check("prefill", token=2731)


def test_fullsize_skewed_relu2_m16384():
    wl = WORKLOADS["skewed_relu2"]
    from synth import make_routing
    ids, _ = make_routing(wl, 0)
    loc = (ids >= wl.local_offset) & (ids < wl.local_offset + wl.n_local)
    token = int(np.nonzero(loc.sum(axis=1) >= 3)[0][7])
    _check("skewed_relu2", token=token)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_fullsize_w4a16_decode_m8(fmt, n_hidden=512):
    wl = WORKLOADS["decode"]
    token = 5
    say("full-size weight-only decode", fmt, "token", token)
    p = Problem(wl)
    M, k, H, I, N1 = wl.M, wl.top_k, wl.H, wl.I, wl.N1
    if fmt == "mxfp4":
        pw, lin = runner.prepare_weights_mxfp4(p.w1, p.w2, gated=wl.gated, keep_linear=True)
    else:
        pw, lin = runner.prepare_weights(p.w1, p.w2, gated=wl.gated, keep_linear=True)
    fwd = runner.MoeForwardW4A16(pw, M, k, wl.E, wl.block_m, wl.local_offset, act=wl.act_code)
    cap = fwd.plan.capacity
    dbg = dict(preact=torch.full((cap, N1), float("nan"), device="cuda"),
               inter=torch.zeros((cap, I), dtype=torch.bfloat16, device="cuda"))
    out = fwd(p.x, p.ids_d, p.w_d, debug=dbg)
    fwd_u = runner.MoeForwardW4A16(pw, M, k, wl.E, wl.block_m, wl.local_offset,
                                   do_finalize=False, act=wl.act_code)
    y, wts, ttr_d = fwd_u(p.x, p.ids_d, p.w_d)
    out_u = torch.zeros_like(out)
    bf.bfp4_moe_finalize(y, wts, runner.weights_dtype(wts), ttr_d, M, H, k, 1.0, out_u)
    torch.cuda.synchronize()
    out_bits = np_bits(out)

    srt, eids, P, ttr = p.oracle_plan(wl.block_m)
    assert np.array_equal(fwd.plan.token_to_row.cpu().numpy(), ttr)
    assert np.array_equal(np_bits(out_u), out_bits)
    ybits = np_bits(y)
    ydict = {int(r): bf16_bits_to_f32(ybits[r]).astype(np.float64) for r in ttr.reshape(-1) if r >= 0}
    assert np.array_equal(oracle.combine(np.zeros((M, H), np.uint16), ydict, p.w, ttr), out_bits)

    rng = np.random.default_rng(token)
    hs = np.sort(rng.choice(H, n_hidden, replace=False))
    rows_t = [int(r) for r in ttr[token] if r >= 0]
    pre_gpu = dbg["preact"][rows_t].cpu().numpy()
    h_gpu = bf16_bits_to_f32(np_bits(dbg["inter"][rows_t]))
    pre_ref, h_ref, ys = [], [], {}
    for j in range(k):
        r = int(ttr[token, j])
        if r < 0:
            continue
        e = int(eids[r // wl.block_m])
        b1, b2 = np_bits(p.w1[e]), np_bits(p.w2[e][torch.from_numpy(hs).cuda()])
        if fmt == "mxfp4":
            q1, s1 = oracle.quantize_mxfp4(bf16_bits_to_f32(b1))
            q2, s2 = oracle.quantize_mxfp4(bf16_bits_to_f32(b2))
            a1 = a2 = 1.0
        else:
            q1, s1, a1 = oracle.quantize_expert_rows(np_bits(p.w1[e]), np.arange(N1))
            q2, s2, a2 = oracle.quantize_expert_rows(np_bits(p.w2[e]), hs)
        # the GPU's weight quantization is the oracle's, bit for bit, on these rows
        assert np.array_equal(np_u8(lin[0][e]), q1) and np.array_equal(np_u8(lin[1][e]), s1)
        hs_d = torch.from_numpy(hs).cuda()
        assert np.array_equal(np_u8(lin[2][e][hs_d]), q2)
        assert np.array_equal(np_u8(lin[3][e][hs_d]), s2)
        o = oracle.expert_rows_forward_w16(p.x_bits[token:token + 1], q1, s1, q2, s2, a1, a1, a2,
                                           wl.act_code, weight_format=fmt)
        pre_ref.append(o["pre"][0])
        h_ref.append(o["h"][0])
        ys[r] = o["y"][0]
    e_pre = rel_fro(pre_gpu, np.stack(pre_ref))
    e_h = rel_fro(h_gpu, np.stack(h_ref))
    ref = oracle.combine(np.zeros((1, len(hs)), np.uint16), ys, p.w[token:token + 1],
                         ttr[token:token + 1])
    e_out = rel_fro(bf16_bits_to_f32(out_bits[token, hs]), bf16_bits_to_f32(ref[0]))
    say("w4a16 %s: pre %.3e  h %.3e  out(sampled) %.3e" % (fmt, e_pre, e_h, e_out))
    assert e_pre <= 1e-5
    assert e_h <= 2e-3
    assert e_out <= 2e-2


@pytest.mark.parametrize("name", ["prefill", "skewed_relu2"])
def test_fullsize_permute(name):
    """The standalone permutation at full size (every element, bit-exact): plan rows below the
    extent take their token's packed row, scale row and decode scale; sentinel rows and rows past
    the extent are zero."""
    from synth import make_activations, make_routing

    wl = WORKLOADS[name]
    say("full-size permute", name)
    M, k, H, bm = wl.M, wl.top_k, wl.H, wl.block_m
    x_bits = make_activations(wl, 0)
    ids, _ = make_routing(wl, 0)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    q, sf, dec = runner.quantize(x)
    pb = runner.MoePlanBuffers(M, k, wl.n_local, bm, "cuda")
    pb.build(torch.from_numpy(ids).cuda(), wl.E, wl.local_offset)
    cap = pb.capacity
    qp = torch.full((cap, H // 2), 0xAB, dtype=torch.uint8, device="cuda")
    sp = torch.full((cap, H // 16), 0xAB, dtype=torch.uint8, device="cuda")
    spd = torch.full((cap,), float("nan"), dtype=torch.float32, device="cuda")
    bf.bfp4_moe_permute(q, sf, dec, M, H, k, pb.sorted_token_ids, pb.num_tokens_post_padded, cap,
                        qp, sp, spd)
    torch.cuda.synchronize()
    srt, _, P, _ = oracle.moe_plan(ids, wl.E, wl.local_offset, wl.n_local, bm)
    oq, osf, odec = oracle.quantize_nvfp4(bf16_bits_to_f32(x_bits), oracle.SCALE_PER_ROW)
    wq, wsf, wsd = oracle.moe_permute(oq, osf, odec, srt, P, k)
    assert np.array_equal(np_u8(qp), wq)
    assert np.array_equal(np_u8(sp), wsf)
    assert np.array_equal(spd.cpu().numpy().view(np.uint32), wsd.view(np.uint32))
