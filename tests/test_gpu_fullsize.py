"""Full-size GPU parity, in the launch configuration bench.py times.

For the decode (M=8), prefill (M=4096) and skewed squared-ReLU (M=16384, 144 of 288 experts
local) workloads: the whole plan, the activation quantization, the combine of the GPU's own
expert outputs and finalize(unfinalized) are checked over every element.  The expert computation
is checked on every local expert with routed rows: on its first routed row, the last routed row
of every 256-row tile of its segment and a few random rows, at sampled columns, against the
oracle, which quantizes those weight rows itself with the whole matrix's scale: the GEMM1
pre-activation element by element within the FP32-summation bound (and within 1e-5 relative
Frobenius), the requantization of the GPU's BF16 intermediate bit-exact, the tiled down GEMM's
FP16 operand bit-exact, and the BF16 expert outputs (GEMM2 on the GPU's own intermediate) within
the FP32-summation bound plus one BF16 step.  A sampled token's final output is within 2e-2.

The standalone permutation is checked over every element at the prefill and skewed sizes.
The weight-only mode (BF16 activations, NVFP4 or MXFP4 weights) is checked at the decode shape:
pre-activation within 1e-5, BF16 intermediate within 2e-3, sampled output within 2e-2, the
combine and finalize(unfinalized) over every element.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import bf16_bits_to_f32
from synth import WORKLOADS

from gpu_common import Problem, check_down, check_gate_up, np_bits, np_u8, rel_fro, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_scaled_fp4_plan_amd as bf
    from block_scaled_fp4_plan_amd import runner


def _sample_rows(rows_e, seg_start, rng, extra):
    """Plan rows of one expert segment to check: its first routed row, the last routed row of
    every 256-row tile of the segment (the tiled kernels' tile height), and `extra` more."""
    pick = {rows_e[0], rows_e[-1]}
    for t0 in range(seg_start, rows_e[-1] + 1, 256):
        inside = [r for r in rows_e if t0 <= r < t0 + 256]
        if inside:
            pick.add(inside[-1])
    pick.update(int(r) for r in rng.choice(rows_e, min(extra, len(rows_e)), replace=False))
    return sorted(pick)


def _check(name, token, n_cols=64, extra_rows=6):
    wl = WORKLOADS[name]
    say("full-size", name)
    p = Problem(wl)
    M, k, H, I, N1, bm = wl.M, wl.top_k, wl.H, wl.I, wl.N1, wl.block_m
    act = wl.act_code
    pw, lin = runner.prepare_weights(p.w1, p.w2, gated=wl.gated, keep_linear=True)
    fwd = runner.MoeForward(pw, M, k, wl.E, bm, wl.local_offset)
    cap = fwd.plan.capacity
    dbg = dict(preact=torch.empty((cap, N1), dtype=torch.float32, device="cuda"),
               inter=torch.empty((cap, I), dtype=torch.bfloat16, device="cuda"),
               inter_q=torch.empty((cap, I // 2), dtype=torch.uint8, device="cuda"),
               inter_sf=torch.empty((cap, I // 16), dtype=torch.uint8, device="cuda"))
    out = fwd(p.x, p.ids_d, p.w_d, debug=dbg)
    # the unfinalized run of the same call: y, and the intermediate its down GEMM read
    fwd_u = runner.MoeForward(pw, M, k, wl.E, bm, wl.local_offset, do_finalize=False)
    dbg_u = dict(inter_q=torch.empty((cap, I // 2), dtype=torch.uint8, device="cuda"),
                 inter_sf=torch.empty((cap, I // 16), dtype=torch.uint8, device="cuda"))
    if bm > 32:
        dbg_u["inter_f16"] = torch.empty((cap, I), dtype=torch.float16, device="cuda")
    y, wts, ttr_d = fwd_u(p.x, p.ids_d, p.w_d, debug=dbg_u)
    out_u = torch.zeros_like(out)
    bf.bfp4_moe_finalize(y, wts, runner.weights_dtype(wts), ttr_d, M, H, k, 1.0, out_u)
    torch.cuda.synchronize()
    out_bits = np_bits(out)

    say(name, "plan + activation quantization (all elements)")
    srt, eids, P, ttr = p.oracle_plan(bm)
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

    # every local expert with routed rows: sampled rows of every tile, sampled output columns
    rng = np.random.default_rng(17)
    seg = {}
    for r in range(P):
        if srt[r] < M * k:
            seg.setdefault(int(eids[r // bm]), []).append(r)
    say(name, "expert computation: %d experts" % len(seg))
    hq_u, hsf_u = np_u8(dbg_u["inter_q"]), np_u8(dbg_u["inter_sf"])
    hq_f, hsf_f = np_u8(dbg["inter_q"]), np_u8(dbg["inter_sf"])
    pre_sq = err_sq = 0.0
    flips = total = 0
    worst1 = worst2 = 0.0
    n_rows = 0
    for e, rows_e in sorted(seg.items()):
        seg_start = rows_e[0]                  # segments hold their routed rows first
        rs = _sample_rows(rows_e, seg_start, rng, extra_rows)
        n_rows += len(rs)
        toks = srt[rs] // k
        if wl.gated:
            ii = np.sort(rng.choice(I, n_cols // 2, replace=False))
            cols = np.concatenate([ii, I + ii])
        else:
            cols = np.sort(rng.choice(N1, n_cols, replace=False))
        hs = np.sort(rng.choice(H, n_cols, replace=False))
        q1, s1, a1 = oracle.quantize_expert_rows(np_bits(p.w1[e]), cols)
        q2, s2, a2 = oracle.quantize_expert_rows(np_bits(p.w2[e]), hs)
        cols_d, hs_d = torch.from_numpy(cols).cuda(), torch.from_numpy(hs).cuda()
        # the GPU's weight quantization is the oracle's, bit for bit, on these rows
        assert np.array_equal(np_u8(lin[0][e][cols_d]), q1)
        assert np.array_equal(np_u8(lin[1][e][cols_d]), s1)
        assert np.array_equal(np_u8(lin[2][e][hs_d]), q2)
        assert np.array_equal(np_u8(lin[3][e][hs_d]), s2)
        assert pw.alpha1_gate[e].item() == float(a1) and pw.alpha2[e].item() == float(a2)
        rs_d = torch.tensor(rs, device="cuda")
        # GEMM1 pre-activation (sampled columns) against the oracle
        alpha_rows = np.full(len(cols), float(a1))
        pre_ref = oracle.expert_gate_up_projection(aq[toks], asf[toks], adec[toks], q1, s1,
                                                    alpha_rows)
        pre_gpu = dbg["preact"][rs_d][:, cols_d].cpu().numpy().astype(np.float64)
        worst1 = max(worst1, check_gate_up(pre_gpu, pre_ref, aq[toks], asf[toks], adec[toks],
                                           q1, s1, alpha_rows))
        pre_sq += float(np.sum(pre_ref ** 2))
        err_sq += float(np.sum((pre_gpu - pre_ref) ** 2))
        # requantization of the GPU's BF16 intermediate (whole rows), both runs alike
        inter_bits = np_bits(dbg["inter"][rs_d])
        rq, rsf, _ = oracle.quantize_nvfp4(bf16_bits_to_f32(inter_bits), oracle.SCALE_FIXED,
                                           None, 1.0)
        assert np.array_equal(hq_f[rs], rq) and np.array_equal(hsf_f[rs], rsf)
        assert np.array_equal(hq_u[rs], rq) and np.array_equal(hsf_u[rs], rsf)
        if bm > 32:          # the tiled down GEMM's FP16 operand: the exact decode of (hq, hsf)
            h16 = dbg_u["inter_f16"][rs_d].cpu().numpy().astype(np.float64)
            assert np.array_equal(h16, oracle.dequantize_nvfp4(rq, rsf))
        # GEMM2 (sampled output columns) on the GPU's own intermediate
        ref = oracle.expert_down_projection(rq, rsf, q2, s2, a2, 1.0)
        got = bf16_bits_to_f32(ybits[rs][:, hs]).astype(np.float64)
        f, t, w = check_down(got, ref, rq, rsf, q2, s2, a2)
        flips, total, worst2 = flips + f, total + t, max(worst2, w)
    e_pre = (err_sq / pre_sq) ** 0.5
    say("%s: %d rows of %d experts; pre rel. Frobenius %.3e (worst %.2f of the FP32 bound); "
        "y %d of %d one BF16 step off (worst %.2f of the bound)"
        % (name, n_rows, len(seg), e_pre, worst1, flips, total, worst2))
    assert e_pre <= 1e-5
    assert flips <= 0.01 * total

    say(name, "final output of token", token)
    rows_t = [int(r) for r in ttr[token] if r >= 0]
    assert rows_t, "sampled token has no routed slot"
    hs = np.sort(rng.choice(H, 512, replace=False))
    ys = {}
    for j in range(k):
        r = int(ttr[token, j])
        if r < 0:
            continue
        e = int(eids[r // bm])
        q1, s1, a1 = oracle.quantize_expert_rows(np_bits(p.w1[e]), np.arange(N1))
        q2, s2, a2 = oracle.quantize_expert_rows(np_bits(p.w2[e]), hs)
        o = oracle.expert_rows_forward(aq[token:token + 1], asf[token:token + 1],
                                       adec[token:token + 1], q1, s1, q2, s2, a1, a1, a2, 1.0, act)
        ys[r] = o["y"][0]
    ref = oracle.combine(np.zeros((1, len(hs)), np.uint16), ys, p.w[token:token + 1],
                         ttr[token:token + 1])
    e_out = rel_fro(bf16_bits_to_f32(out_bits[token, hs]), bf16_bits_to_f32(ref[0]))
    say("%s: out(token %d, sampled) %.3e" % (name, token, e_out))
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
