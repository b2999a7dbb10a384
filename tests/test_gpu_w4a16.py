"""GPU parity of the NVFP4 weight-only mode on BF16 activations (bfp4_fused_moe_w4a16) against
the oracle's fused_moe_w4a16, through the C ABI.

Bars: GEMM1 pre-activation (FP32, before its BF16 rounding) within 1e-5 relative Frobenius; the
BF16 intermediate within 2e-3 (both sides round act(bf16(pre)) to BF16 from pre-activations 1e-5
apart, so elements differ by at most one BF16 step, and rarely); the final output within 2e-2;
the combine of the GPU's own expert outputs bit-exact; finalize(unfinalized) == finalized; two
runs bit-identical.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import bf16_bits_to_f32
from synth import WORKLOADS
from synth.workloads import Workload

from gpu_common import Problem, np_bits, rel_fro, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_scaled_fp4_plan_amd as bf
    from block_scaled_fp4_plan_amd import runner

SKEWED = Workload("w16_skewed", M=96, H=256, I=128, E=24, top_k=4, block_m=16, act="relu2",
                  routing="zipf", local_offset=4, num_local=12)
WL = {
    "tiny": WORKLOADS["tiny"],
    "tiny_geglu": dataclasses.replace(WORKLOADS["tiny"], name="tiny_geglu", act="geglu"),
    "decode_ll": WORKLOADS["decode_ll"],
    "skewed_relu2": SKEWED,
    "skewed_gelu": dataclasses.replace(SKEWED, name="skewed_gelu", act="gelu"),
    "skewed_identity": dataclasses.replace(SKEWED, name="skewed_identity", act="identity"),
    "decode_m2": WORKLOADS["decode"],
}
CASES = [("tiny", 8), ("tiny", 32), ("tiny_geglu", 8), ("decode_ll", 8), ("skewed_relu2", 16),
         ("skewed_gelu", 16), ("skewed_identity", 32), ("decode_m2", 8)]


@pytest.mark.parametrize("name,bm", CASES, ids=["%s-bm%d" % c for c in CASES])
def test_w4a16_matches_oracle(name, bm):
    wl = WL[name]
    M = 2 if name == "decode_m2" else None        # the decode shape on two tokens
    say("w4a16", name, "block_m", bm)
    p = Problem(wl, M=M)
    k = wl.top_k
    pw = runner.prepare_weights(p.w1, p.w2, gated=wl.gated)
    fwd = runner.MoeForwardW4A16(pw, p.M, k, wl.E, bm, wl.local_offset, act=wl.act_code)
    cap = fwd.plan.capacity
    dbg = dict(preact=torch.full((cap, wl.N1), float("nan"), device="cuda"),
               inter=torch.zeros((cap, wl.I), dtype=torch.bfloat16, device="cuda"))
    out = fwd(p.x, p.ids_d, p.w_d, debug=dbg)
    torch.cuda.synchronize()
    out_bits = np_bits(out)
    srt, eids, P, ttr = p.oracle_plan(bm)
    assert int(fwd.plan.num_tokens_post_padded.item()) == P
    experts = sorted(set(int(e) for e in eids[:P // bm]))
    a1, a2 = p.oracle_alphas(experts)
    res = oracle.fused_moe_w4a16(p.x_bits, lambda e: p.oracle_expert(e)[0], a1, a1, a2, srt, eids,
                                 P, ttr, p.w, k, bm, wl.act_code)
    rows = sorted(res["pre"].keys())
    e_pre = rel_fro(dbg["preact"].cpu().numpy()[rows], np.stack([res["pre"][r] for r in rows]))
    h_gpu = bf16_bits_to_f32(np_bits(dbg["inter"])[rows])
    e_h = rel_fro(h_gpu, np.stack([res["h"][r] for r in rows]))
    e_out = rel_fro(bf16_bits_to_f32(out_bits), bf16_bits_to_f32(res["out"]).astype(np.float64))
    say("pre %.3e  h %.3e  out %.3e" % (e_pre, e_h, e_out))
    assert e_pre <= 1e-5
    assert e_h <= 2e-3
    assert e_out <= 2e-2
    assert np.any(out_bits != 0)
    # unfinalized triple: its combine is the oracle's combine bit for bit, and finalize of it is
    # the finalized output
    fwd_u = runner.MoeForwardW4A16(pw, p.M, k, wl.E, bm, wl.local_offset, do_finalize=False,
                                   act=wl.act_code)
    y, wts, ttr_d = fwd_u(p.x, p.ids_d, p.w_d)
    out2 = torch.zeros_like(out)
    bf.bfp4_moe_finalize(y, wts, runner.weights_dtype(wts), ttr_d, p.M, wl.H, k, 1.0, out2)
    torch.cuda.synchronize()
    assert np.array_equal(np_bits(out2), out_bits)
    ttr_np = ttr_d.cpu().numpy()
    ybits = np_bits(y)
    ydict = {int(r): bf16_bits_to_f32(ybits[r]).astype(np.float64)
             for r in ttr_np.reshape(-1) if r >= 0}
    comb = oracle.combine(np.zeros((p.M, wl.H), np.uint16), ydict, p.w, ttr_np)
    assert np.array_equal(comb, out_bits)
    out3 = fwd(p.x, p.ids_d, p.w_d)
    torch.cuda.synchronize()
    assert np.array_equal(np_bits(out3), out_bits)


def test_w4a16_strided_rows_and_nothing_local():
    """Activations read through a row stride larger than H; a batch whose assignments are all
    non-local leaves out unchanged."""
    wl = WORKLOADS["tiny"]
    say("w4a16 strided rows / nothing local")
    p = Problem(wl)
    pw = runner.prepare_weights(p.w1, p.w2)
    fwd = runner.MoeForwardW4A16(pw, p.M, wl.top_k, wl.E, 8)
    wide = torch.zeros((p.M, wl.H + 64), dtype=torch.bfloat16, device="cuda")
    wide[:, :wl.H] = p.x
    out_a = fwd(p.x, p.ids_d, p.w_d)
    out_b = fwd(wide[:, :wl.H], p.ids_d, p.w_d)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    fwd_off = runner.MoeForwardW4A16(pw, p.M, wl.top_k, wl.E + 8, 8, local_expert_offset=wl.E)
    out0 = torch.randn((p.M, wl.H), device="cuda").to(torch.bfloat16)
    out_c = out0.clone()
    fwd_off(p.x, p.ids_d, p.w_d, out=out_c)
    torch.cuda.synchronize()
    assert torch.equal(out_c.view(torch.int16), out0.view(torch.int16))


# ----------------------------------------------------------------------------- MXFP4 weights

def _gpu_mx(bits, pad=0):
    R, C = bits.shape
    wide = np.zeros((R, C + pad), np.uint16)
    wide[:, :C] = bits
    x = torch.from_numpy(wide.view(np.int16)).view(torch.bfloat16).cuda()[:, :C]
    q = torch.empty((R, C // 2), dtype=torch.uint8, device="cuda")
    sf = torch.empty((R, C // 32), dtype=torch.uint8, device="cuda")
    bf.bfp4_quantize_mxfp4(x, R, C, x.stride(0), q, sf)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy()


def test_mxfp4_quantize_bit_exact():
    """Every finite BF16 value (rows of 128: one sign and two exponents per row, then shuffled),
    all-zero and signed-zero blocks, BF16 subnormals next to normal values: GPU codes and UE8M0
    scales equal the oracle's."""
    say("mxfp4 quantize")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f32(bits)
    bits = np.where(np.isfinite(v), bits, 0).astype(np.uint16)
    rng = np.random.default_rng(1)
    edge = np.zeros((4, 128), np.uint16)
    edge[1, :] = 0x8000                                   # negative zeros
    edge[2, :32] = 0x0001                                 # BF16 subnormals only
    edge[2, 32:64] = np.array([0x0001, 0x3F80] * 16)      # subnormals beside 1.0
    edge[3, :] = 0x7F7F                                   # largest finite BF16
    for rows, pad in ((bits.reshape(512, 128), 0), (rng.permutation(bits).reshape(512, 128), 0),
                      (edge, 0), (rng.permutation(bits).reshape(256, 256), 40)):
        q, sf = _gpu_mx(rows, pad)                 # pad: rows read through a wider row stride
        oq, osf = oracle.quantize_mxfp4(bf16_bits_to_f32(rows))
        assert np.array_equal(sf, osf)
        assert np.array_equal(q, oq)


def _mx_expert(p, e):
    key = ("mx", e)
    if key not in p._host_w:
        b1, b2 = p.host_weight_bits(e)
        q1, s1 = oracle.quantize_mxfp4(bf16_bits_to_f32(b1))
        q2, s2 = oracle.quantize_mxfp4(bf16_bits_to_f32(b2))
        p._host_w[key] = (q1, s1, q2, s2)
    return p._host_w[key]


MX_CASES = [("tiny", 8), ("tiny_geglu", 16), ("decode_ll", 8), ("skewed_relu2", 16),
            ("decode_m2", 8)]


@pytest.mark.parametrize("name,bm", MX_CASES, ids=["%s-bm%d" % c for c in MX_CASES])
def test_w4a16_mxfp4_matches_oracle(name, bm):
    wl = WL[name]
    M = 2 if name == "decode_m2" else None
    say("w4a16 mxfp4", name, "block_m", bm)
    p = Problem(wl, M=M)
    k = wl.top_k
    pw, lin = runner.prepare_weights_mxfp4(p.w1, p.w2, gated=wl.gated, keep_linear=True)
    fwd = runner.MoeForwardW4A16(pw, p.M, k, wl.E, bm, wl.local_offset, act=wl.act_code)
    cap = fwd.plan.capacity
    dbg = dict(preact=torch.full((cap, wl.N1), float("nan"), device="cuda"),
               inter=torch.zeros((cap, wl.I), dtype=torch.bfloat16, device="cuda"))
    out = fwd(p.x, p.ids_d, p.w_d, debug=dbg)
    torch.cuda.synchronize()
    out_bits = np_bits(out)
    srt, eids, P, ttr = p.oracle_plan(bm)
    experts = sorted(set(int(e) for e in eids[:P // bm]))
    for e in experts[:3]:                       # the GPU's MXFP4 weights are the oracle's
        q1, s1, q2, s2 = _mx_expert(p, e)
        assert np.array_equal(lin[0][e].cpu().numpy(), q1)
        assert np.array_equal(lin[1][e].cpu().numpy(), s1)
        assert np.array_equal(lin[2][e].cpu().numpy(), q2)
        assert np.array_equal(lin[3][e].cpu().numpy(), s2)
    ones = np.ones(wl.n_local, np.float32)
    res = oracle.fused_moe_w4a16(p.x_bits, lambda e: _mx_expert(p, e), ones, ones, ones, srt, eids,
                                 P, ttr, p.w, k, bm, wl.act_code, weight_format="mxfp4")
    rows = sorted(res["pre"].keys())
    e_pre = rel_fro(dbg["preact"].cpu().numpy()[rows], np.stack([res["pre"][r] for r in rows]))
    e_h = rel_fro(bf16_bits_to_f32(np_bits(dbg["inter"])[rows]),
                  np.stack([res["h"][r] for r in rows]))
    e_out = rel_fro(bf16_bits_to_f32(out_bits), bf16_bits_to_f32(res["out"]).astype(np.float64))
    say("pre %.3e  h %.3e  out %.3e" % (e_pre, e_h, e_out))
    assert e_pre <= 1e-5
    assert e_h <= 2e-3
    assert e_out <= 2e-2
    assert np.any(out_bits != 0)
