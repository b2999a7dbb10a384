"""GPU parity of the MX mode (MXFP4 weights on MXFP8 activations, the block-scaled MFMA path)
against the oracle, through the C ABI.

Bars: MXFP8 activation quantization bit-exact (every finite BF16 value, workload rows, edge
rows); the GPU's MXFP4 weight quantization bit-exact; GEMM1 pre-activation element by element
within MX_SUM_REL * sum |products| of the exact sum; the BF16 intermediate within 2e-3 relative
Frobenius and its MXFP8 requantization bit-exact; the expert outputs against the oracle's down
projection of the GPU's own intermediate within the same bound plus one BF16 step; the final
output within 2e-2; the combine of the GPU's expert outputs and finalize(unfinalized) bit-exact.

MX_SUM_REL: the block-scaled MFMA does not sum a 64-product chunk exactly to FP32.  An in-bounds
probe of the instruction (random FP4 x FP8 operands and E8M0 scales, compared with the exact
sum) measured errors up to 2^-13.4 of the chunk's sum of |products|; chunk results are then added
in FP32 (at most K/64 roundings).  The bar takes 2^-12 (2.6 times the measured worst) plus the
FP32 term; the pre-activation's relative Frobenius error is reported, not gated at 1e-5.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import bf16_bits_to_f32
from oracle.mx import mx_dot, mxfp4_int, mxfp8_int
from synth import WORKLOADS
from synth.workloads import Workload

from gpu_common import Problem, np_bits, np_u8, rel_fro, say, ulp_bf16

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_scaled_fp4_plan_amd as bf
    from block_scaled_fp4_plan_amd import runner


def _gpu_mxfp8(x_bits):
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()
    q, sf = runner.quantize_mxfp8(x)
    torch.cuda.synchronize()
    return np_u8(q), np_u8(sf)


def _check_mxfp8(x_bits):
    q, sf = _gpu_mxfp8(x_bits)
    oq, osf = oracle.quantize_mxfp8(bf16_bits_to_f32(x_bits))
    assert np.array_equal(q, oq)
    assert np.array_equal(sf, osf)


def test_quantize_mxfp8_all_bf16_bit_patterns():
    """Every finite BF16 value, in rows of 128 (each row one sign and two exponents), also
    shuffled; and the workload shapes."""
    say("mxfp8 all bf16 patterns")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f32(bits)
    bits = np.where(np.isfinite(v), bits, 0).astype(np.uint16)
    _check_mxfp8(bits.reshape(512, 128))
    _check_mxfp8(np.random.default_rng(0).permutation(bits).reshape(512, 128))
    from synth import make_activations
    for name in ("tiny", "decode_ll", "decode"):
        _check_mxfp8(make_activations(WORKLOADS[name], 0))


def test_quantize_mxfp8_edge_rows():
    say("mxfp8 edge rows")
    from synth import bf16_bits
    x = np.zeros((5, 64))
    x[1, :32] = 1e-40                       # BF16 subnormals: amax below the FP32 normal range
    x[2, :32] = np.linspace(-3.9, 3.9, 32)  # values that saturate at 448 * 2^X
    x[3, 5] = 3.0e38
    x[3, 40:] = -1e-30
    b = bf16_bits(x)
    b[0, 3] = 0x8000                        # -0.0
    b[4, :] = 0x8001                        # negative subnormals
    _check_mxfp8(b)


SKEWED_MX = Workload("skewed_mx", M=96, H=256, I=128, E=24, top_k=4, block_m=16, act="relu2",
                     routing="zipf", local_offset=4, num_local=12)
ONE_TOKEN = Workload("one_token", M=1, H=256, I=128, E=8, top_k=1, block_m=8)
MX_WORKLOADS = {
    "skewed_mx": SKEWED_MX, "one_token": ONE_TOKEN,
    "tiny_geglu": dataclasses.replace(WORKLOADS["tiny"], name="tiny_geglu", act="geglu"),
    "ll_gelu": dataclasses.replace(WORKLOADS["decode_ll"], name="ll_gelu", act="gelu", M=3),
    "wide": Workload("wide", M=6, H=1280, I=384, E=40, top_k=24, block_m=32, act="silu"),
}
# the tiled (block_m > 32) kernels: tiles of 1 to 8 token fragments (Zipf loads), K = 1280 and
# 640 (10 and 5 stages of 128, no multiple of the weight prefetch depth), gated and one-projection
RAGGED_MX = Workload("ragged_mx", M=384, H=1280, I=640, E=6, top_k=3, block_m=128, routing="zipf")
MX_WORKLOADS.update({
    "ragged_mx": RAGGED_MX,
    "ragged_mx_relu2": dataclasses.replace(RAGGED_MX, name="ragged_mx_relu2", act="relu2"),
    "skewed_mx_tiled": dataclasses.replace(SKEWED_MX, name="skewed_mx_tiled", M=700, block_m=128),
    # one expert with about 98 % of the tokens: a segment of five tiles
    "hot_expert_mx": Workload("hot_expert_mx", M=1100, H=256, I=128, E=4, top_k=1, block_m=128,
                              routing="zipf", zipf_s=6.0),
})
MX_CASES = [("tiny", 8), ("decode_ll", 8), ("skewed_mx", 16), ("one_token", 8),
            ("tiny_geglu", 16), ("ll_gelu", 8), ("wide", 32), ("tiny", 32),
            ("tiny", 128), ("ragged_mx", 128), ("ragged_mx_relu2", 128), ("skewed_mx_tiled", 128),
            ("one_token", 128), ("tiny_geglu", 136), ("hot_expert_mx", 128)]


def _workload(name):
    return MX_WORKLOADS.get(name) or WORKLOADS[name]


def _mx_expert(p, e):
    key = ("mx", e)
    if key not in p._host_w:
        b1, b2 = p.host_weight_bits(e)
        p._host_w[key] = (oracle.quantize_mxfp4(bf16_bits_to_f32(b1)) +
                          oracle.quantize_mxfp4(bf16_bits_to_f32(b2)))
    return p._host_w[key]


MX_SUM_REL = 2.0 ** -12


def _mx_bound(sabs, K):
    """Largest distance of a GPU sum over K products from the exact sum: the per-chunk error of
    the block-scaled MFMA plus the FP32 additions of the K/64 chunk results."""
    return (MX_SUM_REL + (K // 64) * 2.0 ** -24) * sabs


def _check_mx_down(y_gpu, hq, hsf, q2, s2):
    """Expert outputs of the GPU against the exact down projection of the GPU's own MXFP8
    intermediate: within _mx_bound of the exact sum, then one BF16 rounding each.  Returns
    (outputs that differ, outputs)."""
    a_int, a_exp = mxfp8_int(hq, hsf)
    w_int, w_exp = mxfp4_int(q2, s2)
    exact = mx_dot(a_int, a_exp, w_int, w_exp)
    ref = oracle.round_to_bf16(exact)
    sabs = mx_dot(np.abs(a_int), a_exp, np.abs(w_int), w_exp)
    bound = _mx_bound(sabs, hq.shape[1]) + ulp_bf16(ref)
    d = np.abs(y_gpu - ref)
    assert np.all(d <= bound), float((d / bound).max())
    return int(np.count_nonzero(d)), d.size


@pytest.mark.parametrize("name,bm", MX_CASES, ids=["%s-bm%d" % c for c in MX_CASES])
def test_fused_moe_mx_matches_oracle(name, bm):
    wl = _workload(name)
    say("fused MX", name, "block_m", bm)
    p = Problem(wl)
    M, k, H, I, N1 = p.M, wl.top_k, wl.H, wl.I, wl.N1
    pw, lin = runner.prepare_weights_mxfp4(p.w1, p.w2, gated=wl.gated, keep_linear=True)
    fwd = runner.MoeForwardMX(pw, M, k, wl.E, bm, wl.local_offset, act=wl.act_code)
    cap = fwd.plan.capacity
    dbg = dict(preact=torch.full((cap, N1), float("nan"), device="cuda"),
               inter=torch.zeros((cap, I), dtype=torch.bfloat16, device="cuda"),
               inter_q=torch.zeros((cap, I), dtype=torch.uint8, device="cuda"),
               inter_sf=torch.zeros((cap, I // 32), dtype=torch.uint8, device="cuda"))
    out = fwd(p.x, p.ids_d, p.w_d, debug=dbg)
    fwd_u = runner.MoeForwardMX(pw, M, k, wl.E, bm, wl.local_offset, do_finalize=False,
                                act=wl.act_code)
    y, wts, ttr_d = fwd_u(p.x, p.ids_d, p.w_d)
    out_u = torch.zeros_like(out)
    bf.bfp4_moe_finalize(y, wts, runner.weights_dtype(wts), ttr_d, M, H, k, 1.0, out_u)
    torch.cuda.synchronize()
    out_bits = np_bits(out)

    aq, asf = oracle.quantize_mxfp8(bf16_bits_to_f32(p.x_bits))
    assert np.array_equal(np_u8(fwd.a_q)[:M], aq) and np.array_equal(np_u8(fwd.a_sf)[:M], asf)
    srt, eids, P, ttr = p.oracle_plan(bm)
    experts = sorted(set(int(e) for e in eids[:P // bm]))
    for e in experts[:4]:                       # the GPU's MXFP4 weights are the oracle's
        q1, s1, q2, s2 = _mx_expert(p, e)
        assert np.array_equal(np_u8(lin[0][e]), q1) and np.array_equal(np_u8(lin[1][e]), s1)
        assert np.array_equal(np_u8(lin[2][e]), q2) and np.array_equal(np_u8(lin[3][e]), s2)
    res = oracle.fused_moe_mx(p.x_bits, lambda e: _mx_expert(p, e), srt, eids, P, ttr, p.w, k, bm,
                              wl.act_code)
    rows = sorted(res["pre"].keys())
    pre_gpu = dbg["preact"].cpu().numpy()[rows].astype(np.float64)
    hq, hsf = np_u8(dbg["inter_q"]), np_u8(dbg["inter_sf"])
    ybits = np_bits(y)
    ent = np.asarray(srt)
    flips = total = 0
    for e in experts:
        q1, s1, q2, s2 = _mx_expert(p, e)
        rs = [r for r in rows if int(eids[r // bm]) == e]
        toks = ent[rs] // k
        a_int, a_exp = mxfp8_int(aq[toks], asf[toks])
        w_int, w_exp = mxfp4_int(q1, s1)
        ref = mx_dot(a_int, a_exp, w_int, w_exp)
        sabs = mx_dot(np.abs(a_int), a_exp, np.abs(w_int), w_exp)
        got = pre_gpu[[rows.index(r) for r in rs]]
        bound = _mx_bound(sabs, H) + 1e-300
        assert np.all(np.abs(got - ref) <= bound), (e, float((np.abs(got - ref) / bound).max()))
        f, t = _check_mx_down(bf16_bits_to_f32(ybits[rs]).astype(np.float64), hq[rs], hsf[rs],
                              q2, s2)
        flips, total = flips + f, total + t
    e_pre = rel_fro(pre_gpu, np.stack([res["pre"][r] for r in rows]))
    inter = np_bits(dbg["inter"])[rows]
    rq, rsf = oracle.quantize_mxfp8(bf16_bits_to_f32(inter))
    assert np.array_equal(hq[rows], rq) and np.array_equal(hsf[rows], rsf)
    e_h = rel_fro(bf16_bits_to_f32(inter), np.stack([res["h"][r] for r in rows]))
    e_out = rel_fro(bf16_bits_to_f32(out_bits), bf16_bits_to_f32(res["out"]))
    say("MX %s bm%d: pre %.3e  h %.3e  y %d/%d one step off  out %.3e"
        % (name, bm, e_pre, e_h, flips, total, e_out))
    assert e_h <= 2e-3
    assert flips <= 0.1 * total
    assert e_out <= 2e-2
    assert np.array_equal(np_bits(out_u), out_bits)
    ttr_np = ttr_d.cpu().numpy()
    ydict = {int(r): bf16_bits_to_f32(ybits[r]).astype(np.float64)
             for r in ttr_np.reshape(-1) if r >= 0}
    assert np.array_equal(oracle.combine(np.zeros((M, H), np.uint16), ydict, p.w, ttr_np),
                          out_bits)


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_fullsize_mx(name, n_cols=64, extra_rows=4):
    """The MX mode at the full decode and prefill sizes, in the launch configuration the bench
    times: activation quantization and the combine of the GPU's expert outputs over every
    element; on every local expert with routed rows (first and last routed row of each 256-row
    tile and a few more), at sampled columns: the GPU's MXFP4 weight rows bit-exact with the
    oracle's, GEMM1 pre-activations and the expert outputs (on the GPU's own MXFP8 intermediate)
    within the MX bound, the intermediate's requantization bit-exact."""
    wl = WORKLOADS[name]
    say("full-size MX", name)
    p = Problem(wl)
    M, k, H, I, N1, bm = wl.M, wl.top_k, wl.H, wl.I, wl.N1, wl.block_m
    pw, lin = runner.prepare_weights_mxfp4(p.w1, p.w2, gated=wl.gated, keep_linear=True)
    fwd = runner.MoeForwardMX(pw, M, k, wl.E, bm, wl.local_offset, do_finalize=False)
    cap = fwd.plan.capacity
    dbg = dict(preact=torch.empty((cap, N1), device="cuda"),
               inter=torch.empty((cap, I), dtype=torch.bfloat16, device="cuda"),
               inter_q=torch.empty((cap, I), dtype=torch.uint8, device="cuda"),
               inter_sf=torch.empty((cap, I // 32), dtype=torch.uint8, device="cuda"))
    y, wts, ttr_d = fwd(p.x, p.ids_d, p.w_d, debug=dbg)
    out = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    bf.bfp4_moe_finalize(y, wts, runner.weights_dtype(wts), ttr_d, M, H, k, 1.0, out)
    torch.cuda.synchronize()
    aq, asf = oracle.quantize_mxfp8(bf16_bits_to_f32(p.x_bits))
    assert np.array_equal(np_u8(fwd.a_q), aq) and np.array_equal(np_u8(fwd.a_sf), asf)
    srt, eids, P, ttr = p.oracle_plan(bm)
    assert np.array_equal(ttr_d.cpu().numpy(), ttr)
    ybits = np_bits(y)
    ydict = {int(r): bf16_bits_to_f32(ybits[r]).astype(np.float64)
             for r in ttr.reshape(-1) if r >= 0}
    assert np.array_equal(oracle.combine(np.zeros((M, H), np.uint16), ydict, p.w, ttr),
                          np_bits(out))
    rng = np.random.default_rng(19)
    seg = {}
    for r in range(P):
        if srt[r] < M * k:
            seg.setdefault(int(eids[r // bm]), []).append(r)
    hq, hsf = np_u8(dbg["inter_q"]), np_u8(dbg["inter_sf"])
    flips = total = 0
    for e, rows_e in sorted(seg.items()):
        pick = {rows_e[0], rows_e[-1]}
        for t0 in range(rows_e[0], rows_e[-1] + 1, 256):
            inside = [r for r in rows_e if t0 <= r < t0 + 256]
            if inside:
                pick.add(inside[-1])
        pick.update(int(r) for r in rng.choice(rows_e, min(extra_rows, len(rows_e)), replace=False))
        rs = sorted(pick)
        toks = srt[rs] // k
        if wl.gated:
            ii = np.sort(rng.choice(I, n_cols // 2, replace=False))
            cols = np.concatenate([ii, I + ii])
        else:
            cols = np.sort(rng.choice(N1, n_cols, replace=False))
        hs = np.sort(rng.choice(H, n_cols, replace=False))
        cols_d, hs_d = torch.from_numpy(cols).cuda(), torch.from_numpy(hs).cuda()
        # MXFP4 is per row and per 32 values: the oracle quantizes just these rows
        q1, s1 = oracle.quantize_mxfp4(bf16_bits_to_f32(np_bits(p.w1[e][cols_d])))
        q2, s2 = oracle.quantize_mxfp4(bf16_bits_to_f32(np_bits(p.w2[e][hs_d])))
        assert np.array_equal(np_u8(lin[0][e][cols_d]), q1)
        assert np.array_equal(np_u8(lin[1][e][cols_d]), s1)
        assert np.array_equal(np_u8(lin[2][e][hs_d]), q2)
        assert np.array_equal(np_u8(lin[3][e][hs_d]), s2)
        rs_d = torch.tensor(rs, device="cuda")
        a_int, a_exp = mxfp8_int(aq[toks], asf[toks])
        w_int, w_exp = mxfp4_int(q1, s1)
        ref = mx_dot(a_int, a_exp, w_int, w_exp)
        sabs = mx_dot(np.abs(a_int), a_exp, np.abs(w_int), w_exp)
        got = dbg["preact"][rs_d][:, cols_d].cpu().numpy().astype(np.float64)
        bound = _mx_bound(sabs, H) + 1e-300
        assert np.all(np.abs(got - ref) <= bound), (e, float((np.abs(got - ref) / bound).max()))
        rq, rsf = oracle.quantize_mxfp8(bf16_bits_to_f32(np_bits(dbg["inter"][rs_d])))
        assert np.array_equal(hq[rs], rq) and np.array_equal(hsf[rs], rsf)
        f, t = _check_mx_down(bf16_bits_to_f32(ybits[rs][:, hs]).astype(np.float64), rq, rsf,
                              q2, s2)
        flips, total = flips + f, total + t
    say("full-size MX %s: %d experts; y %d of %d one BF16 step off" % (name, len(seg), flips, total))
    assert flips <= 0.1 * total
