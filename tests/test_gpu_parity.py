"""GPU parity of the HIP path against the oracle, through the C ABI.

Bars (per workload): routing plan, permutation and quantization bit-exact; GEMM1
pre-activation within 1e-5 relative Frobenius; final output within 2e-2 relative Frobenius;
requantization of the GPU's own BF16 intermediate and the combine of the GPU's own expert outputs
bit-exact; finalize(unfinalized) == finalized; two runs bit-identical.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import bf16_bits_to_f32
from synth import WORKLOADS
from synth.workloads import Workload

from gpu_common import Problem, check_down, np_bits, np_u8, rel_fro, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_scaled_fp4_plan_amd as bf
    from block_scaled_fp4_plan_amd import runner


# ----------------------------------------------------------------------------- quantization

def _gpu_quant(x_bits, mode=0, group_rows=0, c=1.0):
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()
    q, sf, dec = runner.quantize(x, mode, group_rows, c)
    torch.cuda.synchronize()
    return np_u8(q), np_u8(sf), dec.cpu().numpy()


def _check_quant(x_bits, mode=0, group_rows=0, c=1.0):
    q, sf, dec = _gpu_quant(x_bits, mode, group_rows, c)
    oq, osf, odec = oracle.quantize_nvfp4(bf16_bits_to_f32(x_bits), mode, group_rows or None, c)
    assert np.array_equal(q, oq)
    assert np.array_equal(sf, osf)
    if mode == oracle.SCALE_FIXED:
        assert dec[0] == odec[0]
    else:
        assert np.array_equal(dec[:len(odec)].view(np.uint32), odec.view(np.uint32))


def test_quantize_per_row_workload_shapes():
    for name in ("tiny", "decode_ll", "decode"):
        wl = WORKLOADS[name]
        say("quantize per-row", name)
        from synth import make_activations
        _check_quant(make_activations(wl, 0))


def test_quantize_all_bf16_bit_patterns():
    """Every finite BF16 value, in rows of 256, at several row magnitudes."""
    say("quantize all bf16 patterns")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f32(bits)
    bits = np.where(np.isfinite(v), bits, 0).astype(np.uint16)
    rng = np.random.default_rng(0)

    def in_contract(r):   # row amax 0 or >= 2**-106
        a = np.abs(bf16_bits_to_f32(r)).max(axis=1)
        return r[(a == 0) | (a >= 2.0 ** -106)]

    rows = in_contract(bits.reshape(512, 128))     # each row: one sign, two exponents
    assert rows.shape[0] > 460
    _check_quant(rows)
    _check_quant(in_contract(rng.permutation(bits).reshape(512, 128)))
    _check_quant(bits.reshape(512, 128), oracle.SCALE_FIXED, 0, 1.0)
    _check_quant(bits.reshape(1024, 64), oracle.SCALE_FIXED, 0, 0.37)


def test_quantize_edge_rows():
    say("quantize edge rows")
    from synth import bf16_bits
    x = np.zeros((6, 64))
    x[1] = -0.0
    x[2, :16] = 1e-40                       # BF16 subnormals next to a tiny in-contract amax
    x[2, 20] = -2.0 ** -106
    x[3] = np.linspace(-6, 6, 64)
    x[4, 5] = 3.0e38
    x[5, ::7] = -1e-30
    b = bf16_bits(x)
    b[1] = 0x8000
    _check_quant(b)


def test_quantize_per_group_and_fixed():
    say("quantize per-group")
    rng = np.random.default_rng(3)
    from synth import bf16_bits
    w = bf16_bits(rng.standard_normal((8 * 96, 256)) * rng.uniform(0.001, 10, (8 * 96, 1)))
    _check_quant(w, oracle.SCALE_PER_GROUP, 96)
    _check_quant(w, oracle.SCALE_PER_GROUP, 1)
    say("quantize fixed")
    _check_quant(w, oracle.SCALE_FIXED, 0, 1.0)


# ----------------------------------------------------------------------------- plan / permute

def _gpu_plan(ids, E, off, nloc, bm):
    M, k = ids.shape
    pb = runner.MoePlanBuffers(M, k, nloc, bm, "cuda")
    pb.build(torch.from_numpy(ids).cuda(), E, off)
    torch.cuda.synchronize()
    return (pb.sorted_token_ids.cpu().numpy()[:pb.capacity], pb.expert_ids.cpu().numpy()[:pb.capacity // bm],
            int(pb.num_tokens_post_padded.item()), pb.token_to_row.cpu().numpy()[:M])


PLAN_CASES = [  # (M, top_k, E, offset, nloc, block_m, kind)
    (16, 2, 8, 0, 8, 8, "distinct"), (16, 2, 8, 0, 8, 128, "distinct"),
    (4, 10, 128, 0, 128, 8, "distinct"), (8, 8, 256, 0, 256, 8, "distinct"),
    (300, 6, 288, 0, 144, 128, "zipf"), (37, 3, 8, 2, 4, 16, "noisy"),
    (4096, 8, 256, 0, 256, 128, "distinct"), (16384, 6, 288, 0, 144, 128, "zipf"),
    (2000, 4, 64, 16, 32, 24, "noisy"), (1, 1, 4, 0, 4, 8, "distinct"),
    # 65536 and 65544 slots, 512 and 513 local experts, just past the one-workgroup kernel
    (8192, 8, 256, 0, 256, 128, "distinct"), (8193, 8, 256, 0, 256, 128, "distinct"),
    (700, 8, 600, 40, 512, 8, "noisy"), (700, 8, 600, 40, 513, 8, "noisy"),
    (257, 8, 64, 0, 64, 16, "distinct"),
    # 32 chunks of slots x 1024 local experts: more chunk counts than the scan keeps in LDS
    (4096, 8, 1024, 0, 1024, 16, "distinct"),
    # chunk counts kept in LDS, split over 3 threads per expert (71 chunks) and over all 1024
    # threads for a single local expert (69 chunks, most threads with none)
    (9000, 8, 300, 0, 300, 64, "zipf"), (70000, 1, 4, 0, 1, 8, "noisy"),
]


@pytest.mark.parametrize("case", PLAN_CASES, ids=[str(c) for c in PLAN_CASES])
def test_plan_bit_exact(case):
    M, k, E, off, nloc, bm, kind = case
    say("plan", case)
    rng = np.random.default_rng(M * 7 + k)
    if kind == "distinct":
        ids = np.argsort(rng.random((M, E)), axis=1)[:, :k].astype(np.int32)
    elif kind == "zipf":
        from synth.workloads import make_routing
        wl = Workload("z", M=M, H=256, I=128, E=E, top_k=k, block_m=bm, routing="zipf",
                      num_local=nloc)
        ids, _ = make_routing(wl, 0)
    else:
        ids = rng.integers(-2, E + 3, (M, k)).astype(np.int32)   # duplicates, -1, out of range
    got = _gpu_plan(ids, E, off, nloc, bm)
    want = oracle.moe_plan(ids, E, off, nloc, bm)
    assert got[2] == want[2]
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1], want[1])
    assert np.array_equal(got[3], want[3])


PQ_CASES = [  # (workload, M): one launch (decode sizes), the two-call fallback, an empty batch
    ("decode", 8), ("decode_ll", 4), ("tiny", 16), ("decode", 300), ("decode", 0)]


@pytest.mark.parametrize("name,M", PQ_CASES, ids=["%s-M%d" % c for c in PQ_CASES])
def test_plan_quantize_equals_separate_calls(name, M):
    """bfp4_moe_plan_quantize writes exactly what bfp4_moe_plan and bfp4_quantize_nvfp4 (per row)
    write: checked bit for bit against the two calls and against the oracle, in one launch
    (M * top_k <= 2048 slots) and through the two-call path above that."""
    from synth import make_activations, make_routing
    wl = WORKLOADS[name]
    say("plan+quantize", name, "M", M)
    Mg = max(M, 1)
    x_bits = make_activations(wl, 0, Mg)[:M]
    ids, _ = make_routing(wl, 0, Mg)
    ids = np.ascontiguousarray(ids[:M])
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()
    x = x.reshape(M, wl.H)
    idd = torch.from_numpy(ids).cuda().reshape(M, wl.top_k)
    outs = []
    for fused in (True, False):
        pb = runner.MoePlanBuffers(M, wl.top_k, wl.n_local, wl.block_m, "cuda")
        q = torch.full((Mg, wl.H // 2), 0xAB, dtype=torch.uint8, device="cuda")
        sf = torch.full((Mg, wl.H // 16), 0xAB, dtype=torch.uint8, device="cuda")
        dec = torch.full((Mg,), float("nan"), device="cuda")
        if fused:
            bf.bfp4_moe_plan_quantize(idd, M, wl.top_k, wl.E, wl.local_offset, wl.n_local,
                                      wl.block_m, pb.sorted_token_ids, pb.expert_ids,
                                      pb.num_tokens_post_padded, pb.token_to_row, pb.capacity,
                                      pb.ws, pb.ws_bytes, x, wl.H, wl.H, q, sf, dec)
        else:
            pb.build(idd, wl.E, wl.local_offset)
            if M:
                bf.bfp4_quantize_nvfp4(x, M, wl.H, wl.H, bf.BFP4_SCALE_PER_ROW, 0, 1.0, q, sf, dec,
                                       None, 0)
        torch.cuda.synchronize()
        cap = pb.capacity
        outs.append((pb.sorted_token_ids.cpu().numpy()[:cap],
                     pb.expert_ids.cpu().numpy()[:cap // wl.block_m],
                     int(pb.num_tokens_post_padded.item()), pb.token_to_row.cpu().numpy()[:M],
                     np_u8(q)[:M], np_u8(sf)[:M], dec.cpu().numpy()[:M].view(np.uint32)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    srt, eids, P, ttr = oracle.moe_plan(ids.reshape(M, wl.top_k), wl.E, wl.local_offset,
                                        wl.n_local, wl.block_m)
    assert outs[0][2] == P and np.array_equal(outs[0][0], srt) and np.array_equal(outs[0][3], ttr)
    if M:
        oq, osf, odec = oracle.quantize_nvfp4(bf16_bits_to_f32(x_bits), oracle.SCALE_PER_ROW)
        assert np.array_equal(outs[0][4], oq) and np.array_equal(outs[0][5], osf)
        assert np.array_equal(outs[0][6], odec.view(np.uint32))


def test_permute_bit_exact():
    wl = WORKLOADS["decode_ll"]
    say("permute", wl.name)
    p = Problem(wl, M=48)
    q, sf, dec = runner.quantize(p.x)
    pb = runner.MoePlanBuffers(48, wl.top_k, wl.n_local, 8, "cuda").build(p.ids_d, wl.E)
    cap = pb.capacity
    qp = torch.empty((cap, wl.H // 2), dtype=torch.uint8, device="cuda")
    sp = torch.empty((cap, wl.H // 16), dtype=torch.uint8, device="cuda")
    spd = torch.empty(cap, dtype=torch.float32, device="cuda")
    bf.bfp4_moe_permute(q, sf, dec, 48, wl.H, wl.top_k, pb.sorted_token_ids,
                        pb.num_tokens_post_padded, cap, qp, sp, spd)
    torch.cuda.synchronize()
    srt, eids, P, ttr = oracle.moe_plan(p.ids, wl.E, 0, wl.n_local, 8)
    oq, osf, odec = p.oracle_activations()
    wq, wsf, wsd = oracle.moe_permute(oq, osf, odec, srt, P, wl.top_k)
    assert np.array_equal(np_u8(qp), wq)
    assert np.array_equal(np_u8(sp), wsf)
    assert np.array_equal(spd.cpu().numpy().view(np.uint32), wsd.view(np.uint32))


# ----------------------------------------------------------------------------- weights layout

def test_prepare_weights_layout():
    """Panels hold exactly the linear NVFP4 bytes, rearranged (layout re-derived here)."""
    say("prepare layout")
    rng = np.random.default_rng(5)
    E, H, I = 2, 512, 384                     # K = 512 (one full superchunk), I = 384 (partial)
    for gated in (1, 0):
        N1 = 2 * I if gated else I
        w1q = rng.integers(0, 256, (E, N1, H // 2), dtype=np.uint8)
        w1s = rng.integers(0, 256, (E, N1, H // 16), dtype=np.uint8)
        w2q = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
        w2s = rng.integers(0, 256, (E, H, I // 16), dtype=np.uint8)
        nb = bf.bfp4_panel_bytes(E, H, I, gated)
        panels = torch.empty(nb, dtype=torch.uint8, device="cuda")
        t = [torch.from_numpy(a).cuda() for a in (w1q, w1s, w2q, w2s)]
        bf.bfp4_prepare_weights(*t, E, H, I, gated, panels, nb)
        torch.cuda.synchronize()
        got = np_u8(panels)
        off = 0
        for (q, s, rows, K, half) in ((w1q, w1s, N1, H, I if gated else 0), (w2q, w2s, H, I, 0)):
            nch, ng = K // 64, rows // 32
            nsc = (nch + 7) // 8
            for e in range(E):
                for g in range(ng):
                    for rho in range(32):
                        perm = 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3)
                        # gated W1: gate rows 16g.. in logical rows 0..15, up rows of the same
                        # intermediate indices in logical rows 16..31
                        lr = ((half if perm >= 16 else 0) + 16 * g + (perm & 15)) if half else g * 32 + perm
                        for hh in range(2):
                            lane = hh * 32 + rho
                            for c in range(nch):
                                sc, j = divmod(c, 8)
                                base = off + ((e * ng + g) * (nsc + nch) + sc * 9) * 1024
                                d = base + 1024 * (1 + j) + lane * 16
                                assert np.array_equal(got[d:d + 16], q[e, lr, 32 * c + 16 * hh: 32 * c + 16 * hh + 16])
                                sidx = base + lane * 16 + 2 * j
                                assert got[sidx] == s[e, lr, 4 * c + 2 * hh]
                                assert got[sidx + 1] == s[e, lr, 4 * c + 2 * hh + 1]
            off += E * ng * (nsc + nch) * 1024
        assert off == nb


# ----------------------------------------------------------------------------- full path

SMALL_SKEWED = Workload("skewed_small", M=96, H=256, I=128, E=24, top_k=4, block_m=16,
                        act="relu2", routing="zipf", local_offset=4, num_local=12)
TINY_RELU2 = Workload("tiny_relu2", M=40, H=512, I=256, E=8, top_k=3, block_m=128, act="relu2")
# K = 1280 and 640: 10 and 5 stages of 128, not a multiple of any prefill prefetch depth (2 to 8
# stages), with skewed expert loads giving tiles of 1 to 8 token fragments
RAGGED_K = Workload("ragged_k", M=384, H=1280, I=640, E=6, top_k=3, block_m=128, routing="zipf")
# down GEMM with 4 n-tiles of 4 stages: each tile's n-tiles run as one stage stream
CHAIN_N = Workload("chain_n", M=320, H=1024, I=512, E=5, top_k=2, block_m=128, routing="zipf")

# degenerate and limit shapes: one token with one slot; 24 of 40 experts per token; the largest
# hidden size whose routed rows fit the decode kernels' LDS at block_m 32 (32 rows x 5040 bytes
# + 256 = 161536 of 163840 bytes)
ONE_TOKEN = Workload("one_token", M=1, H=256, I=128, E=8, top_k=1, block_m=8)
WIDE_TOPK = Workload("wide_topk", M=6, H=512, I=256, E=40, top_k=24, block_m=16)
LDS_LIMIT = Workload("lds_limit", M=40, H=8960, I=128, E=4, top_k=2, block_m=32)
# few tokens on few row groups: the decode kernels split K over the waves of a workgroup, here
# in parts of unequal length (GEMM1: 10 stages of 128 over 4 waves; GEMM2: 5 over 2)
KS_RAGGED = Workload("ks_ragged", M=3, H=1280, I=640, E=12, top_k=3, block_m=8)

# one expert takes about 98 % of the tokens (Zipf exponent 6 over 4 experts): its segment spans
# five tiles of up to 256 rows, handed out one after another from the tile list beside the
# other experts' short tiles
HOT_EXPERT = Workload("hot_expert", M=1100, H=256, I=128, E=4, top_k=1, block_m=128,
                      routing="zipf", zipf_s=6.0)

# the other activations, on the decode (block_m 8, 16) and the tiled (block_m 128) kernels
ACT_WORKLOADS = {
    "tiny_geglu": dataclasses.replace(WORKLOADS["tiny"], name="tiny_geglu", act="geglu"),
    "ll_geglu": dataclasses.replace(WORKLOADS["decode_ll"], name="ll_geglu", act="geglu"),
    "ragged_geglu": dataclasses.replace(RAGGED_K, name="ragged_geglu", act="geglu"),
    "gelu": dataclasses.replace(TINY_RELU2, name="gelu", act="gelu"),
    "relu": dataclasses.replace(TINY_RELU2, name="relu", act="relu"),
    "silu": dataclasses.replace(TINY_RELU2, name="silu", act="silu"),
    "identity": dataclasses.replace(TINY_RELU2, name="identity", act="identity"),
    "skewed_gelu": dataclasses.replace(SMALL_SKEWED, name="skewed_gelu", act="gelu"),
}

MOE_CASES = [
    ("tiny", 8), ("tiny", 128), ("decode_ll", 8), ("skewed_small", 16), ("tiny_relu2", 128),
    ("tiny", 32), ("tiny", 136), ("ragged_k", 128), ("chain_n", 128),
    ("tiny_geglu", 8), ("tiny_geglu", 128), ("ll_geglu", 8), ("ragged_geglu", 128),
    ("gelu", 8), ("gelu", 128), ("relu", 16), ("relu", 128), ("silu", 8), ("silu", 128),
    ("identity", 8), ("identity", 128), ("skewed_gelu", 16),
    ("one_token", 8), ("one_token", 128), ("wide_topk", 16), ("wide_topk", 128), ("lds_limit", 32),
    ("ks_ragged", 8), ("hot_expert", 128), ("hot_expert", 8),
]


def _workload(name):
    return ({"skewed_small": SMALL_SKEWED, "tiny_relu2": TINY_RELU2, "ragged_k": RAGGED_K,
             "chain_n": CHAIN_N, "one_token": ONE_TOKEN, "wide_topk": WIDE_TOPK,
             "lds_limit": LDS_LIMIT, "ks_ragged": KS_RAGGED, "hot_expert": HOT_EXPERT,
             **ACT_WORKLOADS}.get(name) or WORKLOADS[name])


def check_gemm2(p, eids, bm, rows, dbg, y, c2=1.0, max_flip_frac=0.01):
    """GEMM2 (down projection) against the oracle on the GPU's own intermediate: for every routed
    plan row r of expert e, y_gpu[r] against oracle.expert_down_projection of (hq[r], hsf[r]) as
    the GPU wrote them, with W2_e quantized by the oracle, within the FP32-summation bound of
    check_down; at most max_flip_frac of the outputs may be one BF16 step off.  With block_m > 32
    the FP16 copy that the tiled down GEMM reads must be the exact decode of (hq, hsf) on every
    routed row."""
    hq = np_u8(dbg["inter_q"])
    hsf = np_u8(dbg["inter_sf"])
    if "inter_f16" in dbg:
        h16 = dbg["inter_f16"].cpu().numpy()[rows].astype(np.float64)
        assert np.array_equal(h16, oracle.dequantize_nvfp4(hq[rows], hsf[rows]))
    ybits = np_bits(y)
    by_e = {}
    for r in rows:
        by_e.setdefault(int(eids[r // bm]), []).append(r)
    flips = total = 0
    worst = 0.0
    for e, rs in sorted(by_e.items()):
        (_, _, q2, s2), _, a2 = p.oracle_expert(e)
        ref = oracle.expert_down_projection(hq[rs], hsf[rs], q2, s2, a2, c2)
        got = bf16_bits_to_f32(ybits[rs]).astype(np.float64)
        f, t, w = check_down(got, ref, hq[rs], hsf[rs], q2, s2, a2, c2)
        flips, total, worst = flips + f, total + t, max(worst, w)
    say("gemm2: %d of %d outputs one BF16 step off (worst %.2f of the bound)"
        % (flips, total, worst))
    assert flips <= max_flip_frac * total


def run_gpu_moe(p, block_m, do_finalize=True, debug=True, rsf=1.0):
    wl = p.wl
    pw, lin = runner.prepare_weights(p.w1, p.w2, gated=wl.gated, keep_linear=True)
    fwd = runner.MoeForward(pw, p.M, wl.top_k, wl.E, block_m, wl.local_offset, do_finalize,
                            act=wl.act_code)
    cap = fwd.plan.capacity
    dbg = None
    if debug:
        dbg = dict(preact=torch.full((cap, wl.N1), float("nan"), device="cuda"),
                   inter=torch.zeros((cap, wl.I), dtype=torch.bfloat16, device="cuda"),
                   inter_q=torch.zeros((cap, wl.I // 2), dtype=torch.uint8, device="cuda"),
                   inter_sf=torch.zeros((cap, wl.I // 16), dtype=torch.uint8, device="cuda"))
    res = fwd(p.x, p.ids_d, p.w_d, debug=dbg, routed_scaling_factor=rsf)
    torch.cuda.synchronize()
    return fwd, pw, lin, dbg, res


@pytest.mark.parametrize("name,bm", MOE_CASES, ids=["%s-bm%d" % c for c in MOE_CASES])
def test_fused_moe_matches_oracle(name, bm):
    wl = _workload(name)
    say("fused_moe", name, "block_m", bm)
    p = Problem(wl)
    fwd, pw, lin, dbg, out = run_gpu_moe(p, bm)
    out_bits = np_bits(out)
    M, k = p.M, wl.top_k
    # activations and plan: bit-exact
    oq, osf, odec = p.oracle_activations()
    assert np.array_equal(np_u8(fwd.a_q), oq) and np.array_equal(np_u8(fwd.a_sf), osf)
    assert np.array_equal(fwd.a_dec.cpu().numpy().view(np.uint32), odec.view(np.uint32))
    srt, eids, P, ttr = p.oracle_plan(bm)
    assert int(fwd.plan.num_tokens_post_padded.item()) == P
    assert np.array_equal(fwd.plan.sorted_token_ids.cpu().numpy()[:len(srt)], srt)
    assert np.array_equal(fwd.plan.token_to_row.cpu().numpy(), ttr)
    # weights: the GPU's per-expert quantization is bit-exact for the routed experts
    experts = sorted(set(int(e) for e in eids[:P // bm]))
    for e in experts[:4]:
        (q1, s1, q2, s2), a1, a2 = p.oracle_expert(e)
        assert np.array_equal(np_u8(lin[0][e]), q1) and np.array_equal(np_u8(lin[1][e]), s1)
        assert np.array_equal(np_u8(lin[2][e]), q2) and np.array_equal(np_u8(lin[3][e]), s2)
        assert pw.alpha1_gate[e].item() == a1 and pw.alpha2[e].item() == a2
    # oracle forward with its own quantized weights
    a1, a2 = p.oracle_alphas(experts)
    act = wl.act_code
    res = oracle.fused_moe_nvfp4(oq, osf, odec, lambda e: p.oracle_expert(e)[0], a1, a1, a2, 1.0,
                                 srt, eids, P, ttr, p.w, k, bm, act)
    rows = sorted(res["pre"].keys())
    # GEMM1 pre-activation
    pre_gpu = dbg["preact"].cpu().numpy()[rows]
    pre_ref = np.stack([res["pre"][r] for r in rows])
    e_pre = rel_fro(pre_gpu, pre_ref)
    # requantization of the GPU's own BF16 intermediate
    inter = np_bits(dbg["inter"])[rows]
    rq, rsf_, _ = oracle.quantize_nvfp4(bf16_bits_to_f32(inter), oracle.SCALE_FIXED, None, 1.0)
    assert np.array_equal(np_u8(dbg["inter_q"])[rows], rq)
    assert np.array_equal(np_u8(dbg["inter_sf"])[rows], rsf_)
    e_h = rel_fro(bf16_bits_to_f32(inter), np.stack([res["h"][r] for r in rows]))
    # final output
    out_ref = bf16_bits_to_f32(res["out"]).astype(np.float64)
    e_out = rel_fro(bf16_bits_to_f32(out_bits), out_ref)
    # NVFP4 vs unquantized FP64 gap of the oracle itself (reported)
    ref64 = oracle.unquantized_moe_f64(p.x_bits, lambda e: p.host_weight_bits(e)[0],
                                       lambda e: p.host_weight_bits(e)[1], p.ids, p.w, wl.E,
                                       wl.local_offset, wl.n_local, act)
    ref64 = np.stack([ref64[t] for t in range(M)])
    gap = rel_fro(out_ref, ref64)
    say("pre %.3e  h %.3e  out %.3e  oracle-vs-fp64 gap %.3f" % (e_pre, e_h, e_out, gap))
    assert e_pre <= 1e-5
    # the activation itself: both sides round act(pre) to BF16 from pre-activations 1e-5 apart,
    # so an element differs by at most one BF16 step (2^-8 relative) and rarely; 2e-3 would take
    # a quarter of the elements a step apart, a wrong activation is ~1e-1 off
    assert e_h <= 2e-3
    assert e_out <= 2e-2
    # unfinalized triple -> finalize == finalized, bit for bit; run-twice determinism
    fwd2 = runner.MoeForward(pw, p.M, k, wl.E, bm, wl.local_offset, do_finalize=False,
                             act=wl.act_code)
    cap = fwd2.plan.capacity
    dbg2 = dict(inter_q=torch.zeros((cap, wl.I // 2), dtype=torch.uint8, device="cuda"),
                inter_sf=torch.zeros((cap, wl.I // 16), dtype=torch.uint8, device="cuda"))
    if bm > 32:
        dbg2["inter_f16"] = torch.full((cap, wl.I), float("nan"), dtype=torch.float16,
                                       device="cuda")
    y, wts, ttr_d = fwd2(p.x, p.ids_d, p.w_d, debug=dbg2)
    torch.cuda.synchronize()
    assert np.array_equal(np_u8(dbg2["inter_q"])[rows], np_u8(dbg["inter_q"])[rows])
    # GEMM2 on its own: the expert outputs against the oracle's down projection of the GPU's own
    # requantized intermediate, every routed row (and the tiled kernels' FP16 operand is the
    # exact decode of that intermediate)
    check_gemm2(p, eids, bm, rows, dbg2, y)
    out2 = torch.zeros_like(out)
    bf.bfp4_moe_finalize(y, wts, runner.weights_dtype(wts), ttr_d, M, wl.H, k, 1.0, out2)
    torch.cuda.synchronize()
    assert np.array_equal(np_bits(out2), out_bits)
    # the combine of the GPU's own expert outputs is the oracle's combine, bit for bit
    ttr_np = ttr_d.cpu().numpy()
    ybits = np_bits(y)
    ydict = {int(r): bf16_bits_to_f32(ybits[r]).astype(np.float64) for r in ttr_np.reshape(-1) if r >= 0}
    comb = oracle.combine(np.zeros((M, wl.H), np.uint16), ydict, p.w, ttr_np)
    assert np.array_equal(comb, out_bits)
    out3 = fwd(p.x, p.ids_d, p.w_d)
    torch.cuda.synchronize()
    assert np.array_equal(np_bits(out3), out_bits)


def test_out_accumulates_and_rsf():
    wl = WORKLOADS["tiny"]
    say("out accumulation / routed_scaling_factor")
    p = Problem(wl)
    pw = runner.prepare_weights(p.w1, p.w2)
    fwd = runner.MoeForward(pw, p.M, wl.top_k, wl.E, 8)
    rng = np.random.default_rng(1)
    from synth import bf16_bits
    o0 = bf16_bits(rng.standard_normal((p.M, wl.H)))
    out = torch.from_numpy(o0.view(np.int16)).view(torch.bfloat16).cuda()
    fwd(p.x, p.ids_d, p.w_d, out=out, routed_scaling_factor=0.75)
    fwd2 = runner.MoeForward(pw, p.M, wl.top_k, wl.E, 8, do_finalize=False)
    y, wts, ttr = fwd2(p.x, p.ids_d, p.w_d)
    torch.cuda.synchronize()
    ttr_np = ttr.cpu().numpy()
    ybits = np_bits(y)
    ydict = {int(r): bf16_bits_to_f32(ybits[r]).astype(np.float64) for r in ttr_np.reshape(-1) if r >= 0}
    want = oracle.combine(o0, ydict, p.w, ttr_np, 0.75)
    assert np.array_equal(np_bits(out), want)


@pytest.mark.parametrize("bm", [8, 128])
def test_bf16_routing_weights(bm):
    """BF16 routing weights ([cuDNN] routing weights bullet) combine as their exact FP32 values:
    the finalized output equals the FP32-weight call on those values and the oracle's combine of
    the GPU's expert outputs, bit for bit; the unfinalized triple returns the BF16 weights and
    bfp4_moe_finalize with them reproduces the finalized output."""
    wl = WORKLOADS["tiny"]
    say("bf16 routing weights, block_m", bm)
    p = Problem(wl)
    pw = runner.prepare_weights(p.w1, p.w2)
    w_bf = p.w_d.to(torch.bfloat16)
    w_exact = w_bf.float()
    fwd = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm)
    out_bf = fwd(p.x, p.ids_d, w_bf)
    torch.cuda.synchronize()
    out_f32 = fwd(p.x, p.ids_d, w_exact)
    torch.cuda.synchronize()
    assert torch.equal(out_bf.view(torch.int16), out_f32.view(torch.int16))
    fwd_u = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm, do_finalize=False)
    y, wts, ttr_d = fwd_u(p.x, p.ids_d, w_bf)
    out2 = torch.zeros_like(out_bf)
    bf.bfp4_moe_finalize(y, wts, bf.BFP4_WEIGHTS_BF16, ttr_d, p.M, wl.H, wl.top_k, 1.0, out2)
    torch.cuda.synchronize()
    assert wts.dtype == torch.bfloat16 and torch.equal(wts, w_bf)
    assert torch.equal(out2.view(torch.int16), out_bf.view(torch.int16))
    ttr_np = ttr_d.cpu().numpy()
    ybits = np_bits(y)
    ydict = {int(r): bf16_bits_to_f32(ybits[r]).astype(np.float64)
             for r in ttr_np.reshape(-1) if r >= 0}
    comb = oracle.combine(np.zeros((p.M, wl.H), np.uint16), ydict, w_exact.cpu().numpy(), ttr_np)
    assert np.array_equal(comb, np_bits(out_bf))
    assert np.any(comb != 0)


def test_unpack_routing_bit_exact():
    """bfp4_unpack_routing ([cuDNN] routing weights bullet; [Frost] numerics paragraph: packed
    scores keep their BF16 rounding) equals oracle.unpack_routing bit for bit on every word of a
    random sample and on the edge words (ids -1, -32768, 32767 and past the experts; NaN, infinite,
    subnormal and negative scores); the unpacked routing of the tiny workload then gives the same
    output as the BF16-weight call on the oracle's unpacking of the same words."""
    rng = np.random.default_rng(11)
    M, k = 1000, 7
    words = rng.integers(-(1 << 31), 1 << 31, (M, k), dtype=np.int64)
    edge = np.array([0x3F80FFFF, 0x7FC08000, 0x7F807FFF, 0xFF800010, 0x00010000, 0x80000005,
                     0xBF800100], dtype=np.uint32).view(np.int32)
    words[0] = edge
    words = words.astype(np.int32)
    ids_d = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((M, k), dtype=torch.int16, device="cuda")
    bf.bfp4_unpack_routing(torch.from_numpy(words).cuda(), M, k, ids_d, w_d)
    torch.cuda.synchronize()
    want_ids, want_w = oracle.unpack_routing(words)
    assert np.array_equal(ids_d.cpu().numpy(), want_ids)
    assert np.array_equal(w_d.cpu().numpy().view(np.uint16), want_w)

    wl = WORKLOADS["tiny"]
    p = Problem(wl)
    w_bf16 = np_bits(p.w_d.to(torch.bfloat16)).astype(np.int64)
    packed = ((w_bf16 << 16) | (p.ids.astype(np.int64) & 0xFFFF)).astype(np.uint32).view(np.int32)
    packed[0, 1] = np.uint32(0x7FC0FFFF).view(np.int32)          # an empty slot with a NaN score
    ids_g = torch.empty_like(p.ids_d)
    w_g = torch.empty((p.M, wl.top_k), dtype=torch.bfloat16, device="cuda")
    bf.bfp4_unpack_routing(torch.from_numpy(packed).cuda(), p.M, wl.top_k, ids_g, w_g)
    oid, ow = oracle.unpack_routing(packed)
    pw = runner.prepare_weights(p.w1, p.w2)
    for bm in (8, 128):
        fwd = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm)
        got = fwd(p.x, ids_g, w_g)
        torch.cuda.synchronize()
        got = got.clone()
        want = fwd(p.x, torch.from_numpy(oid).cuda(),
                   torch.from_numpy(ow.view(np.int16)).cuda().view(torch.bfloat16))
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        assert torch.any(got != 0)


def test_masked_slots_nan_weights_and_all_masked_token():
    wl = SMALL_SKEWED
    say("masking with NaN weights")
    p = Problem(wl)
    pw = runner.prepare_weights(p.w1, p.w2, gated=False)
    fwd = runner.MoeForward(pw, p.M, wl.top_k, wl.E, wl.block_m, wl.local_offset)
    base = np_bits(fwd(p.x, p.ids_d, p.w_d))
    loc = p.ids - wl.local_offset
    masked = (loc < 0) | (loc >= wl.n_local)
    assert masked.any()
    w = p.w.copy()
    w[masked] = np.nan
    ids = p.ids.copy()
    ids[0, :] = -1
    w[0, :] = np.inf
    o0 = np.full((p.M, wl.H), 0x3F80, np.uint16)
    out = torch.from_numpy(o0.view(np.int16)).view(torch.bfloat16).cuda()
    fwd(p.x, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), out=out)
    got = np_bits(out)
    torch.cuda.synchronize()
    assert np.all(got[0] == 0x3F80)
    assert np.all(np.isfinite(bf16_bits_to_f32(got)))
    # with all NaNs on masked slots, unmasked tokens match the plain run with out0 = 1.0 added
    fwd_plain = runner.MoeForward(pw, p.M, wl.top_k, wl.E, wl.block_m, wl.local_offset)
    out_b = torch.from_numpy(o0.view(np.int16)).view(torch.bfloat16).cuda()
    fwd_plain(p.x, torch.from_numpy(ids).cuda(), p.w_d, out=out_b)
    torch.cuda.synchronize()
    assert np.array_equal(np_bits(out_b), got)
    assert base.shape == got.shape


# ----------------------------------------------------------------------------- exact GEMM1 case

EXACT_GRID = Workload("exact_grid", M=48, H=2048, I=256, E=4, top_k=2, block_m=8)
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _grid_rows(rng, rows, cols, big_rows, zero_blocks, big_block, pow2):
    """Values on the NVFP4 grid: every 16-value block holds E2M1 values with block scale 1 and
    one element of magnitude 6, except zero_blocks (all zero) and, in big_rows, big_block (block
    scale 448, so the row maximum is 6 * 448); all times 2**pow2."""
    v = _E2M1[rng.integers(0, 8, (rows, cols))] * rng.choice([-1.0, 1.0], (rows, cols))
    v = v.reshape(rows, cols // 16, 16)
    v[:, :, 0] = 6.0 * rng.choice([-1.0, 1.0], (rows, cols // 16))
    for b in zero_blocks:
        v[:, b, :] = 0.0
    for r in big_rows:
        v[r, big_block, :] *= 448.0
    return (v.reshape(rows, cols) * 2.0 ** pow2)


@pytest.mark.parametrize("bm", [8, 128])
def test_gemm1_exact_on_grid(bm):
    """GEMM1 pre-activation bit-exact in a case where FP32 accumulation is exact.

    Activations and W1 lie on the NVFP4 grid with power-of-two token and expert scales (row
    maxima 2688 * 2^-9 and 2688 * 2^-10, so the decode scales are 2^-9 and 2^-10); the scale-448
    blocks of activations (K block 0) and of W1 (K block 1, row 0) meet only zeros, so every
    surviving product is a multiple of 1/4 of magnitude <= 36 and every partial sum over
    K = 2048 is an exact FP32 number in any order.  The GPU's pre-activation must then equal the
    oracle's exact value bit for bit, on the decode (block_m 8) and the tiled (block_m 128)
    kernels."""
    from synth import bf16_bits
    wl = EXACT_GRID
    say("exact GEMM1 on grid, block_m", bm)
    rng = np.random.default_rng(11)
    p = Problem(wl)
    x = _grid_rows(rng, wl.M, wl.H, range(wl.M), [1], 0, -9)
    p.x_bits = bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(p.x_bits).astype(np.float64), x)   # exact in BF16
    p.x = torch.from_numpy(p.x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    w1 = np.stack([_grid_rows(rng, wl.N1, wl.H, [0], [0], 1, -10) for _ in range(wl.E)])
    wb = bf16_bits(w1)
    assert np.array_equal(bf16_bits_to_f32(wb).astype(np.float64), w1)
    p.w1 = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).cuda()
    p._host_w = {}
    fwd, pw, lin, dbg, out = run_gpu_moe(p, bm)
    oq, osf, odec = p.oracle_activations()
    assert np.all(odec == np.float32(2.0 ** -9))
    srt, eids, P, ttr = p.oracle_plan(bm)
    experts = sorted(set(int(e) for e in eids[:P // bm]))
    a1, a2 = p.oracle_alphas(experts)
    assert all(a1[e] == np.float32(2.0 ** -10) for e in experts)
    res = oracle.fused_moe_nvfp4(oq, osf, odec, lambda e: p.oracle_expert(e)[0], a1, a1, a2, 1.0,
                                 srt, eids, P, ttr, p.w, wl.top_k, bm, oracle.ACT_SWIGLU)
    rows = sorted(res["pre"].keys())
    pre_ref = np.stack([res["pre"][r] for r in rows])
    assert np.array_equal(pre_ref.astype(np.float32).astype(np.float64), pre_ref)  # FP32-exact
    pre_gpu = dbg["preact"].cpu().numpy()[rows].astype(np.float64)
    bad = int(np.count_nonzero(pre_gpu != pre_ref))
    say("exact GEMM1 block_m %d: %d of %d pre-activations differ" % (bm, bad, pre_ref.size))
    assert bad == 0


# ----------------------------------------------------------------------------- empty inputs

@pytest.mark.parametrize("bm", [8, 128])
def test_nothing_local_and_empty_batch(bm):
    """No routed slot is local (every expert id below the local range): the plan is empty, out
    keeps its previous contents bit for bit and the unfinalized triple names no row.  M = 0: every
    call succeeds and touches nothing."""
    wl = WORKLOADS["tiny"]
    say("nothing local / empty batch, block_m", bm)
    p = Problem(wl)
    half = wl.E // 2                     # local experts [half, E); every routed id below half
    pw = runner.prepare_weights(p.w1[half:], p.w2[half:], gated=True)
    ids = torch.from_numpy(p.ids % half).cuda()
    fwd = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm, local_expert_offset=half)
    o0 = np.random.default_rng(2).integers(0, 0x3F00, (p.M, wl.H)).astype(np.uint16)
    out = torch.from_numpy(o0.view(np.int16)).view(torch.bfloat16).cuda()
    fwd(p.x, ids, p.w_d, out=out)
    torch.cuda.synchronize()
    assert int(fwd.plan.num_tokens_post_padded.item()) == 0
    assert np.array_equal(np_bits(out), o0)
    fwd_u = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm, local_expert_offset=half,
                              do_finalize=False)
    y, wts, ttr = fwd_u(p.x, ids, p.w_d)
    torch.cuda.synchronize()
    assert np.all(ttr.cpu().numpy() == -1)
    # an empty batch
    fwd0 = runner.MoeForward(pw, 0, wl.top_k, wl.E, bm)
    x0 = torch.empty((0, wl.H), dtype=torch.bfloat16, device="cuda")
    out0 = torch.empty((0, wl.H), dtype=torch.bfloat16, device="cuda")
    fwd0(x0, torch.empty((0, wl.top_k), dtype=torch.int32, device="cuda"),
         torch.empty((0, wl.top_k), dtype=torch.float32, device="cuda"), out=out0)
    torch.cuda.synchronize()
    assert int(fwd0.plan.num_tokens_post_padded.item()) == 0
