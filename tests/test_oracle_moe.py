"""Pins of the oracle's plan, permutation, expert projections, activation and combine.

Sources by page title: "flashinfer.fused_moe.alphamoe_nvfp4_aligned_moe" (aligned plan arrays,
[gate; up] row order, per-expert output scales, accumulation into out),
"flashinfer.fused_moe.CudnnGroupedGemmNvfp4Config" (expert-sorted permutation, segments padded,
masking of non-local experts, unfinalized triple, distinct experts per token),
"flashinfer.fused_moe.FrostLowLatencyConfig" (BF16 intermediate and expert outputs, ordered
separate FP32 multiply/add combine, unrouted slots ignored with their scores),
Megatron-Core "core.inference.moe.flashinfer_nvfp4" (-1 routing entries contribute zero).
"""

import dataclasses
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import bf16_bits_to_f32
from synth import WORKLOADS, make_activations, make_routing, make_weights, to_bits
from synth.workloads import Workload

GOLDEN_COMBINE = os.path.join(os.path.dirname(__file__), "golden", "combine_order.txt")
GOLDEN_PACKED = os.path.join(os.path.dirname(__file__), "golden", "packed_routing.txt")


# ----------------------------------------------------------------------------- plan

def _plan_bruteforce(ids, E, off, nloc, bm):
    """Stable argsort of the local expert id over the flat slot index (a different algorithm)."""
    flat = ids.reshape(-1).astype(np.int64)
    loc = flat - off
    ok = (flat >= 0) & (flat < E) & (loc >= 0) & (loc < nloc)
    key = np.where(ok, loc, nloc)                        # unrouted slots sort last
    order = np.argsort(key, kind="stable")
    order = order[ok[order]]
    rows, eids = [], []
    for e in range(nloc):
        seg = [int(f) for f in order if loc[f] == e]
        if not seg:
            continue
        pad = -len(seg) % bm
        rows += seg + [flat.size] * pad
        eids += [e] * ((len(seg) + pad) // bm)
    return rows, eids


@pytest.mark.parametrize("bm", [8, 16, 128])
@pytest.mark.parametrize("off,nloc", [(0, 8), (2, 4), (6, 2)])
def test_plan_matches_bruteforce(bm, off, nloc):
    rng = np.random.default_rng(bm + off)
    M, k, E = 37, 3, 8
    ids = np.stack([rng.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
    ids[3, 1] = -1
    ids[5, 0] = 99
    srt, eids, P, ttr = oracle.moe_plan(ids, E, off, nloc, bm)
    rows, beids = _plan_bruteforce(ids, E, off, nloc, bm)
    cap = oracle.plan_capacity(M, k, nloc, bm)
    assert srt.shape == (cap,) and eids.shape == (cap // bm,)
    assert P == len(rows) <= cap and P % bm == 0
    assert list(srt[:P]) == rows
    assert np.all(srt[P:] == M * k)
    assert list(eids[:P // bm]) == beids and np.all(eids[P // bm:] == -1)
    # token_to_row inverts the plan; unrouted slots are -1
    for t in range(M):
        for j in range(k):
            r = ttr[t, j]
            loc = ids[t, j] - off
            if 0 <= ids[t, j] < E and 0 <= loc < nloc:
                assert srt[r] == t * k + j and eids[r // bm] == loc
            else:
                assert r == -1


def test_plan_capacity_is_tight_upper_bound():
    # every non-empty expert needs bm-1 padding rows: the bound is reached
    M, k, bm = 8, 1, 8
    ids = np.arange(8, dtype=np.int32).reshape(8, 1)
    _, _, P, _ = oracle.moe_plan(ids, 8, 0, 8, bm)
    assert P == oracle.plan_capacity(M, k, 8, bm) == 64


def test_plan_empty_and_all_masked():
    ids = np.full((4, 2), -1, dtype=np.int32)
    srt, eids, P, ttr = oracle.moe_plan(ids, 8, 0, 8, 8)
    assert P == 0 and np.all(ttr == -1) and np.all(eids == -1)
    srt, eids, P, ttr = oracle.moe_plan(np.zeros((0, 2), np.int32), 8, 0, 8, 8)
    assert P == 0 and srt.shape == (0,)


def test_generator_topk_distinct():
    for name in ("tiny", "decode_ll", "decode", "prefill"):
        ids, w = make_routing(WORKLOADS[name])
        s = np.sort(ids, axis=1)
        assert np.all(s[:, 1:] != s[:, :-1]), name
        assert np.allclose(w.sum(axis=1), 1, atol=1e-6)
    ids, w = make_routing(WORKLOADS["skewed_relu2"], M=2048)
    s = np.sort(ids, axis=1)
    assert np.all(s[:, 1:] != s[:, :-1])
    assert ids.min() >= 0 and ids.max() < 288


def test_routing_violations_pins():
    """Hand-counted example; the generated routings of every workload are clean; and on random
    small id matrices the counts equal a second formulation (sorted rows, adjacent equal ids)."""
    ids = np.array([[0, 1], [2, 2], [-1, -1], [5, -3], [3, 3], [-1, 0]], np.int32)
    # token 1 and token 4 repeat an id; ids 5 and -3 (token 3) are outside [-1, 4)
    assert oracle.routing_violations(ids, 4) == (2, 2, 1)
    assert oracle.routing_violations(np.array([[-1, -1]], np.int32), 4) == (0, 0, None)
    assert oracle.routing_violations(np.array([[0, 7]], np.int32), 4) == (0, 1, 0)
    assert oracle.routing_violations(np.zeros((0, 3), np.int32), 4) == (0, 0, None)
    for name, wl in WORKLOADS.items():
        r, _ = make_routing(wl, M=min(wl.M, 2048))
        assert oracle.routing_violations(r, wl.E) == (0, 0, None), name
    rng = np.random.default_rng(3)
    for _ in range(20):
        E = int(rng.integers(2, 9))
        ids = rng.integers(-3, E + 3, size=(50, 4)).astype(np.int32)
        inr = (ids >= 0) & (ids < E)
        s_ = np.sort(np.where(inr, ids, -10 - np.arange(4)), axis=1)   # out-of-range ids distinct
        dup = np.any(s_[:, 1:] == s_[:, :-1], axis=1)
        bad = (ids < -1) | (ids >= E)
        bad_tok = bad.any(axis=1)
        flagged = np.nonzero(dup | bad_tok)[0]
        first = int(flagged[0]) if flagged.size else None
        assert oracle.routing_violations(ids, E) == (int(dup.sum()), int(bad.sum()), first)


def test_plan_violations_pins():
    """Every oracle plan is clean; each planted breach is counted once, and entries at or past
    the extent are not looked at."""
    rng = np.random.default_rng(4)
    for bm, off, nloc in ((8, 0, 8), (16, 2, 4), (128, 0, 8)):
        M, k, E = 37, 3, 8
        ids = np.stack([rng.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
        srt, eids, P, _ = oracle.moe_plan(ids, E, off, nloc, bm)
        cap = oracle.plan_capacity(M, k, nloc, bm)
        assert oracle.plan_violations(srt, eids, P, cap, M, k, nloc, bm) == (0, 0, 0)
    M, k, nloc, bm = 37, 3, 8, 8
    ids = np.stack([rng.permutation(8)[:k] for _ in range(M)]).astype(np.int32)
    srt, eids, P, _ = oracle.moe_plan(ids, 8, 0, nloc, bm)
    cap = oracle.plan_capacity(M, k, nloc, bm)
    assert P < cap
    s2, e2 = srt.copy(), eids.copy()
    s2[0], s2[P - 1] = -1, M * k + 1                  # two bad entries inside the extent
    s2[P] = -7                                        # past the extent: not counted
    e2[1] = nloc                                      # one bad block inside the extent
    e2[P // bm] = 99                                  # past the extent: not counted
    assert oracle.plan_violations(s2, e2, P, cap, M, k, nloc, bm) == (2, 1, 0)
    # bad extents: not a multiple of block_m (checked below P rounded down), above capacity
    # (checked below capacity), negative (nothing checked)
    assert oracle.plan_violations(s2, e2, P + 3, cap, M, k, nloc, bm) == (2, 1, 1)
    # past the real extent the blocks hold -1, so each of them counts
    assert oracle.plan_violations(s2, e2, cap + bm, cap, M, k, nloc, bm) == \
        (3, 1 + (cap - P) // bm, 1)
    assert oracle.plan_violations(s2, e2, -bm, cap, M, k, nloc, bm) == (0, 0, 1)


def test_permute_rows():
    rng = np.random.default_rng(2)
    M, k = 6, 2
    q = rng.integers(0, 256, (M, 8), dtype=np.uint8)
    sf = rng.integers(1, 127, (M, 1), dtype=np.uint8)
    s = rng.uniform(0.1, 1, M).astype(np.float32)
    ids = np.array([[0, 1], [1, 2], [2, 0], [0, 3], [3, 1], [2, 3]], np.int32)
    srt, eids, P, ttr = oracle.moe_plan(ids, 4, 0, 4, 4)
    qp, sp, spd = oracle.moe_permute(q, sf, s, srt, P, k)
    for r in range(srt.shape[0]):
        f = srt[r]
        if r < P and f < M * k:
            assert np.array_equal(qp[r], q[f // k]) and sp[r, 0] == sf[f // k, 0] and spd[r] == s[f // k]
        else:
            assert not qp[r].any() and not sp[r].any() and spd[r] == 0


# ----------------------------------------------------------------------------- experts

def _rand_nvfp4(rng, R, C):
    q = rng.integers(0, 256, (R, C // 2), dtype=np.uint8)
    sf = rng.integers(0x10, 0x60, (R, C // 16), dtype=np.uint8)
    return q, sf


def _exact_matrix(q, sf):
    """Fractions from an explicit E2M1 dict and torch's float8_e4m3fn decode of the scales."""
    e2m1 = {0: Fraction(0), 1: Fraction(1, 2), 2: Fraction(1), 3: Fraction(3, 2), 4: Fraction(2),
            5: Fraction(3), 6: Fraction(4), 7: Fraction(6)}
    sfv = torch.from_numpy(sf.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    R, Ch = q.shape
    out = []
    for r in range(R):
        row = []
        for c in range(2 * Ch):
            byte = int(q[r, c // 2])
            code = byte & 0xF if c % 2 == 0 else byte >> 4
            v = e2m1[code & 7] * (-1 if code & 8 else 1)
            row.append(v * Fraction(float(sfv[r, c // 16])))
        out.append(row)
    return out


def _act_ref(act, g, u=None):
    """Textbook activations on one float (math module only): silu(x) = x / (1 + e^-x),
    gelu(x) = x * Phi(x) with Phi(x) = (1 + erf(x / sqrt 2)) / 2."""
    silu = lambda x: x / (1 + math.exp(-x))                       # noqa: E731
    gelu = lambda x: x * 0.5 * (1 + math.erf(x / math.sqrt(2)))    # noqa: E731
    return {oracle.ACT_SWIGLU: lambda: silu(g) * u, oracle.ACT_GEGLU: lambda: gelu(g) * u,
            oracle.ACT_RELU2: lambda: max(g, 0.0) ** 2, oracle.ACT_RELU: lambda: max(g, 0.0),
            oracle.ACT_SILU: lambda: silu(g), oracle.ACT_GELU: lambda: gelu(g),
            oracle.ACT_IDENTITY: lambda: g}[act]()


@pytest.mark.parametrize("act", oracle.ACTS)
def test_expert_projection_brute_force(act):
    """pre, h and y against exact rational arithmetic on a tiny expert (H=32, I=16)."""
    rng = np.random.default_rng(11 + act)
    R, H, I = 3, 32, 16
    gated = oracle.is_gated(act)
    N1 = 2 * I if gated else I
    aq, asf = _rand_nvfp4(rng, R, H)
    w1q, w1sf = _rand_nvfp4(rng, N1, H)
    w2q, w2sf = _rand_nvfp4(rng, H, I)
    adec = rng.uniform(0.01, 0.1, R).astype(np.float32)
    ag, au, a2 = np.float32(0.003), np.float32(0.005), np.float32(0.007)
    o = oracle.expert_rows_forward(aq, asf, adec, w1q, w1sf, w2q, w2sf, ag, au, a2, 1.0, act)
    A = _exact_matrix(aq, asf)
    W1 = _exact_matrix(w1q, w1sf)
    for r in range(R):
        pre = []
        for n in range(N1):
            s = sum(A[r][h] * W1[n][h] for h in range(H))
            alpha = (ag if n < I else au) if gated else au
            pre.append(s * Fraction(float(adec[r])) * Fraction(float(alpha)))
        got = o["pre"][r]
        for n in range(N1):
            assert abs(got[n] - float(pre[n])) <= 4e-16 * abs(float(pre[n])) + 1e-300
        # activation from the exact pre-activation with math.exp: gate rows first, then up
        for i in range(I):
            h = _act_ref(act, float(pre[i]), float(pre[I + i]) if gated else None)
            hb = o["h"][r, i]
            assert abs(hb - h) <= abs(h) * 2.0 ** -8 * 1.0001 + 1e-300
    # the intermediate is requantized with the fixed encode scale 1 (CudnnGroupedGemmNvfp4Config,
    # permutation bullet): block scale = E4M3(fl32(bmax / 6)), elements = E2M1(h / scale)
    hb32 = o["h"].astype(np.float32)
    bmax = np.abs(hb32.reshape(R, -1, 16)).max(axis=2)
    assert np.array_equal(o["hsf"], oracle.e4m3_encode((bmax / np.float32(6)).astype(np.float32)))
    deq = oracle.dequantize_nvfp4(o["hq"], o["hsf"])
    sfv = np.repeat(oracle.e4m3_decode(o["hsf"]), 16, axis=1)
    # within one E2M1 step of the block scale; a zero block scale only when bmax/6 rounds to 0
    bound = np.where(sfv == 0, 6 * 2.0 ** -10, sfv)
    assert np.all(np.abs(deq - o["h"]) <= bound)
    # y from the oracle's own requantized intermediate, exactly
    HQ = _exact_matrix(o["hq"], o["hsf"])
    W2 = _exact_matrix(w2q, w2sf)
    for r in range(R):
        for hh in range(H):
            s = sum(HQ[r][i] * W2[hh][i] for i in range(I)) * Fraction(float(a2))
            ref = float(s)
            assert abs(o["y"][r, hh] - ref) <= abs(ref) * 2.0 ** -8 * 1.0001 + 1e-300


def _bf16_rne(v):
    """Exact round-to-nearest-even of a Fraction onto the BF16 grid (8 significant bits)."""
    if v == 0:
        return Fraction(0)
    m = abs(v)
    e = m.numerator.bit_length() - m.denominator.bit_length()     # 2^e <= m < 2^(e+2)
    if Fraction(2) ** e > m:
        e -= 1
    if Fraction(2) ** (e + 1) <= m:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    r = round(m / ulp) * ulp                                      # Fraction round: half to even
    return r if v > 0 else -r


@pytest.mark.parametrize("c2", [1.0, 0.37, 3.0])
def test_expert_down_projection_brute_force(c2):
    """GEMM2 on its own: y[r, k] = bf16(sum_i deq(hq[r, i]) deq(w2[k, i]) * fl32(1 / c2) *
    alpha2) against exact rational arithmetic, the BF16 rounding done exactly on the rational
    value; c2 != 1 pins the decode factor of the intermediate's fixed scale, and the [H, I]
    orientation of W2 (output k reads W2 row k) is fixed by its non-square shape."""
    rng = np.random.default_rng(23)
    R, H, I = 3, 48, 32
    hq, hsf = _rand_nvfp4(rng, R, I)
    w2q, w2sf = _rand_nvfp4(rng, H, I)
    a2 = np.float32(0.0071)
    y = oracle.expert_down_projection(hq, hsf, w2q, w2sf, a2, c2)
    assert y.shape == (R, H)
    HQ = _exact_matrix(hq, hsf)
    W2 = _exact_matrix(w2q, w2sf)
    dec = Fraction(float(np.float32(1) / np.float32(c2)))
    for r in range(R):
        for k in range(H):
            exact = sum(HQ[r][i] * W2[k][i] for i in range(I)) * dec * Fraction(float(a2))
            assert Fraction(float(y[r, k])) == _bf16_rne(exact), (r, k)
    # the same step inside the whole expert forward
    aq, asf = _rand_nvfp4(rng, R, H)
    w1q, w1sf = _rand_nvfp4(rng, 2 * I, H)
    o = oracle.expert_rows_forward(aq, asf, np.full(R, 0.05, np.float32), w1q, w1sf, w2q, w2sf,
                                   np.float32(0.004), np.float32(0.004), a2, c2, oracle.ACT_SWIGLU)
    assert np.array_equal(o["y"], oracle.expert_down_projection(o["hq"], o["hsf"], w2q, w2sf, a2,
                                                                c2))


def test_gate_up_projection_on_row_subsets():
    """GEMM1 on a subset of W1's rows (with their per-row scales) equals the same columns of the
    whole expert's pre-activation, and the row scales multiply their own columns only."""
    rng = np.random.default_rng(29)
    R, H, I = 4, 64, 32
    aq, asf = _rand_nvfp4(rng, R, H)
    w1q, w1sf = _rand_nvfp4(rng, 2 * I, H)
    w2q, w2sf = _rand_nvfp4(rng, H, I)
    adec = rng.uniform(0.01, 0.1, R).astype(np.float32)
    ag, au = np.float32(0.003), np.float32(0.005)
    o = oracle.expert_rows_forward(aq, asf, adec, w1q, w1sf, w2q, w2sf, ag, au, np.float32(1),
                                   1.0, oracle.ACT_SWIGLU)
    cols = np.array([0, 7, I - 1, I, I + 5, 2 * I - 1])
    alpha_rows = np.where(cols < I, ag, au)
    sub = oracle.expert_gate_up_projection(aq, asf, adec, w1q[cols], w1sf[cols], alpha_rows)
    assert np.array_equal(sub, o["pre"][:, cols])
    ones = oracle.expert_gate_up_projection(aq, asf, adec, w1q[cols], w1sf[cols], np.ones(6))
    assert np.array_equal(ones * alpha_rows.astype(np.float64), sub)


def test_activation_closed_forms():
    """Values of the typed activations fixed by their definitions: Phi(1) = 0.841344746068543,
    Phi(2) = 0.977249868051821 (standard normal CDF); the odd parts gelu(x) - gelu(-x) = x and
    silu(x) - silu(-x) = x; logistic(1) = 1 / (1 + 1/e); gated forms take the gate half first."""
    act = oracle.moe._activation
    x = np.array([[1.0, -1.0, 2.0, 0.0, 10.0]])
    assert np.allclose(act(x, 5, oracle.ACT_GELU),
                       [[0.8413447460685429, -0.15865525393145707, 1.9544997361036416, 0.0, 10.0]],
                       rtol=1e-15, atol=0)
    assert np.allclose(act(x, 5, oracle.ACT_SILU)[0, 0], 0.7310585786300049, rtol=1e-15)
    v = np.linspace(-8, 8, 33).reshape(1, -1)
    for a in (oracle.ACT_GELU, oracle.ACT_SILU):
        assert np.allclose(act(v, 33, a) - act(-v, 33, a), v, rtol=1e-14, atol=1e-14)
    assert np.array_equal(act(v, 33, oracle.ACT_RELU), np.maximum(v, 0))
    assert np.array_equal(act(v, 33, oracle.ACT_RELU2), np.maximum(v, 0) ** 2)
    assert np.array_equal(act(v, 33, oracle.ACT_IDENTITY), v)
    gu = np.array([[1.0, 3.0]])                  # I = 1: gate 1, up 3
    assert np.isclose(act(gu, 1, oracle.ACT_SWIGLU)[0, 0], 3 * 0.7310585786300049, rtol=1e-15)
    assert np.isclose(act(gu, 1, oracle.ACT_GEGLU)[0, 0], 3 * 0.8413447460685429, rtol=1e-15)
    assert np.isclose(act(gu[:, ::-1], 1, oracle.ACT_GEGLU)[0, 0], 0.9986501019683699 * 3,
                      rtol=1e-15)                # gelu(3) * 1 = 3 Phi(3)
    with pytest.raises(ValueError):
        act(v, 33, 7)


def test_gemm1_exact_grid_case():
    """Grid-valued operands with unit scales: the pre-activation is an exactly representable sum."""
    rng = np.random.default_rng(12)
    H, I = 64, 16
    aq = rng.integers(0, 256, (2, H // 2), dtype=np.uint8)
    asf = np.full((2, H // 16), 0x38, np.uint8)                 # E4M3 1.0
    w1q = rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8)
    w1sf = np.full((2 * I, H // 16), 0x38, np.uint8)
    w2q = rng.integers(0, 256, (H, I // 2), dtype=np.uint8)
    w2sf = np.full((H, I // 16), 0x38, np.uint8)
    o = oracle.expert_rows_forward(aq, asf, np.ones(2, np.float32), w1q, w1sf, w2q, w2sf,
                                   1.0, 1.0, 1.0, 1.0, oracle.ACT_SWIGLU)
    a = oracle.e2m1_decode(oracle.quant.unpack_codes(aq))
    w = oracle.e2m1_decode(oracle.quant.unpack_codes(w1q))
    exact = np.array([[math.fsum(a[r] * w[n]) for n in range(2 * I)] for r in range(2)])
    assert np.array_equal(o["pre"], exact)


def _small_problem(wl, seed=0, M=None):
    M = wl.M if M is None else M
    x = make_activations(wl, seed, M)
    ids, w = make_routing(wl, seed, M)
    w1, w2 = make_weights(wl, seed, "cpu")
    w1q, w1sf, a1 = oracle.quantize_expert_weights(to_bits(w1))
    w2q, w2sf, a2 = oracle.quantize_expert_weights(to_bits(w2))
    aq, asf, adec = oracle.quantize_nvfp4(bf16_bits_to_f32(x), oracle.SCALE_PER_ROW)
    return dict(x=x, ids=ids, w=w, w1=w1, w2=w2, W=(w1q, w1sf, w2q, w2sf), a1=a1, a2=a2,
                aq=aq, asf=asf, adec=adec, M=M)


def _run(wl, p, bm, out0=None, ids=None, w=None, rsf=1.0):
    ids = p["ids"] if ids is None else ids
    w = p["w"] if w is None else w
    act = wl.act_code
    srt, eids, P, ttr = oracle.moe_plan(ids, wl.E, wl.local_offset, wl.n_local, bm)
    return oracle.fused_moe_nvfp4(p["aq"], p["asf"], p["adec"], p["W"], p["a1"], p["a1"], p["a2"],
                                  1.0, srt, eids, P, ttr, w, wl.top_k, bm, act, rsf, out0)


SHRUNK_SKEWED = Workload("skewed_small", M=48, H=128, I=64, E=24, top_k=4, block_m=16,
                         act="relu2", routing="zipf", local_offset=4, num_local=12)


ACT_VARIANTS = [WORKLOADS["tiny"], SHRUNK_SKEWED,
                dataclasses.replace(WORKLOADS["tiny"], name="tiny_geglu", act="geglu"),
                dataclasses.replace(SHRUNK_SKEWED, name="skewed_gelu", act="gelu"),
                dataclasses.replace(SHRUNK_SKEWED, name="skewed_silu", act="silu"),
                dataclasses.replace(SHRUNK_SKEWED, name="skewed_relu", act="relu"),
                dataclasses.replace(SHRUNK_SKEWED, name="skewed_identity", act="identity")]


@pytest.mark.parametrize("wl", ACT_VARIANTS, ids=[w.name for w in ACT_VARIANTS])
def test_dense_loop_equals_plan_path(wl):
    p = _small_problem(wl)
    act = wl.act_code
    res = _run(wl, p, wl.block_m)
    dense = oracle.dense_loop_moe(p["aq"], p["asf"], p["adec"], p["W"], p["a1"], p["a1"], p["a2"],
                                  1.0, p["ids"], p["w"], wl.E, wl.local_offset, wl.n_local, act)
    assert np.array_equal(res["out"], dense)
    assert np.any(res["out"] != 0)


def test_padding_rows_contribute_nothing():
    wl = WORKLOADS["tiny"]
    p = _small_problem(wl)
    outs = [_run(wl, p, bm)["out"] for bm in (8, 16, 32, 128)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_masked_slots_ignored_with_nan_weights():
    wl = SHRUNK_SKEWED
    p = _small_problem(wl)
    base = _run(wl, p, wl.block_m)["out"]
    w = p["w"].copy()
    loc = p["ids"] - wl.local_offset
    masked = (loc < 0) | (loc >= wl.n_local)
    assert masked.any()
    w[masked] = np.nan
    w[np.nonzero(masked)[0][:1], np.nonzero(masked)[1][:1]] = np.inf
    assert np.array_equal(_run(wl, p, wl.block_m, w=w)["out"], base)
    # a token whose slots are all unrouted keeps out0
    ids = p["ids"].copy()
    ids[0, :] = -1
    out0 = np.full((wl.M, wl.H), 0x3F80, np.uint16)
    res = _run(wl, p, wl.block_m, out0=out0, ids=ids)
    assert np.all(res["out"][0] == 0x3F80)


def test_out_accumulation_and_combine_closed_form():
    wl = WORKLOADS["tiny"]
    p = _small_problem(wl)
    res0 = _run(wl, p, 8)
    rng = np.random.default_rng(9)
    out0 = to_bits(torch.from_numpy(rng.standard_normal((wl.M, wl.H)).astype(np.float32)).to(torch.bfloat16))
    res1 = _run(wl, p, 8, out0=out0)
    # closed form of the ordered FP32 combine, token by token
    y, w, ttr = res1["unfinalized"]
    for t in range(wl.M):
        acc = bf16_bits_to_f32(out0[t]).copy()
        for j in range(wl.top_k):
            acc = acc + np.float32(w[t, j]) * y[ttr[t, j]].astype(np.float32)
        want = oracle.f64_to_bf16_bits(acc.astype(np.float64))
        assert np.array_equal(res1["out"][t], want)
    assert not np.array_equal(res0["out"], res1["out"])
    # finalize(unfinalized) reproduces the finalized output
    again = oracle.combine(out0, y, w, ttr)
    assert np.array_equal(again, res1["out"])


def test_routed_scaling_factor_placement():
    wl = WORKLOADS["tiny"]
    p = _small_problem(wl)
    r2 = _run(wl, p, 8, rsf=2.0)["out"]
    r1 = _run(wl, p, 8)["out"]
    # multiplying every product by 2 in FP32 is exact, so the result doubles exactly
    assert np.array_equal(bf16_bits_to_f32(r2), 2 * bf16_bits_to_f32(r1))


def test_token_permutation_equivariance():
    wl = WORKLOADS["tiny"]
    p = _small_problem(wl)
    base = _run(wl, p, 8)["out"]
    perm = np.random.default_rng(5).permutation(wl.M)
    q = dict(p, aq=p["aq"][perm], asf=p["asf"][perm], adec=p["adec"][perm])
    res = _run(wl, q, 8, ids=p["ids"][perm], w=p["w"][perm])
    assert np.array_equal(res["out"], base[perm])


def test_golden_combine_order():
    slots, outs = [], {}
    for line in open(GOLDEN_COMBINE):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        if parts[0] == "slot":
            slots.append(parts[1:])
        else:
            outs[int(parts[1])] = int(parts[2], 16)
    M, k = 3, 3
    ttr = np.full((M, k), -1, np.int64)
    w = np.zeros((M, k), np.float32)
    y = {}
    for t, j, r, wh, yh in slots:
        t, j, r = int(t), int(j), int(r)
        ttr[t, j] = r
        w[t, j] = np.array([int(wh, 16)], np.uint32).view(np.float32)[0]
        if r >= 0:
            y[r] = bf16_bits_to_f32(np.array([int(yh, 16)], np.uint16)).astype(np.float64)
    out = oracle.combine(np.zeros((M, 1), np.uint16), y, w, ttr)
    for t in range(M):
        assert int(out[t, 0]) == outs[t], t


def test_gap_to_unquantized_reference():
    """The NVFP4 result stays close to the unquantized float64 MoE (three ~1-bit operands)."""
    wl = WORKLOADS["tiny"]
    p = _small_problem(wl)
    out = bf16_bits_to_f32(_run(wl, p, 8)["out"]).astype(np.float64)
    w1b, w2b = to_bits(p["w1"]), to_bits(p["w2"])
    ref = oracle.unquantized_moe_f64(p["x"], lambda e: w1b[e], lambda e: w2b[e], p["ids"], p["w"],
                                     wl.E, 0, wl.n_local, oracle.ACT_SWIGLU)
    ref = np.stack([ref[t] for t in range(wl.M)])
    gap = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert 0.02 < gap < 0.35, gap


# ----------------------------------------------------------------------------- weight-only mode

@pytest.mark.parametrize("act", [oracle.ACT_SWIGLU, oracle.ACT_GEGLU, oracle.ACT_RELU2,
                                 oracle.ACT_IDENTITY])
def test_w16_expert_brute_force(act):
    """NVFP4 weight-only expert on BF16 rows (FrostLowLatencyConfig, FP4 weight-only paragraph)
    against exact rational arithmetic: pre from Fractions of the BF16 inputs and the exactly
    decoded weights; the BF16 rounding of pre and of the activation; y from the oracle's own
    BF16 intermediate, exactly."""
    rng = np.random.default_rng(31 + act)
    R, H, I = 3, 32, 16
    gated = oracle.is_gated(act)
    N1 = 2 * I if gated else I
    x_bits = to_bits(torch.from_numpy(rng.standard_normal((R, H))).to(torch.bfloat16))
    w1q, w1sf = _rand_nvfp4(rng, N1, H)
    w2q, w2sf = _rand_nvfp4(rng, H, I)
    ag, au, a2 = np.float32(0.03), np.float32(0.05), np.float32(0.07)
    o = oracle.expert_rows_forward_w16(x_bits, w1q, w1sf, w2q, w2sf, ag, au, a2, act)
    X = [[Fraction(float(v)) for v in row] for row in bf16_bits_to_f32(x_bits)]
    W1 = _exact_matrix(w1q, w1sf)
    W2 = _exact_matrix(w2q, w2sf)
    for r in range(R):
        pre = [sum(X[r][h] * W1[n][h] for h in range(H)) *
               Fraction(float((ag if n < I else au) if gated else au)) for n in range(N1)]
        for n in range(N1):
            assert abs(o["pre"][r, n] - float(pre[n])) <= 1e-15 * abs(float(pre[n])) + 1e-300
            # pre-activation rounded to BF16: within half a BF16 step of the exact value
            assert abs(o["pre_b"][r, n] - float(pre[n])) <= abs(float(pre[n])) * 2.0 ** -8 + 1e-300
            assert o["pre_b"][r, n] == oracle.round_to_bf16(np.array([float(pre[n])]))[0]
        for i in range(I):
            h = _act_ref(act, float(o["pre_b"][r, i]),
                         float(o["pre_b"][r, I + i]) if gated else None)
            assert abs(o["h"][r, i] - h) <= abs(h) * 2.0 ** -8 * 1.0001 + 1e-300
        for hh in range(H):
            s = sum(Fraction(float(o["h"][r, i])) * W2[hh][i] for i in range(I)) * Fraction(float(a2))
            assert abs(o["y"][r, hh] - float(s)) <= abs(float(s)) * 2.0 ** -8 * 1.0001 + 1e-300
    # every rounded value is a BF16 value
    for k in ("pre_b", "h", "y"):
        v = o[k].astype(np.float32)
        assert np.array_equal(v.view(np.uint32) & 0xFFFF, np.zeros_like(v.view(np.uint32)))


def test_w16_unit_vector_reads_weight_column():
    """A BF16 row equal to the unit vector e_k gives pre = alpha1 * W1[:, k] (exact), and with the
    identity activation and alpha = 1 the intermediate is the BF16 of that column."""
    rng = np.random.default_rng(7)
    H, I = 64, 16
    w1q, w1sf = _rand_nvfp4(rng, I, H)
    w2q, w2sf = _rand_nvfp4(rng, H, I)
    w1 = oracle.dequantize_nvfp4(w1q, w1sf)
    for k in (0, 17, 63):
        x = np.zeros((1, H))
        x[0, k] = 1.0
        o = oracle.expert_rows_forward_w16(oracle.f64_to_bf16_bits(x), w1q, w1sf, w2q, w2sf,
                                           np.float32(1), np.float32(1), np.float32(1),
                                           oracle.ACT_IDENTITY)
        assert np.array_equal(o["pre"][0], w1[:, k])
        assert np.array_equal(o["h"][0], w1[:, k])          # E2M1 x E4M3 values are BF16 values


@pytest.mark.parametrize("wl", [WORKLOADS["tiny"], SHRUNK_SKEWED], ids=["tiny", "skewed_small"])
def test_w16_plan_path_equals_per_token_loop(wl):
    """The plan-driven weight-only forward equals a per-token loop over the routed slots (each
    slot's row through its expert, then the ordered combine), and block_m 8 / 16 / 32 give the
    same output bit for bit (padding rows contribute nothing)."""
    p = _small_problem(wl)
    act = wl.act_code
    outs = []
    for bm in (8, 16, 32):
        srt, eids, P, ttr = oracle.moe_plan(p["ids"], wl.E, wl.local_offset, wl.n_local, bm)
        res = oracle.fused_moe_w4a16(p["x"], p["W"], p["a1"], p["a1"], p["a2"], srt, eids, P, ttr,
                                     p["w"], wl.top_k, bm, act)
        outs.append(res["out"])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # per-token loop
    M, k = p["ids"].shape
    get = lambda e: (p["W"][0][e], p["W"][1][e], p["W"][2][e], p["W"][3][e])   # noqa: E731
    acc = np.zeros((M, wl.H), np.float32)
    for t in range(M):
        for j in range(k):
            e = int(p["ids"][t, j]) - wl.local_offset
            if not (0 <= int(p["ids"][t, j]) < wl.E and 0 <= e < wl.n_local):
                continue
            o = oracle.expert_rows_forward_w16(p["x"][t:t + 1], *get(e), p["a1"][e], p["a1"][e],
                                               p["a2"][e], act)
            prod = np.float32(p["w"][t, j]) * o["y"][0].astype(np.float32)
            acc[t] = (acc[t] + prod).astype(np.float32)
    dense = oracle.f64_to_bf16_bits(acc.astype(np.float64))
    assert np.array_equal(outs[0], dense)
    assert np.any(outs[0] != 0)


def test_golden_packed_routing():
    """oracle.unpack_routing against hand-derived words (tests/golden/packed_routing.txt): ids
    sign-extended from the low 16 bits, BF16 score bits from the high 16, values as written."""
    rows = []
    with open(GOLDEN_PACKED) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                w, e, sb, v = line.split()
                rows.append((int(w, 16), int(e), int(sb, 16), float(v)))
    words = np.array([r[0] for r in rows], dtype=np.uint32).view(np.int32).reshape(1, -1)
    ids, scores = oracle.unpack_routing(words)
    assert ids.dtype == np.int32 and scores.dtype == np.uint16
    assert ids.tolist() == [[r[1] for r in rows]]
    assert scores.tolist() == [[r[2] for r in rows]]
    vals = bf16_bits_to_f32(scores[0])
    for got, (_, _, _, want) in zip(vals, rows):
        assert (np.isnan(got) and np.isnan(want)) or got == want

