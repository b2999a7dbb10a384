"""Pins of the oracle's MXFP4 codec (oracle/mx.py) and of the weight-only forward on MXFP4
weights: the E8M0 code of 1.0 printed on the pages, the format definition, brute force over the
E2M1 grid, grid round trips and the quantization error bound, exact rational arithmetic."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import E2M1_MAGNITUDES, bf16_bits_to_f32
from synth import to_bits


def test_e8m0_decode():
    # vLLM flashinfer_utils page: padded scales are 127, "UE8M0 for 1.0"
    assert oracle.e8m0_decode(np.array([127]))[0] == 1.0
    v = oracle.e8m0_decode(np.arange(255))
    assert np.array_equal(v, np.ldexp(1.0, np.arange(255) - 127))      # pure powers of two
    assert np.isnan(oracle.e8m0_decode(np.array([255]))[0])


def _codes(q):
    return oracle.quant.unpack_codes(q)


def test_quantize_mxfp4_brute_force():
    """Every scale code is floor(log2 amax) - 2 + 127 (frexp); every element code is the nearest
    E2M1 code to x * 2**-X, ties to the even code, magnitudes above 6 saturating."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((6, 128)) * np.exp(rng.uniform(-8, 8, (6, 1)))).astype(np.float32)
    x[0, :32] = 0.0
    x[0, 3] = -0.0
    x[1, 32:64] = np.float32(6.0)                 # block whose amax is exactly on the grid
    q, sf = oracle.quantize_mxfp4(x)
    codes = _codes(q)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                assert sf[r, b] == 0
                assert np.all((codes[r, 32 * b:32 * b + 32] & 7) == 0)
                continue
            m, e = math.frexp(amax)                   # amax = m * 2**e, 0.5 <= m < 1
            X = (e - 1) - 2
            assert sf[r, b] == X + 127
            for i in range(32):
                y = blk[i] * 2.0 ** -X
                # nearest magnitude (ties to the even code), sign bit from the input's sign
                d = np.abs(E2M1_MAGNITUDES - abs(y))
                best = np.flatnonzero(d == d.min())
                want = int(best[0] if len(best) == 1 else best[best % 2 == 0][0])
                if math.copysign(1.0, blk[i]) < 0:
                    want |= 8
                assert codes[r, 32 * b + i] == want, (r, b, i, y)
    assert (codes[0, 3] == 8)                          # sign of -0.0 kept


def test_mxfp4_grid_round_trip_and_error_bound():
    rng = np.random.default_rng(4)
    R, C = 8, 256
    k = rng.integers(-20, 20, (R, C // 32))
    mags = E2M1_MAGNITUDES[rng.integers(0, 8, (R, C))]
    sign = np.where(rng.random((R, C)) < 0.5, -1.0, 1.0)
    x = sign * mags * np.repeat(np.ldexp(1.0, k), 32, axis=1)
    x.reshape(R, C // 32, 32)[:, :, 0] = 6.0 * np.ldexp(1.0, k)      # amax = 6 * 2**k per block
    q, sf = oracle.quantize_mxfp4(x.astype(np.float32))
    assert np.array_equal(oracle.dequantize_mxfp4(q, sf), x)
    assert np.array_equal(sf, (k + 127).astype(np.uint8))
    # arbitrary values: within half an E2M1 step (0.25, 0.5, 1 by magnitude) times 2**X unless
    # saturated (|x| * 2**-X in (6, 8)), then within 2 * 2**X
    y = (rng.standard_normal((R, C)) * 3.0).astype(np.float32)
    q, sf = oracle.quantize_mxfp4(y)
    d = oracle.dequantize_mxfp4(q, sf)
    s = np.repeat(oracle.e8m0_decode(sf), 32, axis=1)
    t = np.abs(y) / s
    half = np.where(t < 2, 0.25, np.where(t < 4, 0.5, 1.0))
    bound = np.where(t > 6, 2.0, half) * s
    assert np.all(np.abs(d - y) <= bound + 1e-30)


def test_w16_forward_on_mxfp4_weights_brute_force():
    """The weight-only forward with MXFP4 weights against exact rational arithmetic."""
    rng = np.random.default_rng(9)
    R, H, I = 2, 64, 32
    x_bits = to_bits(torch.from_numpy(rng.standard_normal((R, H))).to(torch.bfloat16))
    w1 = (rng.standard_normal((2 * I, H)) * 0.05).astype(np.float32)
    w2 = (rng.standard_normal((H, I)) * 0.05).astype(np.float32)
    w1q, w1s = oracle.quantize_mxfp4(w1)
    w2q, w2s = oracle.quantize_mxfp4(w2)
    one = np.float32(1.0)
    o = oracle.expert_rows_forward_w16(x_bits, w1q, w1s, w2q, w2s, one, one, one,
                                       oracle.ACT_SWIGLU, weight_format="mxfp4")

    def exact(q, sf):
        c = _codes(q)
        mag = {0: Fraction(0), 1: Fraction(1, 2), 2: Fraction(1), 3: Fraction(3, 2),
               4: Fraction(2), 5: Fraction(3), 6: Fraction(4), 7: Fraction(6)}
        return [[mag[int(c[r, j]) & 7] * (-1 if c[r, j] & 8 else 1) *
                 Fraction(2) ** (int(sf[r, j // 32]) - 127) for j in range(c.shape[1])]
                for r in range(c.shape[0])]

    W1, W2 = exact(w1q, w1s), exact(w2q, w2s)
    X = [[Fraction(float(v)) for v in row] for row in bf16_bits_to_f32(x_bits)]
    for r in range(R):
        for n in range(2 * I):
            pre = sum(X[r][h] * W1[n][h] for h in range(H))
            assert abs(o["pre"][r, n] - float(pre)) <= 1e-15 * abs(float(pre)) + 1e-300
        for hh in range(H):
            s_ = sum(Fraction(float(o["h"][r, i])) * W2[hh][i] for i in range(I))
            assert abs(o["y"][r, hh] - float(s_)) <= abs(float(s_)) * 2.0 ** -8 * 1.0001 + 1e-300


def test_mxfp4_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_mxfp4(np.zeros((1, 48), np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_mxfp4(np.full((1, 32), np.inf, np.float32))


# ----------------------------------------------------------------------------- MXFP8 activations

E4M3_POS = np.array([oracle.e4m3_decode(np.array([c]))[0] for c in range(0x7F)])   # 0 .. 448


def test_quantize_mxfp8_brute_force():
    """Every scale code is floor(log2 amax) - 8 + 127 (frexp; 8 = the exponent of E4M3's largest
    magnitude 448); every element code is the nearest E4M3 magnitude to |x| * 2**-X with ties to
    the even code, saturating at 448, with the input's sign bit."""
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((6, 128)) * np.exp(rng.uniform(-30, 30, (6, 1)))).astype(np.float32)
    x[0, :32] = 0.0
    x[0, 5] = -0.0
    x[1, 32:64] = np.float32(448.0)               # block whose amax is exactly E4M3's maximum
    x[2, 64] = np.float32(3.75)                   # 3.75 * 2**-X = 480 -> saturates at 448
    x[2, 65:96] = np.float32(0.001)
    q, sf = oracle.quantize_mxfp8(x)
    assert q.shape == x.shape and sf.shape == (6, 4)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                assert sf[r, b] == 0
                assert np.all((q[r, 32 * b:32 * b + 32] & 0x7F) == 0)
                continue
            m, e = math.frexp(amax)                   # amax = m * 2**e, 0.5 <= m < 1
            X = (e - 1) - 8
            assert sf[r, b] == X + 127
            for i in range(32):
                y = abs(blk[i]) * 2.0 ** -X
                d = np.abs(E4M3_POS - y)
                best = np.flatnonzero(d == d.min())
                want = int(best[0] if len(best) == 1 else best[best % 2 == 0][0])
                if math.copysign(1.0, blk[i]) < 0:
                    want |= 0x80
                assert q[r, 32 * b + i] == want, (r, b, i, y)
    assert q[0, 5] == 0x80                             # sign of -0.0 kept
    assert q[2, 64] == 0x7E                            # saturated to 448


def test_mxfp8_elements_match_torch_float8():
    """Element codes equal torch's float8_e4m3fn conversion of x * 2**-X wherever that value is
    inside E4M3's range (torch rounds to nearest even; above 448 the oracle saturates)."""
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((64, 256)) * 3.0).astype(np.float32)
    q, sf = oracle.quantize_mxfp8(x)
    X = np.repeat(sf.astype(np.int64) - 127, 32, axis=1)
    y = (x.astype(np.float64) * np.ldexp(1.0, -X))
    inside = np.abs(y) <= 448.0
    t = torch.from_numpy(y[inside]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q[inside], t)
    assert inside.mean() > 0.9


def test_mxfp8_grid_round_trip_and_error_bound():
    rng = np.random.default_rng(33)
    R, C = 8, 256
    k = rng.integers(-30, 30, (R, C // 32))
    codes = rng.integers(0, 0x7F, (R, C))
    sign = np.where(rng.random((R, C)) < 0.5, -1.0, 1.0)
    x = sign * E4M3_POS[codes] * np.repeat(np.ldexp(1.0, k), 32, axis=1)
    x.reshape(R, C // 32, 32)[:, :, 0] = 448.0 * np.ldexp(1.0, k)     # amax = 448 * 2**k
    q, sf = oracle.quantize_mxfp8(x.astype(np.float32))
    assert np.array_equal(oracle.dequantize_mxfp8(q, sf), x)
    assert np.array_equal(sf, (k + 127).astype(np.uint8))
    # arbitrary values: within half an E4M3 step at their magnitude unless saturated
    y = (rng.standard_normal((R, C)) * 3.0).astype(np.float32)
    q, sf = oracle.quantize_mxfp8(y)
    d = oracle.dequantize_mxfp8(q, sf)
    s = np.repeat(oracle.e8m0_decode(sf), 32, axis=1)
    t = np.abs(y) / s
    step = np.ldexp(1.0, (np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 3).astype(np.int64))
    bound = np.where(t > 448, t - 448 + 1e-9, step / 2) * s
    assert np.all(np.abs(d - y) <= bound + 1e-30)


def _exact_mx(q, sf, fmt):
    """Fractions of an MX operand: element values from explicit tables, scales 2**(code-127)."""
    if fmt == "fp4":
        c = _codes(q)
        mag = {0: Fraction(0), 1: Fraction(1, 2), 2: Fraction(1), 3: Fraction(3, 2),
               4: Fraction(2), 5: Fraction(3), 6: Fraction(4), 7: Fraction(6)}
        val = lambda r, j: mag[int(c[r, j]) & 7] * (-1 if c[r, j] & 8 else 1)   # noqa: E731
        ncol = c.shape[1]
    else:
        tv = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        val = lambda r, j: Fraction(float(tv[r, j]))                           # noqa: E731
        ncol = q.shape[1]
    return [[val(r, j) * Fraction(2) ** (int(sf[r, j // 32]) - 127) for j in range(ncol)]
            for r in range(q.shape[0])]


def test_mx_dot_exact_with_wide_exponents():
    """mx_dot returns the exact sum rounded once: blocks whose scales lie far apart (beyond what
    a plain float64 sum would keep) are summed correctly as well."""
    rng = np.random.default_rng(34)
    a = (rng.standard_normal((3, 128)) * np.exp(rng.uniform(-40, 40, (3, 128)))).astype(np.float32)
    w = (rng.standard_normal((5, 128)) * 0.1).astype(np.float32)
    aq, asf = oracle.quantize_mxfp8(a)
    wq, wsf = oracle.quantize_mxfp4(w)
    from oracle.mx import mx_dot, mxfp4_int, mxfp8_int
    got = mx_dot(*mxfp8_int(aq, asf), *mxfp4_int(wq, wsf))
    A = _exact_mx(aq, asf, "fp8")
    W = _exact_mx(wq, wsf, "fp4")
    for r in range(3):
        for n in range(5):
            exact = sum(A[r][h] * W[n][h] for h in range(128))
            assert got[r, n] == float(exact), (r, n)


@pytest.mark.parametrize("act", [oracle.ACT_SWIGLU, oracle.ACT_RELU2, oracle.ACT_GELU])
def test_mx_expert_forward_brute_force(act):
    """MXFP4-weight x MXFP8-activation expert against exact rational arithmetic: the activation
    codec of the rows, pre exactly, h the BF16 rounding of the activation, the intermediate's
    MXFP8 codec, y the BF16 rounding of the exact down projection of that intermediate."""
    rng = np.random.default_rng(35 + act)
    R, H, I = 2, 64, 32
    gated = oracle.is_gated(act)
    N1 = 2 * I if gated else I
    x_bits = to_bits(torch.from_numpy(rng.standard_normal((R, H))).to(torch.bfloat16))
    w1q, w1s = oracle.quantize_mxfp4((rng.standard_normal((N1, H)) * 0.1).astype(np.float32))
    w2q, w2s = oracle.quantize_mxfp4((rng.standard_normal((H, I)) * 0.1).astype(np.float32))
    o = oracle.expert_rows_forward_mx(x_bits, w1q, w1s, w2q, w2s, act)
    aq, asf = oracle.quantize_mxfp8(bf16_bits_to_f32(x_bits))
    assert np.array_equal(o["a_q"], aq) and np.array_equal(o["a_sf"], asf)
    A, W1, W2 = _exact_mx(aq, asf, "fp8"), _exact_mx(w1q, w1s, "fp4"), _exact_mx(w2q, w2s, "fp4")
    silu = lambda v: v / (1 + math.exp(-v))                                      # noqa: E731
    gelu = lambda v: v * 0.5 * (1 + math.erf(v / math.sqrt(2)))                  # noqa: E731
    for r in range(R):
        pre = [sum(A[r][h] * W1[n][h] for h in range(H)) for n in range(N1)]
        for n in range(N1):
            assert o["pre"][r, n] == float(pre[n])
        for i in range(I):
            g = float(pre[i])
            ref = {oracle.ACT_SWIGLU: lambda: silu(g) * float(pre[I + i]),
                   oracle.ACT_RELU2: lambda: max(g, 0.0) ** 2,
                   oracle.ACT_GELU: lambda: gelu(g)}[act]()
            assert abs(o["h"][r, i] - ref) <= abs(ref) * 2.0 ** -8 * 1.0001 + 1e-300
    hq, hsf = oracle.quantize_mxfp8(o["h"].astype(np.float32))
    assert np.array_equal(o["hq"], hq) and np.array_equal(o["hsf"], hsf)
    HQ = _exact_mx(hq, hsf, "fp8")
    for r in range(R):
        for hh in range(H):
            s_ = sum(HQ[r][i] * W2[hh][i] for i in range(I))
            assert o["y"][r, hh] == oracle.round_to_bf16(np.array([float(s_)]))[0]


def _mx_problem(wl, seed=0):
    from synth import make_activations, make_routing
    rng = np.random.default_rng(seed + 100)
    x_bits = make_activations(wl, seed)
    ids, w = make_routing(wl, seed)
    N1 = 2 * wl.I if wl.gated else wl.I
    ws = []
    for e in range(wl.n_local):
        w1 = (rng.standard_normal((N1, wl.H)) * 0.02).astype(np.float32)
        w2 = (rng.standard_normal((wl.H, wl.I)) * 0.02).astype(np.float32)
        ws.append(oracle.quantize_mxfp4(w1) + oracle.quantize_mxfp4(w2))
    return x_bits, ids, w, (lambda e: ws[e])


@pytest.mark.parametrize("wl_name", ["tiny", "skewed_small"])
def test_mx_plan_path_equals_dense_loop_and_padding(wl_name):
    """The plan-driven MX forward equals the per-token loop bit for bit, and padding rows
    contribute nothing (block_m 8 and 128 give the same output)."""
    from synth import WORKLOADS
    from synth.workloads import Workload
    wl = WORKLOADS["tiny"] if wl_name == "tiny" else Workload(
        "skewed_small", M=24, H=256, I=128, E=12, top_k=3, block_m=16, act="relu2",
        routing="zipf", local_offset=2, num_local=6)
    x_bits, ids, w, get = _mx_problem(wl)
    outs = []
    for bm in (8, 128):
        srt, eids, P, ttr = oracle.moe_plan(ids, wl.E, wl.local_offset, wl.n_local, bm)
        outs.append(oracle.fused_moe_mx(x_bits, get, srt, eids, P, ttr, w, wl.top_k, bm,
                                        wl.act_code)["out"])
    dense = oracle.dense_loop_moe_mx(x_bits, get, ids, w, wl.E, wl.local_offset, wl.n_local,
                                     wl.act_code)
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0], dense)
    assert np.any(dense != 0)
