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
