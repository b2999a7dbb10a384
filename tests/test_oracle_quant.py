"""Pins of the oracle's NVFP4 quantizer.

* tests/golden/nvfp4_pack_example.txt: hand-derived bytes, scales and decode scales (format
  constants from Megatron-Core "core.inference.moe.flashinfer_nvfp4"; nibble order and linear
  per-16 scales from "flashinfer.fused_moe.alphamoe_nvfp4_aligned_moe"; decode-scale return from
  vLLM "flashinfer_utils" quantize_nvfp4_per_token_input).
* Lossless round trip for values that already lie on the NVFP4 grid.
* Error bound for random values: half the E2M1 spacing times the block scale, except where the
  block maximum saturates at 6 after E4M3 rounding of the block scale.
"""

import os

import numpy as np
import pytest

import oracle
from oracle.quant import dequantize_int, unpack_codes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_pack_example.txt")


def _read_golden():
    rows = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tag, idx, _, *rest = line.split()
        rows.setdefault(int(idx), {})[tag] = rest
    return rows


def test_golden_pack_example():
    g = _read_golden()
    x0 = np.array([float(v) for v in g[0]["x"]], dtype=np.float32)
    xs = {0: x0, 1: np.array([float(v) for v in g[1]["x"]], dtype=np.float32)}
    assert g[2]["x"][0] == "scaled"
    xs[2] = (xs[int(g[2]["x"][1])] * np.float32(2.0 ** int(g[2]["x"][2]))).astype(np.float32)
    x = np.stack([xs[0], xs[1], xs[2]])
    q, sf, dec = oracle.quantize_nvfp4(x, oracle.SCALE_PER_ROW)
    for r in range(3):
        assert [int(b, 16) for b in g[r]["q"]] == list(q[r]), r
        assert [int(b, 16) for b in g[r]["sf"]] == list(sf[r]), r
        num, den, ex = (int(v) for v in g[r]["dec"])
        want = (np.float32(num) / np.float32(den)) * np.float32(2.0 ** ex)
        assert dec[r] == want, r
    # -0.0 keeps its sign bit (code 0x8) even in an all-zero block
    assert q[0, 31] == 0x80


def _grid_row(rng, C, p):
    """A row whose values lie on the NVFP4 grid with encode scale exactly 2**p (see below)."""
    nb = C // 16
    e4 = oracle.e4m3_decode(np.arange(0x7F))
    codes = rng.integers(0, 16, size=(nb, 16))
    bscale = e4[rng.integers(1, 0x7F, size=nb)]                # nonzero E4M3 block scales
    bscale[0] = 448.0                                          # the row maximum block
    codes[0, 0] = 7                                            # |6| in the maximum block
    for b in range(nb):                                        # each block reaches its max
        codes[b, 1] = 7 | (codes[b, 1] & 8)
    vals = oracle.e2m1_decode(codes) * bscale[:, None] * 2.0 ** -p
    return vals.reshape(-1).astype(np.float32)


@pytest.mark.parametrize("p", [0, 3, -5])
def test_round_trip_lossless_on_grid(p):
    rng = np.random.default_rng(p + 10)
    x = np.stack([_grid_row(rng, 256, p) for _ in range(6)])
    q, sf, dec = oracle.quantize_nvfp4(x, oracle.SCALE_PER_ROW)
    back = oracle.dequantize_nvfp4(q, sf, dec)
    assert np.array_equal(back, x.astype(np.float64))
    assert np.all(dec == np.float32(2.0 ** -p) / np.float32(448 * 6 / 2688))   # = 2**-p exactly


def test_error_bound_random():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 512)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    q, sf, dec = oracle.quantize_nvfp4(x, oracle.SCALE_PER_ROW)
    back = oracle.dequantize_nvfp4(q, sf, dec)
    sfv = np.repeat(oracle.e4m3_decode(sf), 16, axis=1) * dec[:, None]
    y = np.abs(x.astype(np.float64)) / sfv                     # position on the E2M1 grid
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, 6])
    idx = np.clip(np.searchsorted(grid, y) - 1, 0, 7)
    half_gap = (grid[idx + 1] - grid[idx]) / 2
    half_gap = np.where(y >= 6, y - 6, half_gap)               # saturated elements
    err = np.abs(back - x)
    assert np.all(err <= half_gap * sfv * (1 + 1e-6) + 1e-30)
    # the block scale never exceeds bmax/6 by more than half an E4M3 step
    bmax = np.abs(x.reshape(64, -1, 16)).max(axis=2)
    assert np.all(oracle.e4m3_decode(sf) * dec[:, None] <= bmax / 6 * (1 + 1 / 16) * (1 + 1e-6))


def test_per_group_equals_per_row_for_single_row_groups():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    a = oracle.quantize_nvfp4(x, oracle.SCALE_PER_ROW)
    b = oracle.quantize_nvfp4(x, oracle.SCALE_PER_GROUP, group_rows=1)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_per_group_uses_group_amax():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 32)).astype(np.float32)
    x[4, 7] = 50.0
    q, sf, dec = oracle.quantize_nvfp4(x, oracle.SCALE_PER_GROUP, group_rows=3)
    assert dec.shape == (2,)
    assert dec[1] == np.float32(1) / (np.float32(2688) / np.float32(50.0))
    assert dec[0] == np.float32(1) / (np.float32(2688) / np.float32(np.abs(x[:3]).max()))


def test_fixed_scale_mode():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 32)).astype(np.float32)
    q, sf, dec = oracle.quantize_nvfp4(x, oracle.SCALE_FIXED, fixed_encode_scale=1.0)
    assert dec.shape == (1,) and dec[0] == 1.0
    # with encode scale 1 the block scale is fl32(bmax/6)
    bmax = np.abs(x.reshape(4, 2, 16)).max(axis=2)
    assert np.array_equal(sf, oracle.e4m3_encode((bmax / np.float32(6)).astype(np.float32)))


def test_dequantize_int_is_exact():
    rng = np.random.default_rng(7)
    q = rng.integers(0, 256, (5, 16), dtype=np.uint8)
    sf = rng.integers(0, 0x7F, (5, 2), dtype=np.uint8)
    n = dequantize_int(q, sf)
    assert np.array_equal(n.astype(np.float64) * 2.0 ** -10, oracle.dequantize_nvfp4(q, sf))
    assert np.abs(n).max() < 2 ** 22


def test_unpack_even_value_low_nibble():
    codes = unpack_codes(np.array([[0x21, 0xF7]], dtype=np.uint8))
    assert list(codes[0]) == [1, 2, 7, 15]


def test_expert_rows_subset_matches_whole_matrix():
    """Quantizing selected rows with the whole matrix's scale equals slicing the full result."""
    rng = np.random.default_rng(8)
    from synth import bf16_bits
    w = bf16_bits(rng.standard_normal((64, 128)) * 0.02)
    q, sf, a = oracle.quantize_expert_weights(w[None])
    rows = [3, 17, 40, 63]
    q2, sf2, a2 = oracle.quantize_expert_rows(w, rows)
    assert np.array_equal(q2, q[0, rows]) and np.array_equal(sf2, sf[0, rows]) and a2 == a[0]
    # the largest magnitude negative, in a row that is not selected, next to BF16 subnormals
    w[9, 5] = bf16_bits(np.array([-0.75]))[0]
    w[2, :4] = bf16_bits(np.array([1e-40, -1e-40, 3e-39, 0.0]))
    q, sf, a = oracle.quantize_expert_weights(w[None])
    q2, sf2, a2 = oracle.quantize_expert_rows(w, rows + [2])
    assert a2 == a[0] and a2 == np.float32(1) / (np.float32(2688) / np.float32(0.75))
    assert np.array_equal(q2, q[0, rows + [2]]) and np.array_equal(sf2, sf[0, rows + [2]])
