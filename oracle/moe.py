"""Routing plan, permutation, the two expert projections, activation, requantization, combine.

Test infrastructure (see the package docstring).  Everything is float64 except the rounding
points the pages name (BF16 intermediate and expert outputs, FP32 combine), which are applied
exactly.  The projections are computed exactly: every dequantized operand is an integer times
2**-10 (quant.dequantize_int), so a dot product is an exact int64 sum times 2**-20, rounded once
to float64.
"""

import numpy as np

from .formats import bf16_bits_to_f32, round_to_bf16
from .quant import SCALE_FIXED, SCALE_PER_GROUP, dequantize_int, quantize_nvfp4

# Typed activations.  CudnnGroupedGemmNvfp4Config, activation bullet: SwiGLU with default
# scalars, GeGLU, GELU, ReLU, SiLU and Identity; Megatron-Core flashinfer_nvfp4: squared ReLU.
# The two GLU forms are gated (W1 rows [gate; up], N1 = 2 I); the others take one projection.
ACT_SWIGLU = 0
ACT_RELU2 = 1
ACT_GEGLU = 2
ACT_GELU = 3
ACT_RELU = 4
ACT_SILU = 5
ACT_IDENTITY = 6
ACTS = (ACT_SWIGLU, ACT_RELU2, ACT_GEGLU, ACT_GELU, ACT_RELU, ACT_SILU, ACT_IDENTITY)


def is_gated(act):
    return act in (ACT_SWIGLU, ACT_GEGLU)

_TWO_M20 = 2.0 ** -20


def _round_up(v, a):
    return (v + a - 1) // a * a


def plan_capacity(M, top_k, num_local_experts, block_m):
    """Largest plan extent any routing can produce (capacity of the plan arrays).

    Each non-empty local segment adds at most block_m - 1 padding rows, and at most
    min(num_local_experts, M * top_k) segments are non-empty.
    """
    A = M * top_k
    return _round_up(A + min(num_local_experts, A) * (block_m - 1), block_m)


def moe_plan(topk_ids, num_experts, local_expert_offset, num_local_experts, block_m):
    """The aligned expert-sorted routing plan (alphamoe_nvfp4_aligned_moe page, plan paragraph).

    A slot (t, j) is routed to this device when its expert id lies in
    [local_expert_offset, local_expert_offset + num_local_experts) (CudnnGroupedGemmNvfp4Config:
    non-local assignments are masked out; FrostLowLatencyConfig: ids outside the routed range mark
    unrouted slots; Megatron-Core: -1 entries contribute zero).  Readings taken where the pages
    leave the plan open:
    * segments in ascending local expert id; each padded to a multiple of block_m; empty experts
      get no blocks;
    * a plan entry is the flat slot index f = t * top_k + j, ascending inside a segment;
      padding entries and entries in [extent, capacity) hold the sentinel M * top_k;
    * expert_ids[b] is the local expert id of block b, -1 past the extent;
    * token_to_row[t, j] is the plan position of slot (t, j), -1 for unrouted slots.
    Returns (sorted_token_ids int32 [cap], expert_ids int32 [cap/block_m],
             num_tokens_post_padded int, token_to_row int32 [M, top_k]).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    M, k = ids.shape
    cap = plan_capacity(M, k, num_local_experts, block_m)
    sentinel = M * k
    flat = ids.reshape(-1)
    local = flat - local_expert_offset
    valid = (flat >= 0) & (flat < num_experts) & (local >= 0) & (local < num_local_experts)
    sorted_ids = np.full(cap, sentinel, dtype=np.int64)
    expert_ids = np.full(cap // block_m if block_m else 0, -1, dtype=np.int64)
    token_to_row = np.full(M * k, -1, dtype=np.int64)
    pos = 0
    for e in range(num_local_experts):
        fs = np.nonzero(valid & (local == e))[0]          # ascending flat indices
        if len(fs) == 0:
            continue
        seg = _round_up(len(fs), block_m)
        sorted_ids[pos:pos + len(fs)] = fs
        token_to_row[fs] = pos + np.arange(len(fs))
        expert_ids[pos // block_m:(pos + seg) // block_m] = e
        pos += seg
    return (sorted_ids.astype(np.int32), expert_ids.astype(np.int32), int(pos),
            token_to_row.reshape(M, k).astype(np.int32))


def unpack_routing(packed):
    """Packed routing slots -> (topk_ids int32, topk_weights as BF16 bit patterns uint16).

    CudnnGroupedGemmNvfp4Config, routing weights bullet, accepts routing weights packed as well as
    unpacked; FrostLowLatencyConfig, numerics paragraph, says packed routing scores keep their BF16
    rounding.  Neither page gives the bit layout.  Reading used here: one 32-bit word per
    (token, slot), the score's BF16 bits in the high 16 bits and the expert id as a two's-complement
    16-bit integer in the low 16 bits (so an empty slot, id -1, has low half 0xFFFF).  The id is
    sign-extended; the score bits are returned unchanged (their value is the exact FP32 of a BF16,
    which the combine then uses as it does for unpacked BF16 weights).
    """
    w = np.asarray(packed).astype(np.int64) & 0xFFFFFFFF
    low = w & 0xFFFF
    ids = np.where(low >= 0x8000, low - 0x10000, low).astype(np.int32)
    scores = (w >> 16).astype(np.uint16)
    return ids, scores


def routing_violations(topk_ids, num_experts):
    """Breaches of the routing's preconditions (CudnnGroupedGemmNvfp4Config, topk_ids bullet:
    each token's top_k experts are distinct; -1 marks an empty slot).

    Returns (number of tokens holding some id >= 0 more than once,
             number of ids outside [-1, num_experts),
             smallest token index counted in either, or None).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    dup_tokens, bad_ids, first = 0, 0, None
    for t in range(ids.shape[0]):
        row = [int(v) for v in ids[t]]
        bad = sum(1 for v in row if v < -1 or v >= num_experts)
        ok = [v for v in row if 0 <= v < num_experts]
        dup = len(set(ok)) < len(ok)
        dup_tokens += int(dup)
        bad_ids += bad
        if (dup or bad) and first is None:
            first = t
    return dup_tokens, bad_ids, first


def plan_violations(sorted_token_ids, expert_ids, num_tokens_post_padded, capacity, M, top_k,
                    num_local_experts, block_m):
    """Breaches of what the fused computation requires of a pre-aligned plan it did not build
    (alphamoe_nvfp4_aligned_moe page, plan paragraph and parameters): entries name a flat slot
    f < M * top_k or the padding sentinel M * top_k, every block names a local expert, and the
    extent num_tokens_post_padded is a multiple of block_m within the capacity.

    Returns (entries below the extent outside [0, M * top_k],
             blocks below the extent whose expert id is outside [0, num_local_experts),
             1 if the extent is negative, above capacity or not a multiple of block_m, else 0).
    With a bad extent, entries and blocks are checked below the extent clamped to
    [0, capacity] and rounded down to a multiple of block_m.
    """
    P = int(num_tokens_post_padded)
    bad_extent = int(not (0 <= P <= capacity and P % block_m == 0))
    ext = (min(max(P, 0), capacity) // block_m) * block_m
    sentinel = M * top_k
    bad_entries = sum(1 for f in np.asarray(sorted_token_ids[:ext], dtype=np.int64)
                      if not 0 <= int(f) <= sentinel)
    bad_blocks = sum(1 for e in np.asarray(expert_ids[:ext // block_m], dtype=np.int64)
                     if not 0 <= int(e) < num_local_experts)
    return bad_entries, bad_blocks, bad_extent


def moe_permute(q, sf, dec_scale, sorted_token_ids, num_tokens_post_padded, top_k):
    """Gather quantized token rows into plan order (CudnnGroupedGemmNvfp4Config: rows and scale
    rows are permuted into expert order).  Row r < extent takes token f // top_k of its entry f;
    sentinel rows and rows past the extent are all-zero bytes with scale 0.
    Returns (q_perm [cap, H/2], sf_perm [cap, H/16], s_perm float32 [cap]).
    """
    q = np.asarray(q)
    sf = np.asarray(sf)
    M = q.shape[0]
    ent = np.asarray(sorted_token_ids, dtype=np.int64)
    cap = ent.shape[0]
    qp = np.zeros((cap, q.shape[1]), dtype=np.uint8)
    sp = np.zeros((cap, sf.shape[1]), dtype=np.uint8)
    s = np.zeros(cap, dtype=np.float32)
    for r in range(min(num_tokens_post_padded, cap)):
        f = ent[r]
        if f < M * top_k:
            t = f // top_k
            qp[r] = q[t]
            sp[r] = sf[t]
            s[r] = dec_scale[t]
    return qp, sp, s


def quantize_expert_weights(w_bf16_bits):
    """Per-expert NVFP4 of a BF16 stack [E, rows, cols]: one encode scale per expert matrix
    (Megatron-Core flashinfer_nvfp4: a single FP32 global scale for each expert;
    _global_encode_scale / _quantize_expert).
    Returns (q [E, rows, cols/2], sf [E, rows, cols/16], alpha float32 [E]) where alpha is the
    decode scale of each expert matrix.
    """
    w = bf16_bits_to_f32(w_bf16_bits)
    E, R, C = w.shape
    q, sf, dec = quantize_nvfp4(w.reshape(E * R, C), SCALE_PER_GROUP, group_rows=R)
    return q.reshape(E, R, C // 2), sf.reshape(E, R, C // 16), dec.astype(np.float32)


def quantize_expert_rows(w_bf16_bits, rows):
    """Selected rows of one expert matrix [R, C] quantized exactly as quantize_expert_weights
    quantizes the whole matrix: the encode scale comes from the amax of the full matrix, and each
    row is then quantized on its own (the per-block steps only read the row).
    Returns (q [len(rows), C/2], sf [len(rows), C/16], alpha)."""
    from .quant import _encode_scale, quantize_rows

    bits = np.asarray(w_bf16_bits, dtype=np.uint16)
    # amax of the whole matrix: for finite BF16 values the magnitude order is the integer order
    # of the 15 low bits, so the largest magnitude is the value of the largest such pattern
    amax = bf16_bits_to_f32(np.array([np.max(bits & np.uint16(0x7FFF))], np.uint16))[0]
    s_enc = _encode_scale(amax)
    sel = bf16_bits_to_f32(bits[np.asarray(rows)])
    q, sf = quantize_rows(sel, np.full(sel.shape[0], s_enc, dtype=np.float32))
    return q, sf, (np.float32(1) / s_enc).astype(np.float32)


def _silu(x):
    """silu(x) = x / (1 + e^-x) (x * logistic(x))."""
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def _gelu(x):
    """GELU in its exact form x * Phi(x) = x / 2 * (1 + erf(x / sqrt(2))), Phi the standard
    normal CDF.  Reading taken: the pages list GELU and GeGLU beside a separate tanh variant
    (GeGLUTanh), so the plain names are the erf form."""
    return 0.5 * x * (1.0 + _erf(x / np.sqrt(2.0)))


def _erf(x):
    from scipy.special import erf

    return erf(x)


def _activation(pre, I, act):
    """Typed activation on float64 pre-activations [rows, N1].

    Gated forms split W1's rows as [gate; up] (alphamoe page: the usual gate-then-up row
    order): SwiGLU with default scalars (CudnnGroupedGemmNvfp4Config activation bullet)
    h = silu(gate) * up; GeGLU h = gelu(gate) * up.  One-projection forms: squared ReLU
    (Megatron-Core module) h = max(pre, 0)**2; ReLU max(pre, 0); SiLU silu(pre); GELU gelu(pre);
    Identity h = pre.
    """
    if act == ACT_SWIGLU:
        return _silu(pre[:, :I]) * pre[:, I:2 * I]
    if act == ACT_GEGLU:
        return _gelu(pre[:, :I]) * pre[:, I:2 * I]
    if act == ACT_RELU2:
        return np.maximum(pre, 0.0) ** 2
    if act == ACT_RELU:
        return np.maximum(pre, 0.0)
    if act == ACT_SILU:
        return _silu(pre)
    if act == ACT_GELU:
        return _gelu(pre)
    if act == ACT_IDENTITY:
        return pre.copy()
    raise ValueError("unknown activation")


def expert_rows_forward(a_q, a_sf, a_dec, w1_q, w1_sf, w2_q, w2_sf, alpha1_gate, alpha1_up,
                        alpha2, c2, act):
    """One expert applied to rows of NVFP4 activations (the rows all route to this expert).

    a_q [R, H/2], a_sf [R, H/16], a_dec float32 [R]; w1 [N1, H/2] / [N1, H/16];
    w2 [H, I/2] / [H, I/16]; alpha1_gate, alpha1_up, alpha2: this expert's FP32 scales.
    Steps (pages' order: GEMM1, typed activation, requantize, GEMM2):
      pre  = (sum_h deq(a) deq(w1)) * a_dec * alpha1   (gate rows * alpha1_gate, up rows *
             alpha1_up: alphamoe page, output1_scale_gate_scalar / output1_scale_scalar)
      h    = activation(pre), rounded to BF16 (FrostLowLatencyConfig: intermediate rounding)
      hq   = NVFP4 of h with fixed encode scale c2 (CudnnGroupedGemmNvfp4Config, permutation
             bullet: the intermediate's global scale is one; c2 = 1 unless a caller folds
             another constant in)
      y    = bf16((sum_i deq(hq) deq(w2)) * dec(c2) * alpha2)  (alphamoe page,
             output2_scale_scalar; expert outputs BF16 per FrostLowLatencyConfig)
    Returns dict(pre float64 [R, N1], h float64 (BF16 values) [R, I], hq, hsf, y float64
    (BF16 values) [R, H]).
    """
    R = a_q.shape[0]
    N1 = w1_q.shape[0]
    I = w2_q.shape[1] * 2
    gated = is_gated(act)
    if N1 != (2 * I if gated else I):
        raise ValueError("W1 rows do not match the activation")
    # Non-gated FC1 has a single projection; it takes the up/FC1 scale (output1_scale_scalar).
    alpha_rows = np.full(N1, float(alpha1_up), dtype=np.float64)
    if gated:
        alpha_rows[:I] = float(alpha1_gate)
    pre = expert_gate_up_projection(a_q, a_sf, a_dec, w1_q, w1_sf, alpha_rows)
    h = round_to_bf16(_activation(pre, I, act))
    hq, hsf, _ = quantize_nvfp4(h.astype(np.float32), SCALE_FIXED, fixed_encode_scale=c2)
    y = expert_down_projection(hq, hsf, w2_q, w2_sf, alpha2, c2)
    return dict(pre=pre, h=h, hq=hq, hsf=hsf, y=y)


def expert_gate_up_projection(a_q, a_sf, a_dec, w1_q, w1_sf, alpha_rows):
    """GEMM1 pre-activation of one expert (the first step of expert_rows_forward, on its own so
    that a caller can take any subset of W1's rows):
      pre[r, n] = (sum_h deq(a[r, h]) deq(w1[n, h])) * a_dec[r] * alpha_rows[n]
    a_q [R, H/2], a_sf [R, H/16], a_dec float32 [R]; w1_q [N, H/2], w1_sf [N, H/16];
    alpha_rows [N]: the FP32 scale of each W1 row (alphamoe page, output1_scale_gate_scalar for
    gate rows, output1_scale_scalar otherwise).  The sum is exact (int64), then two float64
    products.  Returns float64 [R, N].
    """
    R = a_q.shape[0]
    N = w1_q.shape[0]
    s1 = dequantize_int(a_q, a_sf) @ dequantize_int(w1_q, w1_sf).T          # exact int64
    pre = (s1.astype(np.float64) * _TWO_M20) * np.asarray(a_dec, np.float64).reshape(R, 1)
    return pre * np.asarray(alpha_rows, np.float64).reshape(1, N)


def expert_down_projection(hq, hsf, w2_q, w2_sf, alpha2, c2):
    """GEMM2 of one expert on rows of the requantized intermediate (the last step of
    expert_rows_forward, on its own so that a caller can apply it to any NVFP4 intermediate):
      y = bf16((sum_i deq(hq) deq(w2)) * dec(c2) * alpha2)
    with dec(c2) = fl32(1 / c2), the decode scale the fixed-scale quantizer returns for encode
    scale c2 (alphamoe page, output2_scale_scalar; expert outputs rounded to BF16 per
    FrostLowLatencyConfig numerics).  hq [R, I/2], hsf [R, I/16]; w2 [H, I/2] / [H, I/16].
    Returns float64 BF16 values [R, H].
    """
    s2 = dequantize_int(hq, hsf) @ dequantize_int(w2_q, w2_sf).T            # exact int64
    hdec = np.float32(1) / np.float32(c2)
    return round_to_bf16((s2.astype(np.float64) * _TWO_M20) * float(hdec) * float(alpha2))


def combine(out0_bits, y_rows, topk_weights, token_to_row, routed_scaling_factor=1.0):
    """Finalize: out[t] = bf16(f32(out0[t]) (+) sum_j fl32(w[t,j] * y[row(t,j)])).

    FrostLowLatencyConfig numerics: each product and each sum rounded to FP32 on its own, in
    slot order; alphamoe page:
    contributions are added to the existing out values in FP32, converted to BF16 once.
    Reading taken: j ascending; unrouted slots (token_to_row == -1) are skipped and their weights
    never read (FrostLowLatencyConfig: scores of unrouted slots may be NaN/Inf);
    routed_scaling_factor multiplies each product when it is not 1 (alphamoe page: applied to each
    routed contribution); no flush of subnormals.
    y_rows: float64 BF16 values indexed by plan row (dict or array).  Returns uint16 BF16 bits.
    """
    acc = bf16_bits_to_f32(out0_bits).astype(np.float32).copy()
    w = np.asarray(topk_weights, dtype=np.float32)
    ttr = np.asarray(token_to_row)
    M, k = ttr.shape
    rsf = np.float32(routed_scaling_factor)
    for t in range(M):
        for j in range(k):
            r = int(ttr[t, j])
            if r < 0:
                continue
            p = np.float32(w[t, j]) * np.asarray(y_rows[r], dtype=np.float32)     # fp32 product
            if rsf != np.float32(1.0):
                p = (p * rsf).astype(np.float32)
            acc[t] = (acc[t] + p).astype(np.float32)                             # fp32 sum
    r = round_to_bf16(acc.astype(np.float64)).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def _experts_from(weights):
    """Accept either a tuple of stacked arrays or a callable e -> per-expert tuple."""
    if callable(weights):
        return weights

    w1_q, w1_sf, w2_q, w2_sf = weights
    return lambda e: (w1_q[e], w1_sf[e], w2_q[e], w2_sf[e])


def fused_moe_nvfp4(a_q, a_sf, a_dec, weights, alpha1_gate, alpha1_up, alpha2, c2,
                    sorted_token_ids, expert_ids, num_tokens_post_padded, token_to_row,
                    topk_weights, top_k, block_m, act, routed_scaling_factor=1.0, out0_bits=None,
                    do_finalize=True, rows=None):
    """Plan-driven forward: permute, per-block expert compute, finalize (or the unfinalized triple).

    weights: (w1_q [E,N1,H/2], w1_sf [E,N1,H/16], w2_q [E,H,I/2], w2_sf [E,H,I/16]) indexed by
    local expert id, or a callable local id -> that tuple.  ``rows``: optional iterable of plan
    rows to compute (the others are skipped; for sampling large workloads).
    Returns dict(out (uint16 [M,H] or None), y {row: BF16 float64 [H]}, pre {row: [N1]},
    h {row: [I]}, hq {row}, hsf {row}, unfinalized=(y, topk_weights, token_to_row)).
    """
    get = _experts_from(weights)
    M = a_q.shape[0]
    H = a_q.shape[1] * 2
    qp, sp, spd = moe_permute(a_q, a_sf, a_dec, sorted_token_ids, num_tokens_post_padded, top_k)
    ent = np.asarray(sorted_token_ids, dtype=np.int64)
    eids = np.asarray(expert_ids, dtype=np.int64)
    wanted = None if rows is None else set(int(r) for r in rows)
    by_expert = {}
    for b in range(num_tokens_post_padded // block_m):
        e = int(eids[b])
        for r in range(b * block_m, (b + 1) * block_m):
            if ent[r] >= M * top_k:
                continue                                   # padding rows contribute nothing
            if wanted is not None and r not in wanted:
                continue
            by_expert.setdefault(e, []).append(r)
    res = dict(y={}, pre={}, h={}, hq={}, hsf={})
    for e, rs in sorted(by_expert.items()):
        w1q, w1s, w2q, w2s = get(e)
        rs = np.array(rs)
        o = expert_rows_forward(qp[rs], sp[rs], spd[rs], w1q, w1s, w2q, w2s,
                                alpha1_gate[e], alpha1_up[e], alpha2[e], c2, act)
        for i, r in enumerate(rs):
            res["y"][int(r)] = o["y"][i]
            res["pre"][int(r)] = o["pre"][i]
            res["h"][int(r)] = o["h"][i]
            res["hq"][int(r)] = o["hq"][i]
            res["hsf"][int(r)] = o["hsf"][i]
    res["unfinalized"] = (res["y"], np.asarray(topk_weights, np.float32), np.asarray(token_to_row))
    res["out"] = None
    if do_finalize and rows is None:
        if out0_bits is None:
            out0_bits = np.zeros((M, H), dtype=np.uint16)
        res["out"] = combine(out0_bits, res["y"], topk_weights, token_to_row,
                             routed_scaling_factor)
    return res


def dense_loop_moe(a_q, a_sf, a_dec, weights, alpha1_gate, alpha1_up, alpha2, c2, topk_ids,
                   topk_weights, num_experts, local_expert_offset, num_local_experts, act,
                   routed_scaling_factor=1.0, out0_bits=None):
    """Per-token reference with no plan: for each token and each of its slots in order, run the
    routed expert on that token's row and combine (ordered FP32 multiply then add).
    Must equal fused_moe_nvfp4 bit for bit."""
    get = _experts_from(weights)
    M, k = np.asarray(topk_ids).shape
    H = a_q.shape[1] * 2
    acc = bf16_bits_to_f32(np.zeros((M, H), np.uint16) if out0_bits is None else out0_bits)
    acc = acc.astype(np.float32).copy()
    w = np.asarray(topk_weights, dtype=np.float32)
    rsf = np.float32(routed_scaling_factor)
    for t in range(M):
        for j in range(k):
            gid = int(topk_ids[t, j])
            e = gid - local_expert_offset
            if not (0 <= gid < num_experts and 0 <= e < num_local_experts):
                continue
            w1q, w1s, w2q, w2s = get(e)
            o = expert_rows_forward(a_q[t:t + 1], a_sf[t:t + 1], np.asarray(a_dec)[t:t + 1],
                                    w1q, w1s, w2q, w2s, alpha1_gate[e], alpha1_up[e], alpha2[e],
                                    c2, act)
            p = np.float32(w[t, j]) * o["y"][0].astype(np.float32)
            if rsf != np.float32(1.0):
                p = (p * rsf).astype(np.float32)
            acc[t] = (acc[t] + p).astype(np.float32)
    r = round_to_bf16(acc.astype(np.float64)).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def _dequantize_weights(q, sf, weight_format):
    """float64 weights of one matrix: NVFP4 (E4M3 per 16) or MXFP4 (E8M0 per 32)."""
    if weight_format == "nvfp4":
        return dequantize_int(q, sf).astype(np.float64) * 2.0 ** -10
    if weight_format == "mxfp4":
        from .mx import dequantize_mxfp4

        return dequantize_mxfp4(q, sf)
    raise ValueError("unknown weight format")


def expert_rows_forward_w16(x_bits, w1_q, w1_sf, w2_q, w2_sf, alpha1_gate, alpha1_up, alpha2, act,
                            weight_format="nvfp4"):
    """One expert in the NVFP4 weight-only mode on BF16 rows (FrostLowLatencyConfig, FP4
    weight-only paragraph: canonical E2M1 payloads with linear E4M3 K16 scales, BF16 input,
    pre-activation and intermediate rounding, BF16 expert outputs).

    x_bits: BF16 bit patterns [R, H] of the rows routed to this expert.  Steps:
      pre   = (sum_h x deq(W1)) * alpha1            (float64; gate rows alpha1_gate, up rows
                                                     alpha1_up, one-projection alpha1_up)
      pre_b = bf16(pre)                              (pre-activation rounding)
      h     = bf16(activation(pre_b))                (intermediate rounding)
      y     = bf16((sum_i h deq(W2)) * alpha2)       (BF16 expert output)
    Reading taken: the expert's FP32 global weight scale multiplies the sum before the rounding,
    as in the NVFP4 x NVFP4 mode.  Each product of a BF16 value and a dequantized weight is exact
    in float64 and the sums are float64.  weight_format "mxfp4": E8M0 scales per 32 values
    (the same paragraph: MXFP4 uses E8M0 K32 scales, dequantized in FP32; oracle.mx), with the
    alphas as given (1 for MXFP4 weights, which carry no global scale).
    Returns dict(pre, pre_b, h, y) as float64 arrays.
    """
    x = bf16_bits_to_f32(np.asarray(x_bits, np.uint16)).astype(np.float64)
    N1 = w1_q.shape[0]
    I = w2_q.shape[1] * 2
    gated = is_gated(act)
    if N1 != (2 * I if gated else I):
        raise ValueError("W1 rows do not match the activation")
    w1 = _dequantize_weights(w1_q, w1_sf, weight_format)
    w2 = _dequantize_weights(w2_q, w2_sf, weight_format)
    alpha_rows = np.full(N1, float(alpha1_up), dtype=np.float64)
    if gated:
        alpha_rows[:I] = float(alpha1_gate)
    pre = (x @ w1.T) * alpha_rows.reshape(1, N1)
    pre_b = round_to_bf16(pre)
    h = round_to_bf16(_activation(pre_b, I, act))
    y = round_to_bf16((h @ w2.T) * float(alpha2))
    return dict(pre=pre, pre_b=pre_b, h=h, y=y)


def fused_moe_w4a16(x_bits, weights, alpha1_gate, alpha1_up, alpha2, sorted_token_ids,
                    expert_ids, num_tokens_post_padded, token_to_row, topk_weights, top_k, block_m,
                    act, routed_scaling_factor=1.0, out0_bits=None, do_finalize=True,
                    weight_format="nvfp4"):
    """Plan-driven NVFP4 weight-only forward on BF16 activations: every valid plan row r of
    expert e takes token t = entry // top_k through expert_rows_forward_w16, then the same
    ordered combine as the NVFP4 mode (or the unfinalized triple).
    Returns dict(out, y {row}, pre {row}, h {row}, unfinalized)."""
    get = _experts_from(weights)
    xb = np.asarray(x_bits, np.uint16)
    M, H = xb.shape
    ent = np.asarray(sorted_token_ids, dtype=np.int64)
    eids = np.asarray(expert_ids, dtype=np.int64)
    by_expert = {}
    for b in range(num_tokens_post_padded // block_m):
        for r in range(b * block_m, (b + 1) * block_m):
            if ent[r] < M * top_k:                     # padding rows contribute nothing
                by_expert.setdefault(int(eids[b]), []).append(r)
    res = dict(y={}, pre={}, h={})
    for e, rs in sorted(by_expert.items()):
        w1q, w1s, w2q, w2s = get(e)
        rs = np.array(rs)
        o = expert_rows_forward_w16(xb[ent[rs] // top_k], w1q, w1s, w2q, w2s, alpha1_gate[e],
                                    alpha1_up[e], alpha2[e], act, weight_format)
        for i, r in enumerate(rs):
            res["y"][int(r)] = o["y"][i]
            res["pre"][int(r)] = o["pre"][i]
            res["h"][int(r)] = o["h"][i]
    res["unfinalized"] = (res["y"], np.asarray(topk_weights, np.float32), np.asarray(token_to_row))
    res["out"] = None
    if do_finalize:
        if out0_bits is None:
            out0_bits = np.zeros((M, H), dtype=np.uint16)
        res["out"] = combine(out0_bits, res["y"], topk_weights, token_to_row,
                             routed_scaling_factor)
    return res


def expert_rows_forward_mx(x_bits, w1_q, w1_sf, w2_q, w2_sf, act):
    """One expert with MXFP4 weights on MXFP8 activations (FrostLowLatencyConfig, MX paragraph:
    MXFP4 weights with MXFP8 inputs, the same typed activations, BF16 expert outputs, ordered FP32
    combine; an MX intermediate quantization contract of its own).

    x_bits: BF16 bit patterns [R, H] of the rows routed to this expert; w1 [N1, H/2] / [N1, H/32]
    and w2 [H, I/2] / [H, I/32] MXFP4.  Steps (readings taken, mirroring the NVFP4 recipe with the
    MX formats; MX weights carry no FP32 global scale):
      a     = MXFP8 of the rows (oracle.mx.quantize_mxfp8, one E8M0 scale per 32 values of H)
      pre   = sum_h deq(a) deq(W1)          exact, rounded once to float64 (oracle.mx.mx_dot)
      h     = bf16(activation(pre))         (BF16 intermediate, as in the NVFP4 mode)
      hq    = MXFP8 of h                    (the MX intermediate quantization, per 32 values of I)
      y     = bf16(sum_i deq(hq) deq(W2))   (BF16 expert output)
    Returns dict(a_q, a_sf, pre, h, hq, hsf, y).
    """
    from .mx import mx_dot, mxfp4_int, mxfp8_int, quantize_mxfp8

    x = bf16_bits_to_f32(np.asarray(x_bits, np.uint16))
    N1 = w1_q.shape[0]
    I = w2_q.shape[1] * 2
    if N1 != (2 * I if is_gated(act) else I):
        raise ValueError("W1 rows do not match the activation")
    aq, asf = quantize_mxfp8(x)
    pre = mx_dot(*mxfp8_int(aq, asf), *mxfp4_int(w1_q, w1_sf))
    h = round_to_bf16(_activation(pre, I, act))
    hq, hsf = quantize_mxfp8(h.astype(np.float32))
    y = round_to_bf16(mx_dot(*mxfp8_int(hq, hsf), *mxfp4_int(w2_q, w2_sf)))
    return dict(a_q=aq, a_sf=asf, pre=pre, h=h, hq=hq, hsf=hsf, y=y)


def fused_moe_mx(x_bits, weights, sorted_token_ids, expert_ids, num_tokens_post_padded,
                 token_to_row, topk_weights, top_k, block_m, act, routed_scaling_factor=1.0,
                 out0_bits=None, do_finalize=True):
    """Plan-driven forward with MXFP4 weights and MXFP8 activations: every valid plan row r of
    expert e takes token t = entry // top_k through expert_rows_forward_mx, then the ordered
    combine of the NVFP4 mode (or the unfinalized triple).
    weights: (w1_q, w1_sf, w2_q, w2_sf) stacks indexed by local expert, or a callable.
    Returns dict(out, y {row}, pre {row}, h {row}, hq {row}, hsf {row}, unfinalized)."""
    get = _experts_from(weights)
    xb = np.asarray(x_bits, np.uint16)
    M, H = xb.shape
    ent = np.asarray(sorted_token_ids, dtype=np.int64)
    eids = np.asarray(expert_ids, dtype=np.int64)
    by_expert = {}
    for b in range(num_tokens_post_padded // block_m):
        for r in range(b * block_m, (b + 1) * block_m):
            if ent[r] < M * top_k:                     # padding rows contribute nothing
                by_expert.setdefault(int(eids[b]), []).append(r)
    res = dict(y={}, pre={}, h={}, hq={}, hsf={})
    for e, rs in sorted(by_expert.items()):
        w1q, w1s, w2q, w2s = get(e)
        rs = np.array(rs)
        o = expert_rows_forward_mx(xb[ent[rs] // top_k], w1q, w1s, w2q, w2s, act)
        for i, r in enumerate(rs):
            for key in ("y", "pre", "h", "hq", "hsf"):
                res[key][int(r)] = o[key][i]
    res["unfinalized"] = (res["y"], np.asarray(topk_weights, np.float32), np.asarray(token_to_row))
    res["out"] = None
    if do_finalize:
        if out0_bits is None:
            out0_bits = np.zeros((M, H), dtype=np.uint16)
        res["out"] = combine(out0_bits, res["y"], topk_weights, token_to_row,
                             routed_scaling_factor)
    return res


def dense_loop_moe_mx(x_bits, weights, topk_ids, topk_weights, num_experts, local_expert_offset,
                      num_local_experts, act, routed_scaling_factor=1.0):
    """Per-token reference of the MX mode with no plan (each token and slot in order, then the
    ordered combine); must equal fused_moe_mx bit for bit."""
    get = _experts_from(weights)
    xb = np.asarray(x_bits, np.uint16)
    M, k = np.asarray(topk_ids).shape
    acc = np.zeros((M, xb.shape[1]), np.float32)
    w = np.asarray(topk_weights, dtype=np.float32)
    rsf = np.float32(routed_scaling_factor)
    for t in range(M):
        for j in range(k):
            gid = int(topk_ids[t, j])
            e = gid - local_expert_offset
            if not (0 <= gid < num_experts and 0 <= e < num_local_experts):
                continue
            w1q, w1s, w2q, w2s = get(e)
            o = expert_rows_forward_mx(xb[t:t + 1], w1q, w1s, w2q, w2s, act)
            p = np.float32(w[t, j]) * o["y"][0].astype(np.float32)
            if rsf != np.float32(1.0):
                p = (p * rsf).astype(np.float32)
            acc[t] = (acc[t] + p).astype(np.float32)
    r = round_to_bf16(acc.astype(np.float64)).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def unquantized_moe_f64(x_bits, w1_bits_of, w2_bits_of, topk_ids, topk_weights, num_experts,
                        local_expert_offset, num_local_experts, act, routed_scaling_factor=1.0,
                        tokens=None):
    """The same routed MoE with BF16 inputs and weights taken as float64 and no quantization or
    intermediate rounding (reported alongside the NVFP4 result, not gated).
    w1_bits_of(e) / w2_bits_of(e): BF16 bit arrays of local expert e."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    M, k = np.asarray(topk_ids).shape
    toks = range(M) if tokens is None else tokens
    out = {}
    for t in toks:
        acc = np.zeros(x.shape[1])
        for j in range(k):
            gid = int(topk_ids[t, j])
            e = gid - local_expert_offset
            if not (0 <= gid < num_experts and 0 <= e < num_local_experts):
                continue
            w1 = bf16_bits_to_f32(w1_bits_of(e)).astype(np.float64)
            w2 = bf16_bits_to_f32(w2_bits_of(e)).astype(np.float64)
            pre = (w1 @ x[t]).reshape(1, -1)
            I = w2.shape[1]
            h = _activation(pre, I, act)[0]
            acc += float(topk_weights[t, j]) * routed_scaling_factor * (w2 @ h)
        out[t] = acc
    return out
