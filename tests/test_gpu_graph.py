"""The whole forward (routing plan, activation quantization, fused experts and combine) captured
once in a HIP graph and replayed with new contents in the same input buffers: every replay
equals the eager call on the same inputs, bit for bit, and is checked against the oracle on that
replay's inputs (pre-activations of sampled tokens through a captured debug buffer within the
FP32-summation bound; for the small workloads the whole output within 2e-2).

The library allocates nothing on this path, never synchronizes and clears its counters with
kernels (no memset nodes), and its grids are sized by the plan capacity, so one captured graph
serves any routing of the same shape.  Replays alternate with eager work and synchronizations.
"""

import numpy as np
import pytest
import torch

from synth import WORKLOADS, make_activations, make_routing
from synth.workloads import Workload

import oracle
from oracle.formats import bf16_bits_to_f32

from gpu_common import Problem, check_gate_up, np_bits, np_u8, rel_fro, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_scaled_fp4_plan_amd import runner

# several tiles of 1 to 8 token fragments and K not a multiple of the prefetch depth
SKEWED = Workload("graph_skewed", M=384, H=1280, I=640, E=6, top_k=3, block_m=128,
                  routing="zipf")

# the last two: the decode and prefill workloads at full size, as the bench replays them
CASES = [("tiny", 8, True), ("tiny", 128, True), ("tiny", 128, False), ("decode_ll", 8, True),
         ("graph_skewed", 128, True), ("decode", 8, True), ("prefill", 128, True)]


def _inputs(wl, seed, M):
    x_bits = make_activations(wl, seed, M)
    ids, w = make_routing(wl, seed, M)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    return x, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()


def _bits(t):
    return t.view(torch.int16)


def _oracle_replay_check(p, wl, bm, seed, pre_d, out_g=None, y_g=None, n_cols=48):
    """One replay against the oracle on that replay's inputs (the oracle quantizes the
    activations and, at sampled columns, each expert's weights with the whole matrix's scale):
    the captured pre-activation buffer of every routed row of the sampled tokens within the FP32
    summation bound; for small workloads also the whole output within 2e-2 (finalized) or every
    routed row's expert output through the oracle's own forward (unfinalized)."""
    M, k, I, N1 = p.M, wl.top_k, wl.I, wl.N1
    x_bits = make_activations(wl, seed, M)
    ids, w = make_routing(wl, seed, M)
    aq, asf, adec = oracle.quantize_nvfp4(bf16_bits_to_f32(x_bits), oracle.SCALE_PER_ROW)
    srt, eids, P, ttr = oracle.moe_plan(ids, wl.E, wl.local_offset, wl.n_local, bm)
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(M, min(M, 4 if wl.H * N1 <= 1 << 22 else 2), replace=False))
    cols = np.sort(np.random.default_rng(99).choice(N1, min(N1, n_cols), replace=False))
    pre = pre_d.cpu().numpy()
    cache = p.__dict__.setdefault("_rows_q", {})     # expert -> its W1 rows `cols`, quantized
    for t in toks:
        for j in range(k):
            r = int(ttr[t, j])
            if r < 0:
                continue
            e = int(eids[r // bm])
            if e not in cache:
                cache[e] = oracle.quantize_expert_rows(np_bits(p.w1[e]), cols)
            q1, s1, a1 = cache[e]
            alpha_rows = np.full(len(cols), float(a1))
            ref = oracle.expert_gate_up_projection(aq[t:t + 1], asf[t:t + 1], adec[t:t + 1], q1,
                                                    s1, alpha_rows)
            check_gate_up(pre[r:r + 1, cols].astype(np.float64), ref, aq[t:t + 1],
                          asf[t:t + 1], adec[t:t + 1], q1, s1, alpha_rows)
    if wl.H * N1 > 1 << 22:        # the full oracle forward only where experts are small
        return
    experts = sorted(set(int(e) for e in eids[:P // bm]))
    a1, a2 = p.oracle_alphas(experts)
    res = oracle.fused_moe_nvfp4(aq, asf, adec, lambda e: p.oracle_expert(e)[0], a1, a1, a2, 1.0,
                                 srt, eids, P, ttr, w, k, bm, wl.act_code)
    if out_g is not None:
        e_out = rel_fro(bf16_bits_to_f32(np_bits(out_g)), bf16_bits_to_f32(res["out"]))
        assert e_out <= 2e-2, (seed, e_out)
    if y_g is not None:
        yb = np_bits(y_g)
        rows = sorted(res["y"].keys())
        e_y = rel_fro(bf16_bits_to_f32(yb[rows]), np.stack([res["y"][r] for r in rows]))
        assert e_y <= 2e-2, (seed, e_y)


@pytest.mark.parametrize("name,bm,fin", CASES,
                         ids=["%s-bm%d-%s" % (n, b, "fin" if f else "unfin") for n, b, f in CASES])
def test_graph_replay_matches_eager(name, bm, fin):
    wl = SKEWED if name == "graph_skewed" else WORKLOADS[name]
    say("graph replay", name, "block_m", bm, "finalize", fin)
    p = Problem(wl)
    pw = runner.prepare_weights(p.w1, p.w2, gated=wl.gated)
    fwd_e = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm, wl.local_offset, fin)
    fwd_g = runner.MoeForward(pw, p.M, wl.top_k, wl.E, bm, wl.local_offset, fin)
    x, ids, w = p.x.clone(), p.ids_d.clone(), p.w_d.clone()      # the graph's input buffers
    out_g = torch.zeros((p.M, wl.H), dtype=torch.bfloat16, device="cuda")
    # a captured debug buffer: the replay's pre-activations, checked against the oracle
    dbg = dict(preact=torch.zeros((fwd_g.plan.capacity, wl.N1), device="cuda"))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd_g(x, ids, w, out=out_g, debug=dbg)       # first call outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res_g = fwd_g(x, ids, w, out=out_g, debug=dbg)

    for seed in (1, 2, 0, 3, 1):
        xs, idss, ws = _inputs(wl, seed, p.M)
        x.copy_(xs)
        ids.copy_(idss)
        w.copy_(ws)
        out_g.zero_()
        graph.replay()
        res_e = fwd_e(xs, idss, ws)
        torch.cuda.synchronize()
        _oracle_replay_check(p, wl, bm, seed, dbg["preact"], out_g if fin else None,
                             None if fin else res_g[0])
        if fin:
            assert torch.equal(_bits(out_g), _bits(res_e)), seed
        else:
            (y_g, w_g, ttr_g), (y_e, w_e, ttr_e) = res_g, res_e
            assert torch.equal(ttr_g, ttr_e), seed
            assert torch.equal(w_g, ws) and torch.equal(w_e, ws)
            rows = ttr_e.reshape(-1)
            rows = rows[rows >= 0].long()
            assert rows.numel() > 0
            assert torch.equal(_bits(y_g[rows]), _bits(y_e[rows])), seed


@pytest.mark.parametrize("bm", [8, 128])
def test_graph_stable_dispatcher_buffer(bm):
    """Bounded execution over a graph-stable dispatcher buffer ([MCore] flashinfer_routed_nvfp4_moe:
    rows whose routing entries are -1 contribute zero; with a token capacity only that fixed prefix
    is processed and rows past it are left untouched in out).  One graph is captured over a
    48-row buffer with a 32-row prefix; each replay routes a different number of leading rows and
    marks the rest -1.  Routed rows equal the eager call on the same rows, unrouted prefix rows
    keep their previous out values, and rows past the prefix are never written."""
    wl = WORKLOADS["tiny"]
    rows_buf, cap_rows = 48, 32
    say("graph dispatcher buffer, block_m", bm)
    p = Problem(wl, M=rows_buf)
    pw = runner.prepare_weights(p.w1, p.w2, gated=wl.gated)
    fwd_g = runner.MoeForward(pw, cap_rows, wl.top_k, wl.E, bm)
    fwd_e = runner.MoeForward(pw, cap_rows, wl.top_k, wl.E, bm)
    x, ids, w = p.x.clone(), p.ids_d.clone(), p.w_d.clone()
    g = torch.Generator(device="cuda").manual_seed(5)
    out0 = torch.randn((rows_buf, wl.H), device="cuda", generator=g).to(torch.bfloat16)
    out = out0.clone()

    def call(f, xs, idss, ws, o):
        return f(xs[:cap_rows], idss[:cap_rows], ws[:cap_rows], out=o[:cap_rows])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(fwd_g, x, ids, w, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(fwd_g, x, ids, w, out)

    for n_routed in (32, 5, 0, 17):
        xs, idss, ws = _inputs(wl, n_routed + 1, rows_buf)
        idss[n_routed:] = -1
        x.copy_(xs)
        ids.copy_(idss)
        w.copy_(ws)
        o0 = out0.clone()
        o0[:n_routed] = 0                   # routed rows start from zero: the oracle's bar
        out.copy_(o0)
        graph.replay()
        ref = o0.clone()
        call(fwd_e, xs, idss, ws, ref)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), n_routed
        assert torch.equal(_bits(out[n_routed:]), _bits(out0[n_routed:])), n_routed
        if n_routed:
            assert not torch.equal(_bits(out[:n_routed]), _bits(o0[:n_routed]))
            # the routed prefix rows against the oracle on the same rows (plan over the
            # 32-row prefix, -1 rows unrouted)
            ids_np = idss[:cap_rows].cpu().numpy()
            x_bits = np_bits(xs[:cap_rows])
            aq, asf, adec = oracle.quantize_nvfp4(bf16_bits_to_f32(x_bits), oracle.SCALE_PER_ROW)
            srt, eids, P, ttr = oracle.moe_plan(ids_np, wl.E, 0, wl.n_local, bm)
            experts = sorted(set(int(e) for e in eids[:P // bm]))
            a1, a2 = p.oracle_alphas(experts)
            res = oracle.fused_moe_nvfp4(aq, asf, adec, lambda e: p.oracle_expert(e)[0], a1, a1,
                                         a2, 1.0, srt, eids, P, ttr, ws[:cap_rows].cpu().numpy(),
                                         wl.top_k, bm, wl.act_code)
            assert np.all(res["out"][n_routed:] == 0)
            e_out = rel_fro(bf16_bits_to_f32(np_bits(out[:n_routed])),
                            bf16_bits_to_f32(res["out"][:n_routed]))
            say("dispatcher buffer: %d routed rows, out vs oracle %.3e" % (n_routed, e_out))
            assert e_out <= 2e-2


def test_graph_in_place_weight_refresh():
    """In-place weight refresh under a captured graph: new weights are quantized and laid out
    into the panel buffer and alpha arrays the graph already points to (bfp4_prepare_weights
    writes caller-owned memory), and the next replay computes with them, bit for bit as an eager
    call with freshly prepared copies of the same weights."""
    import block_scaled_fp4_plan_amd as bf

    wl = WORKLOADS["tiny"]
    say("graph in-place weight refresh")
    p = Problem(wl)
    pw = runner.prepare_weights(p.w1, p.w2)
    fwd_g = runner.MoeForward(pw, p.M, wl.top_k, wl.E, 8)
    out_g = torch.zeros((p.M, wl.H), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd_g(p.x, p.ids_d, p.w_d, out=out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd_g(p.x, p.ids_d, p.w_d, out=out_g)

    for step in range(2):
        g = torch.Generator(device="cuda").manual_seed(11 + step)
        w1n = (torch.randn(p.w1.shape, device="cuda", generator=g) * 0.03).to(torch.bfloat16)
        w2n = (torch.randn(p.w2.shape, device="cuda", generator=g) * 0.03).to(torch.bfloat16)
        E, N1, H = w1n.shape
        I = w2n.shape[2]
        q1, s1, a1 = runner.quantize(w1n.reshape(E * N1, H), bf.BFP4_SCALE_PER_GROUP, N1)
        q2, s2, a2 = runner.quantize(w2n.reshape(E * H, I), bf.BFP4_SCALE_PER_GROUP, H)
        bf.bfp4_prepare_weights(q1, s1, q2, s2, E, H, I, 1, pw.panels, pw.panels_bytes)
        pw.alpha1_gate.copy_(a1)
        pw.alpha1_up.copy_(a1)
        pw.alpha2.copy_(a2)
        out_g.zero_()
        graph.replay()
        ref = runner.MoeForward(runner.prepare_weights(w1n, w2n), p.M, wl.top_k, wl.E, 8)(
            p.x, p.ids_d, p.w_d)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_g), _bits(ref)), step
        # the replay against the oracle, which quantizes the refreshed weights itself
        o1 = oracle.quantize_expert_weights(np_bits(w1n))
        o2 = oracle.quantize_expert_weights(np_bits(w2n))
        assert np.array_equal(np_u8(q1).reshape(o1[0].shape), o1[0])
        assert np.array_equal(np_u8(s2).reshape(o2[1].shape), o2[1])
        aq, asf, adec = p.oracle_activations()
        srt, eids, P, ttr = p.oracle_plan(8)
        res = oracle.fused_moe_nvfp4(aq, asf, adec, (o1[0], o1[1], o2[0], o2[1]), o1[2], o1[2],
                                     o2[2], 1.0, srt, eids, P, ttr, p.w, wl.top_k, 8,
                                     oracle.ACT_SWIGLU)
        e_out = rel_fro(bf16_bits_to_f32(np_bits(out_g)), bf16_bits_to_f32(res["out"]))
        say("in-place refresh step %d: out vs oracle %.3e" % (step, e_out))
        assert e_out <= 2e-2


W16_CASES = [("tiny", 8, "nvfp4"), ("decode", 8, "nvfp4"), ("decode", 8, "mxfp4")]


@pytest.mark.parametrize("name,bm,fmt", W16_CASES, ids=["%s-bm%d-%s" % c for c in W16_CASES])
def test_graph_replay_w4a16_matches_eager(name, bm, fmt):
    """The weight-only forward (plan + bfp4_fused_moe_w4a16) captured once and replayed with new
    inputs equals the eager call bit for bit (the decode case at full size, NVFP4 and MXFP4
    weights)."""
    wl = WORKLOADS[name]
    say("graph replay w4a16", name, "block_m", bm, fmt)
    p = Problem(wl)
    prep = runner.prepare_weights_mxfp4 if fmt == "mxfp4" else runner.prepare_weights
    pw = prep(p.w1, p.w2, gated=wl.gated)
    fwd_e = runner.MoeForwardW4A16(pw, p.M, wl.top_k, wl.E, bm, wl.local_offset)
    fwd_g = runner.MoeForwardW4A16(pw, p.M, wl.top_k, wl.E, bm, wl.local_offset)
    x, ids, w = p.x.clone(), p.ids_d.clone(), p.w_d.clone()
    out_g = torch.zeros((p.M, wl.H), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd_g(x, ids, w, out=out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd_g(x, ids, w, out=out_g)
    for seed in (1, 2, 0, 1):
        xs, idss, ws = _inputs(wl, seed, p.M)
        x.copy_(xs)
        ids.copy_(idss)
        w.copy_(ws)
        out_g.zero_()
        graph.replay()
        res_e = fwd_e(xs, idss, ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_g), _bits(res_e)), seed
        assert torch.any(_bits(res_e) != 0)
