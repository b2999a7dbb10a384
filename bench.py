"""Benchmark of the NVFP4 routed-MoE hot path on one MI355X.

One step = the whole per-call path on one batch of synthetic input already resident in HBM:
routing plan + per-token NVFP4 quantization of the activations + fused experts (GEMM1 with
SwiGLU and requantization, GEMM2, ordered FP32 finalize).  Weight quantization and panel
preparation happen once, before timing (offline in a serving system).

Workloads (synthetic, seeded inputs from synth/):
  decode    : M=8,    H=7168, I=2048, E=256, top_k=8, block_m=8   (primary: value = tokens/s)
  decode_ll : M=4,    H=2048, I=512,  E=128, top_k=10, block_m=8  (reported in "decode_ll")
  prefill   : M=4096, H=7168, I=2048, E=256, top_k=8, block_m=128 (reported in "prefill")
  skewed    : M=16384, H=4096, I=1536, E=288 (144 local), top_k=6, squared ReLU, Zipf routing,
              block_m=128 (reported in "skewed_relu2")
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|decode_ll|prefill|
       skewed|all]
Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-MoE tokens/s + HBM GB/s (M=8) and TFLOP/s (M=4096), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense FP16/BF16 MFMA (the issued dtype)
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (the MX mode's FP4 x FP8 products)
MXFP4_BYTES = 0.5 + 1.0 / 32   # E2M1 data + one E8M0 scale per 32 values
NVFP4_BYTES = 9.0 / 16.0       # 0.5 B data + 1/16 B E4M3 scale per element


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    choices=["decode", "decode_ll", "prefill", "skewed", "mx", "all", "both"],
                    help="all (or both): decode, decode-LL, prefill, the skewed squared-ReLU "
                         "workload and the MX mode (decode and prefill); the first of them gives "
                         "the headline value")
    ap.add_argument("--replicas", type=int, default=2,
                    help="weight panel copies rotated across steps (defeats the 256 MB MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-skewed", action="store_true",
                    help="leave the skewed squared-ReLU workload out of the default run")
    ap.add_argument("--no-w4a16", action="store_true",
                    help="skip the weight-only (BF16 activation) decode measurement")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing (for counter-collection runs)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the achievable-peak context (read stream, vendor BF16 GEMM)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--digest-counters", nargs="+", metavar="NAME:FETCH_DIR:WRITE_DIR",
                    help="only write profiles/traffic.json from rocprofv3 FETCH_SIZE / WRITE_SIZE "
                         "runs: one NAME:FETCH_DIR:WRITE_DIR per workload run (NAME one of "
                         "decode, decode_ll, prefill, skewed, mx) and copy:FETCH_DIR:WRITE_DIR "
                         "for the --calibrate-copy runs; prints the summary table")
    ap.add_argument("--graph-vs-eager", action="store_true",
                    help="only run the workload's step eagerly, pause, then as HIP-graph replays "
                         "(for a kernel trace comparing the two)")
    return ap.parse_args()


def calibrate_copy(copies=4):
    """A plain device-to-device copy of 1 GiB, the known-size reference against which the
    FETCH_SIZE / WRITE_SIZE counters of the kernels are scaled."""
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(copies):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": copies}))


def graph_vs_eager(wl, steps, warmup):
    """The step `steps` times eagerly, a 50 ms pause, then `steps` replays of the same step
    captured in HIP graphs (one per weight copy): under a kernel tracer the two phases show the
    kernels' durations and the idle time between steps of each."""
    import torch

    s = Setup(wl, 2)
    for i in range(warmup):
        s.step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        s.step(i)
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / steps * 1e3
    time.sleep(0.05)
    graph = time_graph(s, steps, warmup) / steps * 1e3
    print(json.dumps({"workload": wl.name, "eager_ms_per_step": eager,
                      "graph_replay_ms_per_step": graph}))


def kernel_source_digest():
    """Digest of the code (comments and whitespace removed) of the sources that define the GEMM
    kernels: device helpers and gemm.hip."""
    h = hashlib.sha256()
    for f in ("device.h", "gemm.hip"):
        with open(os.path.join(ROOT, "block_scaled_fp4_plan_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


# rocprofv3 kernel symbols of the GEMMs, per workload run, and the names the bench's event table
# gives the same launches
COUNTER_KERNELS = {
    # moe_gemv_kernel<FN, KS, EPI, RING, OCC>: decode-LL splits K over 4 (gate/up) and 2 (down)
    # waves
    "decode": {"moe_gemv_kernel<2, 1, 0, 2, 4>": "gemm1_swiglu_decode",
               "moe_gemv_kernel<2, 1, 2, 2, 4>": "gemm2_down_decode"},
    "decode_ll": {"moe_gemv_kernel<1, 4, 0, 3, 4>": "gemm1_swiglu_decode",
                  "moe_gemv_kernel<1, 2, 2, 3, 4>": "gemm2_down_decode"},
    "prefill": {"moe_gemm_kernel<0>": "gemm1_swiglu_prefill",
                "moe_gemm_kernel<2>": "gemm2_down_prefill"},
    "skewed": {"moe_gemm_kernel<1>": "gemm1_relu2_prefill",
               "moe_gemm_kernel<2>": "gemm2_down_prefill"},
    "mx": {"moe_gemv_mx_kernel<0, 2>": "gemm1_swiglu_mx_decode",
           "moe_gemv_mx_kernel<2, 2>": "gemm2_down_mx_decode",
           "moe_gemm_mx_kernel<0>": "gemm1_swiglu_mx_prefill",
           "moe_gemm_mx_kernel<2>": "gemm2_down_mx_prefill"},
}


def _counter_rows(d):
    """(kernel name, counter name, value) of every dispatch in a rocprofv3 csv output dir."""
    import csv
    import glob

    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def digest_counters(specs, out_path=None):
    """profiles/traffic.json from rocprofv3 counter runs: per workload and GEMM kernel, the mean
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) over every dispatch of the run, scaled by what
    the same counters read for a plain 1 GiB device copy (bytes moved / counter reading), with the
    digest of the kernel sources they were taken on.  Prints a markdown table of the result."""
    runs = {}
    for spec in specs:
        name, fdir, wdir = spec.split(":")
        runs[name] = (_counter_rows(fdir), _counter_rows(wdir))
    if "copy" not in runs:
        raise SystemExit("--digest-counters needs the copy:FETCH_DIR:WRITE_DIR calibration runs")

    def mean(rows, counter, key):
        v = [x for k, c, x in rows if c == counter and key in k]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    n = 1 << 30
    fk, _ = mean(runs["copy"][0], "FETCH_SIZE", "opy")
    wk, _ = mean(runs["copy"][1], "WRITE_SIZE", "opy")
    fscale, wscale = n / (fk * 1024.0), n / (wk * 1024.0)
    digest = kernel_source_digest()
    out = {"about": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per "
                    "dispatch, one counter per pass, mean over every dispatch of the kernel in the "
                    "run), scaled by the same counters' readings for a plain 1 GiB device copy "
                    "(bench.py --calibrate-copy): FETCH_SIZE x %.3f, WRITE_SIZE x %.3f.  "
                    "source_digest = bench.py kernel_source_digest() of the sources the counters "
                    "were taken on; bench.py reports traffic only while it matches."
                    % (fscale, wscale),
           "commands": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- "
                        "python3 -u bench.py --workload <w> --steps 3 --warmup 1 "
                        "--no-cpu-baseline --no-context --no-graph --no-w4a16",
                        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- "
                        "python3 -u bench.py --workload <w> --steps 3 --warmup 1 "
                        "--no-cpu-baseline --no-context --no-graph --no-w4a16",
                        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- "
                        "python3 -u bench.py --calibrate-copy",
                        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- "
                        "python3 -u bench.py --calibrate-copy",
                        "python3 bench.py --digest-counters <w>:<fetch dir>:<write dir> ... "
                        "copy:<fetch dir>:<write dir>"],
           "copy_reference": {"bytes_read": n, "bytes_written": n, "fetch_kib": fk,
                              "write_kib": wk},
           "fetch_scale": fscale, "write_scale": wscale}
    lines = ["| workload / kernel | dispatches | FETCH_SIZE raw (KiB) | WRITE_SIZE raw (KiB) | "
             "HBM bytes per launch (scaled) |", "|---|---|---|---|---|"]
    for wl_name, (frows, wrows) in runs.items():
        if wl_name == "copy":
            continue
        for sym, kname in COUNTER_KERNELS[wl_name].items():
            f, nf = mean(frows, "FETCH_SIZE", sym)
            w, _ = mean(wrows, "WRITE_SIZE", sym)
            if f is None or w is None:
                continue
            fb, wb = f * 1024.0 * fscale, w * 1024.0 * wscale
            out["%s/%s" % (wl_name, kname)] = {
                "kernel": sym, "fetch_bytes": int(fb), "write_bytes": int(wb),
                "bytes_per_launch": int(fb + wb), "fetch_kib_raw": f, "write_kib_raw": w,
                "dispatches": nf, "source_digest": digest}
            lines.append("| %s/%s `%s` | %d | %.4g | %.4g | %.4g GB |"
                         % (wl_name, kname, sym, nf, f, w, (fb + wb) / 1e9))
    with open(out_path or os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print("\n".join(lines))
    print("\nsource_digest %s; FETCH_SIZE x %.4f, WRITE_SIZE x %.4f" % (digest, fscale, wscale))
    return out


def traffic_for(kernel, workload, path=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources; else None."""
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    ent = d.get("%s/%s" % (workload, kernel))
    if not ent or ent.get("source_digest") != kernel_source_digest():
        return None
    return ent["bytes_per_launch"]


class Setup:
    def __init__(self, wl, replicas, seed=0):
        import torch

        from block_scaled_fp4_plan_amd import runner
        from synth import make_activations, make_routing, make_weights

        self.wl = wl
        dev = "cuda"
        self.x_bits = make_activations(wl, seed)
        self.ids, self.w = make_routing(wl, seed)
        self.x = torch.from_numpy(self.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        self.ids_d = torch.from_numpy(self.ids).to(dev)
        self.w_d = torch.from_numpy(self.w).to(dev)
        self.w1, self.w2 = make_weights(wl, seed, dev)
        pw = runner.prepare_weights(self.w1, self.w2, gated=wl.gated)
        self.weights = [pw]
        for _ in range(replicas - 1):
            self.weights.append(runner.PreparedWeights(pw.panels.clone(), pw.panels_bytes,
                                                       pw.alpha1_gate, pw.alpha1_up, pw.alpha2,
                                                       pw.num_local_experts, pw.H, pw.I,
                                                       pw.gated))
        self.fwd = runner.MoeForward(pw, wl.M, wl.top_k, wl.E, wl.block_m, wl.local_offset)
        self.out = torch.zeros((wl.M, wl.H), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        loc = self.ids.reshape(-1) - wl.local_offset
        ok = (loc >= 0) & (loc < wl.n_local)
        self.A = int(ok.sum())                               # valid local assignments
        self.touched = len(set(loc[ok].tolist()))            # distinct routed experts

    def step(self, i):
        self.fwd(self.x, self.ids_d, self.w_d, out=self.out,
                 weights=self.weights[i % len(self.weights)])


_SPIN_RATE = []


def spin_cycles(seconds):
    """Argument of torch.cuda._sleep that keeps the GPU busy for about `seconds` (its cycle rate
    measured once)."""
    import torch

    if not _SPIN_RATE:
        n = 1 << 22
        torch.cuda._sleep(n)                    # warm
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(n)
        b.record()
        torch.cuda.synchronize()
        _SPIN_RATE.append(n / max(a.elapsed_time(b) * 1e-3, 1e-6))
    return int(min(seconds * _SPIN_RATE[0], 2 ** 62))


def time_workload(wl, steps, warmup, replicas, timed_prefix="gemm1"):
    """Times `steps` whole steps with nothing but the steps on the stream, then repeats them with
    one HIP event pair around each launch of the dominant GEMM (kernels whose name starts with
    `timed_prefix`) for that kernel's live average duration.  Each event marker costs several
    microseconds of queue time, so the step time comes from the first, uninstrumented pass; the
    second pass's own GPU time per step is returned as well.  A last pass outside both records
    every kernel for the per-kernel breakdown."""
    import torch

    import block_scaled_fp4_plan_amd as bf

    s = Setup(wl, replicas)
    for i in range(warmup):
        s.step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        s.step(i)
    t_enq = time.perf_counter() - t0           # host time to enqueue the steps
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    table, dt_ev = {}, None
    if timed_prefix is not None:
        # When the host's launches pace the GPU (the short decode-LL step: enqueueing took most of
        # the pass), the instrumented steps are queued behind a spin kernel that outlasts their
        # host-side launches, so the GPU runs them back to back and the event pairs time the
        # kernel, not the launch rate.  GPU-bound workloads run as they are.
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        bf.bfp4_profile_begin(steps * 4 + 16, timed_prefix)
        torch.cuda.synchronize()
        if t_enq > 0.5 * dt:
            torch.cuda._sleep(spin_cycles(min(2.0 * t_enq + 0.002, 0.05)))
        ev0.record()
        for i in range(steps):
            s.step(i)
        ev1.record()
        torch.cuda.synchronize()
        dt_ev = ev0.elapsed_time(ev1) * 1e-3
        table = bf.bfp4_profile_end()[1]
    nb = min(steps, 20)                      # per-kernel breakdown, outside the timed passes
    bf.bfp4_profile_begin(nb * 16 + 64)
    for i in range(nb):
        s.step(i)
    torch.cuda.synchronize()
    breakdown = bf.bfp4_profile_end()[1]
    return s, dt, dt_ev, table, breakdown


def time_graph(s, steps, warmup):
    """The same step captured once per weight replica in a HIP graph (plan, activation
    quantization, fused experts, finalize: the library allocates nothing and never synchronizes,
    so the capture holds exactly the eager step's kernels), then `steps` replays timed."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for r in range(len(s.weights)):
            s.step(r)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for r in range(len(s.weights)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s.step(r)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    del graphs
    return dt


def time_w4a16(s, steps, warmup, mxfp4=False):
    """The decode step in the weight-only mode on BF16 activations (routing plan + fused
    weight-only experts + finalize, no activation quantization) with NVFP4 or MXFP4 weights, on
    the same inputs and rotating weight replicas: step time of an uninstrumented pass, then the weight-only GEMM1's average
    launch duration from a pass with HIP events around it."""
    import torch

    import block_scaled_fp4_plan_amd as bf
    from block_scaled_fp4_plan_amd import runner

    wl = s.wl
    weights = s.weights
    if mxfp4:                # the same BF16 weights as MXFP4 (E8M0 per 32), same replica count
        pw = runner.prepare_weights_mxfp4(s.w1, s.w2, gated=wl.gated)
        weights = [pw] + [runner.PreparedWeights(pw.panels.clone(), pw.panels_bytes,
                                                 pw.alpha1_gate, pw.alpha1_up, pw.alpha2,
                                                 pw.num_local_experts, pw.H, pw.I, pw.gated,
                                                 pw.fmt) for _ in range(len(s.weights) - 1)]
    f = runner.MoeForwardW4A16(weights[0], wl.M, wl.top_k, wl.E, wl.block_m, wl.local_offset)

    def step(i):
        f(s.x, s.ids_d, s.w_d, out=s.out, weights=weights[i % len(weights)])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    bf.bfp4_profile_begin(steps * 4 + 16, "gemm1_swiglu_w16")
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    g1_ms, _, name = kernel_ms(bf.bfp4_profile_end()[1], "gemm1")
    # algorithmic bytes: the weights in their format (MXFP4: one scale byte per 32 values; the
    # panels store it in both 16-value slots, so the kernel moves 1/32 B per value more)
    q = NVFP4_BYTES if not mxfp4 else 0.5 + 1.0 / 32
    g1_bytes = (s.touched * wl.N1 * wl.H * q + wl.M * wl.H * 2 + s.A * wl.I * 2)
    ach = g1_bytes / (g1_ms * 1e-3) / 1e9
    del weights, f
    torch.cuda.empty_cache()
    return {"value": wl.M / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "weights": "MXFP4 (E8M0 per 32)" if mxfp4 else "NVFP4 (E4M3 per 16)",
            "roofline": {"bound": "hbm", "kernel": name, "achieved": ach, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "bytes_per_launch": g1_bytes,
                         "avg_launch_ms": g1_ms}}


def achievable_context(reps=5):
    """Achievable-peak context on this GPU: plain read streams over 4 GiB (torch's sum of FP32,
    and the library's XOR-checksum diagnostic, which reads with the decode GEMMs' 16-byte lane
    loads), a device copy, and a BF16 GEMM of the prefill's GEMM1 shape through torch.matmul
    (the vendor BLAS)."""
    import torch

    import block_scaled_fp4_plan_amd as bf

    x = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    x.sum()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        x.sum()
    torch.cuda.synchronize()
    read_gbs = x.numel() * 4 * reps / (time.perf_counter() - t0) / 1e9
    partial = torch.zeros(bf.XOR_PARTIALS, dtype=torch.int32, device="cuda")
    nbytes = x.numel() * 4
    bf.bfp4_xor_checksum(x, nbytes, partial)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps * 4):
        bf.bfp4_xor_checksum(x, nbytes, partial)
    e1.record()
    torch.cuda.synchronize()
    xor_gbs = nbytes * reps * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # 2^30 copies of one word: their XOR is zero
    xor_ok = int(np.bitwise_xor.reduce(partial.cpu().numpy().view(np.uint32))) == 0
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    copy_gbs = 2 * x.numel() * 4 * reps / (time.perf_counter() - t0) / 1e9
    del x, y
    m, n, k = 4096, 4096, 7168
    a = torch.randn(m, k, device="cuda").to(torch.bfloat16)
    b = torch.randn(k, n, device="cuda").to(torch.bfloat16)
    (a @ b)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps * 4):
        (a @ b)
    torch.cuda.synchronize()
    gemm_tf = 2.0 * m * n * k * reps * 4 / (time.perf_counter() - t0) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"read_stream_gbs": read_gbs, "read_stream": "torch sum over 4 GiB FP32",
            "read_stream_lane16_gbs": xor_gbs if xor_ok else None,
            "read_stream_lane16": "bfp4_xor_checksum over 4 GiB (16-byte loads per lane, four in "
                                  "flight per wave, 16384 waves)",
            "copy_gbs": copy_gbs, "copy": "torch copy of 4 GiB, bytes read + written",
            "bf16_gemm_tflops": gemm_tf,
            "bf16_gemm": "torch.matmul BF16 %dx%dx%d (vendor BLAS)" % (m, n, k)}


def gemm_bytes(wl, touched, A, which):
    H, I, N1 = wl.H, wl.I, wl.N1
    if which == 1:   # W1 of routed experts + routed token rows + requantized intermediate
        return (touched * N1 * H * NVFP4_BYTES + wl.M * (H * NVFP4_BYTES + 4) +
                A * I * NVFP4_BYTES)
    return touched * H * I * NVFP4_BYTES + A * I * NVFP4_BYTES + A * H * 2


def kernel_rooflines(wl, s, breakdown):
    """Every kernel of the step against its own roofline: the average duration from the breakdown
    pass and the algorithmic bytes (HBM- and latency-bound kernels) or flops (the tiled GEMMs) of
    one launch, as in the kernel table of the design notes."""
    M, H, I, N1, k, A, q = wl.M, wl.H, wl.I, wl.N1, wl.top_k, s.A, NVFP4_BYTES
    work = {
        "plan": ("latency", M * k * 12),                  # id read, plan entry, token_to_row
        "quantize_rows": ("hbm", M * H * 2 + M * H * q + M * 4),
        "tile_list_decode_tokens": ("hbm", M * H * (q + 2)),   # the FP16 token copy's bytes
        "tile_list": ("latency", 0),
        "gemm1_%s_decode" % wl.act: ("hbm", gemm_bytes(wl, s.touched, A, 1)),
        "gemm2_down_decode": ("hbm", gemm_bytes(wl, s.touched, A, 2)),
        "gemm1_%s_prefill" % wl.act: ("mfma", 2.0 * A * H * N1),
        "gemm2_down_prefill": ("mfma", 2.0 * A * H * I),
        "finalize": ("hbm", A * H * 2 + 2 * M * H * 2 + M * k * 8),
    }
    out = {}
    for name, (cnt, tot) in breakdown.items():
        ms = tot / cnt
        key = "plan" if name.startswith("plan_") else name
        ent = {"ms": ms}
        if key in work:
            bound, units = work[key]
            ent["bound"] = bound
            if bound == "mfma":
                ach = units / (ms * 1e-3) / 1e12
                ent.update(achieved=ach, unit="TFLOP/s", frac=ach / F16_MFMA_PEAK_TFLOPS)
            elif units:
                ach = units / (ms * 1e-3) / 1e9
                ent.update(achieved=ach, unit="GB/s", frac=ach / HBM_PEAK_GBS)
        out[name] = ent
    return out


def step_bytes(wl, touched):
    """Whole-step algorithmic HBM bytes: routed experts' weights, x, out read+write, ids+weights."""
    return (touched * (wl.N1 * wl.H + wl.H * wl.I) * NVFP4_BYTES + wl.M * wl.H * 2 +
            2 * wl.M * wl.H * 2 + wl.M * wl.top_k * 8)


def step_flops(wl, A):
    return 2.0 * A * wl.H * wl.N1 + 2.0 * A * wl.I * wl.H


def kernel_ms(table, prefix):
    for name, (cnt, tot) in table.items():
        if name.startswith(prefix):
            return tot / cnt, cnt, name
    return None, 0, None


def cpu_baseline(s, runs=3, max_experts=None):
    """The oracle (float64 / exact int64 numpy, as it stands) on the per-call path of this
    workload: activation quantization, plan, permutation, every routed expert's projections,
    activation and requantization (oracle.expert_rows_forward, one call per expert, the calls
    spread over a thread pool of all host cores: numpy's integer matrix products release the
    interpreter lock), then the ordered combine.  Weight quantization is offline on both sides
    and excluded.  With max_experts, only that many experts (spread over the range of routed
    rows per expert) run and the time is extrapolated to all assignments linearly in the number
    of assignments; the sample is stated.  Returns the median of `runs` timed runs."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from oracle.formats import bf16_bits_to_f32
    from synth import to_bits

    wl = s.wl
    threads = len(os.sched_getaffinity(0))
    srt, eids, P, ttr = oracle.moe_plan(s.ids, wl.E, wl.local_offset, wl.n_local, wl.block_m)
    rows_of = {}
    for r in range(P):
        if srt[r] < wl.M * wl.top_k:
            rows_of.setdefault(int(eids[r // wl.block_m]), []).append(r)
    experts = sorted(rows_of)
    if max_experts is not None and len(experts) > max_experts:
        by_size = sorted(experts, key=lambda e: len(rows_of[e]))
        pick = np.linspace(0, len(by_size) - 1, max_experts).round().astype(int)
        experts = sorted(set(by_size[i] for i in pick))
    A_all = sum(len(v) for v in rows_of.values())
    A_run = sum(len(rows_of[e]) for e in experts)

    host_w = {e: (to_bits(s.w1[e]), to_bits(s.w2[e])) for e in experts}

    def quant(e):                                                # offline part (untimed)
        q1, s1, a1 = oracle.quantize_expert_weights(host_w[e][0][None])
        q2, s2, a2 = oracle.quantize_expert_weights(host_w[e][1][None])
        return e, ((q1[0], s1[0], q2[0], s2[0]), a1[0], a2[0])

    with ThreadPoolExecutor(threads) as ex:
        wq = dict(ex.map(quant, experts))
    del host_w
    x = bf16_bits_to_f32(s.x_bits)

    def one_run():
        t0 = time.perf_counter()
        aq, asf, adec = oracle.quantize_nvfp4(x, oracle.SCALE_PER_ROW)
        srt_, eids_, P_, ttr_ = oracle.moe_plan(s.ids, wl.E, wl.local_offset, wl.n_local,
                                               wl.block_m)
        qp, sp, spd = oracle.moe_permute(aq, asf, adec, srt_, P_, wl.top_k)

        def expert(e):
            rs = np.array(rows_of[e])
            (w1q, w1s, w2q, w2s), a1, a2 = wq[e]
            return rs, oracle.expert_rows_forward(qp[rs], sp[rs], spd[rs], w1q, w1s, w2q, w2s,
                                                  a1, a1, a2, 1.0, wl.act_code)["y"]

        y = {}
        with ThreadPoolExecutor(threads) as ex:
            for rs, ye in ex.map(expert, experts):
                for i, r in enumerate(rs):
                    y[int(r)] = ye[i]
        if max_experts is None:
            out = oracle.combine(np.zeros((wl.M, wl.H), np.uint16), y, s.w, ttr_)
        else:
            out = None
        return time.perf_counter() - t0, out

    times, out = [], None
    for _ in range(runs):
        dt, out = one_run()
        times.append(dt)
    dt = float(np.median(times))
    flops = 2.0 * A_run * (wl.N1 * wl.H + wl.H * wl.I)
    full_dt = dt * A_all / A_run
    res = dict(value=wl.M / full_dt, unit="tokens/s", cores=threads, kind="oracle",
               runs=runs, run_seconds=times, gflops=flops / dt / 1e9,
               blas_threads="none: the oracle's projections are exact int64 matrix products")
    if max_experts is None:
        res["sample"] = ("the whole per-call path of the %s workload (%d tokens, %d experts, %d "
                         "assignments), median of %d runs, %d threads; weight quantization "
                         "excluded" % (wl.name, wl.M, len(experts), A_all, runs, threads))
        import torch

        o = torch.zeros_like(s.out)                   # one fresh GPU forward for the comparison
        s.fwd(s.x, s.ids_d, s.w_d, out=o, weights=s.weights[0])
        torch.cuda.synchronize()
        got = bf16_bits_to_f32(to_bits(o)).astype(np.float64)
        ref = bf16_bits_to_f32(out).astype(np.float64)
        res["gpu_vs_oracle_rel_fro"] = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    else:
        res["sample"] = ("%d of the %d routed experts of the %s workload (%d of %d assignments, "
                         "chosen across the range of rows per expert), activation quantization "
                         "and plan over all %d tokens; %.2f s median of %d runs on %d threads, "
                         "extrapolated to all assignments linearly in their number (%.1f s); "
                         "weight quantization excluded"
                         % (len(experts), len(rows_of), wl.name, A_run, A_all, wl.M, dt, runs,
                            threads, full_dt))
    return res


def time_tiled(wl, label, args, desc):
    """One compute-bound workload (tiled prefill kernels): step time and throughput, the dominant
    GEMM1 launch against the FP16 MFMA peak, every kernel against its own roofline."""
    import torch

    s, dt, dt_ev, table, breakdown = time_workload(wl, args.steps, args.warmup, 1)
    ms = dt / args.steps * 1e3
    gdt = None if args.no_graph else time_graph(s, args.steps, args.warmup)
    g1_ms, _, g1_name = kernel_ms(table, "gemm1")
    g1_flops = 2.0 * s.A * wl.H * wl.N1
    ach = g1_flops / (g1_ms * 1e-3) / 1e12
    tf = step_flops(wl, s.A) / (ms * 1e-3) / 1e12
    res = dict(
        value=wl.M / (ms * 1e-3), unit="tokens/s", ms_per_step=ms, tflops=tf,
        tflops_frac=tf / F16_MFMA_PEAK_TFLOPS,
        config={"workload": desc, "assignments": s.A,
                "padded_rows": int(s.fwd.plan.num_tokens_post_padded.item()),
                "ms_per_step_with_gemm1_events": dt_ev / args.steps * 1e3,
                "graph_replay_ms_per_step": gdt and gdt / args.steps * 1e3,
                "graph_replay_tokens_per_s": gdt and wl.M / (gdt / args.steps),
                "kernels": kernel_rooflines(wl, s, breakdown)},
        roofline={"bound": "mfma", "kernel": g1_name, "achieved": ach,
                  "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": ach / F16_MFMA_PEAK_TFLOPS,
                  "traffic": traffic_for(g1_name, label), "flops_per_launch": g1_flops,
                  "avg_launch_ms": g1_ms})
    if not args.no_cpu_baseline:
        log("oracle CPU baseline (sample):", wl.name)
        res["cpu_baseline"] = cpu_baseline(s, runs=1, max_experts=8)
    del s
    torch.cuda.empty_cache()
    return res


def cpu_baseline_mx(wl, ids, w, x_bits, w1, w2, runs=3, max_experts=None, gpu_out=None,
                    central=False):
    """The oracle on the MX mode's per-call path (plan, then per routed expert the MXFP8
    quantization of its rows, the exact MX projections, activation and MXFP8 requantization,
    oracle.expert_rows_forward_mx, one call per expert over a thread pool of all host cores;
    then the ordered combine), as cpu_baseline does for the NVFP4 mode; the MXFP4 weight
    quantization is offline and excluded.  w1 / w2: the BF16 weights (device tensors).  With
    central, the sampled experts come from the middle half of the range of rows per expert
    (the oracle's MX path is slow enough that the largest experts alone would take a minute)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from oracle.formats import bf16_bits_to_f32
    from synth import to_bits

    threads = len(os.sched_getaffinity(0))
    srt, eids, P, ttr = oracle.moe_plan(ids, wl.E, wl.local_offset, wl.n_local, wl.block_m)
    rows_of = {}
    for r in range(P):
        if srt[r] < wl.M * wl.top_k:
            rows_of.setdefault(int(eids[r // wl.block_m]), []).append(r)
    experts = sorted(rows_of)
    if max_experts is not None and len(experts) > max_experts:
        by_size = sorted(experts, key=lambda e: len(rows_of[e]))
        lo, hi = (len(by_size) // 4, (3 * len(by_size)) // 4) if central else (0, len(by_size) - 1)
        pick = np.linspace(lo, hi, max_experts).round().astype(int)
        experts = sorted(set(by_size[i] for i in pick))
    A_all = sum(len(v) for v in rows_of.values())
    A_run = sum(len(rows_of[e]) for e in experts)

    def quant(e):                                                # offline part (untimed)
        q1, s1 = oracle.quantize_mxfp4(bf16_bits_to_f32(to_bits(w1[e])))
        q2, s2 = oracle.quantize_mxfp4(bf16_bits_to_f32(to_bits(w2[e])))
        return e, (q1, s1, q2, s2)

    with ThreadPoolExecutor(threads) as ex:
        wq = dict(ex.map(quant, experts))

    def one_run():
        t0 = time.perf_counter()
        srt_, eids_, P_, ttr_ = oracle.moe_plan(ids, wl.E, wl.local_offset, wl.n_local,
                                               wl.block_m)

        def expert(e):
            rs = np.array(rows_of[e])
            return rs, oracle.expert_rows_forward_mx(x_bits[srt_[rs] // wl.top_k], *wq[e],
                                                     wl.act_code)["y"]

        y = {}
        with ThreadPoolExecutor(threads) as ex:
            for rs, ye in ex.map(expert, experts):
                for i, r in enumerate(rs):
                    y[int(r)] = ye[i]
        out = (oracle.combine(np.zeros((wl.M, wl.H), np.uint16), y, w, ttr_)
               if max_experts is None else None)
        return time.perf_counter() - t0, out

    times, out = [], None
    for _ in range(runs):
        dt, out = one_run()
        times.append(dt)
    dt = float(np.median(times))
    flops = 2.0 * A_run * (wl.N1 * wl.H + wl.H * wl.I)
    full_dt = dt * A_all / A_run
    res = dict(value=wl.M / full_dt, unit="tokens/s", cores=threads, kind="oracle",
               runs=runs, run_seconds=times, gflops=flops / dt / 1e9,
               blas_threads="none: the oracle's MX projections are exact int64 matrix products")
    if max_experts is None:
        res["sample"] = ("the whole per-call path of the %s workload in the MX mode (%d tokens, "
                         "%d experts, %d assignments), median of %d runs, %d threads; MXFP4 weight "
                         "quantization excluded" % (wl.name, wl.M, len(experts), A_all, runs,
                                                    threads))
        if gpu_out is not None:
            got = bf16_bits_to_f32(to_bits(gpu_out)).astype(np.float64)
            ref = bf16_bits_to_f32(out).astype(np.float64)
            res["gpu_vs_oracle_rel_fro"] = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    else:
        res["sample"] = ("%d of the %d routed experts of the %s workload in the MX mode (%d of %d "
                         "assignments, chosen across the %s of rows per expert), plan over all "
                         "%d tokens; %.2f s median of %d runs on %d threads, extrapolated to all "
                         "assignments linearly in their number (%.1f s); MXFP4 weight "
                         "quantization excluded"
                         % (len(experts), len(rows_of), wl.name, A_run, A_all,
                            "middle half of the range" if central else "range", wl.M, dt, runs,
                            threads, full_dt))
    return res


def time_mx(wl, args, label, desc):
    """The MX mode (MXFP4 weights, MXFP8 activations, block-scaled MFMA) on a workload: plan,
    MXFP8 activation quantization and the fused MX call (+ finalize) per step, with the same
    inputs; the dominant GEMM1 against the FP8 MFMA peak (tiled, block_m > 32) or the HBM peak
    (decode), every kernel's average duration."""
    import torch

    import block_scaled_fp4_plan_amd as bf
    from block_scaled_fp4_plan_amd import runner
    from synth import make_activations, make_routing, make_weights

    x_bits = make_activations(wl, 0)
    ids, w = make_routing(wl, 0)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    ids_d, w_d = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    w1, w2 = make_weights(wl, 0, "cuda")
    pw = runner.prepare_weights_mxfp4(w1, w2, gated=wl.gated)
    if args.no_cpu_baseline:                     # else kept for the oracle's weight quantization
        del w1, w2
        w1 = w2 = None
    replicas = [pw]
    decode = wl.block_m <= 32
    if decode:                                   # weights from HBM on every step
        replicas.append(runner.PreparedWeights(pw.panels.clone(), pw.panels_bytes, pw.alpha1_gate,
                                               pw.alpha1_up, pw.alpha2, pw.num_local_experts, pw.H,
                                               pw.I, pw.gated, pw.fmt))
    f = runner.MoeForwardMX(pw, wl.M, wl.top_k, wl.E, wl.block_m, wl.local_offset)
    out = torch.zeros((wl.M, wl.H), dtype=torch.bfloat16, device="cuda")

    def step(i):
        f(x, ids_d, w_d, out=out, weights=replicas[i % len(replicas)])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    t_enq = time.perf_counter() - t0
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    bf.bfp4_profile_begin(args.steps * 4 + 16, "gemm1")
    torch.cuda.synchronize()
    if t_enq > 0.5 * ms * 1e-3 * args.steps:                          # as in time_workload
        torch.cuda._sleep(spin_cycles(min(2.0 * t_enq + 0.002, 0.05)))
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    g1_ms, _, g1_name = kernel_ms(bf.bfp4_profile_end()[1], "gemm1")
    nb = min(args.steps, 20)
    bf.bfp4_profile_begin(nb * 16 + 64)
    for i in range(nb):
        step(i)
    torch.cuda.synchronize()
    breakdown = {k: {"ms": tot / c} for k, (c, tot) in bf.bfp4_profile_end()[1].items()}
    loc = ids.reshape(-1) - wl.local_offset
    ok = (loc >= 0) & (loc < wl.n_local)
    A, touched = int(ok.sum()), len(set(loc[ok].tolist()))
    res = dict(value=wl.M / (ms * 1e-3), unit="tokens/s", ms_per_step=ms,
               config={"workload": desc, "assignments": A, "touched_experts": touched,
                       "kernels": breakdown})
    if decode:
        g1_bytes = (touched * wl.N1 * wl.H * MXFP4_BYTES + wl.M * wl.H * (1 + 1.0 / 32) +
                    A * wl.I * (1 + 1.0 / 32))
        step_b = (touched * (wl.N1 * wl.H + wl.H * wl.I) * MXFP4_BYTES + wl.M * wl.H * 2 +
                  2 * wl.M * wl.H * 2 + wl.M * wl.top_k * 8)
        ach = g1_bytes / (g1_ms * 1e-3) / 1e9
        res["config"]["step_hbm_frac"] = step_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
        res["roofline"] = {"bound": "hbm", "kernel": g1_name, "achieved": ach,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                           "traffic": traffic_for(g1_name, "mx"), "bytes_per_launch": g1_bytes,
                           "avg_launch_ms": g1_ms}
    else:
        g1_flops = 2.0 * A * wl.H * wl.N1
        ach = g1_flops / (g1_ms * 1e-3) / 1e12
        tf = step_flops(wl, A) / (ms * 1e-3) / 1e12
        res.update(tflops=tf, tflops_frac=tf / FP8_MFMA_PEAK_TFLOPS)
        res["roofline"] = {"bound": "mfma", "kernel": g1_name, "achieved": ach,
                           "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / FP8_MFMA_PEAK_TFLOPS, "traffic": traffic_for(g1_name, "mx"),
                           "flops_per_launch": g1_flops, "avg_launch_ms": g1_ms}
    if not args.no_cpu_baseline:
        log("oracle CPU baseline (MX mode):", wl.name)
        if decode:
            o = torch.zeros_like(out)                 # one fresh GPU forward for the comparison
            f(x, ids_d, w_d, out=o, weights=replicas[0])
            torch.cuda.synchronize()
            # one run: the oracle's MX dot products are several times slower than its NVFP4
            # ones, and one run of this path already takes seconds
            res["cpu_baseline"] = cpu_baseline_mx(wl, ids, w, x_bits, w1, w2, runs=1, gpu_out=o)
        else:
            res["cpu_baseline"] = cpu_baseline_mx(wl, ids, w, x_bits, w1, w2, runs=1,
                                                  max_experts=4, central=True)
    del f, replicas, pw, w1, w2
    torch.cuda.empty_cache()
    return res


def log(*a):
    """Progress of the run on stderr (the JSON result is the only line on stdout)."""
    print("[bench]", *a, file=sys.stderr, flush=True)


def time_hbm(wl, args, replicas, desc, label, cpu_runs=3):
    """One weight-streaming (decode) workload: step time with `replicas` rotated copies of the
    weight panels, the whole step's algorithmic bytes against the HBM peak, the dominant GEMM1
    launch against its roofline, every kernel's average duration, HIP-graph replay timing and the
    oracle's CPU baseline of the same call."""
    import torch

    s, dt, dt_ev, table, breakdown = time_workload(wl, args.steps, args.warmup, replicas)
    ms = dt / args.steps * 1e3
    g1_ms, _, g1_name = kernel_ms(table, "gemm1")
    g1_bytes = gemm_bytes(wl, s.touched, s.A, 1)
    ach = g1_bytes / (g1_ms * 1e-3) / 1e9
    sb = step_bytes(wl, s.touched)
    res = dict(value=wl.M / (ms * 1e-3), unit="tokens/s", ms_per_step=ms,
               config={"workload": desc, "touched_experts": s.touched, "assignments": s.A,
                       "step_algorithmic_bytes": sb,
                       "step_hbm_gbs": sb / (ms * 1e-3) / 1e9,
                       "step_hbm_frac": sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "weight_replicas": replicas,
                       "ms_per_step_with_gemm1_events": dt_ev / args.steps * 1e3,
                       "kernels": kernel_rooflines(wl, s, breakdown)},
               roofline={"bound": "hbm", "kernel": g1_name, "achieved": ach,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                         "traffic": traffic_for(g1_name, label), "bytes_per_launch": g1_bytes,
                         "avg_launch_ms": g1_ms})
    if not args.no_graph:
        gdt = time_graph(s, args.steps, args.warmup)
        res["config"]["graph_replay_ms_per_step"] = gdt / args.steps * 1e3
        res["config"]["graph_replay_tokens_per_s"] = wl.M / (gdt / args.steps)
    if not args.no_w4a16 and label == "decode":
        log("weight-only decode (NVFP4, MXFP4 weights)")
        res["w4a16_decode"] = time_w4a16(s, args.steps, args.warmup)
        res["w4a16_mxfp4_decode"] = time_w4a16(s, args.steps, args.warmup, mxfp4=True)
    if not args.no_cpu_baseline:
        log("oracle CPU baseline:", wl.name)
        res["cpu_baseline"] = cpu_baseline(s, runs=cpu_runs)
    del s
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on exactly one GPU (expert parallelism is reduced to "
              "masking non-local experts); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.digest_counters:                   # reads counter files only: no GPU needed
        digest_counters(args.digest_counters)
        return
    import torch

    from synth import WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.graph_vs_eager:
        graph_vs_eager(WORKLOADS["decode" if args.workload in ("all", "both") else
                                 args.workload], args.steps, args.warmup)
        return
    want = {"all": ("decode", "decode_ll", "prefill", "skewed", "mx"),
            "both": ("decode", "decode_ll", "prefill", "skewed", "mx")}.get(args.workload,
                                                                      (args.workload,))
    if args.no_skewed:
        want = tuple(w for w in want if w != "skewed")
    parts = []          # (key of the nested object, result), in order; the first is the headline
    if "decode" in want:
        log("decode M=8")
        parts.append(("decode", time_hbm(
            WORKLOADS["decode"], args, args.replicas,
            "decode: M=8 H=7168 I=2048 E=256 top_k=8 block_m=8 SwiGLU NVFP4", "decode")))
    if "decode_ll" in want:
        log("decode-LL M=4")
        # 128 experts x 1.77 MB = 226 MB of weights fit the 256 MB MALL: rotate >= 9 copies so
        # that every step streams its weights from HBM
        parts.append(("decode_ll", time_hbm(
            WORKLOADS["decode_ll"], args, max(args.replicas, 10),
            "decode-LL: M=4 H=2048 I=512 E=128 top_k=10 block_m=8 SwiGLU NVFP4", "decode_ll")))
    if "prefill" in want:
        log("prefill M=4096")
        parts.append(("prefill", time_tiled(
            WORKLOADS["prefill"], "prefill", args,
            "prefill: M=4096 H=7168 I=2048 E=256 top_k=8 block_m=128 SwiGLU NVFP4")))
    if "mx" in want:
        log("MX mode: decode M=8 and prefill M=4096")
        parts.append(("mx_decode", time_mx(
            WORKLOADS["decode"], args, "decode",
            "MX decode: M=8 H=7168 I=2048 E=256 top_k=8 block_m=8 SwiGLU, MXFP4 weights x "
            "MXFP8 activations (block-scaled MFMA)")))
        parts.append(("mx_prefill", time_mx(
            WORKLOADS["prefill"], args, "prefill",
            "MX prefill: M=4096 H=7168 I=2048 E=256 top_k=8 block_m=128 SwiGLU, MXFP4 weights "
            "x MXFP8 activations (block-scaled MFMA)")))
    if "skewed" in want:
        log("skewed M=16384")
        parts.append(("skewed_relu2", time_tiled(
            WORKLOADS["skewed_relu2"], "skewed", args,
            "skewed: M=16384 H=4096 I=1536 E=288 (experts 0-143 local) top_k=6 block_m=128 "
            "squared-ReLU NVFP4, Zipf(1.2) routing")))
    head = parts[0][1]
    result = dict(metric=METRIC, value=head["value"], unit="tokens/s", n_gpus=1,
                  steps=args.steps, warmup=args.warmup, ms_per_step=head["ms_per_step"],
                  higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f16",
                  data="synthetic")
    for k in ("config", "roofline", "cpu_baseline", "w4a16_decode", "w4a16_mxfp4_decode"):
        if k in head:
            result[k] = head[k]
    for key, r in parts[1:]:
        result[key] = r
    if not args.no_context:
        log("achievable-peak context")
        result["context"] = achievable_context()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
