"""Helpers shared by the GPU parity tests: run the HIP path on seeded synthetic inputs and hand
identical inputs to the oracle.  Each GPU step prints what it runs (flushed) first."""

import sys

import numpy as np
import torch

import oracle
from oracle.formats import bf16_bits_to_f32
from synth import make_activations, make_routing, make_weights, to_bits


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def np_u8(t):
    return t.detach().cpu().numpy().astype(np.uint8)


def np_bits(t):
    return to_bits(t)


class Problem:
    """Seeded inputs of one workload on the GPU (torch) and on the host (numpy)."""

    def __init__(self, wl, seed=0, M=None, device="cuda"):
        self.wl = wl
        self.M = wl.M if M is None else M
        self.x_bits = make_activations(wl, seed, self.M)
        self.ids, self.w = make_routing(wl, seed, self.M)
        self.x = torch.from_numpy(self.x_bits.view(np.int16)).view(torch.bfloat16).to(device)
        self.ids_d = torch.from_numpy(self.ids).to(device)
        self.w_d = torch.from_numpy(self.w).to(device)
        self.w1, self.w2 = make_weights(wl, seed, device)        # BF16 on the GPU
        self._host_w = {}

    def host_weight_bits(self, e):
        if e not in self._host_w:
            self._host_w[e] = (np_bits(self.w1[e]), np_bits(self.w2[e]))
        return self._host_w[e]

    def oracle_expert(self, e):
        """Oracle NVFP4 of local expert e (its own quantizer, one scale per expert matrix)."""
        key = ("q", e)
        if key not in self._host_w:
            b1, b2 = self.host_weight_bits(e)
            q1, s1, a1 = oracle.quantize_expert_weights(b1[None])
            q2, s2, a2 = oracle.quantize_expert_weights(b2[None])
            self._host_w[key] = ((q1[0], s1[0], q2[0], s2[0]), float(a1[0]), float(a2[0]))
        return self._host_w[key]

    def oracle_alphas(self, experts):
        n = self.wl.n_local
        a1 = np.zeros(n, np.float32)
        a2 = np.zeros(n, np.float32)
        for e in experts:
            _, x1, x2 = self.oracle_expert(e)
            a1[e], a2[e] = x1, x2
        return a1, a2

    def oracle_activations(self):
        return oracle.quantize_nvfp4(bf16_bits_to_f32(self.x_bits), oracle.SCALE_PER_ROW)

    def oracle_plan(self, block_m):
        wl = self.wl
        return oracle.moe_plan(self.ids, wl.E, wl.local_offset, wl.n_local, block_m)


def ulp_bf16(v):
    """Spacing of the BF16 grid at |v| (the normal spacing below the normal range)."""
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _abs_products(q_a, sf_a, q_w, sf_w):
    """sum_k |deq(a[r, k]) deq(w[n, k])| for every (r, n), exactly (float64 of an int64 sum)."""
    from oracle.quant import dequantize_int

    return (np.abs(dequantize_int(q_a, sf_a)) @ np.abs(dequantize_int(q_w, sf_w)).T).astype(
        np.float64) * 2.0 ** -20


def check_gate_up(pre_gpu, ref, aq, asf, adec, q1, s1, alpha_rows):
    """GEMM1 pre-activations of the GPU against the oracle's, element by element: the GPU sums
    the exact products in FP32 in its own order (each addition rounded, at most K of them), then
    multiplies by the token and expert scales (two FP32 roundings), so
    |pre_gpu - ref| <= (K * 2^-23 * sum |products|) * s_tok * alpha + 2^-22 |ref|.
    Returns the largest error as a fraction of its bound."""
    K = aq.shape[1] * 2
    sabs = _abs_products(aq, asf, q1, s1)
    scale = np.asarray(adec, np.float64).reshape(-1, 1) * np.asarray(alpha_rows, np.float64)
    bound = K * 2.0 ** -23 * sabs * scale + 2.0 ** -22 * np.abs(ref) + 1e-300
    d = np.abs(np.asarray(pre_gpu, np.float64) - ref)
    assert np.all(d <= bound), float((d / bound).max())
    return float((d / bound).max())


def check_down(y_gpu, ref, hq, hsf, q2, s2, alpha2, c2=1.0):
    """GEMM2 (BF16 expert outputs) of the GPU against oracle.expert_down_projection of the same
    intermediate: the pre-rounding values differ by at most (I * 2^-23 * sum |products| + 2^-22
    |ref|) * fl32(1/c2) * alpha2, so after the BF16 rounding by at most that plus one BF16 step.
    Returns (elements that differ, elements, largest error as a fraction of its bound)."""
    I = hq.shape[1] * 2
    sabs = _abs_products(hq, hsf, q2, s2)
    scale = float(np.float32(1) / np.float32(c2)) * float(alpha2)
    bound = (I * 2.0 ** -23 * sabs + 2.0 ** -22 * np.abs(ref)) * scale + ulp_bf16(ref)
    d = np.abs(np.asarray(y_gpu, np.float64) - ref)
    assert np.all(d <= bound), float((d / bound).max())
    return int(np.count_nonzero(d)), d.size, float((d / bound).max())
