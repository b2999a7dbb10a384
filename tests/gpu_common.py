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
