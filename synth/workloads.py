"""The five workload shapes and their seeded input recipes.

Recipe (fixed draw order, numpy PCG64 ``default_rng``):
* activations x [M, H]: standard normals drawn in float64, rounded to float32 then BF16 (RNE);
* router: logits [M, E] ~ N(0, 1) (prefill adds a per-expert bias ~ N(0, 0.5) drawn after the
  logits); softmax over experts; the top_k distinct experts by descending probability
  (stable argsort); weights = chosen probabilities renormalised to sum to one, as float32;
* skewed workload: a random permutation of the experts, then per token top_k distinct ranks
  1..E drawn without replacement with probability proportional to rank**-1.2 (Gumbel top-k on
  -1.2*ln(rank)); the expert is perm[rank-1]; weights = softmax of top_k N(0, 1) draws;
* weights: per expert and tensor, ``torch.randn`` on the requested device with a generator
  seeded from (seed, tensor id, expert), times 0.02, rounded to BF16.  CPU and GPU generators
  give different numbers; tests that compare the GPU path with the oracle draw on the GPU and
  hand the same tensors to both.
"""

from dataclasses import dataclass, field

import numpy as np


# Activation names in the order of their codes in the C ABI and in the oracle.
ACT_NAMES = ("swiglu", "relu2", "geglu", "gelu", "relu", "silu", "identity")


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    H: int
    I: int
    E: int
    top_k: int
    block_m: int
    act: str = "swiglu"              # one of ACT_NAMES; "swiglu" and "geglu" are gated
    routing: str = "softmax"         # "softmax", "softmax_bias", "zipf"
    local_offset: int = 0
    num_local: int = -1              # -1: all experts are local
    zipf_s: float = 1.2
    bias_std: float = 0.5
    extra_block_m: tuple = field(default_factory=tuple)

    @property
    def n_local(self):
        return self.E if self.num_local < 0 else self.num_local

    @property
    def gated(self):
        return self.act in ("swiglu", "geglu")

    @property
    def act_code(self):
        return ACT_NAMES.index(self.act)

    @property
    def N1(self):
        return 2 * self.I if self.gated else self.I


WORKLOADS = {
    # Tiny parity case; segments padded to block_m = 8 and, separately, to 128 rows.
    "tiny": Workload("tiny", M=16, H=256, I=128, E=8, top_k=2, block_m=8, extra_block_m=(128,)),
    # Low-latency decode shape H=2048 / I=512 / top-10 (FrostLowLatencyConfig shape list).
    "decode_ll": Workload("decode_ll", M=4, H=2048, I=512, E=128, top_k=10, block_m=8),
    # Decode shape H=7168 / I=2048 / top-8, M=8 tokens.
    "decode": Workload("decode", M=8, H=7168, I=2048, E=256, top_k=8, block_m=8),
    # Prefill, same expert shape, 4096 tokens, segments padded to 128 rows.
    "prefill": Workload("prefill", M=4096, H=7168, I=2048, E=256, top_k=8, block_m=128,
                        routing="softmax_bias"),
    # Skewed non-gated squared-ReLU: 288 experts, experts 0..143 local.
    "skewed_relu2": Workload("skewed_relu2", M=16384, H=4096, I=1536, E=288, top_k=6,
                             block_m=128, act="relu2", routing="zipf", local_offset=0,
                             num_local=144),
}


def bf16_bits(a_f64):
    """float64 array -> uint16 BF16 bit patterns via float32 (both steps round to nearest even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a_f64, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_activations(wl, seed=0, M=None):
    """x [M, H] as uint16 BF16 bits."""
    rng = np.random.default_rng([seed, 1])
    M = wl.M if M is None else M
    return bf16_bits(rng.standard_normal((M, wl.H)))


def make_routing(wl, seed=0, M=None):
    """(topk_ids int32 [M, top_k], topk_weights float32 [M, top_k])."""
    rng = np.random.default_rng([seed, 2])
    M = wl.M if M is None else M
    k = wl.top_k
    if wl.routing in ("softmax", "softmax_bias"):
        logits = rng.standard_normal((M, wl.E))
        if wl.routing == "softmax_bias":
            logits = logits + wl.bias_std * rng.standard_normal(wl.E)[None, :]
        z = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        ids = np.argsort(-p, axis=1, kind="stable")[:, :k]
        w = np.take_along_axis(p, ids, axis=1)
        w = w / w.sum(axis=1, keepdims=True)
        return ids.astype(np.int32), w.astype(np.float32)
    if wl.routing == "zipf":
        perm = rng.permutation(wl.E)
        ranks = np.arange(1, wl.E + 1, dtype=np.float64)
        logw = -wl.zipf_s * np.log(ranks)
        g = rng.gumbel(size=(M, wl.E))
        chosen = np.argsort(-(logw[None, :] + g), axis=1, kind="stable")[:, :k]   # rank - 1
        ids = perm[chosen]
        s = rng.standard_normal((M, k))
        z = np.exp(s - s.max(axis=1, keepdims=True))
        w = z / z.sum(axis=1, keepdims=True)
        return ids.astype(np.int32), w.astype(np.float32)
    raise ValueError(wl.routing)


def _expert_generator(seed, tensor_id, e, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(tensor_id) * 10_007 + int(e))
    return g


def make_expert_weight(wl, tensor_id, e, seed=0, device="cpu"):
    """One expert's BF16 weight as a torch tensor on ``device``.

    tensor_id 1: W1 [N1, H] ([gate; up] rows when gated); tensor_id 2: W2 [H, I].
    """
    import torch

    shape = (wl.N1, wl.H) if tensor_id == 1 else (wl.H, wl.I)
    g = _expert_generator(seed, tensor_id, e, device)
    w = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * 0.02
    return w.to(torch.bfloat16)


def make_weights(wl, seed=0, device="cpu", experts=None):
    """Stacked BF16 weights (W1 [E', N1, H], W2 [E', H, I]) for the local experts, or for the
    given list of global expert ids, in that order."""
    import torch

    if experts is None:
        experts = [wl.local_offset + i for i in range(wl.n_local)]     # global expert ids
    experts = list(experts)
    w1 = torch.empty((len(experts), wl.N1, wl.H), dtype=torch.bfloat16, device=device)
    w2 = torch.empty((len(experts), wl.H, wl.I), dtype=torch.bfloat16, device=device)
    for i, e in enumerate(experts):
        w1[i] = make_expert_weight(wl, 1, e, seed, device)
        w2[i] = make_expert_weight(wl, 2, e, seed, device)
    return w1, w2


def to_bits(t):
    """torch BF16 tensor -> numpy uint16 bits (host copy)."""
    import torch

    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16).copy()
