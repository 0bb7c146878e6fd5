"""Seeded synthetic workloads for the chunked GRPO policy loss.

This module only draws inputs.  It holds none of the loss arithmetic, so the
float64 oracle and the HIP path can both be fed from it without sharing any
of the method's code.

The workload table mirrors the shapes the pages discuss: a Qwen2.5-1.5B-sized
LM head (Unsloth "Long-context GRPO" blog, opening section: GRPO for the 1.5B
Qwen model in 5 GB), a Llama-3.1-8B-sized head at 20K context with eight
generations per prompt (same blog, section "90% less VRAM for long context"),
and a gpt-oss-20b-sized head (Unsloth docs "GRPO with 7x longer context",
section "Flattened sequence length chunking").  No model weights or datasets
are used: every tensor below is drawn from a seeded generator.

Recipe (all workloads):
  * H      ~ N(0, 1) per element, then each row divided by its RMS
             (h / sqrt(mean(h^2)), no gain, no epsilon), then cast to dtype.
  * H_ref  = cast(float32(H) + N(0, 0.01)); not re-normalised.
  * W      ~ N(0, 0.02) of shape [V, d], cast to dtype.
  * y      uniform in [0, V), or (targets="softmax") one draw per token from
             softmax(W h / 1.0) using the Gumbel-max construction
             argmax_v(z_v + g_v), g = -log(-log(u)), u ~ U[0, 1).
  * rewards uniform integers in {0, 1, 2, 3}, one per sequence, as float32.
  * mask   prefix mask per sequence: length uniform in [len_lo, len_hi]
             (inclusive), m[b, j] = 1 iff j < length_b.
Each tensor has its own torch.Generator seeded with (seed, tensor index), so
one tensor's draw never shifts another's.  Values depend on the device the
generator runs on (CPU and GPU Philox streams differ); a test always feeds the
oracle the very tensors it hands the GPU path.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

BETA = 0.04
EPS = 1e-4


@dataclass(frozen=True)
class Workload:
    name: str
    prompts: int          # P
    G: int                # generations per prompt (group size)
    L: int                # padded completion length
    d: int                # hidden size
    V: int                # vocabulary size
    dtype: str            # "f32" or "bf16"
    chunk: int            # flattened tokens per chunk
    len_lo: int           # completion length range, inclusive
    len_hi: int
    targets: str = "uniform"   # "uniform" or "softmax"

    @property
    def B(self) -> int:
        return self.prompts * self.G

    @property
    def N(self) -> int:
        return self.B * self.L

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = [
    Workload("tiny-f32", 2, 4, 64, 256, 1024, "f32", 128, 32, 64),
    Workload("qwen2.5-1.5b-bf16", 4, 8, 1024, 1536, 151936, "bf16", 4096, 512, 1024),
    Workload("llama3.1-8b-bf16", 1, 8, 4096, 4096, 128256, "bf16", 4096, 2048, 4096),
    Workload("llama3.1-8b-20k-bf16", 1, 8, 20480, 4096, 128256, "bf16", 8192, 10240, 20480),
    Workload("gpt-oss-20b-16k-bf16", 1, 4, 16384, 2880, 201088, "bf16", 8192, 8192, 16384,
             "softmax"),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def _gen(seed: int, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + index * 7919) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _randn(shape, g, device, block_rows=8192):
    """float32 normals, drawn in row blocks to bound temporaries."""
    rows = shape[0]
    out = torch.empty(shape, dtype=torch.float32, device=device)
    for r0 in range(0, rows, block_rows):
        r1 = min(rows, r0 + block_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                                 device=device, dtype=torch.float32)
    return out


def draw_hidden(N, d, dtype, seed, device, index=0):
    g = _gen(seed, index, device)
    H = _randn((N, d), g, device)
    H.div_(H.square().mean(dim=1, keepdim=True).sqrt_())
    return H.to(dtype)


def perturb(H, sigma, seed, device, index=1):
    g = _gen(seed, index, device)
    noise = _randn(tuple(H.shape), g, device)
    return (H.float() + sigma * noise).to(H.dtype)


def draw_weight(V, d, dtype, seed, device, index=2):
    g = _gen(seed, index, device)
    return (0.02 * _randn((V, d), g, device)).to(dtype)


def draw_uniform_targets(N, V, seed, device, index=3):
    g = _gen(seed, index, device)
    return torch.randint(0, V, (N,), generator=g, device=device, dtype=torch.int64).to(torch.int32)


def draw_sampled_targets(H, W, seed, device, index=3, temperature=1.0, block=1024):
    """One draw per token from softmax(W h / T) via Gumbel-max, on `device`."""
    g = _gen(seed, index, device)
    Wf = W.float()
    N = H.shape[0]
    y = torch.empty(N, dtype=torch.int32, device=device)
    for t0 in range(0, N, block):
        t1 = min(N, t0 + block)
        hT = H[t0:t1].float().t().contiguous()          # [d, b]
        z = torch.mm(Wf, hT) / temperature               # [V, b]
        u = torch.rand(z.shape, generator=g, device=device, dtype=torch.float32)
        z.add_(-torch.log(-torch.log(u)))
        y[t0:t1] = z.argmax(dim=0).to(torch.int32)
    return y


def draw_rewards(B, seed, device, index=4):
    g = _gen(seed, index, device)
    return torch.randint(0, 4, (B,), generator=g, device=device).to(torch.float32)


def draw_mask(B, L, lo, hi, seed, device, index=5):
    g = _gen(seed, index, device)
    lengths = torch.randint(lo, hi + 1, (B,), generator=g, device=device)
    j = torch.arange(L, device=device)
    return (j[None, :] < lengths[:, None]).to(torch.uint8).reshape(-1)


def generate(w: Workload, seed: int = 0, device="cpu", with_ref=True):
    """All inputs of one workload as torch tensors on `device`."""
    H = draw_hidden(w.N, w.d, w.torch_dtype, seed, device)
    H_ref = perturb(H, 0.01, seed, device) if with_ref else None
    W = draw_weight(w.V, w.d, w.torch_dtype, seed, device)
    if w.targets == "softmax":
        y = draw_sampled_targets(H, W, seed, device)
    else:
        y = draw_uniform_targets(w.N, w.V, seed, device)
    rewards = draw_rewards(w.B, seed, device)
    mask = draw_mask(w.B, w.L, w.len_lo, w.len_hi, seed, device)
    return dict(H=H, H_ref=H_ref, W=W, y=y, rewards=rewards, mask=mask)
