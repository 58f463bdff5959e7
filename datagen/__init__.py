"""Seeded synthetic inputs shared by the GPU path, the oracle, the tests and the bench.

This module only draws and rounds random numbers; it contains none of the attention
arithmetic (no feature map, no state, no normalisation), so that the oracle and the HIP
path share nothing beyond their inputs.

Recipe (the same for every workload):
  * draws are IID standard normal in float64 from NumPy's ``Generator(PCG64(seed))``,
    taken in the order q, k, v, each as one full C-order tensor;
  * each tensor is multiplied by ``scale`` (1/sqrt(d) for the workloads whose inputs are
    N(0, 1/d), 1.0 otherwise);
  * the result is rounded once, to nearest-even, to the input dtype (bfloat16 or float32).
    That rounded tensor is the one canonical input: the GPU receives it as is and the
    oracle receives its exact float64 upcast.

The pages publish no dataset and no benchmark suite; these draws stand in for the
"IID Gaussian q, k, v" workloads the sizes below describe.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def normal(shape, seed: int, scale: float = 1.0, dtype: str = "bf16") -> torch.Tensor:
    """One tensor of IID N(0, scale^2) values, rounded to ``dtype`` (CPU tensor)."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=tuple(shape), dtype=np.float64)
    if scale != 1.0:
        x *= scale
    return torch.from_numpy(x).to(DTYPES[dtype])


def qkv(B: int, H: int, N: int, d: int, dv: int, seed: int, scale: float = 1.0,
        dtype: str = "bf16"):
    """q, k: [B,H,N,d]; v: [B,H,N,dv]; drawn from one stream in the order q, k, v."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for shape in ((B, H, N, d), (B, H, N, d), (B, H, N, dv)):
        x = g.standard_normal(size=shape, dtype=np.float64)
        if scale != 1.0:
            x *= scale
        out.append(torch.from_numpy(x).to(DTYPES[dtype]))
    return tuple(out)


def normal_cuda(shape, seed: int, scale: float = 1.0, dtype: str = "f32",
                device: str = "cuda") -> torch.Tensor:
    """One tensor of IID N(0, scale^2) values drawn on the device (torch's seeded Philox
    generator), rounded to ``dtype``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(DTYPES[dtype])


def qkv_cuda(B: int, H: int, N: int, d: int, dv: int, seed: int, scale: float = 1.0,
             dtype: str = "bf16", device: str = "cuda"):
    """Large inputs drawn directly on the device with torch's seeded Philox generator.

    Used where a host draw would take minutes (the decode workload's per-step tokens and
    its 4096-token prior). Same distribution as :func:`qkv`, different stream; a test that
    needs the oracle on such data copies the device tensors back to the host.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    for shape in ((B, H, N, d), (B, H, N, d), (B, H, N, dv)):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        out.append(x.to(DTYPES[dtype]))
    return tuple(out)


# The decode workload's draws (all on the device, torch's seeded Philox generator):
#   * the prior: for each block of DECODE_PRIOR_BLOCK batch rows starting at row b0, one qkv_cuda
#     call of [block, H, prior, d] with seed = seed * 1000 + b0 (its q is drawn and unused);
#     the starting state of those heads is S0 = sum_t phi(k_t) v_t^T, z0 = sum_t phi(k_t)
#     over the block's prior tokens;
#   * the step tokens: one qkv_cuda call of [steps, B * H, 1, d] with seed = seed + 1, viewed
#     as [steps, B, H, d] (token t of head (b, h) is row t of that view).
DECODE_PRIOR_BLOCK = 16


def decode_prior(w: "Workload", b0: int, device: str = "cuda"):
    """k, v [blk, H, prior, d] of the prior tokens of batch rows b0 .. b0 + blk - 1 (blk =
    DECODE_PRIOR_BLOCK, or fewer at the end) of decode workload ``w``."""
    blk = min(DECODE_PRIOR_BLOCK, w.B - b0)
    _, k, v = qkv_cuda(blk, w.H, w.prior, w.d, w.dv, w.seed * 1000 + b0, w.scale, w.dtype,
                       device=device)
    return k, v


def decode_tokens(w: "Workload", steps: int, device: str = "cuda"):
    """q, k, v [steps, B, H, d] of the per-step tokens of decode workload ``w``."""
    toks = qkv_cuda(steps, w.B * w.H, 1, w.d, w.dv, w.seed + 1, w.scale, w.dtype, device=device)
    return tuple(x.view(steps, w.B, w.H, -1) for x in toks)


def projections(m: int, d: int, seed: int, dtype: str = "bf16") -> torch.Tensor:
    """Random-feature projections W [m, d]: IID standard normal rows, rounded to ``dtype``
    (the draw the unbiasedness of positive random features assumes)."""
    return normal((m, d), seed, 1.0, dtype)


def positive(shape, seed: int, scale: float = 1.0, dtype: str = "bf16", floor: float = 0.05):
    """IID |N(0, scale^2)| + floor, rounded to ``dtype``: strictly positive inputs for the
    forms that take q and k as features as given."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = np.abs(g.standard_normal(size=tuple(shape), dtype=np.float64)) * scale + floor
    return torch.from_numpy(x).to(DTYPES[dtype])


def decay_rates(H: int) -> torch.Tensor:
    """Per-head decays for the decayed recurrence, one per head on a multi-scale ladder:
    gamma_h = 1 - 2^-(5 + h) (0.96875 for head 0, closer to 1 for each later head), float32."""
    return torch.tensor([1.0 - 2.0 ** -(5 + h) for h in range(H)], dtype=torch.float32)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 host copy of a bf16/fp32 tensor (both embed exactly in float64). A device
    tensor is widened where it lives and then copied (the host-side widening of the large
    device-drawn tensors is the slow part otherwise); the value of every element is the same
    either way."""
    t = t.detach()
    if t.is_cuda:
        return t.to(torch.float64).cpu().numpy()
    return t.to(torch.float64).numpy()


@dataclass(frozen=True)
class Workload:
    name: str
    form: str          # "causal" | "global" | "decode"
    B: int
    H: int
    N: int
    d: int
    dv: int
    dtype: str
    scale: float
    seed: int
    chunk: int = 0
    steps: int = 1     # decode only
    prior: int = 0     # decode only: tokens summed into the starting state

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.N


# The five workloads: sizes, dtypes and value distributions of the linear-attention
# workloads this library is measured on (seed = 1000 + workload number).
WORKLOADS = {
    1: Workload("causal_b1h1n64_d16_f32", "causal", 1, 1, 64, 16, 16, "f32", 1.0, 1001),
    2: Workload("causal_b4h8n2048_d64_bf16", "causal", 4, 8, 2048, 64, 64, "bf16",
                1.0 / math.sqrt(64), 1002, chunk=64),
    3: Workload("causal_b2h16n8192_d128_bf16", "causal", 2, 16, 8192, 128, 128, "bf16",
                1.0 / math.sqrt(128), 1003),
    4: Workload("global_b1h8n100000_d128_bf16", "global", 1, 8, 100000, 128, 128, "bf16",
                1.0 / math.sqrt(128), 1004),
    5: Workload("decode_b256h32_d128_bf16_state4096", "decode", 256, 32, 1, 128, 128, "bf16",
                1.0 / math.sqrt(128), 1005, steps=1000, prior=4096),
}

# Positive random features over the causal workload's inputs: q and k of workload 3 mapped
# with m = 128 standard normal projections (seed 1006), then causal attention over the
# features.
RF_WORKLOAD = {"name": "favor_causal_b2h16n8192_d128_m128_bf16", "base": 3, "m": 128,
               "seed": 1006}

# The decayed recurrence in its retention form (identity map, no denominator) over the causal
# workload's inputs, per-head decays from decay_rates(16).
DECAY_WORKLOAD = {"name": "retention_causal_b2h16n8192_d128_bf16", "base": 3}
