"""Seeded synthetic inputs for the KDA operator.

This module is the only code shared by the oracle side and the GPU side: it draws
random tensors and holds none of the recurrence's arithmetic.  The recipe follows
the workload descriptions (all values synthetic; no dataset is involved):

* q ~ N(0, 1)
* k ~ N(0, 1), then L2-normalised over d_k per (b, t, h) in fp32
* v ~ N(0, 1)
* alpha = sigmoid(N(mu, 1)) per (b, t, h, channel); mu = 3 (mu = 4 for the
  1M-token long-retention case)
* beta = sigmoid(N(0, 1)) per (b, t, h)
* S0 = 0.1 * N(0, 1) (read as mean 0, variance 0.01), or zeros
* q, k, v are then rounded to bf16 (round-to-nearest-even) for the bf16 cases;
  alpha, beta and the state stay fp32.

Draw order is fixed (q, k, v, alpha, beta, S0) so a (seed, device) pair always
gives the same tensors.  Long sequences are generated in token slices, each with
its own seed (base seed + slice index), to bound transient memory.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    qkv_dtype: torch.dtype
    alpha_mu: float
    s0_std: float  # 0.0 means S0 = zeros
    chunk: int = 64
    decode_steps: int = 0  # > 0: a batched decode workload (T unused)


# The five workloads the operator is specified on.
WORKLOADS = {
    0: Workload("tiny-fp32", 1, 64, 1, 16, 16, torch.float32, 3.0, 0.0),
    1: Workload("prefill-4k", 1, 4096, 8, 128, 128, torch.bfloat16, 3.0, 0.1),
    2: Workload("prefill-64k", 2, 65536, 32, 128, 128, torch.bfloat16, 3.0, 0.1),
    3: Workload("prefill-1m", 1, 1048576, 32, 128, 128, torch.bfloat16, 4.0, 0.1),
    4: Workload("decode-b256", 256, 1, 32, 128, 128, torch.bfloat16, 3.0, 0.1,
                decode_steps=100),
}

SLICE_TOKENS = 65536


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _draw_tokens(B, T, H, dk, dv, qkv_dtype, alpha_mu, g, device):
    f32 = torch.float32
    q = torch.randn(B, T, H, dk, generator=g, device=device, dtype=f32)
    k = torch.randn(B, T, H, dk, generator=g, device=device, dtype=f32)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    v = torch.randn(B, T, H, dv, generator=g, device=device, dtype=f32)
    alpha = torch.sigmoid(torch.randn(B, T, H, dk, generator=g, device=device, dtype=f32) + alpha_mu)
    beta = torch.sigmoid(torch.randn(B, T, H, generator=g, device=device, dtype=f32))
    return q.to(qkv_dtype), k.to(qkv_dtype), v.to(qkv_dtype), alpha, beta


def make_state(B, H, dk, dv, std, seed, device):
    """fp32 state [B,H,dk,dv] = std * N(0,1) (zeros when std == 0)."""
    if std == 0.0:
        return torch.zeros(B, H, dk, dv, device=device, dtype=torch.float32)
    g = _gen(device, seed)
    return std * torch.randn(B, H, dk, dv, generator=g, device=device, dtype=torch.float32)


def make_prefill(B, T, H, dk, dv, qkv_dtype=torch.bfloat16, alpha_mu=3.0, s0_std=0.1,
                 seed=0, device="cpu", slice_tokens=SLICE_TOKENS):
    """Return dict(q, k, v, alpha, beta, S0) for a prefill call.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; alpha: [B,T,H,dk] f32; beta: [B,T,H] f32;
    S0: [B,H,dk,dv] f32 (zeros when s0_std == 0).
    """
    if T <= slice_tokens:
        g = _gen(device, seed)
        q, k, v, alpha, beta = _draw_tokens(B, T, H, dk, dv, qkv_dtype, alpha_mu, g, device)
    else:
        q = torch.empty(B, T, H, dk, device=device, dtype=qkv_dtype)
        k = torch.empty_like(q)
        v = torch.empty(B, T, H, dv, device=device, dtype=qkv_dtype)
        alpha = torch.empty(B, T, H, dk, device=device, dtype=torch.float32)
        beta = torch.empty(B, T, H, device=device, dtype=torch.float32)
        for si, t0 in enumerate(range(0, T, slice_tokens)):
            n = min(slice_tokens, T - t0)
            g = _gen(device, seed * 100003 + si)
            parts = _draw_tokens(B, n, H, dk, dv, qkv_dtype, alpha_mu, g, device)
            for dst, src in zip((q, k, v, alpha, beta), parts):
                dst[:, t0:t0 + n].copy_(src)
            del parts
    S0 = make_state(B, H, dk, dv, s0_std, seed + 7919, device)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)


def make_decode_token(B, H, dk, dv, qkv_dtype=torch.bfloat16, alpha_mu=3.0, seed=0, step=0,
                      device="cpu"):
    """Inputs for one decode step: q, k: [B,H,dk]; v: [B,H,dv]; alpha [B,H,dk]; beta [B,H]."""
    g = _gen(device, seed * 1000003 + step)
    q, k, v, alpha, beta = _draw_tokens(B, 1, H, dk, dv, qkv_dtype, alpha_mu, g, device)
    return dict(q=q[:, 0].contiguous(), k=k[:, 0].contiguous(), v=v[:, 0].contiguous(),
                alpha=alpha[:, 0].contiguous(), beta=beta[:, 0].contiguous())


def make_workload_prefill(idx, seed=0, device="cpu"):
    w = WORKLOADS[idx]
    return make_prefill(w.B, w.T, w.H, w.dk, w.dv, w.qkv_dtype, w.alpha_mu, w.s0_std,
                        seed=seed, device=device)


def make_gate(shape, H, qkv_dtype=torch.bfloat16, seed=0, device="cpu", z_mu=-4.5, z_std=0.4, a_std=0.1):
    """Gate inputs for the fused-gate calls: z ~ N(z_mu, z_std) of the given shape
    (its second-to-last axis is the head axis), rounded to qkv_dtype, and one
    log-scale per head A ~ N(0, a_std) in fp32.  The defaults give a mean log
    retention of about -0.074 per token (per-head means -0.18 .. -0.03), matching
    alpha = sigmoid(N(3, 1)) of the other workloads (-0.075); a smaller z_mu or
    a wider z_std gives faster-forgetting heads."""
    g = _gen(device, seed * 7919 + 13)
    z = (z_mu + z_std * torch.randn(*shape, generator=g, device=device, dtype=torch.float32)).to(qkv_dtype)
    A = a_std * torch.randn(H, generator=g, device=device, dtype=torch.float32)
    return z.contiguous(), A.contiguous()
