"""Seeded input generation.

All draws use one torch.Generator on the requested device, seeded from the
workload key and the seed, in a fixed order, so a (workload, seed, device,
T, B) tuple always yields the same tensors.  CPU and GPU generators give
different streams; a test that compares both sides generates once and hands
the same tensors to each.

Distributions (N(mu, sigma) has standard deviation sigma):
  q, k   : N(0, 1) per element, then scaled to unit L2 norm per (t, b, h)
  v      : N(0, 1)
  beta   : 2 * sigmoid(N(0, 1)) per (t, b, h)           (write gate in (0, 2))
  alpha  : "softplus_step": exp(-softplus(x)), x ~ N(-3, 1) per (t, b, h)
           "uniform_head" : one alpha_h ~ U[lo, hi) per head, constant in (t, b)
           "ssd"          : dt ~ softplus(N(0, 1)) per (t, b, h), A_h ~ U(1, 16),
                            alpha = exp(-dt * A_h) and beta = dt
           "kda_channel"  : exp(-softplus(x)), x ~ N(-4, 1.5) per (t, b, h, j)
bf16 workloads round q, k and v to bfloat16 after normalisation.
"""
import zlib

import torch
import torch.nn.functional as F

from .configs import Workload


def _seed_for(w: Workload, seed: int) -> int:
    return (zlib.crc32(w.key.encode()) * 1000003 + int(seed)) & 0x7FFFFFFFFFFFFFFF


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def make_inputs(w: Workload, seed: int = 0, device="cpu", T=None, B=None):
    """Draw all T decode steps of workload ``w``.

    Returns a dict of tensors with a leading time axis:
      q, k  [T, B, H, dk]   fp32 (bf16 if w.in_bf16)
      v     [T, B, H, dv]   fp32 (bf16 if w.in_bf16)
      alpha [T, B, H] fp32, or [T, B, H, dk] for per-channel decay
      beta  [T, B, H] fp32
    ``T`` and ``B`` override the workload's horizon and batch (the per-head
    draws, alpha_h and A_h, do not depend on them).
    """
    T = w.T if T is None else int(T)
    B = w.B if B is None else int(B)
    H, dk, dv = w.H, w.dk, w.dv
    g = torch.Generator(device=device)
    g.manual_seed(_seed_for(w, seed))
    f32 = torch.float32

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=f32)

    def rand(*shape):
        return torch.rand(*shape, generator=g, device=device, dtype=f32)

    head_u = rand(H)                              # per-head uniform, drawn first
    if w.decay == "uniform_head":
        alpha_h = w.alpha_lo + (w.alpha_hi - w.alpha_lo) * head_u
        alpha = alpha_h.view(1, 1, H).expand(T, B, H).contiguous()
        beta = 2.0 * torch.sigmoid(randn(T, B, H))
    elif w.decay == "softplus_step":
        alpha = torch.exp(-F.softplus(randn(T, B, H) - 3.0))
        beta = 2.0 * torch.sigmoid(randn(T, B, H))
    elif w.decay == "ssd":
        A_h = 1.0 + 15.0 * head_u
        dt = F.softplus(randn(T, B, H))
        alpha = torch.exp(-dt * A_h.view(1, 1, H))
        beta = dt
    elif w.decay == "kda_channel":
        alpha = torch.exp(-F.softplus(1.5 * randn(T, B, H, dk) - 4.0))
        beta = 2.0 * torch.sigmoid(randn(T, B, H))
    else:
        raise ValueError(f"unknown decay kind {w.decay!r}")

    q = _unit(randn(T, B, H, dk))
    k = _unit(randn(T, B, H, dk))
    v = randn(T, B, H, dv)
    if w.in_bf16:
        q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "alpha": alpha.contiguous(), "beta": beta.contiguous()}


def make_random_int_state(n_units: int, dv: int, dk: int, r: int, seed: int = 0,
                          scale_lo: float = 1e-3, scale_hi: float = 1e-1):
    """A random quantized state: codes uniform in [-r, r], scales log-uniform.

    Used as a non-zero starting state for the quantized step.  Returns
    (codes int32 [n, dv, dk], scales fp32 [n, dv]) on the CPU.
    """
    g = torch.Generator().manual_seed(int(seed) * 7919 + r)
    codes = torch.randint(-r, r + 1, (n_units, dv, dk), generator=g, dtype=torch.int32)
    lo, hi = torch.log(torch.tensor(scale_lo)), torch.log(torch.tensor(scale_hi))
    scales = torch.exp(lo + (hi - lo) * torch.rand(n_units, dv, generator=g)).to(torch.float32)
    return codes, scales
