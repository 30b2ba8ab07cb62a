"""Seeded synthetic inputs for the selection and decode workloads.

This module only draws numbers: it holds none of the selection or attention
arithmetic, so the HIP library and the CPU reference can both be fed from it
without sharing any of the method.  Every draw goes through a
``torch.Generator`` seeded from (workload id, seed), on the device asked for.
The same seed on a different device gives different (but equally
distributed) numbers, so a comparison always draws once and copies.

Workloads (the shapes of the pages' top-k and decode settings, synthetic):
  sel-4k     1 x 4096 fp32 Uniform[0,1), k = 64
  vocab-128k 256 x 131072 bf16 ~ N(0, 2^2), k = 64
  mha-32k    decode B16 H32 D128 L32768, 64 keys per head planted at cosine
             0.8 to the query
  gqa-128k   decode B4 Hq32 Hkv8 D128 L131072, 1% of keys scaled 3x
  wide-1m    64 x 2^20 fp32 Uniform[0,1), k = 8192; odd rows hold their top-k
             in the fewest residue classes modulo b (worst case for buckets)
  ar1        fp32 AR(1) Gaussian rows of a chosen correlation (interleaved
             against contiguous bucket assignment)
  vocab-sampling  64 x 128256 fp32 ~ N(0, 2^2), k = 256 (LLM vocabulary
             sampling shape of the runtime/accuracy trade-off)
  kg-2.65m   128 x 2653751 fp32 ~ N(0, 1), k = 100 (knowledge-graph link
             prediction shape of the same trade-off)
  sweep      fp32 N(0, 1) rows of the runtime-versus-(n, k) sweep at m = 1
             and m = 256
"""

import math

import numpy as np
import torch

_WORKLOAD_IDS = {"sel-4k": 1, "vocab-128k": 2, "mha-32k": 3, "gqa-128k": 4, "wide-1m": 5, "ar1": 6, "misc": 9,
                 "vocab-sampling": 10, "kg-2.65m": 11, "sweep": 12}


def generator(workload, seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(2412 * 1_000_003 + _WORKLOAD_IDS[workload] * 10_007 + int(seed))
    return g


def rows_uniform(m, n, seed, device="cpu", workload="sel-4k"):
    """[m, n] fp32 Uniform[0, 1)."""
    g = generator(workload, seed, device)
    return torch.rand((m, n), generator=g, device=device, dtype=torch.float32)


def rows_normal_bf16(m, n, std, seed, device="cpu", workload="vocab-128k"):
    """[m, n] bf16 draws of std * N(0, 1), rounded to nearest even."""
    g = generator(workload, seed, device)
    x = torch.randn((m, n), generator=g, device=device, dtype=torch.float32)
    return (x * std).to(torch.bfloat16)


def rows_normal(m, n, std, seed, device="cpu", workload="kg-2.65m"):
    """[m, n] fp32 draws of std * N(0, 1)."""
    g = generator(workload, seed, device)
    x = torch.randn((m, n), generator=g, device=device, dtype=torch.float32)
    return x.mul_(std) if std != 1.0 else x


def rows_planted_residues(m, n, b, k, seed, device="cpu", workload="wide-1m"):
    """[m, n] fp32 Uniform[0, 1); every odd row carries 1 + Uniform[0, 1) on
    the positions whose residue modulo b is below ceil(k / (n / b)), so its
    k largest values all sit in the fewest possible interleaved buckets."""
    g = generator(workload, seed, device)
    x = torch.rand((m, n), generator=g, device=device, dtype=torch.float32)
    s = n // b
    n_res = -(-k // s)
    pos = torch.arange(n, device=device)
    mask = (pos % b) < n_res
    lift = 1.0 + torch.rand((m, int(mask.sum())), generator=g, device=device, dtype=torch.float32)
    odd = torch.arange(m, device=device) % 2 == 1
    x_odd = x[odd]
    x_odd[:, mask] = lift[odd]
    x[odd] = x_odd
    return x


def rows_ar1(m, n, rho, seed, device="cpu", workload="ar1"):
    """[m, n] fp32 stationary AR(1) Gaussian rows: x_0 ~ N(0, 1) and
    x_i = rho * x_{i-1} + sqrt(1 - rho^2) * e_i with e_i ~ N(0, 1) (the
    correlated-Gaussian inputs of the interleaved / contiguous comparison).
    The recurrence runs on the host in float64 (an IIR filter), then the rows
    go to `device`."""
    from scipy.signal import lfilter

    g = generator(workload, seed, "cpu")
    e = torch.randn((m, n), generator=g, dtype=torch.float64).numpy()
    c = math.sqrt(1.0 - rho * rho)
    if c > 0:
        e[:, 0] /= c  # so that x_0 = e_0 has unit variance
    x = lfilter([c], [1.0, -rho], e, axis=1) if c > 0 else np.repeat(e[:, :1], n, axis=1)
    return torch.from_numpy(x.astype(np.float32)).to(device)


def rows_ties_bf16(m, n, levels, seed, device="cpu"):
    """[m, n] bf16 drawn from a small set of levels (heavy ties), including
    both zeros, infinities and negative values."""
    g = generator("misc", seed, device)
    base = torch.tensor([-math.inf, -2.0, -0.0, 0.0, 0.5, 1.0, 3.0, math.inf], dtype=torch.float32)[:levels]
    pick = torch.randint(0, base.numel(), (m, n), generator=g, device=device)
    return base.to(device)[pick].to(torch.bfloat16)


def decode_mha(bsz, heads, ctx, d, n_plant, cosine, seed, device="cpu", workload="mha-32k"):
    """q [B, H, D], K, V [B, H, L, D] bf16 ~ N(0, 1); in every head n_plant
    distinct key rows are replaced by |K_p| (cosine * q_hat + sqrt(1 -
    cosine^2) * u_p) with u_p a random unit vector orthogonal to q (fp32,
    then rounded to bf16).  Returns (q, K, V, planted positions [B, H, P])."""
    g = generator(workload, seed, device)
    q = torch.randn((bsz, heads, d), generator=g, device=device, dtype=torch.float32)
    kbf = torch.empty((bsz, heads, ctx, d), device=device, dtype=torch.bfloat16)
    vbf = torch.empty_like(kbf)
    planted = torch.empty((bsz, heads, n_plant), device=device, dtype=torch.int64)
    sin = math.sqrt(1.0 - cosine * cosine)
    for bi in range(bsz):
        k0 = torch.randn((heads, ctx, d), generator=g, device=device, dtype=torch.float32)
        pos = torch.rand((heads, ctx), generator=g, device=device).topk(n_plant, dim=1).indices
        qh = q[bi] / q[bi].norm(dim=-1, keepdim=True)
        u = torch.randn((heads, n_plant, d), generator=g, device=device, dtype=torch.float32)
        u = u - (u * qh[:, None, :]).sum(-1, keepdim=True) * qh[:, None, :]
        u = u / u.norm(dim=-1, keepdim=True)
        rows = torch.gather(k0, 1, pos[:, :, None].expand(-1, -1, d))
        new = rows.norm(dim=-1, keepdim=True) * (cosine * qh[:, None, :] + sin * u)
        k0.scatter_(1, pos[:, :, None].expand(-1, -1, d), new)
        kbf[bi] = k0.to(torch.bfloat16)
        del k0
        vbf[bi] = torch.randn((heads, ctx, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        planted[bi] = pos
    return q.to(torch.bfloat16), kbf, vbf, planted


def decode_gqa(bsz, hq, hkv, ctx, d, frac, mult, seed, device="cpu", workload="gqa-128k"):
    """q [B, Hq, D], K, V [B, Hkv, L, D] bf16 ~ N(0, 1); in every (batch, KV
    head) floor(frac * L) distinct key rows are multiplied by `mult` in fp32
    before rounding.  Returns (q, K, V, scaled positions [B, Hkv, P])."""
    g = generator(workload, seed, device)
    q = torch.randn((bsz, hq, d), generator=g, device=device, dtype=torch.float32)
    n_scaled = int(math.floor(frac * ctx))
    kbf = torch.empty((bsz, hkv, ctx, d), device=device, dtype=torch.bfloat16)
    vbf = torch.empty_like(kbf)
    pos_all = torch.empty((bsz, hkv, max(n_scaled, 1)), device=device, dtype=torch.int64)
    for bi in range(bsz):
        k0 = torch.randn((hkv, ctx, d), generator=g, device=device, dtype=torch.float32)
        if n_scaled > 0:
            pos = torch.rand((hkv, ctx), generator=g, device=device).topk(n_scaled, dim=1).indices
            idx = pos[:, :, None].expand(-1, -1, d)
            k0.scatter_(1, idx, torch.gather(k0, 1, idx) * mult)
            pos_all[bi] = pos
        kbf[bi] = k0.to(torch.bfloat16)
        del k0
        vbf[bi] = torch.randn((hkv, ctx, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    return q.to(torch.bfloat16), kbf, vbf, pos_all


# Workload table: sizes of the selection and decode settings.
SELECTION = {
    "sel-4k": dict(m=1, n=4096, k=64, dtype="f32", modes=[(64, 1, False), (32, 2, True)]),
    "vocab-128k": dict(m=256, n=131072, k=64, dtype="bf16", modes=[(64, 1, False), (128, 2, True)]),
    "wide-1m": dict(m=64, n=1 << 20, k=8192, dtype="f32", modes=[(512, 16, True)]),
}
# Runtime/accuracy trade-off shapes: every (b, k_b) with k_b in {1, 2} and
# b * k_b from the smallest power of two >= k up to 8192, final exact top-k.
TRADEOFF = {
    "vocab-sampling": dict(m=64, n=128256, k=256, std=2.0),
    "kg-2.65m": dict(m=128, n=2653751, k=100, std=1.0),
}


def tradeoff_modes(k, max_cand=8192):
    modes = []
    for kb in (1, 2):
        b = 1
        while b * kb < k:
            b *= 2
        while b * kb <= max_cand:
            modes.append((b, kb))
            b *= 2
    return modes


# Runtime versus n and k (fp32 N(0, 1) rows).
SWEEP = dict(ms=(1, 256), log2n=(10, 12, 14, 16, 18, 20, 22), ks=(1, 16, 64, 256, 1024, 4096), max_bytes=1 << 30)
DECODE = {
    "mha-32k": dict(bsz=16, hq=32, hkv=32, ctx=32768, d=128, k_sel=512, b=256, kb=2),
    "gqa-128k": dict(bsz=4, hq=32, hkv=8, ctx=131072, d=128, k_sel=512, b=512, kb=4),
}
