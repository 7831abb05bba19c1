"""Seeded synthetic inputs for the fixed-order row softmax workloads.

This module only draws random numbers and lays them out; it holds none of the
softmax arithmetic.  Both sides use it: the HIP library's tests and benchmark
(on the GPU) and the CPU oracle's checks (on host copies of the same bytes).

Every generator takes a seed and a device and returns torch tensors in the
layouts the library takes: scores / probabilities / gradients as
``[B, H, Sq, N]`` row-major (bf16 or fp32), an additive fp32 mask, per-head fp32
sink logits.  The workloads follow the joint image+text attention shapes of
RL-Kernel PR #453 (16,384 rows of 4,096 image + 256 text keys) and the causal
sink setting of TransformerEngine PR #678; none of the pages ships data, so
all values are drawn here.
"""
import math

import torch

__all__ = [
    "gen", "normal", "grad_check_fp32", "rows_with_outliers_bf16", "joint_attention_bf16", "batch_sweep_fp32",
    "causal_sink_bf16", "long_context_bf16", "synthetic_bwd_inputs", "to_numpy_bits",
    "from_numpy_bits",
]


def gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std, seed, device, dtype=torch.float32):
    """i.i.d. N(0, std^2) drawn in fp32, then rounded (RNE) to ``dtype``."""
    z = torch.randn(shape, generator=gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        z.mul_(float(std))
    return z.to(dtype)


def grad_check_fp32(seed=1, device="cpu", B=2, H=4, S=257, N=257):
    """fp32 scores [B,H,S,N] ~ N(0, 3^2) and upstream gradient ~ N(0, 1)."""
    s = normal((B, H, S, N), 3.0, seed, device)
    g = normal((B, H, S, N), 1.0, seed + 1, device)
    return s, g


def rows_with_outliers_bf16(seed=2, device="cpu", rows=16384, N=4352, outlier_frac=0.001, outlier_mult=8.0):
    """bf16 scores [1,1,rows,N]: z ~ N(0,1) in fp32, multiplied by sqrt(128)
    then by 1/sqrt(128) (the QK scaling of a 128-wide head, done as two fp32
    roundings); exactly round(outlier_frac * E) positions, drawn without
    replacement, multiplied by ``outlier_mult``; then RNE to bf16."""
    E = rows * N
    z = normal((E,), 1.0, seed, device)
    z.mul_(math.sqrt(128.0)).mul_(1.0 / math.sqrt(128.0))
    k = int(round(outlier_frac * E))
    idx = torch.randperm(E, generator=gen(seed + 7, device), device=device)[:k]
    z[idx] = z[idx] * outlier_mult
    return z.to(torch.bfloat16).view(1, 1, rows, N)


def joint_attention_bf16(seed=3, device="cpu", B=1, H=24, S=4352, N=4352, std=2.0, max_pad=255):
    """Joint image+text attention: bf16 scores [B,H,S,N] ~ N(0, std^2); per
    batch entry a text-padding length pad_b ~ U{0..max_pad}, the additive fp32
    mask [B, N] is -inf on the last pad_b keys and 0 elsewhere (broadcast over
    heads and queries: strides (N, 0, 0)); bf16 dP ~ N(0,1)."""
    s = normal((B, H, S, N), std, seed, device, torch.bfloat16)
    g = normal((B, H, S, N), 1.0, seed + 1, device, torch.bfloat16)
    pads = torch.randint(0, max_pad + 1, (B,), generator=gen(seed + 2, "cpu"))
    mask = torch.zeros((B, N), dtype=torch.float32)
    for b in range(B):
        p = int(pads[b])
        if p:
            mask[b, N - p:] = float("-inf")
    return s, mask.to(device), g, [int(p) for p in pads]


def batch_sweep_fp32(n, seed_block=40, seed=41, device="cpu", H=32, N=8449, place_seed=42):
    """Batch-invariance sweep: fp32 [n, H, 1, N].  A fixed block of H rows
    (scores and dP ~ N(0,1) from ``seed_block``) sits at batch index
    p ~ U{0..n-1} (drawn from ``place_seed`` and n); the other rows are drawn
    from a per-n seed.  Returns (scores, dP, p)."""
    blk_s = normal((1, H, 1, N), 1.0, seed_block, device)
    blk_g = normal((1, H, 1, N), 1.0, seed_block + 1, device)
    s = normal((n, H, 1, N), 1.0, seed * 1000 + n, device)
    g = normal((n, H, 1, N), 1.0, seed * 1000 + n + 500, device)
    p = int(torch.randint(0, n, (1,), generator=gen(place_seed * 1000 + n, "cpu")))
    s[p:p + 1] = blk_s
    g[p:p + 1] = blk_g
    return s, g, p


def causal_sink_bf16(seed=5, device="cpu", B=1, H=32, S=8192, N=None):
    """Causal self-attention: bf16 scores [B,H,S,S] ~ N(0,1) with -inf where
    key > query (the causal condition key <= Skv - Sq + query with Sq = Skv),
    per-head fp32 sink logits ~ N(0,1), bf16 dP ~ N(0,1).  The -inf fill runs
    per head to keep the temporary small."""
    N = S if N is None else N
    s = normal((B, H, S, N), 1.0, seed, device, torch.bfloat16)
    qi = torch.arange(S, device=device).view(S, 1)
    kj = torch.arange(N, device=device).view(1, N)
    upper = kj > (N - S) + qi
    ninf = torch.tensor(float("-inf"), dtype=torch.bfloat16, device=device)
    for b in range(B):
        for h in range(H):
            s[b, h].masked_fill_(upper, ninf)
    sink = normal((H,), 1.0, seed + 2, device)
    g = normal((B, H, S, N), 1.0, seed + 1, device, torch.bfloat16)
    return s, sink, g


def long_context_bf16(seed=7, device="cpu", B=1, H=16, S=512, N=65536, std=2.0):
    """Long-context rows: bf16 scores [B,H,S,N] ~ N(0, std^2) and dP ~ N(0,1),
    S queries at the end of N keys (the causal condition key <= N - S + q is
    applied by the library's flag, not written into the scores)."""
    s = normal((B, H, S, N), std, seed, device, torch.bfloat16)
    g = normal((B, H, S, N), 1.0, seed + 1, device, torch.bfloat16)
    return s, g


def synthetic_bwd_inputs(shape, dtype, seed, device, with_sink=False, zero_upper=False):
    """Stand-alone inputs for the backward pass: probabilities P >= 0 drawn as
    |N(0,1)| * 2/N (so a row sums to about 1.6), gradients dP ~ N(0,1), and per
    row p_sink ~ U[0,1).  ``zero_upper`` zeroes P where key > query (the
    causal pattern) to exercise signed zeros in dS."""
    B, H, S, N = shape
    P = normal(shape, 1.0, seed, device).abs_().mul_(2.0 / N)
    if zero_upper:
        qi = torch.arange(S, device=device).view(S, 1)
        kj = torch.arange(N, device=device).view(1, N)
        P.masked_fill_((kj > (N - S) + qi).view(1, 1, S, N), 0.0)
    P = P.to(dtype)
    g = normal(shape, 1.0, seed + 1, device, dtype)
    ps = None
    if with_sink:
        ps = torch.rand((B * H * S,), generator=gen(seed + 2, device), device=device)
    return P, g, ps


def to_numpy_bits(t: torch.Tensor):
    """Host numpy view of a tensor's bytes: bf16 as uint16, fp16 as float16,
    fp32 as float32."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype in (torch.float32, torch.float16):
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def from_numpy_bits(a, device="cpu"):
    """Inverse of :func:`to_numpy_bits`."""
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view("int16").copy()).view(torch.bfloat16).to(device)
    if a.dtype in (np.float32, np.float16):
        return torch.from_numpy(a.copy()).to(device)
    raise TypeError(f"unsupported dtype {a.dtype}")
