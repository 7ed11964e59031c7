"""Seeded synthetic inputs for the sliced-precision linear layer.

This module only *produces inputs*: Gaussian weights (with optional sparse
outliers), the c = 8-bit parent codes with one fp16 scale and zero point per
group made from those weights by a min-max asymmetric quantizer, and Gaussian
activations.  It holds none of the slicing, dequantization or contraction
arithmetic that the library and the oracle implement; both sides receive the
same arrays from here.

Parent quantizer: per group of ``group`` consecutive input (K) indices of one
output row, the observed range [min(0, min w), max(0, max w)] is mapped onto
the 2^c integer levels with a scale and an integer zero point (MatQuant
summary page, section 3.1 "Preliminaries", MinMax quantizer).  Arithmetic is
fp32 with round-to-nearest-even; the scale is stored as fp16 and the zero
point as an integer-valued fp16.

Seeding: every tensor draws from ``numpy.random.default_rng(SeedSequence([0,
cfg_id, tensor_id, *extra]))``; within one layer the draw order is W, then the
outlier positions, then X.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

C_BITS = 8

# Workload shapes.  Llama-3.1-8B FFN: hidden 4096, FFN 14336.  Gemma-2-9B FFN:
# hidden 3584, FFN 14336.
LLAMA8B_FFN = (("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336))
# Llama-3.1-8B attention projections (32 query heads, 8 key/value heads of 128)
LLAMA8B_ATTN = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096))
GEMMA9B_FFN = (("gate", 14336, 3584), ("up", 14336, 3584), ("down", 3584, 14336))
GEMMA9B_BLOCKS = 42


def rng_for(cfg_id: int, tensor_id: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, cfg_id, tensor_id, *extra]))


def gaussian_weights(rng: np.random.Generator, n: int, k: int, std: float = 0.02,
                     outlier_frac: float = 0.0, outlier_mult: float = 10.0) -> np.ndarray:
    """fp32 [n, k] with W ~ N(0, std^2); round(outlier_frac*n*k) distinct entries,
    chosen uniformly, are multiplied by ``outlier_mult`` (sign kept)."""
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    n_out = int(round(outlier_frac * n * k))
    if n_out:
        idx = rng.choice(n * k, size=n_out, replace=False)
        flat = w.reshape(-1)
        flat[idx] *= np.float32(outlier_mult)
    return w


def minmax_parent(w: np.ndarray, group: int, c: int = C_BITS):
    """Asymmetric min-max quantization of fp32 ``w`` [n, k] into unsigned c-bit
    codes with one (scale, zero) per group of ``group`` consecutive k.

    Returns (q uint8 [n,k], scales fp16 [n,k/group], zeros fp16 [n,k/group]).
    """
    n, k = w.shape
    if k % group:
        raise ValueError("k must be a multiple of group")
    qmax = np.float32(2 ** c - 1)
    wg = w.reshape(n, k // group, group).astype(np.float32, copy=False)
    lo = np.minimum(wg.min(axis=-1), np.float32(0))
    hi = np.maximum(wg.max(axis=-1), np.float32(0))
    s16 = ((hi - lo) / qmax).astype(np.float16)
    s16[s16 == 0] = np.float16(1.0)
    sf = s16.astype(np.float32)
    z = np.clip(np.rint(-lo / sf), 0, qmax)
    q = np.clip(np.rint(wg / sf[..., None]) + z[..., None], 0, qmax)
    return (q.astype(np.uint8).reshape(n, k), s16, z.astype(np.float16))


def activations(rng: np.random.Generator, m: int, k: int, dtype: str):
    """X ~ N(0, 1) drawn in fp32 and rounded (RNE) to ``dtype`` ('f16'|'bf16').
    Returns a contiguous CPU torch tensor."""
    import torch
    x = rng.standard_normal((m, k), dtype=np.float32)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(x).to(tdt).contiguous()


@dataclass
class Layer:
    q: np.ndarray        # uint8 [n, k] parent codes
    scales: np.ndarray   # fp16 [n, k/group]
    zeros: np.ndarray    # fp16 [n, k/group], integer-valued
    w: np.ndarray        # fp32 [n, k] the weights the parent was made from
    x: "object"          # torch CPU tensor [m, k], fp16 or bf16
    group: int

    @property
    def n(self):
        return self.q.shape[0]

    @property
    def k(self):
        return self.q.shape[1]


def make_layer(cfg_id: int, tensor_id: int, n: int, k: int, m: int, group: int,
               x_dtype: str = "f16", outlier_frac: float = 0.0, std: float = 0.02,
               extra: tuple = ()) -> Layer:
    rng = rng_for(cfg_id, tensor_id, *extra)
    w = gaussian_weights(rng, n, k, std=std, outlier_frac=outlier_frac)
    q, s, z = minmax_parent(w, group)
    x = activations(rng, m, k, x_dtype) if m > 0 else None
    return Layer(q=q, scales=s, zeros=z, w=w, x=x, group=group)


def all_codes_layer(n: int, k: int, group: int, seed: int = 0) -> Layer:
    """Parent codes that sweep every value 0..255 (each row a rotated ramp) with
    random fp16 scales and integer zero points; used for exhaustive slice and
    dequant checks."""
    rng = np.random.default_rng(np.random.SeedSequence([0, 99, seed]))
    base = np.arange(k, dtype=np.int64)
    q = ((base[None, :] + 37 * np.arange(n, dtype=np.int64)[:, None]) % 256).astype(np.uint8)
    g = k // group
    s = (rng.uniform(1e-4, 4e-2, size=(n, g))).astype(np.float16)
    z = rng.integers(0, 256, size=(n, g)).astype(np.float16)
    return Layer(q=q, scales=s, zeros=z, w=None, x=None, group=group)


def mixnmatch_widths(n_blocks: int = GEMMA9B_BLOCKS, seed: int = 0) -> list[int]:
    """Per-block widths: a seeded permutation of equal counts of 2, 3 and 4 bits
    (mean exactly 3 bits when n_blocks % 3 == 0)."""
    per = n_blocks // 3
    base = np.array([2] * per + [3] * per + [4] * (n_blocks - 2 * per))
    return [int(v) for v in np.random.default_rng(seed).permutation(base)]


def device_weights(seed: int, n: int, k: int, device, std: float = 0.02, outlier_frac: float = 1e-3,
                   outlier_mult: float = 10.0):
    """fp32 [n, k] W ~ N(0, std^2) drawn on `device` with a seeded torch
    generator, with round(outlier_frac*n*k) entries (drawn with replacement)
    multiplied by outlier_mult."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32) * std
    n_out = int(round(outlier_frac * n * k))
    if n_out:
        idx = torch.randint(0, n * k, (n_out,), generator=g, device=device)
        w.view(-1)[idx] *= outlier_mult
    return w


def device_parent(seed: int, n: int, k: int, group: int, device, std: float = 0.02,
                  outlier_frac: float = 1e-3, outlier_mult: float = 10.0, c: int = C_BITS):
    """The same recipe as `make_layer` + `minmax_parent`, drawn on `device` with
    a seeded torch generator (for workloads too large to draw on the host):
    W ~ N(0, std^2) fp32 with round(outlier_frac*n*k) entries x outlier_mult,
    then per-group min-max quantization in fp32 (RNE), fp16 scale, integer zero.
    Returns (q uint8 [n,k], scales fp16 [n,k/group], zeros fp16 [n,k/group])."""
    import torch
    w = device_weights(seed, n, k, device, std, outlier_frac, outlier_mult)
    qmax = float(2 ** c - 1)
    wg = w.view(n, k // group, group)
    lo = torch.clamp(wg.amin(dim=-1), max=0.0)
    hi = torch.clamp(wg.amax(dim=-1), min=0.0)
    s16 = ((hi - lo) / qmax).to(torch.float16)
    s16 = torch.where(s16 == 0, torch.ones_like(s16), s16)
    sf = s16.float()
    z = torch.clamp(torch.round(-lo / sf), 0, qmax)
    q = torch.clamp(torch.round(wg / sf.unsqueeze(-1)) + z.unsqueeze(-1), 0, qmax)
    del w, wg
    return q.to(torch.uint8).view(n, k).contiguous(), s16.contiguous(), z.to(torch.float16).contiguous()
