"""Seeded synthetic inputs for the KDA chunked forward pass.

This module is shared by the oracle side (tests, CPU baseline) and the GPU
side (tests, bench).  It only draws random numbers and shapes them; it holds
none of the method's arithmetic.  The only value transforms here are the
input-distribution recipe itself:

  q, k  ~ N(0, 1), then L2-normalised over d_k per (token, head)
          (ogis-ri NLP primer on Kimi K3, §3.1 "KDA": q and k are
          L2-normalised before use)
  v     ~ N(0, 1)
  beta  = sigmoid(N(0, 1))                    (a write strength in (0, 1))
  g     = -5 * sigmoid(2 * N(0, 1))           (bounded log-decay in (-5, 0);
          ogis-ri §3.1 "chunk 内の減衰と、その数値範囲")
  S0    = s0_std * N(0, 1)  (optional)

Values are drawn in float32 and rounded to the workload dtype
(round-to-nearest-even for bf16), so the float32 arrays returned here hold
exactly the values a kernel sees.  Two backends draw the bulk numbers:

  * "numpy": numpy Generator(PCG64(seed)); used for small workloads and every
    CPU test, draw order lengths -> q -> k -> v -> beta -> g -> pinned
    channels -> S0 -> window.
  * "torch": torch.Generator on the target device seeded with `seed`, same
    order, for the large workloads where host-side drawing would take
    minutes.  Lengths, pinned channels and the window always come from numpy.

Both backends are deterministic for a given seed; they do not produce the
same numbers as each other.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np


@dataclass(frozen=True)
class Spec:
    """Shape and distribution of one synthetic workload."""
    name: str
    dtype: str                      # "f32" or "bf16"
    lengths: tuple                  # per-sequence token counts (packed)
    n_heads: int
    d_k: int
    d_v: int
    s0_std: float = 0.0             # 0 => no initial state (zeros)
    pin_frac: float = 0.0           # fraction of channels per head with g == -5 exactly
    varlen: bool = False            # pass cu_seqlens explicitly
    window: int = 0                 # >0: seeded output window of this many tokens
    seed: int = 0
    chunk: int = 64

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def n_seqs(self) -> int:
        return len(self.lengths)

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(np.asarray(self.lengths, dtype=np.int64))]).astype(np.int64)


def _varlen_lengths(n: int, lo: int, hi: int, seed: int) -> tuple:
    """Lengths uniform in [lo, hi]; redrawn until no length and no interior
    boundary is a multiple of 16, so that sequence edges cut through 16-token
    sub-tiles."""
    rng = np.random.Generator(np.random.PCG64(seed))
    while True:
        lens = rng.integers(lo, hi + 1, size=n)
        cu = np.cumsum(lens)
        if np.all(lens % 16 != 0) and np.all(cu[:-1] % 16 != 0):
            return tuple(int(x) for x in lens)


def headline_configs() -> dict:
    """The five workloads: 0 small fp32; 1 batched bf16; 2 the headline
    H=32, d=128, T=65536 shape; 3 a ragged packed batch; 4 a 1M-token prefill."""
    return {
        0: Spec("fp32 B=1 H=2 T=256 d=64", "f32", (256,), 2, 64, 64),
        1: Spec("bf16 B=4 H=16 T=4096 d=128", "bf16", (4096,) * 4, 16, 128, 128),
        2: Spec("bf16 B=1 H=32 T=65536 d=128", "bf16", (65536,), 32, 128, 128, s0_std=0.02),
        3: Spec("bf16 varlen N=64 L~U[512,16384] H=32 d=128", "bf16",
                _varlen_lengths(64, 512, 16384, seed=0), 32, 128, 128,
                pin_frac=0.25, varlen=True),
        4: Spec("bf16 B=1 H=16 T=1048576 d=128", "bf16", (1048576,), 16, 128, 128,
                s0_std=0.02, window=8192),
    }


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 value (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    spec: Spec
    q: object
    k: object
    v: object
    beta: object
    g: object
    S0: Optional[object]
    cu_seqlens: np.ndarray
    window: tuple = (0, 0)          # [lo, hi) packed-token range of the output window
    pinned: Optional[np.ndarray] = field(default=None, repr=False)   # [H, d_k] bool


def _pinned_mask(spec: Spec, rng: np.random.Generator) -> Optional[np.ndarray]:
    if spec.pin_frac <= 0:
        return None
    n_pin = int(round(spec.pin_frac * spec.d_k))
    mask = np.zeros((spec.n_heads, spec.d_k), dtype=bool)
    for h in range(spec.n_heads):
        mask[h, rng.choice(spec.d_k, size=n_pin, replace=False)] = True
    return mask


def _window(spec: Spec, rng: np.random.Generator) -> tuple:
    if spec.window <= 0:
        return (0, spec.total_tokens)
    lo = int(rng.integers(0, spec.total_tokens - spec.window + 1))
    return (lo, lo + spec.window)


def generate_numpy(spec: Spec) -> Inputs:
    """Host-side draw; all arrays float32 holding values exact in spec.dtype."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    T, H, dk, dv = spec.total_tokens, spec.n_heads, spec.d_k, spec.d_v
    rnd = round_bf16 if spec.dtype == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))

    def unit(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        x /= np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True)).astype(np.float32)
        return rnd(x)

    q = unit((T, H, dk))
    k = unit((T, H, dk))
    v = rnd(rng.standard_normal((T, H, dv), dtype=np.float32))
    beta = rnd(1.0 / (1.0 + np.exp(-rng.standard_normal((T, H), dtype=np.float32))))
    g = rnd(-5.0 / (1.0 + np.exp(-2.0 * rng.standard_normal((T, H, dk), dtype=np.float32))))
    pinned = _pinned_mask(spec, rng)
    if pinned is not None:
        g[:, pinned] = -5.0
    S0 = None
    if spec.s0_std > 0:
        S0 = (spec.s0_std * rng.standard_normal((spec.n_seqs, H, dk, dv), dtype=np.float32)).astype(np.float32)
    win = _window(spec, rng)
    return Inputs(spec, q, k, v, beta.astype(np.float32), g.astype(np.float32), S0,
                  spec.cu_seqlens(), win, pinned)


def generate_torch(spec: Spec, device, block_tokens: int = 1 << 16) -> Inputs:
    """Device-side draw with a seeded torch.Generator (large workloads).

    Tensors are returned on `device` in the workload dtype (torch.float32 or
    torch.bfloat16); S0 is float32.  Drawn in token blocks to bound the
    float32 temporaries."""
    import torch
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed)
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    T, H, dk, dv = spec.total_tokens, spec.n_heads, spec.d_k, spec.d_v

    def draw(shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    def unit_blocks(d):
        out = torch.empty((T, H, d), device=device, dtype=tdt)
        for s in range(0, T, block_tokens):
            e = min(T, s + block_tokens)
            x = draw((e - s, H, d))
            x = x / torch.sqrt(torch.sum(x.double() ** 2, dim=-1, keepdim=True)).float()
            out[s:e] = x.to(tdt)
        return out

    q = unit_blocks(dk)
    k = unit_blocks(dk)
    v = torch.empty((T, H, dv), device=device, dtype=tdt)
    for s in range(0, T, block_tokens):
        e = min(T, s + block_tokens)
        v[s:e] = draw((e - s, H, dv)).to(tdt)
    beta = torch.sigmoid(draw((T, H))).to(tdt)
    g = torch.empty((T, H, dk), device=device, dtype=tdt)
    for s in range(0, T, block_tokens):
        e = min(T, s + block_tokens)
        g[s:e] = (-5.0 * torch.sigmoid(2.0 * draw((e - s, H, dk)))).to(tdt)
    pinned = _pinned_mask(spec, rng)
    if pinned is not None:
        pm = torch.from_numpy(pinned).to(device)
        for s in range(0, T, block_tokens):
            e = min(T, s + block_tokens)
            blk = g[s:e]
            blk[:, pm] = -5.0
    S0 = None
    if spec.s0_std > 0:
        S0 = spec.s0_std * draw((spec.n_seqs, H, dk, dv))
    win = _window(spec, rng)
    return Inputs(spec, q, k, v, beta, g, S0, spec.cu_seqlens(), win, pinned)


def custom(name: str, dtype: str, lengths: Sequence[int], n_heads: int, d: int, **kw) -> Spec:
    """A small ad-hoc workload with the standard distributions."""
    return Spec(name, dtype, tuple(int(x) for x in lengths), n_heads, d, d, **kw)


def generate_grads_numpy(spec: Spec, ds_std: float = 1.0, with_dS_T: bool = True):
    """Seeded upstream gradients for a backward workload: dO ~ N(0, 1) shaped
    like v (rounded to spec.dtype) and dS_T ~ ds_std * N(0, 1) float32 shaped
    like the states (None when with_dS_T is False).  Drawn from its own
    stream, PCG64(seed + 1000003), so the forward inputs are unchanged."""
    rng = np.random.Generator(np.random.PCG64(spec.seed + 1000003))
    T, H, dk, dv = spec.total_tokens, spec.n_heads, spec.d_k, spec.d_v
    rnd = round_bf16 if spec.dtype == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))
    dO = rnd(rng.standard_normal((T, H, dv), dtype=np.float32))
    dS_T = None
    if with_dS_T:
        dS_T = (ds_std * rng.standard_normal((spec.n_seqs, H, dk, dv), dtype=np.float32)).astype(np.float32)
    return dO, dS_T
