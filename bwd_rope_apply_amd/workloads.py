"""Seeded synthetic workloads for exact causal RoPE attention.

This module draws inputs and nothing else: it holds none of the attention or
rotation arithmetic, so both the HIP path and the float64 oracle can take their
inputs from it without sharing any of the method.

Recipe (same for every workload):
  * a numpy PCG64 generator per tensor, seeded from
    ``SeedSequence(seed).spawn(5)`` and used in the fixed order
    [Q, K, V, dO, alpha];
  * draws are float64, then rounded to the storage type with
    round-to-nearest-even (float64 -> float32, and float32 -> bfloat16 for
    bf16 storage);
  * Q, K, V, dO are contiguous [B, H, N, D], D fastest; alpha is one [D/2]
    float32 vector shared by every batch and head.

The five named workloads follow the settings of the pages: one attention
layer at the LeRoPE training length 2048 with head dim 128, a training-step
shape, a long-context shape with bounded entries (the bounded-entries regime
of "RoPE attention can be trained in almost-linear time", Problem definition)
and learned-spectrum-like alpha (LeRoPE, "Main results" on the dominant band
and suppressed slow bands), and a very long context at head dim 64 (LeRoPE,
"Experimental setup").  No dataset is used; the i.i.d. tensors stand in for
activations of those shapes.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

# (kind, a, b): "uniform" U[a,b]; "normal" N(0, a^2) scaled by b; "zero".
Dist = Tuple[str, float, float]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str          # storage type of Q, K, V, dO: "fp32" or "bf16"
    base: float
    causal: bool
    qk: Dist
    v: Dist
    do: Dist
    alpha: Dist
    seed: int
    note: str = ""

    def with_shape(self, B=None, H=None, N=None, seed=None) -> "Workload":
        """Same distributions at another shape (parity cases at reduced size)."""
        return dataclasses.replace(
            self, B=B or self.B, H=H or self.H, N=N or self.N,
            seed=self.seed if seed is None else seed,
            name=f"{self.name}[B{B or self.B},H{H or self.H},N{N or self.N}]")

    @property
    def n_elem(self) -> int:
        return self.B * self.H * self.N * self.D


_INV_SQRT_128 = 1.0 / np.sqrt(128.0)

WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload(
        "tiny_fp32", 1, 1, 128, 64, "fp32", 1e4, True,
        qk=("uniform", -1.0, 1.0), v=("uniform", -1.0, 1.0),
        do=("uniform", -1.0, 1.0), alpha=("zero", 0.0, 0.0), seed=1000,
        note="tiny exact check, standard RoPE (alpha = 0)"),
    "layer_2k": Workload(
        "layer_2k", 1, 16, 2048, 128, "bf16", 1e4, True,
        qk=("normal", 1.0, 1.0), v=("normal", 1.0, 1.0),
        do=("normal", 1.0, 1.0), alpha=("normal", 0.1, 1.0), seed=1001,
        note="single layer at training length 2048"),
    "train_4k": Workload(
        "train_4k", 4, 32, 4096, 128, "bf16", 5e5, True,
        qk=("normal", 1.0, _INV_SQRT_128), v=("normal", 1.0, 1.0),
        do=("normal", 1.0, 1.0), alpha=("zero", 0.0, 0.0), seed=1002,
        note="training-step shape, near-uniform attention"),
    "long_8k": Workload(
        "long_8k", 1, 32, 8192, 128, "bf16", 1e4, True,
        qk=("uniform", -2.0, 2.0), v=("uniform", -2.0, 2.0),
        do=("normal", 1.0, 1.0), alpha=("uniform", -1.0, 0.5), seed=1003,
        note="long-context headline, bounded entries, learned-like alpha"),
    "vlong_32k": Workload(
        "vlong_32k", 1, 8, 32768, 64, "bf16", 1e6, True,
        qk=("normal", 1.0, 1.0), v=("normal", 1.0, 1.0),
        do=("normal", 1.0, 1.0), alpha=("normal", 0.2, 1.0), seed=1004,
        note="very long context, head dim 64"),
}

HEADLINE = "long_8k"


def _draw(rng: np.random.Generator, dist: Dist, shape) -> np.ndarray:
    kind, a, b = dist
    if kind == "uniform":
        return rng.uniform(a, b, size=shape)
    if kind == "normal":
        return rng.normal(0.0, a, size=shape) * b
    if kind == "zero":
        return np.zeros(shape)
    raise ValueError(kind)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Inputs:
    """Stored inputs.  ``q, k, v, do`` hold the storage bits (float32 arrays,
    or uint16 bfloat16 bit patterns); ``alpha`` is float32 [D/2]."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    alpha: np.ndarray

    def f64(self, name: str) -> np.ndarray:
        x = getattr(self, name)
        if x.dtype == np.uint16:
            return bf16_bits_to_f64(x)
        return x.astype(np.float64)


def make_inputs(wl: Workload, which=("q", "k", "v", "do")) -> Inputs:
    """Draw the stored inputs of ``wl``.  Streams are spawned in the fixed
    order [Q, K, V, dO, alpha]; tensors not in ``which`` are not drawn (their
    stream is still consumed by nobody, so the others do not change)."""
    shape = (wl.B, wl.H, wl.N, wl.D)
    streams = np.random.SeedSequence(wl.seed).spawn(5)
    dists = {"q": wl.qk, "k": wl.qk, "v": wl.v, "do": wl.do}
    out = {}
    for idx, name in enumerate(("q", "k", "v", "do")):
        if name not in which:
            out[name] = None
            continue
        x = _draw(np.random.Generator(np.random.PCG64(streams[idx])), dists[name], shape)
        x32 = x.astype(np.float32)
        out[name] = f32_to_bf16_bits(x32) if wl.dtype == "bf16" else x32
    a = _draw(np.random.Generator(np.random.PCG64(streams[4])), wl.alpha, (wl.D // 2,))
    return Inputs(wl, out["q"], out["k"], out["v"], out["do"], a.astype(np.float32))


def get(name: str, B: Optional[int] = None, H: Optional[int] = None,
        N: Optional[int] = None, seed: Optional[int] = None) -> Workload:
    wl = WORKLOADS[name]
    if B is None and H is None and N is None and seed is None:
        return wl
    return wl.with_shape(B, H, N, seed)


def block_lists(B: int, H: int, N: int, retrieved: int, causal: bool, seed: int,
                noise: bool = False, block: int = 128):
    """Seeded key-block lists for block-list attention: ``lists[b][h][qb]``
    names, for each query block of ``block`` rows, ``retrieved`` key blocks
    drawn uniformly without replacement from the other blocks it may see
    (the earlier blocks under the causal mask, any other block otherwise) --
    a stand-in for the retrieved (cluster, block) pairs of Multipole Semantic
    Attention ("Retrieval-augmented approximation"), whose selection depends
    on trained clusters.  The own block is implied and not listed.  With
    ``noise`` each list also gets entries that must be ignored or merged:
    duplicates, out-of-range indices and (causal) later blocks."""
    nb = (N + block - 1) // block
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    out = []
    for _ in range(B):
        per_b = []
        for _ in range(H):
            per_h = []
            for qb in range(nb):
                cand = np.arange(qb) if causal else np.delete(np.arange(nb), qb)
                k = min(retrieved, cand.size)
                sel = [int(x) for x in rng.choice(cand, size=k, replace=False)] if k else []
                if noise:
                    if sel:
                        sel.append(sel[0])
                    sel += [-1, nb, nb + 7, qb]
                    if causal and qb + 1 < nb:
                        sel.append(qb + 1)
                    rng.shuffle(sel)
                per_h.append(sel)
            per_b.append(per_h)
        out.append(per_b)
    return out


# ---------------------------------------------------------------- token sets
# Inputs of Gram-threshold token selection ("Cascade token selection for
# transformer attention acceleration"): one layer's token activations
# [B, T, d] and a stack of layers for the cascade.  The pages measure
# T = 512 with the hidden sizes of GPT-2 (768) and GPT-J / OPT (4096) at
# tau = 0.30, and project to T = 8192 (Experimental results).  Trained
# activations are not available, so tokens are drawn around random
# directions ("topics") with mixed spreads: tight groups make near-duplicates
# (cosine ~0.95-0.99, redundant at tau = 0.30), loose groups do not (~0.6-0.8),
# with per-token gains; deeper layers add a small residual perturbation, the
# depth coherence the cascade relies on (Methodology).


@dataclasses.dataclass(frozen=True)
class TokenWorkload:
    name: str
    B: int
    T: int
    d: int
    dtype: str            # "bf16" or "fp16" storage
    tau: float
    group: int            # mean tokens per direction
    spreads: Tuple[float, ...]   # squared noise-to-signal ratio per direction, drawn from these
    drift: float          # squared relative size of the per-layer residual perturbation
    seed: int
    note: str = ""

    def with_shape(self, B=None, T=None, d=None, seed=None) -> "TokenWorkload":
        return dataclasses.replace(
            self, B=B or self.B, T=T or self.T, d=d or self.d,
            seed=self.seed if seed is None else seed,
            name=f"{self.name}[B{B or self.B},T{T or self.T},d{d or self.d}]")


_SPREADS = (0.01, 0.03, 0.08, 0.12, 0.3)

TOKEN_WORKLOADS: Dict[str, TokenWorkload] = {
    "gram_gpt2_512": TokenWorkload("gram_gpt2_512", 1, 512, 768, "bf16", 0.30, 16, _SPREADS, 0.02,
                                   seed=2001, note="T = 512, GPT-2 hidden size"),
    "gram_gptj_512": TokenWorkload("gram_gptj_512", 1, 512, 4096, "bf16", 0.30, 16, _SPREADS, 0.02,
                                   seed=2002, note="T = 512, GPT-J / OPT hidden size"),
    "gram_8k": TokenWorkload("gram_8k", 1, 8192, 4096, "bf16", 0.30, 16, _SPREADS, 0.02,
                             seed=2003, note="the projected long sequence, T = 8192, d = 4096"),
}

GRAM_HEADLINE = "gram_8k"


def get_tokens(name: str, B=None, T=None, d=None, seed=None) -> TokenWorkload:
    wl = TOKEN_WORKLOADS[name]
    if B is None and T is None and d is None and seed is None:
        return wl
    return wl.with_shape(B, T, d, seed)


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "fp16":
        return x32.astype(np.float16)
    return x32


def storage_to_f64(x: np.ndarray) -> np.ndarray:
    """Exact upcast of stored token bits (bf16 as uint16, fp16, fp32)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


def make_tokens(wl: TokenWorkload, layers: int = 1):
    """Stored tokens of ``layers`` consecutive layers: a list of [B, T, d]
    arrays (bf16 bits as uint16, or fp16).  Streams: one PCG64 per layer,
    spawned from SeedSequence(seed); layer 0 draws the directions, spreads,
    assignments, gains and noise in that order; layer l > 0 adds
    N(0, drift * gain^2 / d) per entry to layer l - 1 (before rounding)."""
    streams = np.random.SeedSequence(wl.seed).spawn(max(1, layers))
    rng = np.random.Generator(np.random.PCG64(streams[0]))
    n_dir = max(1, wl.T // wl.group)
    shape = (wl.B, wl.T, wl.d)
    dirs = rng.normal(size=(wl.B, n_dir, wl.d))
    dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
    spread = rng.choice(np.asarray(wl.spreads), size=(wl.B, n_dir))
    z = rng.integers(0, n_dir, size=(wl.B, wl.T))
    gain = rng.uniform(0.5, 3.0, size=(wl.B, wl.T, 1))
    b = np.arange(wl.B)[:, None]
    x = dirs[b, z] + rng.normal(size=shape) * np.sqrt(spread[b, z] / wl.d)[..., None]
    x = x * gain
    out = [_to_storage(x, wl.dtype)]
    for l in range(1, layers):
        r = np.random.Generator(np.random.PCG64(streams[l]))
        x = x + r.normal(size=shape) * (gain * np.sqrt(wl.drift / wl.d))
        out.append(_to_storage(x, wl.dtype))
    return out
