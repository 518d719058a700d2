"""Seeded synthetic inputs and the workload table.

This module holds no attention arithmetic: it only draws random tensors and
names shapes. Both the HIP path (tests, bench) and the fp64 oracle are fed
from it, so the two sides see bit-identical inputs.

Recipe: config k seeds ``torch.Generator('cpu').manual_seed(k)`` and draws, in
this order, Q, K, V (then dO for a backward workload) with ``torch.randn`` in
float32, i.i.d. N(0, 1); bf16 workloads round these draws to bf16 (round to
nearest even) on the CPU. The oracle receives the same rounded values upcast
exactly to float64. With grouped K/V heads (Hkv < H), K and V are drawn with
Hkv heads and Q, dO with H.
"""

from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    backward: bool
    dtype: str          # "f32" (fp32 in/out, rounded to bf16 on load) or "bf16"
    seed: int
    Hkv: int = 0        # K/V heads shared by groups of query heads; 0: H (multi-head)
    window_left: int = -1   # local window (key j visible to query i iff
    window_right: int = -1  # i-left <= j <= i+right); -1: no bound on that side
    block_density: float = 0.0  # block-sparse: a seeded mask per query head
                                # (draw_block_mask); 0: no block mask

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    @property
    def kv_heads(self):
        return self.Hkv or self.H

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)


# The five workloads the method is measured and checked on.
WORKLOADS = [
    Workload("fwd_b1h1n256d64_f32", 1, 1, 256, 64, False, False, "f32", 1),
    Workload("fwd_b8h16n2048d64", 8, 16, 2048, 64, False, False, "bf16", 2),
    Workload("fwd_causal_b4h32n4096d128", 4, 32, 4096, 128, True, False, "bf16", 3),
    Workload("fwd_causal_b1h16n32768d128", 1, 16, 32768, 128, True, False, "bf16", 4),
    Workload("fwdbwd_causal_b4h16n4096d128", 4, 16, 4096, 128, True, True, "bf16", 5),
]

# Grouped-query attention: 32 query heads sharing 8 K/V heads (groups of 4).
GQA_WORKLOADS = [
    Workload("fwdbwd_causal_gqa_b4h32kv8n4096d128", 4, 32, 4096, 128, True, True, "bf16", 6, 8),
]


# Local attention: every query sees itself and the 1023 keys before it
# (a causal window of 1024 keys).
WINDOW_WORKLOADS = [
    Workload("fwdbwd_window1024_b4h16n4096d128", 4, 16, 4096, 128, True, True, "bf16", 7,
             window_left=1023, window_right=0),
]


# Head dimension 256: the causal forward+backward at the same bytes per
# tensor as the d = 128 bench workload (half the heads).
D256_WORKLOADS = [
    Workload("fwdbwd_causal_b4h8n4096d256", 4, 8, 4096, 256, True, True, "bf16", 8),
]


# Block-sparse attention: under the causal mask, each query head keeps each
# 128 x 128 block below the diagonal with probability 1/2 and every diagonal
# block (so no row is empty).
BLOCK_SPARSE_WORKLOADS = [
    Workload("fwdbwd_causal_blocksparse50_b4h16n4096d128", 4, 16, 4096, 128, True, True, "bf16",
             9, block_density=0.5),
]


def by_name(name: str) -> Workload:
    for w in WORKLOADS + GQA_WORKLOADS + WINDOW_WORKLOADS + D256_WORKLOADS + BLOCK_SPARSE_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def draw(shape, seed, with_grad=False, dtype="bf16", kv_heads=None):
    """Return CPU tensors (q, k, v[, do]) drawn i.i.d. N(0,1) from ``seed``.

    dtype "bf16": rounded to torch.bfloat16; "f32": left in float32.
    kv_heads: heads of k and v (default: those of ``shape``).
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    names = ["q", "k", "v"] + (["do"] if with_grad else [])
    kv_shape = tuple(shape) if kv_heads is None else (shape[0], kv_heads, shape[2], shape[3])
    out = []
    for name in names:
        x = torch.randn(kv_shape if name in ("k", "v") else tuple(shape), generator=g,
                        dtype=torch.float32)
        if dtype == "bf16":
            x = x.to(torch.bfloat16)
        elif dtype != "f32":
            raise ValueError(dtype)
        out.append(x)
    return tuple(out)


def draw_signs(d, seed):
    """d random signs (+1/-1, int8) for the FP8 path's Hadamard rotation: the
    method's own random draw, made here so that both sides receive it."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    bits = torch.randint(0, 2, (d,), generator=g, dtype=torch.int8)
    return (1 - 2 * bits).to(torch.int8)


MASK_BLOCK = 128  # query rows and keys per block of a block-sparse mask


def draw_block_mask(N, seed, density=0.5, heads=(), diagonal=True, empty_rows=0):
    """A seeded block-sparse mask: uint8 CPU tensor [*heads, nb, nb],
    nb = ceil(N / 128), each byte 1 with probability ``density``.

    diagonal: the diagonal blocks are set to 1 (no row is left without keys
    under a causal mask). empty_rows: that many block rows, drawn at random
    per head, are then set to 0 entirely (rows that see no key).
    """
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shape = tuple(heads) + (nb, nb)
    bm = (torch.rand(shape, generator=g) < density).to(torch.uint8)
    if diagonal:
        bm[..., torch.arange(nb), torch.arange(nb)] = 1
    if empty_rows:
        flat = bm.reshape(-1, nb, nb)
        for m in flat:
            rows = torch.randperm(nb, generator=g)[:empty_rows]
            m[rows, :] = 0
    return bm


def draw_segments(N, seed, heads=()):
    """A block-diagonal mask [*heads, nb, nb] of seeded segments: consecutive
    runs of 1 to 4 blocks see each other and nothing else (packed sequences
    at block granularity)."""
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    bm = torch.zeros(tuple(heads) + (nb, nb), dtype=torch.uint8)
    for m in bm.reshape(-1, nb, nb):
        i = 0
        while i < nb:
            n = int(torch.randint(1, 5, (1,), generator=g))
            m[i:i + n, i:i + n] = 1
            i += n
    return bm


def workload_block_mask(w: Workload):
    """The per-query-head block mask [B, H, nb, nb] of a block-sparse workload."""
    return draw_block_mask(w.N, 1000 + w.seed, w.block_density, heads=(w.B, w.H))


def draw_workload(w: Workload):
    return draw(w.shape, w.seed, with_grad=w.backward, dtype=w.dtype, kv_heads=w.kv_heads)


def to_f64(x: torch.Tensor):
    """Exact upcast of a CPU tensor to a float64 numpy array."""
    return x.detach().to("cpu").to(torch.float64).numpy()
