"""Seeded synthetic workloads for the Compressor (shared by tests and bench).

This module only draws random numbers and lays out THD packs; it holds none of
the method's arithmetic (the caller supplies the output row count, which each
side computes itself).  Every tensor is drawn on the CPU from one
``torch.Generator`` per call, in the fixed order kv, score, ape, dout:

  kv, score  bf16 [T_cap, coff*head_dim]   N(0, 1) rounded to nearest-even bf16
  ape        fp32 [ratio, coff*head_dim]   N(0, 1) * 0.02
  dout       bf16 [n_out, head_dim]        N(0, 1)

Workload shapes follow the THD packs the pages measure (single and 3x8192-token
sequences at head_dim 128/512, ratio 4 and 2, coff 2) plus a tiny pack and a
ragged, static-capacity pack.  The ragged pack draws segment lengths uniformly
in [1, 4096] until at least 28000 tokens, and inserts three degenerate
segments so every zero-ownership class occurs: a 1-token segment first, a
(ratio-1)-token segment in the middle and an empty segment last.  It sits in a
32768-row buffer, so the rows past the last segment are static-capacity
padding.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    cu_seqlens: tuple
    total_tokens: int  # row capacity T_cap of kv/score/dkv/dscore
    ratio: int
    coff: int
    head_dim: int
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def num_segments(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def width(self) -> int:
        return self.coff * self.head_dim


def _cu_from_lengths(lengths) -> tuple:
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return tuple(cu)


def ragged_lengths(ratio: int, seed: int = 0, min_tokens: int = 28000, max_len: int = 4096):
    """Uniform segment lengths in [1, max_len] until >= min_tokens, with a
    1-token segment first, a (ratio-1)-token one in the middle and an empty
    one last."""
    rng = np.random.default_rng(seed)
    draws = []
    while sum(draws) < min_tokens:
        draws.append(int(rng.integers(1, max_len + 1)))
    mid = len(draws) // 2
    return [1] + draws[:mid] + [ratio - 1] + draws[mid:] + [0]


def _uniform_pack(n_seq: int, seq_len: int):
    return _cu_from_lengths([seq_len] * n_seq)


def _build_workloads():
    w = {}

    def add(name, cu, T, r, c, d, note=""):
        w[name] = Workload(name, tuple(cu), T, r, c, d, 0, note)

    add("tiny_r4_c2_d16", (0, 37, 64), 64, 4, 2, 16,
        "2 segments, both with a seqlen%ratio tail")
    add("1x8192_d128_r4_c2", _uniform_pack(1, 8192), 8192, 4, 2, 128)
    add("3x8192_d512_r4_c2", _uniform_pack(3, 8192), 24576, 4, 2, 512)
    add("3x8192_d128_r4_c2", _uniform_pack(3, 8192), 24576, 4, 2, 128)
    add("1x8192_d512_r4_c2", _uniform_pack(1, 8192), 8192, 4, 2, 512)
    for n in (1, 3):
        for d in (128, 512):
            add(f"{n}x8192_d{d}_r2_c2", _uniform_pack(n, 8192), 8192 * n, 2, 2, d)
    for c in (1, 2):
        add(f"ragged_d128_r4_c{c}", _cu_from_lengths(ragged_lengths(4)), 32768, 4, c, 128,
            "uniform [1,4096] lengths + 1, ratio-1 and 0-token segments, 32768-row buffer")
    # ratio 128 (windows of 128 * coff rows): the pages time 8k-131k-token
    # packs at coff {1, 2} x head_dim {128, 512}
    for c in (1, 2):
        for d in (128, 512):
            add(f"1x65536_d{d}_r128_c{c}", _uniform_pack(1, 65536), 65536, 128, c, d)
    add("8x8192_d512_r128_c2", _uniform_pack(8, 8192), 65536, 128, 2, 512)
    add("ragged_d128_r128_c2", _cu_from_lengths(ragged_lengths(128)), 32768, 128, 2, 128,
        "uniform [1,4096] lengths + 1, ratio-1 and 0-token segments, 32768-row buffer")
    return w


WORKLOADS = _build_workloads()
HEADLINE = "3x8192_d512_r4_c2"


def custom(name: str, lengths, total_tokens: int, ratio: int, coff: int, head_dim: int,
           seed: int = 0) -> Workload:
    cu = _cu_from_lengths(lengths)
    if cu[-1] > total_tokens:
        raise ValueError("segments exceed the row capacity")
    return Workload(name, cu, total_tokens, ratio, coff, head_dim, seed)


def make_tensors(wl: Workload, n_out: int, seed: int | None = None):
    """Draw (kv, score, ape, dout) on the CPU for workload ``wl``; ``n_out``
    is the number of output rows (dout's first dimension)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.seed if seed is None else seed)
    W = wl.width
    kv = torch.randn(wl.total_tokens, W, generator=g).to(torch.bfloat16)
    score = torch.randn(wl.total_tokens, W, generator=g).to(torch.bfloat16)
    ape = torch.randn(wl.ratio, W, generator=g) * 0.02
    dout = torch.randn(n_out, wl.head_dim, generator=g).to(torch.bfloat16)
    return kv, score, ape, dout


def cu_tensor(wl: Workload) -> torch.Tensor:
    return torch.tensor(wl.cu_seqlens, dtype=torch.int32)


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 CPU tensor."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray) -> torch.Tensor:
    """bf16 CPU tensor from uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
