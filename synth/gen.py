"""Seeded generators for synthetic LittleBit layers and activations.

Distributions (chosen to match the workloads the layer is evaluated on):
  * signs: i.i.d. +-1 with p = 1/2, drawn directly as uniform uint32 words in
    the canonical packed format (row-major, ceil(rank/32) words per row, bit
    j%32 of word j//32 set means -1); bits at positions >= rank are zero;
  * scales h, g, l: fp16 round-to-nearest-even of exp(N(0, 0.5^2));
  * activations: N(0, 1), optionally with a fixed 1 % of input channels
    multiplied by 20, rounded to bf16 (round-to-nearest-even) or kept fp32.

Every tensor comes from its own PCG64 stream keyed by a tuple, so any single
tensor can be regenerated without drawing the others.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_ENTROPY = 0x11781B17  # fixed root entropy of every stream

TENSOR_U, TENSOR_V, TENSOR_H, TENSOR_G, TENSOR_L, TENSOR_X = 0, 1, 2, 3, 4, 9


def rng_for(*key: int) -> np.random.Generator:
    """Independent PCG64 generator for an integer key tuple."""
    ss = np.random.SeedSequence(entropy=_ENTROPY, spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


def _words_per_row(rank: int) -> int:
    return (int(rank) + 31) // 32


def sign_words(key: Sequence[int], rows: int, rank: int) -> np.ndarray:
    """Uniform random sign words, shape [rows, ceil(rank/32)], padding bits zero."""
    w = _words_per_row(rank)
    g = rng_for(*key)
    words = g.integers(0, 1 << 32, size=(rows, w), dtype=np.uint64).astype(np.uint32)
    tail = rank % 32
    if tail and w:
        words[:, -1] &= np.uint32((1 << tail) - 1)
    return words


def int8_signs(key: Sequence[int], rows: int, rank: int) -> np.ndarray:
    """Unpacked i.i.d. +-1 values as int8, shape [rows, rank]."""
    g = rng_for(*key)
    return np.where(g.integers(0, 2, size=(rows, rank)) == 1, -1, 1).astype(np.int8)


def scales_fp16_bits(key: Sequence[int], length: int, sigma: float = 0.5) -> np.ndarray:
    """fp16 bit patterns (uint16) of exp(N(0, sigma^2)) rounded to nearest even."""
    g = rng_for(*key)
    v = np.exp(g.normal(0.0, sigma, size=length))
    return v.astype(np.float16).view(np.uint16)


def signed_scales_fp16_bits(key: Sequence[int], length: int, sigma: float = 0.5,
                           zero_frac: float = 0.05, subnormal_frac: float = 0.05) -> np.ndarray:
    """fp16 bit patterns of scales with every sign and the edge values a
    learned real scale can take: |s| = exp(N(0, sigma^2)) with a random sign,
    except that about zero_frac of the entries are +0 or -0 and about
    subnormal_frac are fp16 subnormals (random sign, magnitude 2^-24 .. 2^-15)."""
    g = rng_for(*key)
    v = np.exp(g.normal(0.0, sigma, size=length)) * np.where(g.integers(0, 2, size=length) == 1, -1.0, 1.0)
    bits = v.astype(np.float16).view(np.uint16).copy()
    kind = g.random(size=length)
    zero = kind < zero_frac
    sub = (kind >= zero_frac) & (kind < zero_frac + subnormal_frac)
    sign = (g.integers(0, 2, size=length).astype(np.uint16) << np.uint16(15))
    bits[zero] = sign[zero]                                                   # +0 / -0
    mant = g.integers(1, 1 << 10, size=length).astype(np.uint16)             # exponent field 0: subnormal
    bits[sub] = sign[sub] | mant[sub]
    return bits


def wide_range_activations(key: Sequence[int], tokens: int, n: int, octaves: int = 12) -> np.ndarray:
    """bf16 bits of N(0, 1) values each multiplied by 2^-u, u uniform in
    [0, octaves]: every block of 32 consecutive elements then spans about
    2^octaves in magnitude."""
    g = rng_for(*key)
    x = g.normal(0.0, 1.0, size=(tokens, n)) * np.exp2(-g.uniform(0.0, octaves, size=(tokens, n)))
    return bf16_bits_from_f32(x.astype(np.float32))


def bf16_bits_from_f32(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def activations(key: Sequence[int], tokens: int, n: int, io: str = "bf16",
                outlier_frac: float = 0.0, outlier_scale: float = 20.0) -> np.ndarray:
    """Activation matrix [tokens, n]: uint16 bf16 bits (io='bf16') or float32.

    With outlier_frac > 0, round(outlier_frac * n) channels (the same for every
    token, drawn without replacement) are multiplied by outlier_scale before
    rounding.
    """
    g = rng_for(*key)
    x = g.normal(0.0, 1.0, size=(tokens, n)).astype(np.float64)
    k = int(round(outlier_frac * n))
    if k:
        ch = g.choice(n, size=k, replace=False)
        x[:, ch] *= outlier_scale
    x32 = x.astype(np.float32)
    if io == "bf16":
        return bf16_bits_from_f32(x32)
    if io == "fp32":
        return x32
    raise ValueError(f"io must be 'bf16' or 'fp32', got {io!r}")


@dataclass(frozen=True)
class MatSpec:
    name: str
    m: int          # d_out (rows of W)
    n: int          # d_in  (columns of W)
    rank_mult: int = 1


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    layers: int
    mats: Tuple[MatSpec, ...]
    bpw: Optional[Fraction]       # sign bits per weight; None when rank is fixed
    fixed_rank: Optional[int]
    tokens: Tuple[int, ...]
    io: str = "bf16"
    outlier_frac: float = 0.0
    note: str = ""

    @property
    def count(self) -> int:
        return self.layers * len(self.mats)

    def entries(self) -> List[Tuple[int, int, MatSpec]]:
        return [(l, j, s) for l in range(self.layers) for j, s in enumerate(self.mats)]


def _llama(d: int, ffn: int, kv: Optional[int] = None, kv_mult: int = 1) -> Tuple[MatSpec, ...]:
    kv = d if kv is None else kv
    return (MatSpec("q", d, d), MatSpec("k", kv, d, kv_mult), MatSpec("v", kv, d, kv_mult),
            MatSpec("o", d, d), MatSpec("gate", ffn, d), MatSpec("up", ffn, d),
            MatSpec("down", d, ffn))


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload(1, "single-512", 1, (MatSpec("w", 512, 512),), None, 16, (4,), io="fp32",
                 note="single 512x512 linear, rank 16 on both paths, 4 tokens, fp32 I/O"),
        Workload(2, "llama2-7b-0.1bpw", 32, _llama(4096, 11008), Fraction(1, 10), None, (1,),
                 outlier_frac=0.01, note="Llama-2-7B-shaped decode stack, batch 1"),
        Workload(3, "llama2-13b-0.55bpw", 40, _llama(5120, 13824), Fraction(55, 100), None, (2048,),
                 note="Llama-2-13B-shaped prefill stack, 2048 tokens"),
        Workload(4, "llama3-8b-0.3bpw", 32, _llama(4096, 14336, kv=1024, kv_mult=2),
                 Fraction(3, 10), None, (16, 2048),
                 note="Llama-3-8B-shaped GQA stack, k/v at twice the formula rank"),
        Workload(5, "llama2-70b-0.1bpw", 80, _llama(8192, 28672, kv=1024), Fraction(1, 10), None,
                 (1, 8, 64), note="Llama-2-70B-shaped stack, decode batch 1/8/64"),
    ]
}


def layer_tensors(wid: int, layer: int, mat: int, m: int, n: int,
                  ranks: Sequence[int]) -> List[Dict[str, np.ndarray]]:
    """Sign words and fp16 scales for every path of one linear.

    Returns one dict per path with keys u_words [m, W], v_words [n, W] (uint32),
    h [m], g [n], l [rank] (uint16 fp16 bits) and rank.
    """
    out = []
    for p, r in enumerate(ranks):
        out.append(dict(
            rank=int(r),
            u_words=sign_words((wid, layer, mat, p, TENSOR_U), m, r),
            v_words=sign_words((wid, layer, mat, p, TENSOR_V), n, r),
            h=scales_fp16_bits((wid, layer, mat, p, TENSOR_H), m),
            g=scales_fp16_bits((wid, layer, mat, p, TENSOR_G), n),
            l=scales_fp16_bits((wid, layer, mat, p, TENSOR_L), r),
        ))
    return out


def layer_activations(wl: Workload, layer: int, mat: int, n: int, tokens: int,
                      io: Optional[str] = None) -> np.ndarray:
    return activations((wl.wid, layer, mat, TENSOR_X, tokens), tokens, n,
                       io=io or wl.io, outlier_frac=wl.outlier_frac)
