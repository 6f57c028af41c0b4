"""CPU fp64 oracle for the forward pass of a LittleBit-factorised linear layer.

TEST INFRASTRUCTURE.  This module is the checker, not the product: only the
test suite, the package's smoke check and the benchmark's CPU-baseline leg may
import it.  It shares no code with the HIP library and imports nothing from it;
both sides read the same seeded inputs from the ``synth`` package.

What it computes (sources are the pages' titles and sections):

* "LittleBit: Ultra Low-Bit Quantization via Latent Factorization" (paper
  notes, NeurIPS 2025), section "Method / Key design / multi-scale
  compensation": the primary path's effective weight is
  diag(h) * U_sign * diag(l) * V_sign^T * diag(g), with a row scale h, a column
  scale g and a latent scale l of length r, and U_sign, V_sign the sign() of
  rank-r factors (section "Method / overall framework", steps 1-3).  The same
  section says the forward pass applies these as successive element-wise
  products and binary matrix products without forming the full weight.
* Same page, section "Residual compensation": the layer's weight is the sum of
  the primary path and a residual path of the same form with its own factors.
* Same page, "overall framework", and the aibk.xyz article's section on how to
  assess an ultra-low-bit scheme (its first point, on how bpp is counted): bits per
  weight is the factorised storage averaged over the original weights.

Readings where the pages are silent (each is listed in the design notes):
* W has shape [d_out, d_in] = [m, n]; h has length m, g length n; y = x W^T.
* The forward consumes +-1 factors only; the sign bit convention of the packed
  interchange format is: bit (j mod 32) of word j//32 of a row is 1 iff the
  entry is -1, padding bits zero.
* Rank per path: r = round(BPW * m * n / (2 (m + n))), exact rational, ties
  rounded up, counting sign bits only.

Every function works in float64 from the exact values of its inputs (bf16 and
fp16 decode exactly into float64).
"""
from __future__ import annotations

from fractions import Fraction
from typing import Dict, Iterable, List, Sequence

import numpy as np

# ----------------------------------------------------------------------------
# exact decoding of the storage formats
# ----------------------------------------------------------------------------


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def decode_fp16(bits: np.ndarray) -> np.ndarray:
    """IEEE half bit patterns (uint16) -> float64, exact."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------------------
# sign factors (pages: U_sign = sign(U), V_sign = sign(V); format is the
# library's interchange format, a reading recorded in the design notes)
# ----------------------------------------------------------------------------


def words_per_row(rank: int) -> int:
    return (int(rank) + 31) // 32


def unpack_signs(words: np.ndarray, rows: int, rank: int) -> np.ndarray:
    """Canonical packed words [rows, ceil(rank/32)] -> int8 +-1 matrix [rows, rank].

    Entry (i, j) is -1 iff bit (j mod 32) of word (i, j // 32) is set.  Padding
    bits must be zero (checked).
    """
    w = words_per_row(rank)
    words = np.asarray(words, dtype=np.uint32).reshape(rows, w)
    out = np.empty((rows, rank), dtype=np.int8)
    for j in range(rank):
        bit = (words[:, j // 32] >> np.uint32(j % 32)) & np.uint32(1)
        out[:, j] = np.where(bit == 1, -1, 1)
    for j in range(rank, 32 * w):
        if np.any((words[:, j // 32] >> np.uint32(j % 32)) & np.uint32(1)):
            raise ValueError("padding bits of packed sign words must be zero")
    return out


def pack_signs(signs: np.ndarray) -> np.ndarray:
    """int8 +-1 matrix [rows, rank] -> canonical packed words [rows, ceil(rank/32)]."""
    s = np.asarray(signs)
    if s.ndim != 2:
        raise ValueError("signs must be 2-D [rows, rank]")
    if not np.all((s == 1) | (s == -1)):
        raise ValueError("sign factors may hold only -1 and +1")
    rows, rank = s.shape
    out = np.zeros((rows, words_per_row(rank)), dtype=np.uint32)
    for j in range(rank):
        out[:, j // 32] |= (s[:, j] == -1).astype(np.uint32) << np.uint32(j % 32)
    return out


def check_sign_factor(s: np.ndarray) -> None:
    """The forward consumes only +-1 factors ("sign(U)"): assert the invariant."""
    if not np.all((s == 1) | (s == -1)):
        raise AssertionError("a sign factor holds a value other than +-1")


# ----------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------


def decode_path(path: Dict, m: int, n: int) -> Dict[str, np.ndarray]:
    """Exact float64 factors of one path from its stored form.

    ``path`` holds rank, u_words [m, W], v_words [n, W] (uint32) and h [m],
    g [n], l [rank] as fp16 bit patterns.
    """
    r = int(path["rank"])
    U = unpack_signs(path["u_words"], m, r).astype(np.float64)
    V = unpack_signs(path["v_words"], n, r).astype(np.float64)
    check_sign_factor(U)
    check_sign_factor(V)
    h = decode_fp16(path["h"])
    g = decode_fp16(path["g"])
    l = decode_fp16(path["l"])
    if h.shape != (m,) or g.shape != (n,) or l.shape != (r,):
        raise ValueError("scale lengths must be h: d_out, g: d_in, l: rank")
    for v in (h, g, l):
        if not np.all(np.isfinite(v)):
            raise ValueError("scales must be finite")
    return dict(U=U, V=V, h=h, g=g, l=l, rank=r)


def reconstruct_w(paths: Sequence[Dict], m: int, n: int) -> np.ndarray:
    """Explicit effective weight W = sum_p diag(h_p) U_p diag(l_p) V_p^T diag(g_p).

    Multi-scale compensation equation (primary path) plus residual compensation
    (sum of the two paths), "LittleBit: Ultra Low-Bit Quantization via Latent
    Factorization", sections "Key design" and "Residual compensation".
    """
    W = np.zeros((m, n), dtype=np.float64)
    for path in paths:
        f = decode_path(path, m, n)
        left = f["h"][:, None] * f["U"] * f["l"][None, :]      # diag(h) U diag(l)
        right = f["V"] * f["g"][:, None]                       # diag(g) V
        W += left @ right.T
    return W


def forward(x: np.ndarray, paths: Sequence[Dict], m: int, n: int) -> np.ndarray:
    """y = x W^T in float64 with W rebuilt explicitly; x is [T, n] float64."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != n:
        raise ValueError("x must be [tokens, d_in]")
    return x @ reconstruct_w(paths, m, n).T


def forward_factored(x: np.ndarray, paths: Sequence[Dict], m: int, n: int) -> np.ndarray:
    """The factorised order the pages describe for inference, in float64.

    Per path: t = x o g, z = t V, z' = z o l, y_p = (z' U^T) o h; y = sum_p y_p.
    The paper notes' section "Key design" describes the inference forward as
    successive element-wise products and binary matrix products that never
    form the full weight.  Equal to ``forward`` up to rounding order: the
    associativity identity the tests check.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.zeros((x.shape[0], m), dtype=np.float64)
    for path in paths:
        f = decode_path(path, m, n)
        t = x * f["g"][None, :]
        z = t @ f["V"]
        zl = z * f["l"][None, :]
        y += (zl @ f["U"].T) * f["h"][None, :]
    return y


# ----------------------------------------------------------------------------
# bit budget (bits per weight) and rank rule
# ----------------------------------------------------------------------------


def rank_for_bpw(m: int, n: int, bpw: Fraction, mult: int = 1) -> int:
    """Per-path rank r = round(BPW * m * n / (2 (m + n))), ties up, times ``mult``.

    Two paths of rank r store 2 r (m + n) sign bits for m n weights, so this r
    spends the budget BPW counting sign bits only (the aibk.xyz article, section
    on how bpp is counted, warns that the scale overhead must be stated; it is
    reported separately by ``scale_bits_per_weight``).  ``mult`` is the GQA k/v
    latent-rank adjustment (paper notes, section "Training strategy": k/v
    projections of GQA models get their own latent rank; the factor is a
    workload choice).
    """
    q = Fraction(bpw) * m * n / (2 * (m + n))
    r = (q + Fraction(1, 2)).numerator // (q + Fraction(1, 2)).denominator
    return int(r) * int(mult)


def sign_bits_per_weight(m: int, n: int, ranks: Iterable[int]) -> Fraction:
    """Sign bits per original weight: sum_p r_p (m + n) / (m n)."""
    return Fraction(sum(int(r) * (m + n) for r in ranks), m * n)


def scale_bits_per_weight(m: int, n: int, ranks: Iterable[int]) -> Fraction:
    """fp16 scale bits per original weight: sum_p 16 (m + n + r_p) / (m n)."""
    return Fraction(sum(16 * (m + n + int(r)) for r in ranks), m * n)


def linear_storage_bytes(m: int, n: int, ranks: Iterable[int]) -> Fraction:
    """Bytes of one factorised linear: sign bits / 8 plus fp16 scales."""
    ranks = list(ranks)
    return Fraction(sum(int(r) * (m + n) for r in ranks), 8) + 2 * sum(m + n + int(r) for r in ranks)


def forward_rows(x: np.ndarray, paths: Sequence[Dict], m: int, n: int, rows: Sequence[int]) -> np.ndarray:
    """y[:, rows] from the explicit rows W[rows, :] of the same weight definition.

    Lets full-size layers be checked on a sample of outputs: only the selected
    rows of W = sum_p diag(h_p) U_p diag(l_p) V_p^T diag(g_p) are formed.
    """
    rows = np.asarray(rows, dtype=np.int64)
    x = np.asarray(x, dtype=np.float64)
    Wr = np.zeros((rows.size, n), dtype=np.float64)
    for path in paths:
        f = decode_path(path, m, n)
        left = f["h"][rows, None] * f["U"][rows] * f["l"][None, :]
        Wr += left @ (f["V"] * f["g"][:, None]).T
    return x @ Wr.T
