"""CPU fp64 reference of the Dual-SVID initialisation of a LittleBit layer.

TEST INFRASTRUCTURE.  Like the forward oracle in this package, this is the
checker, not the product: only the test suite may import it.  It shares no
code with the HIP library.

What it computes ("LittleBit: Ultra Low-Bit Quantization via Latent
Factorization", paper notes, section "Key design / Dual-SVID initialisation"
and section "Residual compensation"):

1. a truncated SVD of W gives factors U', V' of rank r;
2. the sign factors are U_sign = sign(U'), V_sign = sign(V');
3. a rank-1 SVD of |U'| and one of |V'| give the initial row, column and
   latent scales;
4. the residual path is initialised the same way from W - W_pri,0.

Readings where the pages are silent (each is listed in the design notes):
* The singular values are split evenly: U' = U_r diag(sqrt s), V' = V_r
  diag(sqrt s), so that U' V'^T is the rank-r truncation of W.
* |U'| ~ a b^T (its top singular pair, sigma split evenly, signs chosen so the
  sums of a and b are not negative) gives h = a and a latent factor l_u = b;
  |V'| ~ c d^T gives g = c and l_v = d; the latent scale is l = l_u o l_v.
  Then diag(h) U_sign diag(l) V_sign^T diag(g) = (U_sign o h l_u^T)(V_sign o g
  l_v^T)^T, which equals U' V'^T whenever |U'| and |V'| are exactly rank 1.
* sign(0) = +1.
* The residual path starts from W minus the primary path as it will be stored
  (scales rounded to fp16), so that it compensates what the forward computes.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from .littlebit_oracle import pack_signs, reconstruct_w


def truncated_factors(W: np.ndarray, r: int):
    """U' [m, r], V' [n, r] with U' V'^T the rank-r truncated SVD of W."""
    U, s, Vt = np.linalg.svd(np.asarray(W, np.float64), full_matrices=False)
    root = np.sqrt(s[:r])
    return U[:, :r] * root[None, :], Vt[:r, :].T * root[None, :]


def rank1(M: np.ndarray):
    """(a, b) with a b^T the best rank-1 approximation of M (top singular pair,
    sigma split evenly), signs chosen so that sum(a) and sum(b) are not negative."""
    U, s, Vt = np.linalg.svd(np.asarray(M, np.float64), full_matrices=False)
    a = U[:, 0] * np.sqrt(s[0])
    b = Vt[0, :] * np.sqrt(s[0])
    if a.sum() + b.sum() < 0:
        a, b = -a, -b
    return a, b


def sign_pm1(A: np.ndarray) -> np.ndarray:
    """sign() with sign(0) = +1, as int8."""
    return np.where(np.asarray(A) < 0, -1, 1).astype(np.int8)


def dual_svid(W: np.ndarray, r: int) -> Dict[str, np.ndarray]:
    """One path's initial factors in float64: U_sign [m, r], V_sign [n, r]
    (int8 +-1), h [m], g [n], l [r]."""
    Up, Vp = truncated_factors(W, r)
    h, lu = rank1(np.abs(Up))
    g, lv = rank1(np.abs(Vp))
    return dict(U=sign_pm1(Up), V=sign_pm1(Vp), h=h, g=g, l=lu * lv)


def path_weight(f: Dict[str, np.ndarray]) -> np.ndarray:
    """diag(h) U diag(l) V^T diag(g) of float64 factors."""
    return (f["h"][:, None] * f["U"] * f["l"][None, :]) @ (f["V"] * f["g"][:, None]).T


def fp16_bits(v: np.ndarray) -> np.ndarray:
    """Round to IEEE half (nearest, ties to even) and return the bit patterns."""
    return np.asarray(v, np.float64).astype(np.float16).view(np.uint16)


def stored_path(f: Dict[str, np.ndarray]) -> Dict:
    """A path in the library's interchange form: packed signs, fp16 scale bits."""
    U, V = f["U"], f["V"]
    return dict(rank=int(U.shape[1]), u_words=pack_signs(U), v_words=pack_signs(V),
                h=fp16_bits(f["h"]), g=fp16_bits(f["g"]), l=fp16_bits(f["l"]))


def init_paths(W: np.ndarray, ranks: Sequence[int]) -> List[Dict]:
    """Dual-SVID of W for the primary path, then of what the stored paths so
    far leave over for each further path (residual compensation)."""
    W = np.asarray(W, np.float64)
    m, n = W.shape
    paths: List[Dict] = []
    for r in ranks:
        left = W - reconstruct_w(paths, m, n) if paths else W
        paths.append(stored_path(dual_svid(left, int(r))))
    return paths
