"""Helpers shared by the GPU tests: build layers from seeded inputs, run the
oracle, and apply the acceptance criteria."""
from __future__ import annotations

import sys
from typing import Dict, List, Sequence

import numpy as np

import oracle
import synth

# bf16 I/O acceptance (our reading of the 1e-2 accuracy bound; rounding the exact
# result to bf16 alone exceeds 1e-2 * rms when max|y| / rms(y) > ~2.6):
#   (i)  rms(y - y_ref) <= 1e-2 * rms(y_ref)
#   (ii) max|y - y_ref| <= 1e-2 * rms(y_ref) + 2^-7 * max|y_ref|
BF16_ERMS = 1e-2
BF16_EMAX_RMS = 1e-2
BF16_EMAX_ULP = 2.0 ** -7
# fp32 I/O: max|y - y_ref| <= 1e-5 * rms(y_ref)
FP32_EMAX_RMS = 1e-5


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (through fp32, nearest even), as float64."""
    return oracle.decode_bf16(synth.bf16_bits_from_f32(np.asarray(v, np.float32)))


def stats(y: np.ndarray, y_ref: np.ndarray) -> Dict[str, float]:
    """Error statistics of y against the exact y_ref.  emax_rel_rms is the
    literal statistic max|y - y_ref| / rms(y_ref); emax_vs_rounded_rel_rms is
    the same against y_ref rounded to bf16 (output rounding taken out of the
    comparison): both are logged, the acceptance uses erms and emax."""
    y = np.asarray(y, np.float64)
    e = y - y_ref
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    rms_safe = rms if rms > 0 else 1.0
    return dict(rms=rms, erms=float(np.sqrt(np.mean(e ** 2)) / rms_safe), emax=float(np.max(np.abs(e))),
                emax_rel_rms=float(np.max(np.abs(e)) / rms_safe), ymax=float(np.max(np.abs(y_ref))),
                emax_vs_rounded_rel_rms=float(np.max(np.abs(y - bf16_round(y_ref))) / rms_safe))


def assert_bf16_close(y: np.ndarray, y_ref: np.ndarray, what: str = "") -> Dict[str, float]:
    s = stats(y, y_ref)
    bound = BF16_EMAX_RMS * s["rms"] + BF16_EMAX_ULP * s["ymax"]
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert s["erms"] <= BF16_ERMS, f"{what}: E_rms {s['erms']:.3e} > {BF16_ERMS}"
    assert s["emax"] <= bound, f"{what}: E_max {s['emax']:.3e} > bound {bound:.3e} (rms {s['rms']:.3e})"
    log(f"    [{what}] literal max|y-y_ref|/rms = {s['emax_rel_rms']:.4f}, against bf16(y_ref) "
        f"{s['emax_vs_rounded_rel_rms']:.4f}, E_rms {s['erms']:.2e}")
    return s


def assert_fp32_close(y: np.ndarray, y_ref: np.ndarray, what: str = "") -> Dict[str, float]:
    s = stats(y, y_ref)
    assert s["emax"] <= FP32_EMAX_RMS * s["rms"], f"{what}: E_max {s['emax']:.3e} > 1e-5 * rms {s['rms']:.3e}"
    return s


def to_f64(t) -> np.ndarray:
    """A device bf16/fp32 tensor as exact float64 numpy."""
    import torch
    if t.dtype == torch.bfloat16:
        return oracle.decode_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def x_tensor(x_np: np.ndarray, device="cuda"):
    """Generator activations (uint16 bf16 bits or float32) -> device tensor."""
    import torch
    if x_np.dtype == np.uint16:
        return torch.from_numpy(x_np.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x_np, np.float32)).to(device)


def x_f64(x_np: np.ndarray) -> np.ndarray:
    if x_np.dtype == np.uint16:
        return oracle.decode_bf16(x_np)
    return x_np.astype(np.float64)
