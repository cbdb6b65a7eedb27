"""Helpers shared by the GPU parity tests: host<->device moves and comparisons."""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


BF16_ULP = 2.0 ** -7      # one bfloat16 ulp, relative to the value (upper bound)


def assert_close_rms(got: np.ndarray, ref: np.ndarray, tol: float = 2e-2, what: str = "", ulp_rel: float = 0.0,
                     report_only: bool = False):
    """max |got - ref| <= tol * rms(ref), element by element relaxed to
    ulp_rel * |ref| where given: a bfloat16-stored intermediate may sit one
    rounding step away from the reference when the FP32 and float64 sums fall
    on two sides of a rounding boundary (heavy-tailed z has max/rms >> 1/tol)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    d = np.abs(got - ref)
    err = float(np.max(d)) if ref.size else 0.0
    bound = np.maximum(tol * rms, ulp_rel * np.abs(ref))
    worst = float(np.max(d / np.maximum(bound, 1e-300))) if ref.size else 0.0
    say(f"  {what}: max|err| {err:.3e}  rms(ref) {rms:.3e}  ratio {err / max(rms, 1e-300):.2e}  "
        f"worst/bound {worst:.2f}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if report_only:
        return err / max(rms, 1e-300)
    assert np.all(d <= bound), f"{what}: max|err| {err:.4e} > bound (tol {tol} * rms {rms:.4e}, ulp {ulp_rel})"
    return err / max(rms, 1e-300)
