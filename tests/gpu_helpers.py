"""Shared helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle as O
from sparse_mixture_experts_forward_amd import synth

DEV = "cuda:0"

# Tolerances (per-token normwise max relative error, see the design notes):
TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy: bf16 as uint16 patterns, else the same dtype."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def widen_t(t: torch.Tensor) -> np.ndarray:
    """float64 copy of a device tensor (bf16 decoded exactly)."""
    a = to_host_bits(t)
    return O.widen(a, "bf16") if t.dtype == torch.bfloat16 else a.astype(np.float64)


class DeviceExperts:
    """Oracle-side access to generator-made weights living on the GPU: one expert is
    copied to the host and widened to float64 at a time."""

    def __init__(self, layer_w: dict, shared: bool = False):
        self.w = layer_w
        self.p = "shared_" if shared else ""
        self._cache = {}

    def __call__(self, e: int) -> O.ExpertWeights:
        if e not in self._cache:
            if len(self._cache) > 2:
                self._cache.clear()
            g = lambda n: (None if self.w.get(self.p + n) is None else widen_t(self.w[self.p + n][e]))
            b1 = None if self.p else (None if self.w.get("b1") is None else widen_t(self.w["b1"][e]))
            b2 = None if self.p else (None if self.w.get("b2") is None else widen_t(self.w["b2"][e]))
            self._cache[e] = O.ExpertWeights(w1=g("w1"), w2=g("w2"), w3=g("w3"), b1=b1, b2=b2)
        return self._cache[e]


def normwise_err(y_gpu: np.ndarray, y_ref: np.ndarray):
    """max over rows of ||y - ref||_inf / ||ref||_inf over rows whose reference is not 0;
    rows whose reference is exactly 0 must be exactly 0 on the GPU."""
    ref_norm = np.abs(y_ref).max(axis=1)
    nz = ref_norm > 0
    if (~nz).any():
        assert (y_gpu[~nz] == 0).all(), "rows with a zero reference must be exactly zero"
    if not nz.any():
        return 0.0
    return float((np.abs(y_gpu[nz] - y_ref[nz]).max(axis=1) / ref_norm[nz]).max())


def elementwise_err(y_gpu: np.ndarray, y_ref: np.ndarray, floor: float = 1e-2) -> float:
    """max over elements of |y - ref| / max(|ref|, floor * ||ref_t||_inf): the element-wise
    relative error, with an absolute floor scaled to each row's largest value (elements
    far below their row's scale are measured against that floor).  Reported beside the
    normwise error; rows whose reference is 0 are skipped (normwise_err checks them)."""
    ref_norm = np.abs(y_ref).max(axis=1, keepdims=True)
    nz = ref_norm[:, 0] > 0
    if not nz.any():
        return 0.0
    den = np.maximum(np.abs(y_ref[nz]), floor * ref_norm[nz])
    return float((np.abs(y_gpu[nz] - y_ref[nz]) / den).max())


# Parity margins of the tests that ran, printed in the terminal summary (tests/conftest.py).
MARGINS = []


def current_test() -> str:
    """The running test's id (file part dropped)."""
    t = os.environ.get("PYTEST_CURRENT_TEST", "?").split("::")[-1]
    return t.rsplit(" ", 1)[0]


def record_margin(case: str, normwise: float, tol: float, elementwise: float = None,
                  n_tokens: int = None):
    MARGINS.append(dict(case=case, normwise=normwise, tol=tol, elementwise=elementwise,
                        n_tokens=n_tokens))
    el = "" if elementwise is None else f", element-wise {elementwise:.3e}"
    nt = "" if n_tokens is None else f" over {n_tokens} tokens"
    print(f"  {case}: normwise {normwise:.3e} (tolerance {tol:g}){el}{nt}", flush=True)


def logits_tolerance(x64: np.ndarray, wr64: np.ndarray) -> np.ndarray:
    """Bound used for the float32 router product: 1e-5 of sum_c |x_c w_c| plus a floor.
    (Reordered float32 sums of d terms stay far inside d * 2^-24 of that sum.)"""
    return 1e-5 * (np.abs(x64) @ np.abs(wr64)) + 1e-7


def print_case(*parts):
    print("CASE", *parts, flush=True)
