"""Helpers shared by the GPU parity tests: host <-> device copies of the
seeded byte patterns and the element-wise tolerance check."""
import numpy as np
import torch

import oracle

DEV = "cuda:0"


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(DEV).view(torch.bfloat16)


def to_dev_u8(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).to(DEV)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def empty_bf16(m, n, fill_bits=None):
    t = torch.empty((m, n), dtype=torch.int16, device=DEV)
    if fill_bits is not None:
        t.fill_(int(np.int16(np.uint16(fill_bits))))
    return t.view(torch.bfloat16)


def check_close(got_bits: np.ndarray, ref: np.ndarray, k: int, sig_a: float, sig_b: float, what=""):
    """|c - ref| <= 8e-3*|ref| + 4e-3*sqrt(K)*sA*sB element by element where
    ref is finite; where ref is NaN the output must be NaN, and where ref is
    +-Inf the output must be the same infinity."""
    got = oracle.bf16_to_f64(got_bits)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    tol = oracle.tolerance(np.where(fin, ref, 0.0), k, sig_a, sig_b)
    err = np.abs(got - ref)
    bad = np.where(fin, ~(err <= tol), ~((np.isnan(ref) & np.isnan(got)) | (got == ref)))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: got {got[tuple(i)]!r} ref {ref[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; {detail}")
    e = np.where(fin, err / np.maximum(tol, 1e-300), 0.0)
    return float(e.max()) if e.size else 0.0


def assert_values_equal(got_bits: np.ndarray, want_bits: np.ndarray, what=""):
    """BF16 outputs equal as values: NaN matches any NaN, -0 matches +0;
    everything else bit for bit."""
    g = oracle.bf16_to_f64(got_bits)
    w = oracle.bf16_to_f64(want_bits)
    same = (np.isnan(g) & np.isnan(w)) | (g == w)
    if not same.all():
        i = tuple(np.argwhere(~same)[0])
        raise AssertionError(f"{what}: {int((~same).sum())} of {same.size} differ; first at {i}: "
                             f"got {int(got_bits[i]):#x} want {int(want_bits[i]):#x}")


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what=""):
    if not np.array_equal(got, want):
        diff = np.argwhere(got != want)
        i = tuple(diff[0])
        raise AssertionError(f"{what}: {len(diff)} of {got.size} differ; first at {i}: "
                             f"got {int(got[i]):#x} want {int(want[i]):#x}")
