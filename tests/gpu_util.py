"""Helpers of the GPU parity tests: device upload of the seeded inputs, read-back,
and the pass/fail gates.

Gates (the tolerances stated for this path): fp32 inputs, max-abs <= 1e-4;
bf16 / fp16 inputs, max-abs <= 1e-2 and relative L2 <= 5e-3.  Errors are taken
against the unrounded fp64 oracle over every checked element of a case.  The
logsumexp, which the stated tolerances do not name, is gated with the same
bound scaled by max(1, |lse|): its error is that of the fp32 scores it is
made of, which grows with their magnitude (scores of a few hundred carry
errors of a few 1e-4 after an fp32 dot product), and the relative L2 gate
applies to it unchanged.  A failure names the first offending query row and
head dimension.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {
    "f32": dict(max_abs=1e-4, rel_l2=None),
    "bf16": dict(max_abs=1e-2, rel_l2=5e-3),
    "f16": dict(max_abs=1e-2, rel_l2=5e-3),
}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def stats(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    idx = np.unravel_index(int(np.argmax(diff)), diff.shape) if diff.size else ()
    return {
        "max_abs": float(diff.max()) if diff.size else 0.0,
        "rel_l2": float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)),
        "argmax": tuple(int(i) for i in idx),
        "finite": bool(np.all(np.isfinite(got))),
    }


def gate(what: str, got, ref, dtype: str, rows=None, scaled: bool = False, max_abs=None):
    """Assert the tolerance of `dtype`; rows maps the first axis to query rows.
    scaled=True bounds |got - ref| by max_abs * max(1, |ref|) (the logsumexp gate);
    max_abs overrides the element bound for cases outside the stated workloads."""
    s = stats(got, ref)
    tol = dict(TOL[dtype])
    if max_abs is not None:
        tol["max_abs"] = max_abs
    say(f"  {what}: max_abs={s['max_abs']:.3e} rel_l2={s['rel_l2']:.3e}")
    assert s["finite"], f"{what}: non-finite output"
    ref64 = np.asarray(ref, np.float64)
    bound = tol["max_abs"] * (np.maximum(1.0, np.abs(ref64)) if scaled else 1.0)
    bad = np.abs(np.asarray(got, np.float64) - ref64) > bound
    if bad.any():
        first = np.argwhere(bad)[0]
        row = int(first[0]) if rows is None else int(np.asarray(rows)[first[0]])
        col = int(first[-1]) if bad.ndim > 1 else -1
        raise AssertionError(f"{what}: max_abs {s['max_abs']:.3e} > {tol['max_abs']:.0e}; first "
                             f"offending element at query row {row}, head dim {col}")
    # relative L2 is undefined for an all-zero reference (e.g. dQ of one-key rows);
    # the element bound above still applies there
    if tol["rel_l2"] is not None and np.any(ref64 != 0):
        assert s["rel_l2"] <= tol["rel_l2"], f"{what}: rel_l2 {s['rel_l2']:.3e} > {tol['rel_l2']:.0e}"
    return s
