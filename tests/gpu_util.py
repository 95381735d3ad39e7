"""Helpers shared by the GPU tests: upload seeded host inputs, compare."""

from __future__ import annotations

import sys

import numpy as np

import oracle

TOL = {  # max abs error allowed against the fp64 oracle
    "f32": {"o": 1e-5, "lse": 1e-5},
    "bf16": {"o": 1.5e-2, "lse": 1e-3},
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def up(x: np.ndarray, device="cuda"):
    """Host storage array (float32, or bf16 bits in uint16, or int32) -> GPU tensor."""
    torch = torch_mod()
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def down(t) -> np.ndarray:
    """GPU tensor -> float64 numpy (bf16 widened exactly)."""
    torch = torch_mod()
    return t.detach().to(torch.float64).cpu().numpy()


def bits(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def max_err(a, b, mask=None) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if mask is not None:
        a, b = a[mask], b[mask]
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d)) if d.size else 0.0


def lse_of(m, l):
    return oracle.finalize(np.asarray(m, np.float64), np.asarray(l, np.float64))


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def worst(got, ref, mask=None):
    """(max abs error, reference value there) for diagnostics."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    if mask is not None:
        d = np.where(mask, d, -1.0)
    i = np.unravel_index(int(np.argmax(d)), d.shape)
    return float(d[i]), float(ref[i]), tuple(int(x) for x in i)
