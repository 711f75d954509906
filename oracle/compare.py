"""Comparator between a GPU bf16 result and the oracle's unrounded result.

TEST INFRASTRUCTURE ONLY (tests, smoke check).

Gate per element (g = GPU bf16 value, r = oracle value, unrounded):
  |g - r| <= ABS_TOL                                            and
  ulpdist(g, bf16_rne(r)) <= MAX_ULP  or  |g - r| <= ULP_FLOOR
where ulpdist counts steps on the ordered bf16 line (+0 == -0, NaN fails).
ABS_TOL = 2e-2 and MAX_ULP = 2 are the acceptance bound of this build.  The
floor 2**-22 (= 2 bf16 ulps at |r| = 2**-16) keeps references so small that a
bf16 ulp falls below fp32 accumulation noise from failing on noise alone; the
report also counts failures without the floor.

The per-case metrics follow the comparator the pages describe: max_abs,
max_rel and the share of bitwise-identical elements, and a self-test that
plants 1-ulp corruptions at chosen offsets and checks they are localised
[vllm.cpp PR #425, EVIDENCE: kernel numerics table and comparator self-test].
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

ABS_TOL = 2e-2
MAX_ULP = 2
ULP_FLOOR = 2.0 ** -22
REL_FLOOR = 2.0 ** -16


def bf16_rne(r: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, in one
    step (no double rounding through float32).  Returns float64."""
    r = np.asarray(r, np.float64)
    out = r.copy()
    fin = np.isfinite(r) & (r != 0)
    m, e = np.frexp(r[fin])                  # r = m * 2**e, 0.5 <= |m| < 1
    out[fin] = np.ldexp(np.rint(m * 256.0), e - 8)   # 8 significant bits
    return out


def bits_of_bf16_values(x: np.ndarray) -> np.ndarray:
    """uint16 patterns of float64 values that are exactly bf16-representable."""
    f = np.asarray(x, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits(t) -> np.ndarray:
    """uint16 patterns of a bf16 torch tensor (any device)."""
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return np.asarray(t, np.uint16)


def bits_to_f64(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_dist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between two arrays of bf16 bit patterns."""
    def key(u):
        u = u.astype(np.int64)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)
    return np.abs(key(a) - key(b))


@dataclass
class Report:
    n: int
    max_abs: float
    max_rel: float
    bitwise_pct: float
    max_ulp: int
    n_fail: int
    n_fail_unfloored: int
    n_nan: int
    worst: tuple = field(default=())

    @property
    def ok(self) -> bool:
        return self.n_fail == 0

    def __str__(self) -> str:
        return (f"n={self.n} max_abs={self.max_abs:.3e} max_rel={self.max_rel:.3e} "
                f"bitwise={self.bitwise_pct:.4f}% max_ulp={self.max_ulp} fail={self.n_fail} "
                f"(unfloored {self.n_fail_unfloored}) nan={self.n_nan} worst={self.worst}")


def compare(gpu, ref: np.ndarray, abs_tol: float = ABS_TOL, max_ulp: int = MAX_ULP,
            ulp_floor: float = ULP_FLOOR) -> Report:
    g_bits = bf16_bits(gpu).reshape(-1)
    r = np.asarray(ref, np.float64).reshape(-1)
    assert g_bits.shape == r.shape, (g_bits.shape, r.shape)
    g = bits_to_f64(g_bits)
    r_b = bits_of_bf16_values(bf16_rne(r))
    nan = np.isnan(g) | np.isnan(r)
    diff = np.abs(g - r)
    diff = np.where(nan, np.inf, diff)
    ulps = np.where(nan, 1 << 20, ulp_dist(g_bits, r_b))
    ulp_ok = (ulps <= max_ulp)
    ok = (diff <= abs_tol) & (ulp_ok | (diff <= ulp_floor))
    ok_unfloored = (diff <= abs_tol) & ulp_ok
    big = np.abs(r) >= REL_FLOOR
    rel = np.where(big, diff / np.where(big, np.abs(r), 1.0), 0.0)
    worst_i = int(np.argmax(np.where(ok, -1.0, diff))) if (~ok).any() else int(np.argmax(ulps))
    return Report(n=int(r.size), max_abs=float(diff.max()) if r.size else 0.0,
                  max_rel=float(rel.max()) if r.size else 0.0,
                  bitwise_pct=100.0 * float((g_bits == r_b).mean()) if r.size else 100.0,
                  max_ulp=int(ulps.max()) if r.size else 0, n_fail=int((~ok).sum()),
                  n_fail_unfloored=int((~ok_unfloored).sum()), n_nan=int(nan.sum()),
                  worst=(worst_i, float(g[worst_i]) if r.size else 0.0,
                         float(r[worst_i]) if r.size else 0.0))


def mismatch_offsets(gpu, ref: np.ndarray) -> np.ndarray:
    """Flat offsets where the GPU bits differ from bf16_rne(ref)."""
    g_bits = bf16_bits(gpu).reshape(-1)
    r_b = bits_of_bf16_values(bf16_rne(np.asarray(ref, np.float64).reshape(-1)))
    return np.nonzero(g_bits != r_b)[0]


def close_f32(gpu: np.ndarray, ref: np.ndarray, rtol: float = 1e-5, atol: float = 1e-5):
    """Check for fp32 intermediate outputs (split partials): |g-r| <= atol + rtol|r|,
    with +-inf required to match exactly.  Returns (ok, max_err)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    inf = np.isinf(r) | np.isinf(g)
    same_inf = np.where(inf, g == r, True)
    fin = ~inf
    with np.errstate(invalid="ignore"):
        err = np.abs(g - r)
    bound = atol + rtol * np.abs(r)
    ok = bool(same_inf.all() and (err[fin] <= bound[fin]).all() and not np.isnan(g).any())
    return ok, float(err[fin].max()) if fin.any() else 0.0
