"""E8 lattice fields for coset-conditioned entropy coding (test infrastructure only).

EntroPack page: blocks of eight row-normalised weights are quantised to E8 lattice
points identified by invertible integer fields (Section 3.2); a coset-conditioned
model with 17 categorical distributions codes the fields (Section 3.3); parity
reduction codes m in place of the eighth integer coordinate z8 (Section A.3).

E8 = D8 u (D8 + 1/2), D8 = {z in Z^8 : sum z even}.  The page gives no formulas;
the readings used here:

* fields of a point v: coset c = 1 if the coordinates are half-integers, else 0;
  z = v - c/2 (an element of D8); emitted in the order c, z1 .. z7, m with
  m = floor(z8 / 2).  The inverse is z8 = 2m + ((z1 + .. + z7) mod 2), which holds
  because sum z is even.
* table 0 codes c; table 1 + 8c + j codes field j (j = 0..6 -> z_{j+1}, j = 7 -> m)
  given coset c: 1 + 2 * 8 = 17 tables.
* nearest point: Conway and Sloane's decoder -- round every coordinate (half to
  even); for D8, if the sum is odd re-round the coordinate with the largest
  rounding error the other way (lowest index on ties); for E8 take the closer of
  the D8 and D8 + 1/2 answers (coset 0 on ties).
* doubled coordinates 2v = 2z + c are what the decoder rebuilds: INT8 output is
  2v with half the row scale, FP8 output is the nearest E4M3 value of v.
"""
from __future__ import annotations

import numpy as np

N_TABLES = 17


def _nearest_d8(x: np.ndarray) -> np.ndarray:
    f = np.rint(x)
    err = x - f
    odd = (f.sum(axis=-1) % 2) != 0
    worst = np.argmax(np.abs(err), axis=-1)
    g = f.copy()
    idx = np.arange(x.shape[0])
    w_err = err[idx, worst]
    g[idx, worst] = np.where(w_err >= 0, f[idx, worst] + 1, f[idx, worst] - 1)
    return np.where(odd[:, None], g, f)


def nearest_e8(u: np.ndarray):
    """u float [n, 8] -> (coset int [n], z int64 [n, 8]) of the nearest E8 point."""
    u = np.asarray(u, dtype=np.float64).reshape(-1, 8)
    z0 = _nearest_d8(u)
    z1 = _nearest_d8(u - 0.5)
    d0 = ((u - z0) ** 2).sum(axis=1)
    d1 = ((u - (z1 + 0.5)) ** 2).sum(axis=1)
    c = (d1 < d0).astype(np.int64)
    z = np.where(c[:, None] == 1, z1, z0).astype(np.int64)
    return c, z


def point_to_fields(c: np.ndarray, z: np.ndarray) -> np.ndarray:
    """-> int64 [n, 9]: c, z1..z7, m."""
    z = np.asarray(z, dtype=np.int64)
    out = np.empty((z.shape[0], 9), dtype=np.int64)
    out[:, 0] = c
    out[:, 1:8] = z[:, :7]
    out[:, 8] = np.floor_divide(z[:, 7], 2)
    return out


def fields_to_point(fields: np.ndarray):
    f = np.asarray(fields, dtype=np.int64)
    c = f[:, 0]
    z = np.empty((f.shape[0], 8), dtype=np.int64)
    z[:, :7] = f[:, 1:8]
    z[:, 7] = 2 * f[:, 8] + (z[:, :7].sum(axis=1) & 1)
    return c, z


def doubled_coords(c: np.ndarray, z: np.ndarray) -> np.ndarray:
    return 2 * np.asarray(z, dtype=np.int64) + np.asarray(c, dtype=np.int64)[:, None]


def doubled_to_point(v2: np.ndarray):
    """2v int [n, 8] -> (c, z); raises if a block is not an E8 point."""
    v2 = np.asarray(v2, dtype=np.int64).reshape(-1, 8)
    c = v2[:, 0] & 1
    if np.any((v2 & 1) != c[:, None]):
        raise ValueError("block mixes integer and half-integer coordinates")
    z = (v2 - c[:, None]) // 2
    if np.any(z.sum(axis=1) % 2 != 0):
        raise ValueError("block is not in D8 or D8 + 1/2")
    return c, z


def table_of_field(c: np.ndarray, j: int) -> np.ndarray:
    """Table index of field position j in 0..8 (0 = coset)."""
    if j == 0:
        return np.zeros_like(c)
    return 1 + 8 * np.asarray(c) + (j - 1)
