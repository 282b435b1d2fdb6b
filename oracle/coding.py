"""Symbol statistics and frequency tables (test infrastructure only).

* Shannon entropy H(X) = -sum p log2 p: DFloat11 page, "Motivation" paragraph,
  Eq. 2.
* Cross-entropy between the empirical distribution and the table approximation
  f/M as the predicted compressed size (a lower bound): MINE page, Section 4.2,
  "Compressed Size Prediction".
* Table size M = 2^m and the requirement that every occurring symbol receive a
  slot (f >= 1): MINE page Section 4.1 ("Escapes": constructing k-tuples over t
  values calls for M >= t^k) and EntroPack page Section C.1 (precision decides how
  many symbols can receive positive frequencies).

The pages do not fix how counts are quantised to frequencies.  The reading used
here: choose integer f_s >= 1 for every occurring symbol (0 otherwise), sum f = M,
minimising the cross-entropy sum_s c_s * log2(M / f_s).  That objective is
separable and concave in f, so adding one unit at a time to the symbol with the
largest marginal gain c_s * (log2(f_s + 1) - log2(f_s)) is exact.  Ties go to the
smallest symbol index.  A single occurring symbol gets f = M.
"""
from __future__ import annotations

import math

import numpy as np


def histogram(symbols: np.ndarray, alphabet: int) -> np.ndarray:
    s = np.asarray(symbols).ravel().astype(np.int64)
    if s.size and (s.min() < 0 or s.max() >= alphabet):
        raise ValueError("symbol outside alphabet")
    return np.bincount(s, minlength=alphabet).astype(np.int64)


def entropy_bits(counts: np.ndarray) -> float:
    """Empirical Shannon entropy in bits per symbol (Eq. 2 of the DFloat11 page)."""
    c = np.asarray(counts, dtype=np.float64)
    n = c.sum()
    if n == 0:
        return 0.0
    p = c[c > 0] / n
    return float(-(p * np.log2(p)).sum())


def cross_entropy_total_bits(counts: np.ndarray, freq: np.ndarray, log2_m: int) -> float:
    """sum_s c_s * log2(M / f_s): the size predictor of MINE Section 4.2."""
    c = np.asarray(counts, dtype=np.float64)
    f = np.asarray(freq, dtype=np.float64)
    used = c > 0
    if np.any(f[used] <= 0):
        return math.inf
    return float((c[used] * (log2_m - np.log2(f[used]))).sum())


def marginal_log2_table(m_slots: int) -> list[float]:
    """d[f] = log2(f + 1) - log2(f) for f = 1 .. M, using the C library's log2."""
    return [0.0] + [math.log2(f + 1) - math.log2(f) for f in range(1, m_slots + 1)]


def normalise(counts: np.ndarray, log2_m: int) -> np.ndarray:
    """Optimal integer frequencies (see module docstring).  Returns int64 [alphabet]."""
    counts = np.asarray(counts, dtype=np.int64)
    m_slots = 1 << log2_m
    present = counts > 0
    n_present = int(present.sum())
    f = np.zeros(counts.shape[0], dtype=np.int64)
    if n_present == 0:
        return f
    if n_present > m_slots:
        raise ValueError("more occurring symbols than table slots")
    if n_present == 1:
        f[present] = m_slots
        return f
    d = np.array(marginal_log2_table(m_slots), dtype=np.float64)
    f[present] = 1
    cnt = counts.astype(np.float64)
    gain = np.where(present, cnt * d[np.minimum(f, m_slots)], -np.inf)
    for _ in range(m_slots - n_present):
        s = int(np.argmax(gain))          # first maximum = smallest index on ties
        f[s] += 1
        gain[s] = cnt[s] * d[f[s]]
    return f


def cumulative(freq: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum over symbol order."""
    f = np.asarray(freq, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(f)[:-1]]).astype(np.int64)


def slot_to_symbol(freq: np.ndarray) -> np.ndarray:
    """Slots [cum_s, cum_s + f_s) map to symbol s."""
    f = np.asarray(freq, dtype=np.int64)
    return np.repeat(np.arange(f.shape[0], dtype=np.int64), f)


def tuple_mode_legal(values: int, k: int, log2_m: int) -> bool:
    """k-tuples over `values` distinct values fit a table of M slots iff values^k <= M
    (MINE page, Section 4.1 "Escapes" and Section 4.2 "Tuning t")."""
    return values ** k <= (1 << log2_m)
