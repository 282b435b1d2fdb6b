"""Logical tensors <-> symbol streams, and symbol tiling (test infrastructure only).

* Integer codes, k codes per symbol ("Single / Pair / Quad" modes): MINE page,
  Section 4.1, "Data Types" (k-tuples over t values need M >= t^k).  Reading taken:
  a b-bit code q in [-2^(b-1), 2^(b-1)) maps to the unsigned digit q + 2^(b-1), and
  the digit of the i-th column of a k-tuple sits at bits [b*i, b*(i+1)) of the
  symbol (first column in the low bits).
* BF16: sign/exponent/mantissa layout of Eq. 1 on the DFloat11 page; the 8-bit
  exponent is the coded symbol and sign + 7-bit mantissa stay a raw byte, as in the
  DFloat11 format (PackedSignMantissa) and the MINE page, Section 4.1.  The raw
  byte is sign << 7 | mantissa, and the weight is rebuilt with the bit join of the
  DFloat11 page's Algorithm 1: (sign << 8) | (exponent << 7) | mantissa, with the
  sign taken from bit 7 of the raw byte.
* BF16 exponent pairs: two consecutive columns per symbol, each exponent as a
  4-bit digit into the table's t = 16 stored exponents (MINE page, Section 4.1
  "Escapes": a table restricted to the t most frequent values admits pairs when
  t^2 <= M; Section 4.2 "Tuning t": keep the t most frequent codes and always 0,
  which escaped values are coded as).  Readings taken: with at most 256 pair
  symbols per table, t = 16; the stored exponents are 0 and the 15 most frequent
  other exponents (ties to the smaller exponent), ascending, so digit 0 is
  exponent 0; an escaped weight is coded as digit 0 with raw byte 0, i.e. as +0.0,
  and its bf16 bits go to the correction stream (``corrections``).
* Quads of 4-bit codes: four consecutive columns per symbol over a table of t
  stored 4-tuples (MINE page, Section 4.1 "Escapes": restrict the decoding table
  to the most frequent symbols, code an escaped value as 0 and keep the real value
  in the correction stream).  The page builds pairs over t single values and
  limits 4-bit codes to pairs; reading taken here for quads: the table stores the
  t most frequent whole tuples (ties to the smaller tuple, the zero tuple always
  kept), and a tuple outside the table is coded as the stored tuple reached by
  setting the fewest of its codes to 0 (the first such set of positions in
  (count, mask) order); each nonzero code so set is escaped, its record holding the
  code's value as a bf16 number.
* FP8 E4M3: the byte itself is the symbol (MINE page Section 4.1; OCP E4M3 with
  bias 7, no infinities, S.1111.111 = NaN).
* Tiling: rows in groups of 64 (lane l = row r0 + l, the MINE page's lane-per-row
  grid layout, Section 4 "Grid Layout"), columns in slices; the tile of
  (row group g, slice c) has index g * n_slices + c.
"""
from __future__ import annotations

import math

import numpy as np

LANES = 64


# ---------------------------------------------------------------- integer codes
def int_codes_to_symbols(codes: np.ndarray, code_bits: int, k: int) -> np.ndarray:
    q = np.asarray(codes, dtype=np.int64)
    n, K = q.shape
    if K % k:
        raise ValueError("columns not a multiple of k")
    half = 1 << (code_bits - 1)
    if q.size and (q.min() < -half or q.max() >= half):
        raise ValueError("code outside range")
    d = (q + half).reshape(n, K // k, k)
    sym = np.zeros((n, K // k), dtype=np.int64)
    for i in range(k):
        sym |= d[:, :, i] << (code_bits * i)
    return sym


def symbols_to_int_codes(sym: np.ndarray, code_bits: int, k: int) -> np.ndarray:
    s = np.asarray(sym, dtype=np.int64)
    n, ns = s.shape
    half = 1 << (code_bits - 1)
    mask = (1 << code_bits) - 1
    out = np.zeros((n, ns, k), dtype=np.int64)
    for i in range(k):
        out[:, :, i] = ((s >> (code_bits * i)) & mask) - half
    return out.reshape(n, ns * k).astype(np.int8)


# ---------------------------------------------------------------- BF16
def bf16_split(bits: np.ndarray):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    exponent = (b >> 7) & 0xFF
    raw = ((b >> 8) & 0x80) | (b & 0x7F)
    return exponent.astype(np.int64), raw.astype(np.uint8)


def bf16_join(exponent: np.ndarray, raw: np.ndarray) -> np.ndarray:
    e = np.asarray(exponent, dtype=np.uint32)
    r = np.asarray(raw, dtype=np.uint32)
    return (((r & 0x80) << 8) | (e << 7) | (r & 0x7F)).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """Eq. 1 of the DFloat11 page: (-1)^s * 2^(e-127) * 1.m (and the usual specials)."""
    b = np.asarray(bits, dtype=np.uint32)
    s = (b >> 15) & 1
    e = ((b >> 7) & 0xFF).astype(np.int64)
    m = (b & 0x7F).astype(np.float64)
    mag = np.where(e == 0, m / 128.0 * 2.0 ** -126, (1.0 + m / 128.0) * np.exp2(e - 127.0))
    mag = np.where(e == 255, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


PAIR_DIGITS = 16


def bf16_pair_values(exponent_counts: np.ndarray) -> np.ndarray:
    """The 16 exponents of a pair table: 0, then the 15 most frequent nonzero
    exponents (more occurrences first, the smaller exponent on ties), in ascending
    order.  Digits beyond the occurring exponents hold 0 and are never used."""
    c = np.asarray(exponent_counts, dtype=np.int64)
    others = [e for e in range(1, 256) if c[e] > 0]
    others.sort(key=lambda e: (-int(c[e]), e))
    keep = sorted(others[:PAIR_DIGITS - 1])
    v = np.zeros(PAIR_DIGITS, dtype=np.int64)
    v[1:1 + len(keep)] = keep
    return v


def bf16_pair_split(bits: np.ndarray, values: np.ndarray):
    """bf16 bits [N, K] (K even) -> (pair symbols int64 [N, K/2], raw bytes uint8
    [N, K], escaped bool [N, K]).  Exponent e has digit d >= 1 if values[d] == e (the
    first such d); exponent 0 has digit 0; any other exponent is escaped: digit 0 and
    raw byte 0.  The even column's digit is the low nibble."""
    ex, raw = bf16_split(bits)
    if ex.shape[1] % 2:
        raise ValueError("pair mode needs an even column count")
    digit = np.zeros(256, dtype=np.int64)
    known = np.zeros(256, dtype=bool)
    known[0] = True
    for d in range(PAIR_DIGITS - 1, 0, -1):     # descending, so the first match wins
        v = int(values[d])
        if v != 0:
            digit[v] = d
            known[v] = True
    esc = ~known[ex]
    dg = np.where(esc, 0, digit[ex])
    raw = np.where(esc, 0, raw).astype(np.uint8)
    sym = dg[:, 0::2] | (dg[:, 1::2] << 4)
    return sym, raw, esc


def bf16_pair_join(sym: np.ndarray, raw: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Pair symbols [N, K/2] + raw bytes [N, K] -> bf16 bits [N, K] (escapes not yet
    applied: they read as +0.0)."""
    s = np.asarray(sym, dtype=np.int64)
    v = np.asarray(values, dtype=np.int64)
    ex = np.empty((s.shape[0], 2 * s.shape[1]), dtype=np.int64)
    ex[:, 0::2] = v[s & 15]
    ex[:, 1::2] = v[s >> 4]
    return bf16_join(ex, raw)


# ---------------------------------------------------------------- 4-bit code quads
QUAD_ZERO = 0x8888      # the tuple of four zero codes (digit 8 = code 0)


def quad_tuples(codes: np.ndarray) -> np.ndarray:
    """4-bit codes [N, K] (K % 4 == 0) -> tuples int64 [N, K/4], the digit q + 8 of
    column 4j + i at bits [4i, 4i + 4)."""
    return int_codes_to_symbols(codes, 4, 4)


def quad_stored(tuple_counts: np.ndarray, t: int) -> np.ndarray:
    """The stored tuples of a quad table: the t most frequent occurring tuples (more
    occurrences first, the smaller tuple on ties), with the zero tuple taking the
    place of the last one if it is not among them, in ascending order.  MINE page,
    Section 4.1 "Escapes" (a table restricted to the most frequent symbols, 0 always
    kept for the escaped values); read here for whole 4-tuples of codes."""
    c = np.asarray(tuple_counts, dtype=np.int64)
    occ = [int(v) for v in np.nonzero(c)[0]]
    occ.sort(key=lambda v: (-int(c[v]), v))
    keep = occ[:t]
    if QUAD_ZERO not in keep:
        keep = keep[:t - 1] + [QUAD_ZERO]
    return np.array(sorted(keep), dtype=np.int64)


def _zeroed(tup: int, mask: int) -> int:
    for i in range(4):
        if (mask >> i) & 1:
            tup = (tup & ~(15 << (4 * i))) | (8 << (4 * i))
    return tup


# masks over the four codes, fewest codes first, then the smaller mask
QUAD_MASKS = sorted(range(1, 16), key=lambda m: (bin(m).count("1"), m))


def quad_map(tuples: np.ndarray, stored: np.ndarray):
    """Tuples [N, n] -> (symbol ids int64 [N, n], escaped bool [N, 4n]).  A stored
    tuple is its own symbol; any other is coded as the stored tuple reached by
    setting some of its codes to 0, taking the first such set of positions in
    QUAD_MASKS order; its nonzero codes so set are escaped.  (Each distinct tuple is
    mapped once.)"""
    tu = np.asarray(tuples, dtype=np.int64)
    index = {int(v): i for i, v in enumerate(stored)}
    uniq, inv = np.unique(tu, return_inverse=True)
    ids_u = np.zeros(uniq.size, dtype=np.int64)
    esc_u = np.zeros((uniq.size, 4), dtype=bool)
    for n, v in enumerate(uniq.tolist()):
        if v in index:
            ids_u[n] = index[v]
            continue
        for m in QUAD_MASKS:
            z = _zeroed(v, m)
            if z in index:
                ids_u[n] = index[z]
                for p in range(4):
                    esc_u[n, p] = bool((m >> p) & 1) and ((v >> (4 * p)) & 15) != 8
                break
    inv = inv.reshape(tu.shape)
    return ids_u[inv], esc_u[inv].reshape(tu.shape[0], 4 * tu.shape[1])


def quad_join(ids: np.ndarray, stored: np.ndarray) -> np.ndarray:
    """Symbol ids [N, n] -> codes int8 [N, 4n] (escaped codes read as 0)."""
    tu = np.asarray(stored, dtype=np.int64)[np.asarray(ids, dtype=np.int64)]
    return symbols_to_int_codes(tu, 4, 4).astype(np.int8)


def small_int_bf16_bits(q: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of integers |q| <= 256 (exact): the high half of the fp32."""
    return (np.asarray(q, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- FP8 E4M3
def e4m3_value(byte: np.ndarray) -> np.ndarray:
    b = np.asarray(byte, dtype=np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_rne(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 byte, ties to the even code, sign kept (so tiny negatives give
    -0 = 0x80, as IEEE rounding does); |v| <= 448 required."""
    table = e4m3_value(np.arange(256))
    pos = np.array([b for b in range(128) if not math.isnan(table[b])])
    pv = table[pos]
    a = np.abs(np.asarray(v, dtype=np.float64))
    if np.any(a > 448.0):
        raise ValueError("value beyond E4M3 range")
    i = np.searchsorted(pv, a)
    i = np.clip(i, 1, len(pv) - 1)
    lo, hi = pv[i - 1], pv[i]
    pick_hi = (hi - a < a - lo) | ((hi - a == a - lo) & (pos[i] % 2 == 0))
    mag_code = np.where(pick_hi, pos[i], pos[i - 1])
    mag_code = np.where(a == 0, 0, mag_code)
    neg = np.signbit(np.asarray(v, dtype=np.float64))
    return (mag_code | np.where(neg, 0x80, 0)).astype(np.uint8)


# ---------------------------------------------------------------- tiling
def tile_plan(n_rows: int, n_sym: int, syms_per_slice: int):
    n_rg = -(-n_rows // LANES)
    n_sl = -(-n_sym // syms_per_slice) if n_sym else 0
    s_last = n_sym - (n_sl - 1) * syms_per_slice if n_sl else 0
    return n_rg, n_sl, syms_per_slice, s_last


def rows_to_tiles(rows: np.ndarray, syms_per_slice: int, fill=0):
    """[N, n_sym] per-row streams -> list over slice-kind of (tile ids, [T,64,S], active)."""
    rows = np.asarray(rows)
    n, n_sym = rows.shape
    n_rg, n_sl, s_full, s_last = tile_plan(n, n_sym, syms_per_slice)
    pad = np.full((n_rg * LANES, n_sym), fill, dtype=rows.dtype)
    pad[:n] = rows
    active_rows = np.zeros(n_rg * LANES, dtype=bool)
    active_rows[:n] = True
    groups = []
    if n_sl == 0:
        kinds = []
    elif s_last == s_full:
        kinds = [(list(range(n_sl)), s_full)]
    else:
        kinds = [(list(range(n_sl - 1)), s_full)] if n_sl > 1 else []
        kinds.append(([n_sl - 1], s_last))
    for slices, S in kinds:
        ids, data, act = [], [], []
        for g in range(n_rg):
            for c in slices:
                ids.append(g * n_sl + c)
                c0 = c * syms_per_slice
                data.append(pad[g * LANES:(g + 1) * LANES, c0:c0 + S])
                act.append(active_rows[g * LANES:(g + 1) * LANES])
        groups.append((np.array(ids, dtype=np.int64), np.stack(data) if data else
                       np.zeros((0, LANES, S), rows.dtype), np.stack(act) if act else
                       np.zeros((0, LANES), bool)))
    return groups


def tiles_to_rows(n_rows: int, n_sym: int, syms_per_slice: int, groups) -> np.ndarray:
    n_rg, n_sl, _, _ = tile_plan(n_rows, n_sym, syms_per_slice)
    out = None
    for ids, data, _ in groups:
        if out is None:
            out = np.zeros((n_rg * LANES, n_sym), dtype=data.dtype)
        for i, t in enumerate(ids):
            g, c = divmod(int(t), n_sl)
            c0 = c * syms_per_slice
            out[g * LANES:(g + 1) * LANES, c0:c0 + data.shape[2]] = data[i]
    if out is None:
        out = np.zeros((n_rg * LANES, n_sym), dtype=np.int64)
    return out[:n_rows]


def raw_plane_bytes(raw_tiles: np.ndarray, active: np.ndarray) -> np.ndarray:
    """Raw bytes of a group of tiles [T, 64, S] -> [T, G, 64, 16] with G = ceil(S/16).

    Lane l's bytes for steps 16g .. 16g+15 sit contiguously at [t, g, l, :] so one
    wave reads a step group with one 16-byte load per lane.  Padding bytes are 0.
    """
    T, lanes, S = raw_tiles.shape
    G = -(-S // 16)
    buf = np.zeros((T, lanes, G * 16), dtype=np.uint8)
    buf[:, :, :S] = np.where(active[:, :, None], raw_tiles, 0)
    return buf.reshape(T, lanes, G, 16).transpose(0, 2, 1, 3).copy()
