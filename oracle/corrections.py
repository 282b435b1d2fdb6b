"""Sparse correction stream of escaped weights (test infrastructure only).

MINE page, Section 4.1, "Escapes": a value outside the table is coded as 0 in the
dense stream, and its real value goes to a correction stream appended to the
tile's ANS stream, one 32-bit record per escape holding the 16-bit weight, an
11-bit column index relative to the start of the tile's column slice, a flag that
marks the row's last escape (and a 4-bit pause counter).  Each lane handles the
records of its own row; reads are coordinated like the renormalisation reads, so
the wave takes as many rounds as the row with the most records.

Readings taken where the page leaves the layout open:

* Record bits: weight in bits 0..15, column in bits 16..26, last-of-row flag in
  bit 27, bits 28..31 zero (the pause counter schedules records inside the decode
  loop; here all records of a tile are applied after its last symbol, so no pause
  is stored).
* The stream starts with a 64-bit mask (four 16-bit words, least significant
  first): bit l set iff lane l has at least one record.
* Records follow in rounds: round r holds the r-th record of every lane that has
  more than r records, lanes ascending; each record is two words, low half first.
* Within a row, records are in ascending column order.
"""
from __future__ import annotations

import numpy as np

LANES = 64
LAST = 1 << 27
COL_BITS = 11


def record(bits: int, col: int, last: bool) -> int:
    if not 0 <= col < (1 << COL_BITS):
        raise ValueError("column does not fit the record")
    return (int(bits) & 0xFFFF) | (col << 16) | (LAST if last else 0)


def tile_records(bits: np.ndarray, escaped: np.ndarray, active: np.ndarray):
    """bf16 bits and escape flags of one tile [64, W] -> per-lane record lists."""
    out = []
    for lane in range(LANES):
        cols = np.nonzero(escaped[lane])[0] if active[lane] else []
        recs = [record(bits[lane, c], int(c), i + 1 == len(cols)) for i, c in enumerate(cols)]
        out.append(recs)
    return out


def stream_words(per_lane) -> np.ndarray:
    """Per-lane record lists -> the tile's correction stream as 16-bit words."""
    mask = 0
    for lane, recs in enumerate(per_lane):
        if recs:
            mask |= 1 << lane
    words = [(mask >> (16 * i)) & 0xFFFF for i in range(4)]
    rounds = max((len(r) for r in per_lane), default=0)
    for r in range(rounds):
        for lane in range(LANES):
            if len(per_lane[lane]) > r:
                rec = per_lane[lane][r]
                words += [rec & 0xFFFF, rec >> 16]
    return np.array(words, dtype=np.uint16)


def parse(words: np.ndarray, width: int, active: np.ndarray):
    """Read one tile's correction stream (the words after its last ANS word).

    Returns (per-lane list of (column, bits), ok) where ok says the stream is well
    formed: it holds the mask, every lane with a mask bit ends on a last flag, no
    record names a column outside the slice or an inactive lane, and the records
    end exactly at the end of the words."""
    w = [int(v) for v in np.asarray(words, dtype=np.int64)]
    if len(w) < 4:
        return [[] for _ in range(LANES)], False
    mask = w[0] | (w[1] << 16) | (w[2] << 32) | (w[3] << 48)
    pos = 4
    open_lanes = [lane for lane in range(LANES) if (mask >> lane) & 1]
    out = [[] for _ in range(LANES)]
    ok = all(active[lane] for lane in open_lanes)
    while open_lanes:
        still = []
        for lane in open_lanes:
            if pos + 2 > len(w):
                return out, False
            rec = w[pos] | (w[pos + 1] << 16)
            pos += 2
            col = (rec >> 16) & ((1 << COL_BITS) - 1)
            if rec >> 28 or col >= width:
                ok = False
            out[lane].append((col, rec & 0xFFFF))
            if not rec & LAST:
                still.append(lane)
        open_lanes = still
    return out, ok and pos == len(w)
