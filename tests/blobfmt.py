"""Independent reader of blob format v1 for the tests (written from the format
description: 256-byte header, seven 256-byte-aligned sections).  Test code only."""
from __future__ import annotations

import struct
from dataclasses import dataclass

import numpy as np

SECTIONS = ["tables", "lut", "states", "offsets", "words", "raw", "scales"]
HEADER_U32 = ["magic", "version", "header_bytes", "n_sections", "payload", "rows", "cols",
              "weights_per_symbol", "code_bits", "log2_m", "tile_rows", "tile_cols",
              "recon_dtype", "n_tables", "n_row_groups", "n_slices", "n_tiles", "steps_full",
              "steps_last", "lut_entry_bytes", "stored_tuples", "reserved1"]


@dataclass
class Blob:
    h: dict
    sec: dict          # name -> (offset, bytes)
    raw_bytes: np.ndarray

    def section(self, name) -> np.ndarray:
        off, n = self.sec[name]
        return self.raw_bytes[off:off + n]


def parse(blob: np.ndarray) -> Blob:
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    vals = struct.unpack_from("<22I", b.tobytes()[:88])
    h = dict(zip(HEADER_U32, vals))
    h["total_bytes"] = struct.unpack_from("<Q", b.tobytes()[88:96])[0]
    sec = {}
    for i, name in enumerate(SECTIONS):
        off, n = struct.unpack_from("<QQ", b.tobytes()[96 + 16 * i: 112 + 16 * i])
        sec[name] = (off, n)
    return Blob(h, sec, b)


def tables(bl: Blob):
    t = bl.section("tables")
    n = bl.h["n_tables"]
    rec = t[: 520 * n].reshape(n, 520)
    alphabet = rec[:, 0:4].copy().view(np.uint32).ravel().astype(np.int64)
    value_offset = rec[:, 4:8].copy().view(np.int32).ravel().astype(np.int64)
    freq = rec[:, 8:].copy().view(np.uint16).astype(np.int64)
    return alphabet, value_offset, freq


def pair_values(bl: Blob):
    """BF16 pairs: the 16 stored exponents after the table records (else None)."""
    if bl.h["payload"] != 2 or bl.h["weights_per_symbol"] != 2:
        return None
    t = bl.section("tables")
    n = bl.h["n_tables"]
    return t[520 * n: 520 * n + 16].astype(np.int64)


def quad_tables(bl: Blob):
    """INT quads: (stored tuples, their frequencies), the first n of the stored_tuples
    slots after the table record, n = the record's alphabet (else None)."""
    T = bl.h["stored_tuples"]
    if not T:
        return None
    t = bl.section("tables")
    n = int(t[0:4].copy().view(np.uint32)[0])
    tup = t[520:520 + 2 * T].copy().view(np.uint16).astype(np.int64)
    fq = t[520 + 2 * T:520 + 4 * T].copy().view(np.uint16).astype(np.int64)
    return tup[:n], fq[:n], tup[n:], fq[n:]


def states(bl: Blob) -> np.ndarray:
    return bl.section("states").copy().view(np.uint32).reshape(-1, 64)


def offsets(bl: Blob) -> np.ndarray:
    return bl.section("offsets").copy().view(np.uint32).astype(np.int64)


def words(bl: Blob) -> np.ndarray:
    off = offsets(bl)
    n = int(off[-1]) if off.size else 0
    return bl.section("words")[: 2 * n].copy().view(np.uint16)


def lut(bl: Blob) -> np.ndarray:
    return bl.section("lut").copy().view(np.uint32).reshape(bl.h["n_tables"], -1, 2)


def scales(bl: Blob):
    s = bl.section("scales")
    return s.copy().view(np.float16) if s.size else None
