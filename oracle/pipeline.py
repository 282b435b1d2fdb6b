"""Whole-tensor encode / decode / reconstruct (test infrastructure only).

Steps, in the pages' order: map the logical tensor to symbols (``symbols``, ``e8``),
histogram and normalise per table (``coding``; MINE page Section 4.2), cut into
independent 64-row tiles and rANS-encode each (``rans``; EntroPack page Sections
3.6 and C.3).  Decoding reverses these steps and rebuilds the weights (EntroPack
page Section 3.7; DFloat11 page Algorithm 1's bit join; MINE page Section 4.1).

Payload kinds: 1 integer codes, 2 BF16 exponent + raw sign/mantissa byte (one
exponent per symbol, or with k = 2 a pair of exponent digits plus the correction
stream of escaped weights: MINE page Section 4.1 "Escapes"; 4-bit codes with k = 4
likewise over a table of stored 4-tuples), 3 FP8 E4M3 bytes,
4 E8 lattice fields (doubled coordinates as logical tensor).
Reconstruction dtypes for E8: 4 = INT8 (2v), 5 = FP8 E4M3 (nearest to v).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import coding, corrections, e8, rans, symbols

INT_CODES, BF16_EXP, FP8_E4M3, E8_LATTICE = 1, 2, 3, 4
DT_I8, DT_FP8 = 4, 5


@dataclass
class Coding:
    payload: int
    rows: int
    cols: int
    k: int = 1                 # weights per symbol (E8: 8 weights per 9-symbol block)
    code_bits: int = 4         # integer codes only
    log2_m: int = 12
    tile_cols: int = 256
    recon_dtype: int = 0       # E8 only
    stored_tuples: int = 0     # quads of 4-bit codes: t, the tuples the table stores


@dataclass
class Components:
    coding: Coding
    n_tables: int
    alphabet: np.ndarray       # int [n_tables]
    value_offset: np.ndarray   # int [n_tables]
    freq: np.ndarray           # int [n_tables, 256]
    n_rg: int
    n_sl: int
    s_full: int
    s_last: int
    states: np.ndarray         # uint32 [T, 64]
    offsets: np.ndarray        # int64 [T + 1]
    words: np.ndarray          # uint16
    raw: np.ndarray | None     # uint8, BF16 raw plane in tile order
    scales: np.ndarray | None  # float16 [N]
    counts: np.ndarray = field(default=None)   # histogram [n_tables, 256]
    pair_values: np.ndarray | None = None      # BF16 pairs: exponent of each digit
    stored: np.ndarray | None = None           # code quads: the stored tuples, ascending


def syms_per_slice(c: Coding) -> int:
    if c.payload == INT_CODES:
        return c.tile_cols // c.k
    if c.payload == E8_LATTICE:
        return 9 * c.tile_cols // 8
    if c.payload == BF16_EXP:
        return c.tile_cols // c.k
    return c.tile_cols


def _bf16_pairs(c: Coding) -> bool:
    return c.payload == BF16_EXP and c.k == 2


def _quads(c: Coding) -> bool:
    """Quads of 4-bit codes over a table of stored tuples, with escapes."""
    return c.payload == INT_CODES and c.k == 4 and c.code_bits == 4


def _escapes(c: Coding) -> bool:
    return _bf16_pairs(c) or _quads(c)


# ---------------------------------------------------------------- logical -> symbols
def _row_symbols(c: Coding, logical: np.ndarray):
    """-> (symbol-values int64 [N, n_sym], table int64 [N, n_sym], raw uint8 or None)."""
    if c.payload == INT_CODES:
        s = symbols.int_codes_to_symbols(logical, c.code_bits, c.k)
        return s, np.zeros_like(s), None
    if c.payload == BF16_EXP:
        ex, raw = symbols.bf16_split(logical)
        return ex, np.zeros_like(ex), raw
    if c.payload == FP8_E4M3:
        s = np.asarray(logical, dtype=np.uint8).astype(np.int64)
        return s, np.zeros_like(s), None
    if c.payload == E8_LATTICE:
        v2 = np.asarray(logical, dtype=np.int64)
        n, K = v2.shape
        cos, z = e8.doubled_to_point(v2.reshape(-1, 8))
        f = e8.point_to_fields(cos, z)                     # [n*K/8, 9]
        tbl = np.stack([e8.table_of_field(cos, j) for j in range(9)], axis=1)
        return f.reshape(n, K // 8 * 9), tbl.reshape(n, K // 8 * 9), None
    raise ValueError("payload")


def encode(c: Coding, logical: np.ndarray, scales=None) -> Components:
    pair_values = esc = stored = esc_bits = None
    if _bf16_pairs(c):
        ex, _ = symbols.bf16_split(logical)
        pair_values = symbols.bf16_pair_values(coding.histogram(ex, 256))
        vals, raw, esc = symbols.bf16_pair_split(logical, pair_values)
        tbl = np.zeros_like(vals)
        esc_bits = np.asarray(logical, np.uint16)
    elif _quads(c):
        if not 1 <= c.stored_tuples <= (1 << c.log2_m):
            raise ValueError("stored tuples must be in [1, M]")
        tu = symbols.quad_tuples(logical)
        stored = symbols.quad_stored(coding.histogram(tu, 1 << 16), c.stored_tuples)
        vals, esc = symbols.quad_map(tu, stored)
        tbl = np.zeros_like(vals)
        raw = None
        esc_bits = symbols.small_int_bf16_bits(logical)
    else:
        vals, tbl, raw = _row_symbols(c, logical)
    n_tables = e8.N_TABLES if c.payload == E8_LATTICE else 1
    value_offset = np.zeros(n_tables, dtype=np.int64)
    alphabet = np.zeros(n_tables, dtype=np.int64)
    if c.payload == E8_LATTICE:
        for t in range(n_tables):
            sel = vals[tbl == t]
            if sel.size:
                value_offset[t] = sel.min()
                alphabet[t] = sel.max() - sel.min() + 1
        sym = vals - value_offset[tbl]
    elif stored is not None:
        sym = vals
        alphabet[0] = stored.size
    else:
        sym = vals
        alphabet[0] = {INT_CODES: 1 << (c.code_bits * c.k), BF16_EXP: 256, FP8_E4M3: 256}[c.payload]
    width = max(256, int(alphabet.max()))      # only quad tables exceed 256 symbols
    if width > 256 and stored is None:
        raise ValueError("alphabet larger than 256")
    counts = np.zeros((n_tables, width), dtype=np.int64)
    for t in range(n_tables):
        counts[t] = coding.histogram(sym[tbl == t], width)
    freq = np.stack([coding.normalise(counts[t], c.log2_m) for t in range(n_tables)])
    sps = syms_per_slice(c)
    n_rg, n_sl, s_full, s_last = symbols.tile_plan(c.rows, sym.shape[1], sps)
    T = n_rg * n_sl
    states = np.zeros((T, 64), dtype=np.uint32)
    per_tile_words = [None] * T
    raw_tiles = [None] * T
    g_sym = symbols.rows_to_tiles(sym, sps)
    g_tbl = symbols.rows_to_tiles(tbl, sps)
    # raw bytes and escapes are per weight: tiles of tile_cols columns
    g_raw = symbols.rows_to_tiles(raw, c.tile_cols) if raw is not None else [None] * len(g_sym)
    g_esc = [None] * len(g_sym)
    if esc is not None:
        g_esc = list(zip(symbols.rows_to_tiles(esc, c.tile_cols),
                         symbols.rows_to_tiles(esc_bits, c.tile_cols)))
    for (ids, sdat, act), (_, tdat, _), rg, eg in zip(g_sym, g_tbl, g_raw, g_esc):
        st, words, cnt = rans.encode_tiles(sdat, tdat, freq, c.log2_m, act)
        states[ids] = st
        offs = rans.offsets_from_counts(cnt)
        for i, t in enumerate(ids):
            per_tile_words[t] = words[offs[i]:offs[i + 1]]
            if eg is not None:
                recs = corrections.tile_records(eg[1][1][i], eg[0][1][i], act[i])
                per_tile_words[t] = np.concatenate([per_tile_words[t], corrections.stream_words(recs)])
        if rg is not None:
            plane = symbols.raw_plane_bytes(rg[1], act)
            for i, t in enumerate(ids):
                raw_tiles[t] = plane[i].ravel()
    counts_t = np.array([w.size for w in per_tile_words], dtype=np.int64)
    words_all = (np.concatenate(per_tile_words) if T else np.zeros(0, np.uint16)).astype(np.uint16)
    raw_all = np.concatenate(raw_tiles) if raw is not None and T else (
        np.zeros(0, np.uint8) if raw is not None else None)
    sc = None if scales is None else np.asarray(scales, dtype=np.float16)
    return Components(c, n_tables, alphabet, value_offset, freq, n_rg, n_sl, s_full, s_last,
                      states, rans.offsets_from_counts(counts_t), words_all, raw_all, sc, counts,
                      pair_values, stored)


# ---------------------------------------------------------------- symbols -> logical
def decode_symbols(comp: Components):
    """-> (row symbol values int64 [N, n_sym], tile ok flags bool [T])."""
    sym, ok, _ = _decode_all(comp)
    return sym, ok


def _decode_all(comp: Components):
    """-> (row symbols, tile ok flags, {tile: per-lane [(column, bits)]} of the
    correction streams (BF16 pairs; empty otherwise))."""
    c = comp.coding
    sps = syms_per_slice(c)
    pairs = _escapes(c)
    corr = {}
    n_sym = {INT_CODES: c.cols // max(c.k, 1), BF16_EXP: c.cols // c.k, FP8_E4M3: c.cols,
             E8_LATTICE: 9 * c.cols // 8}[c.payload]
    T = comp.n_rg * comp.n_sl
    ok = np.zeros(T, dtype=bool)
    dummy = np.zeros((c.rows, n_sym), dtype=np.int64)
    groups = symbols.rows_to_tiles(dummy, sps)
    active_rows = np.zeros((comp.n_rg * 64,), dtype=bool)
    active_rows[:c.rows] = True
    dec_groups = []
    for ids, sdat, act in groups:
        S = sdat.shape[2]
        # decode each tile against the shared word array using per-tile offsets
        offsets = np.stack([comp.offsets[ids], comp.offsets[ids + 1]], axis=1)
        tos = None
        if c.payload == E8_LATTICE:
            def tos(j, out):
                jj = j % 9
                if jj == 0:
                    return np.zeros(out.shape[:2], np.int64)
                cos = out[:, :, j - jj] + comp.value_offset[0]
                return 1 + 8 * cos + (jj - 1)
        if pairs:
            syms, okg, ptr = _decode_group(comp, comp.states[ids], offsets, S, act, tos, trailing=True)
            for i, t in enumerate(ids):
                b, e = int(comp.offsets[t]), int(comp.offsets[t + 1])
                recs, okc = corrections.parse(comp.words[b + int(ptr[i]):e], c.k * S, act[i])
                okg[i] &= okc
                corr[int(t)] = recs
        else:
            syms, okg = _decode_group(comp, comp.states[ids], offsets, S, act, tos)
        ok[ids] = okg
        dec_groups.append((ids, syms, act))
    sym = symbols.tiles_to_rows(c.rows, n_sym, sps, dec_groups)
    return sym, ok, corr


def _decode_group(comp, states, offsets, S, act, tos, trailing=False):
    # rans.decode_tiles expects offsets as a [T+1] prefix; tiles here may not be
    # contiguous, so decode with explicit (begin, end) pairs gathered into a copy.
    T = states.shape[0]
    lens = offsets[:, 1] - offsets[:, 0]
    words = np.concatenate([comp.words[b:e] for b, e in offsets]) if T else np.zeros(0, np.uint16)
    offs = rans.offsets_from_counts(lens)
    return rans.decode_tiles(states, words, offs, S, comp.freq, comp.coding.log2_m, act, tos,
                             trailing=trailing)


def decode(comp: Components) -> np.ndarray:
    """Bit-exact logical tensor."""
    c = comp.coding
    sym, _, corr = _decode_all(comp)
    if _bf16_pairs(c):
        w = symbols.bf16_pair_join(sym, raw_rows(comp), comp.pair_values)
        for t, per_lane in corr.items():
            g, sl = divmod(t, comp.n_sl)
            for lane, recs in enumerate(per_lane):
                for col, bits in recs:
                    if g * 64 + lane < c.rows:
                        w[g * 64 + lane, sl * c.tile_cols + col] = bits
        return w
    if _quads(c):
        q = symbols.quad_join(sym, comp.stored)
        for t, per_lane in corr.items():
            g, sl = divmod(t, comp.n_sl)
            for lane, recs in enumerate(per_lane):
                for col, bits in recs:
                    if g * 64 + lane < c.rows:
                        q[g * 64 + lane, sl * c.tile_cols + col] = int(np.array([bits << 16], np.uint32)
                                                                       .view(np.float32)[0])
        return q
    if c.payload == INT_CODES:
        return symbols.symbols_to_int_codes(sym, c.code_bits, c.k)
    if c.payload == FP8_E4M3:
        return sym.astype(np.uint8)
    if c.payload == BF16_EXP:
        raw = raw_rows(comp)
        return symbols.bf16_join(sym, raw)
    if c.payload == E8_LATTICE:
        n = c.rows
        f = sym.reshape(n, c.cols // 8, 9)
        cos = f[:, :, 0] + comp.value_offset[0]
        vals = np.empty_like(f)
        vals[:, :, 0] = cos
        for j in range(1, 9):
            t = 1 + 8 * cos + (j - 1)
            vals[:, :, j] = f[:, :, j] + comp.value_offset[t]
        cc, z = e8.fields_to_point(vals.reshape(-1, 9))
        return e8.doubled_coords(cc, z).reshape(n, c.cols).astype(np.int8)
    raise ValueError("payload")


def raw_rows(comp: Components) -> np.ndarray:
    """Inverse of the raw-plane layout -> uint8 [N, K]."""
    c = comp.coding
    out = np.zeros((comp.n_rg * 64, c.cols), dtype=np.uint8)
    pos = 0
    for t in range(comp.n_rg * comp.n_sl):
        g, sl = divmod(t, comp.n_sl)
        S = (comp.s_last if sl == comp.n_sl - 1 else comp.s_full) * c.k     # weights per lane
        G = -(-S // 16)
        blk = comp.raw[pos:pos + G * 1024].reshape(G, 64, 16).transpose(1, 0, 2).reshape(64, G * 16)
        pos += G * 1024
        out[g * 64:(g + 1) * 64, sl * c.tile_cols:sl * c.tile_cols + S] = blk[:, :S]
    return out[:c.rows]


# ---------------------------------------------------------------- reconstruction
def weight_values(c: Coding, logical: np.ndarray, scales=None) -> np.ndarray:
    """Real weight values W_val (float64 [N, K]) of a logical tensor."""
    if c.payload == INT_CODES:
        return logical.astype(np.float64) * np.asarray(scales, np.float64)[:, None]
    if c.payload == BF16_EXP:
        return symbols.bf16_value(logical)
    if c.payload == FP8_E4M3:
        return symbols.e4m3_value(logical) * np.asarray(scales, np.float64)[:, None]
    if c.payload == E8_LATTICE:
        v2 = logical.astype(np.float64)
        if c.recon_dtype == DT_I8:
            return v2 * np.asarray(scales, np.float64)[:, None] / 2.0
        return symbols.e4m3_value(symbols.e4m3_rne(v2 / 2.0)) * np.asarray(scales, np.float64)[:, None]
    raise ValueError("payload")


def dequantized(c: Coding, logical: np.ndarray, scales=None, dtype: str = "f16") -> np.ndarray:
    """The real weight values rounded to nearest even into fp16 or bf16, as uint16
    bits [N, K]: what a dequantising decode hands to a dense GEMM (MINE page, Section
    4.2, the dequant kernel).  Every value of these payloads is exact in fp32 (a
    code or E4M3 significand of at most 4 bits times an 11-bit fp16 scale, or a bf16
    value), so rounding once from float64 and once from float32 agree."""
    import torch
    wv = weight_values(c, logical, scales)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return wv.astype(np.float16).view(np.uint16)
    f32 = wv.astype(np.float32)
    fin = np.isfinite(wv)
    if not np.array_equal(f32.astype(np.float64)[fin], wv[fin]):
        raise ValueError("weight value not exact in fp32")
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def reconstructed_dtype_tensor(c: Coding, logical: np.ndarray) -> np.ndarray:
    """The weights in their reconstruction dtype, bit patterns (what a decoder emits)."""
    if c.payload == E8_LATTICE:
        if c.recon_dtype == DT_I8:
            return logical.astype(np.int8)
        return symbols.e4m3_rne(logical.astype(np.float64) / 2.0)
    return logical
