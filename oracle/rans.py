"""Interleaved rANS over independent 64-lane tiles (test infrastructure only).

Follows the EntroPack page: independent rANS tiles decoded in parallel, one GPU
wave per tile (Section 3.6), 32-bit rANS states, 16-bit payload words and table
precision b = log2 M <= 15 so a symbol needs at most one payload word (Section
C.3).  The ANS state-update rule is Duda's, as summarised in Section 3 of the MINE
page ("tANS": the decoder uses the low m bits of the state as a table index and
rebuilds the next state from the table entry and bits of the stream).

Readings taken where the pages are silent:

* The state interval is [L, 2^32) with L = 2^16 (forced by a 32-bit state that is
  refilled 16 bits at a time).  The decoder renormalises after each symbol.
* A tile holds 64 lanes.  Lane l owns one row; its S symbols are that row's
  symbols in column order inside the tile's column slice.
* Word order inside a tile: step-major, lanes ascending within a step (the order
  in which the decoder reads them).  The encoder runs steps in reverse and lanes
  in descending order, then reverses the list of pushed words.
* Inactive lanes (rows past the end of the matrix) carry state L, are skipped by
  the encoder, and neither decode nor read words.
* Each tile stores the 64 decoder start states and its word offset; a final
  boundary offset closes the last tile (EntroPack page, Section C.3).

Arrays are vectorised over (tile, lane); the step loop is a plain Python loop.
"""
from __future__ import annotations

import numpy as np

L_BITS = 16
L = 1 << L_BITS
WORD_BITS = 16
LANES = 64


def encode_tiles(sym: np.ndarray, tbl: np.ndarray, freq: np.ndarray, log2_m: int,
                 active: np.ndarray):
    """Encode tiles.

    sym, tbl: int [T, 64, S] symbol and table index of lane l at step j.
    freq: int [n_tables, alphabet]; active: bool [T, 64].
    Returns (states uint32 [T, 64], words uint16 [total], counts int64 [T]) with the
    words of all tiles concatenated in tile order.
    """
    sym = np.asarray(sym, dtype=np.int64)
    tbl = np.asarray(tbl, dtype=np.int64)
    T, lanes, S = sym.shape
    assert lanes == LANES
    freq = np.asarray(freq, dtype=np.int64)
    cum = np.concatenate([np.zeros((freq.shape[0], 1), np.int64),
                          np.cumsum(freq, axis=1)[:, :-1]], axis=1)
    M = 1 << log2_m
    x = np.full((T, LANES), L, dtype=np.uint64)
    push_val = np.zeros((T, S, LANES), dtype=np.uint16)
    push_msk = np.zeros((T, S, LANES), dtype=bool)
    act = np.asarray(active, dtype=bool)
    for j in range(S - 1, -1, -1):
        s = sym[:, :, j]
        t = tbl[:, :, j]
        f = np.where(act, freq[t, s], 1)
        c = np.where(act, cum[t, s], 0)
        if np.any(f <= 0):
            raise ValueError("symbol with zero frequency")
        f64 = f.astype(np.uint64)
        x_max = f64 << np.uint64(32 - log2_m)          # (L >> m) << 16, times f
        need = act & (x >= x_max)
        push_val[:, j, :] = np.where(need, x & np.uint64(0xFFFF), 0).astype(np.uint16)
        push_msk[:, j, :] = need
        x = np.where(need, x >> np.uint64(WORD_BITS), x)
        x_new = (x // f64) * np.uint64(M) + (x % f64) + c.astype(np.uint64)
        x = np.where(act, x_new, x)
    # The word pushed by lane l before encoding step j is the word the decoder reads
    # for lane l after decoding step j, so decoder order is (j ascending, l ascending).
    words = push_val[push_msk]          # C order over (tile, step, lane)
    counts = push_msk.reshape(T, -1).sum(axis=1).astype(np.int64)
    assert np.all(x < (1 << 32)) and np.all(x >= L)
    return x.astype(np.uint32), words, counts


def decode_tiles(states: np.ndarray, words: np.ndarray, offsets: np.ndarray, S: int,
                 freq: np.ndarray, log2_m: int, active: np.ndarray, table_of_step=None,
                 trailing: bool = False):
    """Decode tiles; the reference for the GPU decoder.

    states uint32 [T, 64]; words uint16 (all tiles); offsets int [T + 1] word offsets
    of each tile; table_of_step(j, out) -> int [T, 64] table index of step j given the
    symbols decoded so far (default: table 0).
    Returns (symbols int64 [T, 64, S], ok bool [T]) where ok is the end-of-tile
    invariant: every active state back at L and exactly all of the tile's words read.
    trailing: the tile's words may go on after the ANS words (a correction stream);
    then ok leaves out the last condition and the words read per tile are returned
    as a third value.
    """
    states = np.asarray(states, dtype=np.uint64)
    T = states.shape[0]
    freq = np.asarray(freq, dtype=np.int64)
    n_tables, alphabet = freq.shape
    M = 1 << log2_m
    cum = np.concatenate([np.zeros((n_tables, 1), np.int64),
                          np.cumsum(freq, axis=1)[:, :-1]], axis=1)
    slot2sym = np.zeros((n_tables, M), dtype=np.int64)
    for t in range(n_tables):
        if freq[t].sum() == M:
            slot2sym[t] = np.repeat(np.arange(alphabet), freq[t])
    offsets = np.asarray(offsets, dtype=np.int64)
    base = offsets[:-1]
    count = offsets[1:] - offsets[:-1]
    words64 = np.asarray(words, dtype=np.uint64)
    act = np.asarray(active, dtype=bool)
    x = states.copy()
    ptr = np.zeros(T, dtype=np.int64)
    out = np.zeros((T, LANES, S), dtype=np.int64)
    overrun = np.zeros(T, dtype=bool)
    for j in range(S):
        t = np.zeros((T, LANES), np.int64) if table_of_step is None else table_of_step(j, out)
        slot = (x & np.uint64(M - 1)).astype(np.int64)
        s = slot2sym[t, slot]
        f = freq[t, s].astype(np.uint64)
        c = cum[t, s].astype(np.uint64)
        x_new = f * (x >> np.uint64(log2_m)) + slot.astype(np.uint64) - c
        x = np.where(act, x_new, x)
        out[:, :, j] = np.where(act, s, 0)
        need = act & (x < np.uint64(L))
        off = np.cumsum(need, axis=1) - need            # exclusive prefix, lanes ascending
        rel = ptr[:, None] + off
        bad = need & (rel >= count[:, None])
        overrun |= bad.any(axis=1)
        idx = np.where(need & ~bad, base[:, None] + rel, 0)
        w = words64[idx] if words64.size else np.zeros_like(x)
        x = np.where(need, (x << np.uint64(WORD_BITS)) | w, x)
        ptr += need.sum(axis=1)
    ok = (~overrun) & np.all(np.where(act, x == L, True), axis=1)
    if trailing:
        return out, ok, ptr
    return out, ok & (ptr == count)


def offsets_from_counts(counts: np.ndarray) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int64)
