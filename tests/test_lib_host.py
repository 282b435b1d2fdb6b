"""CPU tests of the C-ABI library: symbols, byte parity with the oracle, validation.

No GPU is touched: only the host entry points run, and the device entry points are
called only with arguments they must reject before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import entropy_coded_weight_amd as ecw
from oracle import pipeline as P, rans
from tests import blobfmt, cases

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "ecw.h")).read()
    declared = set(re.findall(r"^\w[\w\s\*]*?\b(\w+)\s*\(", header, flags=re.M))
    declared -= {"if", "while"}
    assert {"enc_build_tables", "enc_encode", "dec_prepare", "dec_gemv", "dec_materialize",
            "dec_gemv_workspace_size", "ecw_last_error", "ecw_abi_version"} <= declared
    L = ecw.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert L.ecw_abi_version() == 3


def test_tile_metadata_bytes_match_page_formula():
    rows = [list(map(int, l.split())) for l in open(os.path.join(GOLDEN, "tile_metadata_bytes.txt"))
            if l.strip() and not l.startswith("#")]
    for lanes, sb, ob, total in rows:
        assert lanes * sb + ob == total
    c = cases.small_cases()[0]
    t = ecw.prepare(ecw.encode(c.lib_coding(), c.logical, c.scales))
    # 64 states + 1 offset per tile, plus the closing boundary offset
    assert t.bytes_tile_meta == t.n_tiles * 260 + 4


@pytest.mark.parametrize("case", cases.small_cases() + cases.e8_cases(), ids=lambda c: c.name)
def test_byte_parity_with_oracle_and_oracle_decodes_library_blob(case):
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    comp = P.encode(case.oracle_coding(), case.logical, case.scales)
    bl = blobfmt.parse(blob)
    assert bl.h["magic"] == 0x31574345 and bl.h["version"] == 2
    assert bl.h["total_bytes"] == blob.size
    alphabet, voff, freq = blobfmt.tables(bl)
    qt = blobfmt.quad_tables(bl)
    if qt is not None:
        assert np.array_equal(qt[0], comp.stored) and not qt[2].any() and not qt[3].any()
        assert not freq.any()
        n = qt[0].size                          # the oracle's table is at least 256 wide
        assert not comp.freq[:, n:].any()
        freq = np.zeros_like(comp.freq)
        freq[0, :n] = qt[1]
    assert np.array_equal(freq, comp.freq)
    assert np.array_equal(voff, comp.value_offset)
    assert np.array_equal(blobfmt.states(bl), comp.states)
    assert np.array_equal(blobfmt.offsets(bl), comp.offsets)
    assert np.array_equal(blobfmt.words(bl), comp.words)
    if comp.raw is not None:
        assert np.array_equal(bl.section("raw"), comp.raw)
    if case.scales is not None:
        assert np.array_equal(blobfmt.scales(bl).view(np.uint16), case.scales.view(np.uint16))
    # code parity: the oracle's decoder reads the library's sections
    comp2 = P.Components(comp.coding, comp.n_tables, alphabet, voff, freq, comp.n_rg, comp.n_sl,
                         comp.s_full, comp.s_last, blobfmt.states(bl), blobfmt.offsets(bl),
                         blobfmt.words(bl), bl.section("raw") if comp.raw is not None else None,
                         blobfmt.scales(bl), pair_values=blobfmt.pair_values(bl),
                         stored=qt[0] if qt is not None else None)
    if comp.pair_values is not None:
        assert np.array_equal(comp2.pair_values, comp.pair_values)
    _, ok = P.decode_symbols(comp2)
    assert ok.all()
    assert np.array_equal(P.decode(comp2), case.logical)


def test_tables_match_oracle_histogram_and_frequencies():
    for case in cases.small_cases()[:6]:
        t = ecw.build_tables(case.lib_coding(), case.logical)
        comp = P.encode(case.oracle_coding(), case.logical, case.scales)
        assert np.array_equal(t.count_array(), comp.counts)
        assert np.array_equal(t.freq_array(), comp.freq)


def test_decode_table_entries_follow_the_frequencies():
    case = cases.small_cases()[1]
    bl = blobfmt.parse(ecw.encode(case.lib_coding(), case.logical, case.scales))
    _, voff, freq = blobfmt.tables(bl)
    lut = blobfmt.lut(bl)[0]
    cum = np.concatenate([[0], np.cumsum(freq[0])[:-1]])
    sym = np.repeat(np.arange(256), freq[0])
    assert np.array_equal(lut[:, 0] & 0xFFFFFF, freq[0][sym])
    assert np.array_equal(lut[:, 1] & 0xFFFF, np.arange(lut.shape[0]) - cum[sym])
    # Pair mode payload: a8 = the symbol (first code in the low digit); h16 holds the
    # high bytes of the two codes' fp16 values (their low bytes are zero)
    assert np.array_equal(lut[:, 0] >> 24, sym)
    h = (lut[:, 1] >> 16).astype(np.uint32)
    f0 = ((h & 0xFF) << 8).astype(np.uint16).view(np.float16).astype(np.float64)
    f1 = (h & 0xFF00).astype(np.uint16).view(np.float16).astype(np.float64)
    assert np.array_equal(f0, (sym & 15) - 8)
    assert np.array_equal(f1, (sym >> 4) - 8)
    # single-code payload: a8 = the code (int8), h16 = its fp16 value
    case1 = cases.small_cases()[0]
    bl1 = blobfmt.parse(ecw.encode(case1.lib_coding(), case1.logical, case1.scales))
    _, _, freq1 = blobfmt.tables(bl1)
    lut1 = blobfmt.lut(bl1)[0]
    sym1 = np.repeat(np.arange(256), freq1[0])
    q = sym1 - 8
    assert np.array_equal((lut1[:, 0] >> 24).astype(np.uint8).view(np.int8), q)
    assert np.array_equal((lut1[:, 1] >> 16).astype(np.uint16).view(np.float16).astype(np.float64), q)


def test_fp8_entry_payload_is_the_code_value():
    case = [c for c in cases.small_cases() if c.name == "fp8_m12"][0]
    bl = blobfmt.parse(ecw.encode(case.lib_coding(), case.logical, case.scales))
    _, _, freq = blobfmt.tables(bl)
    lut = blobfmt.lut(bl)[0]
    sym = np.repeat(np.arange(256), freq[0])
    h = (lut[:, 1] >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    from oracle import symbols
    assert np.array_equal(h, symbols.e4m3_value(sym))
    assert np.array_equal(lut[:, 0] >> 24, sym)


def test_bf16_entry_payload_is_the_rotated_exponent():
    # a8 = the exponent rotated right by one bit, so that together with the raw byte
    # (sign << 7 | mantissa) the bf16 value is sign | a8[6:0] : a8[7] | mantissa, whole
    # bytes; h16 = 0 and the high word is the bias alone
    case = [c for c in cases.small_cases() if c.name == "bf16_m12"][0]
    bl = blobfmt.parse(ecw.encode(case.lib_coding(), case.logical, case.scales))
    _, _, freq = blobfmt.tables(bl)
    lut = blobfmt.lut(bl)[0]
    cum = np.concatenate([[0], np.cumsum(freq[0])[:-1]])
    sym = np.repeat(np.arange(256), freq[0])
    a8 = lut[:, 0] >> 24
    assert np.array_equal(a8, ((sym >> 1) | (sym << 7)) & 0xFF)
    assert np.array_equal(lut[:, 1], np.arange(lut.shape[0]) - cum[sym])
    # the byte join rebuilds every bf16 bit pattern with this exponent
    for e in np.unique(sym):
        r = np.arange(256)
        rot = ((e >> 1) | (e << 7)) & 0xFF
        joined = (((r & 0x80) | (rot & 0x7F)) << 8) | ((rot & 0x80) | (r & 0x7F))
        assert np.array_equal(joined, ((r & 0x80) << 8) | (e << 7) | (r & 0x7F))


def test_e8_nearest_matches_the_oracle():
    # the library's lattice quantiser (the product path's E8 generator step) against
    # the oracle's Conway-Sloane decoder, itself pinned by brute force: random blocks
    # at several scales, exact half-integers (rounding ties), and blocks equidistant
    # from both cosets
    from oracle import e8
    rng = np.random.default_rng([0, 77])
    blocks = [rng.normal(0, s, (20000, 8)) for s in (0.3, 1.0, 4.0, 11.0)]
    blocks.append(rng.integers(-20, 20, (4000, 8)) + 0.5)
    blocks.append(rng.integers(-20, 20, (4000, 8)).astype(np.float64))
    blocks.append(np.full((1, 8), 0.25))                   # equidistant: coset 0 wins
    blocks.append(np.full((1, 8), -0.25))
    blocks.append(rng.integers(-8, 8, (4000, 8)) + 0.25)
    u = np.concatenate(blocks)
    got = ecw.e8_nearest(u).astype(np.int64)
    c, z = e8.nearest_e8(u)
    assert np.array_equal(got, e8.doubled_coords(c, z))
    with pytest.raises(ecw.EcwError):
        ecw.e8_nearest(np.full((1, 8), 100.0))               # 2v = 200 does not fit int8
    with pytest.raises(ecw.EcwError):
        ecw.e8_nearest(np.full((1, 8), np.nan))


def test_prepare_ledger_and_defaults():
    case = cases.small_cases()[0]
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    t = ecw.prepare(blob)
    assert t.blob_bytes == blob.size
    assert t.n_tiles == 16 * 4 and t.steps_full == 256 and t.steps_last == 256
    assert t.bytes_scales == 2 * 1024 and t.bytes_raw == 0
    assert t.bytes_tables == 520 + (1 << 12) * 8
    assert 1 <= t.waves_per_block <= 16 and t.tiles_per_wave >= 1


# ------------------------------------------------------------------ fault injection
def _blob():
    case = cases.small_cases()[2]
    return ecw.encode(case.lib_coding(), case.logical, case.scales)


def _prep_status(blob):
    t = ecw.Tensor()
    b = np.ascontiguousarray(blob)
    return ecw.lib().dec_prepare(b.ctypes.data_as(ctypes.c_void_p), b.size, None, ctypes.byref(t))


def _mutate(fn):
    b = _blob().copy()
    fn(b)
    return b


def _u32(b, off, v):
    b[off:off + 4] = np.array([v], np.uint32).view(np.uint8)


def _u64(b, off, v):
    b[off:off + 8] = np.array([v], np.uint64).view(np.uint8)


def test_prepare_accepts_valid_blob():
    assert _prep_status(_blob()) == 0


@pytest.mark.parametrize("name,fn,expect", [
    ("truncated", None, 3),
    ("bad_magic", lambda b: _u32(b, 0, 0xDEADBEEF), 3),
    ("bad_version", lambda b: _u32(b, 4, 3), 2),
    ("old_version", lambda b: _u32(b, 4, 1), 2),
    ("bad_section_count", lambda b: _u32(b, 12, 6), 3),
    ("bad_tile_rows", lambda b: _u32(b, 40, 32), 2),
    ("geometry_mismatch", lambda b: _u32(b, 64, 7), 3),
    ("section_misaligned", lambda b: _u64(b, 96 + 16 * 2, 300), 3),
    ("section_out_of_range", lambda b: _u64(b, 96 + 16 * 6, 1 << 40), 3),
    ("section_size_overflow", lambda b: _u64(b, 96 + 16 * 4 + 8, (1 << 64) - 16), 3),
    ("sections_overlap", lambda b: _u64(b, 96 + 16 * 3, 256), 3),
])
def test_prepare_rejects_corrupt_header(name, fn, expect):
    if name == "truncated":
        b = _blob()[:-300]
    else:
        b = _mutate(fn)
    assert _prep_status(b) == expect, name
    assert ecw.lib().ecw_last_error()


def test_prepare_rejects_corrupt_contents():
    base = _blob()
    bl = blobfmt.parse(base)
    off_t, _ = bl.sec["tables"]
    off_l, _ = bl.sec["lut"]
    off_s, _ = bl.sec["states"]
    off_o, _ = bl.sec["offsets"]
    # frequencies no longer sum to M
    b = base.copy()
    f = b[off_t + 8: off_t + 10].view(np.uint16)
    f[0] += 1
    assert _prep_status(b) == 3
    # decode entry inconsistent with the frequencies
    b = base.copy()
    b[off_l + 4: off_l + 8] = np.array([5], np.uint32).view(np.uint8)
    assert _prep_status(b) == 3
    # frequency beyond the alphabet
    b = base.copy()
    _u32(b, off_t, 4)
    assert _prep_status(b) == 3
    # start state below L
    b = base.copy()
    _u32(b, off_s + 4 * 5, 123)
    assert _prep_status(b) == 3
    # inactive lane (row >= rows) with a state other than L: last row group of 200 rows
    t = ecw.prepare(base)
    last_rg_tile = (t.n_row_groups - 1) * t.n_slices
    b = base.copy()
    _u32(b, off_s + (last_rg_tile * 64 + 63) * 4, 0x20000)
    assert _prep_status(b) == 3
    # tile offsets not monotone
    b = base.copy()
    offs = b[off_o: off_o + 4 * 3].view(np.uint32)
    offs[1], offs[2] = offs[2] + 1, offs[1]
    assert _prep_status(b) == 3
    # more words than symbols claimed by one tile
    b = base.copy()
    _u32(b, off_o + 4, 10 ** 7)
    assert _prep_status(b) == 3


def test_prepare_rejects_bad_arguments():
    L = ecw.lib()
    t = ecw.Tensor()
    b = _blob()
    assert L.dec_prepare(None, b.size, None, ctypes.byref(t)) == 1
    # misaligned device pointer is rejected before anything else
    assert L.dec_prepare(b.ctypes.data_as(ctypes.c_void_p), b.size, 8, ctypes.byref(t)) == 1


def test_device_entry_points_reject_bad_arguments_without_launching():
    L = ecw.lib()
    b = _blob()
    t = ecw.prepare(b)        # no device blob
    y = ctypes.c_void_p(256)
    assert L.dec_gemv(None, ctypes.byref(t), 256, 1, y, 1, None, 0) == 1
    t.device_blob = 256
    assert L.dec_gemv(None, ctypes.byref(t), 256, 1, y, 5, None, 0) == 1      # batch
    assert L.dec_gemv(None, ctypes.byref(t), 256, 3, y, 1, None, 0) == 1      # x dtype
    assert L.dec_gemv(None, ctypes.byref(t), 8, 1, y, 1, None, 0) == 1        # x misaligned
    t.waves_per_block = 17
    assert L.dec_gemv(None, ctypes.byref(t), 256, 1, y, 1, None, 0) == 1
    t.waves_per_block, t.tiles_per_wave = 1, 1
    n = ctypes.c_size_t()
    assert L.dec_gemv_workspace_size(ctypes.byref(t), 1, ctypes.byref(n)) == 0 and n.value > 0
    assert L.dec_gemv(None, ctypes.byref(t), 256, 1, y, 1, None, 0) == 1      # workspace needed
    assert L.dec_materialize(None, None, None, None, None) == 1


def test_encoder_rejects_bad_inputs():
    c = ecw.Coding(ecw.INT_CODES, 64, 64, 1, 4, 12, 64)
    with pytest.raises(ecw.EcwError):
        ecw.encode(c, np.full((64, 64), 9, np.int8), np.ones(64, np.float16))   # code out of range
    with pytest.raises(ecw.EcwError):
        ecw.encode(ecw.Coding(ecw.INT_CODES, 64, 64, 2, 4, 7, 64), np.zeros((64, 64), np.int8),
                   np.ones(64, np.float16))                                      # M < alphabet^k
    with pytest.raises(ecw.EcwError):
        ecw.encode(ecw.Coding(ecw.INT_CODES, 64, 64, 1, 4, 12, 96), np.zeros((64, 64), np.int8),
                   np.ones(64, np.float16))                                      # tile_cols % 64
    v2 = np.zeros((8, 8), np.int8)
    v2[0, 0] = 1                                                                 # mixed parity
    with pytest.raises(ecw.EcwError):
        ecw.encode(ecw.Coding(ecw.E8_LATTICE, 8, 8, 8, 0, 11, 64, 4), v2, np.ones(8, np.float16))
    # buffer too small in the second call
    c = ecw.Coding(ecw.INT_CODES, 64, 64, 1, 4, 12, 64)
    q = np.zeros((64, 64), np.int8)
    t = ecw.build_tables(c, q)
    buf = np.zeros(512, np.uint8)
    n = ctypes.c_size_t(512)
    st = ecw.lib().enc_encode(ctypes.byref(c), ctypes.byref(t), q.ctypes.data_as(ctypes.c_void_p),
                              np.ones(64, np.float16).ctypes.data_as(ctypes.c_void_p),
                              buf.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n))
    assert st == 4 and n.value > 512


def test_empty_tensor_encodes_and_validates():
    c = ecw.Coding(ecw.INT_CODES, 0, 64, 1, 4, 10, 64)
    blob = ecw.encode(c, np.zeros((0, 64), np.int8), np.zeros(0, np.float16))
    t = ecw.prepare(blob)
    assert t.n_tiles == 0 and t.bytes_words == 0


def test_encode_is_deterministic_and_threads_agree():
    case = cases.small_cases()[1]
    a = ecw.encode(case.lib_coding(), case.logical, case.scales)
    b = ecw.encode(case.lib_coding(), case.logical, case.scales)
    assert np.array_equal(a, b)


def test_group_rejects_mismatched_tensors_without_launching():
    a = ecw.prepare(_blob())
    case = cases.small_cases()[1]                      # different cols
    b = ecw.prepare(ecw.encode(case.lib_coding(), case.logical, case.scales))
    a.device_blob = 256
    b.device_blob = 256
    L = ecw.lib()
    arr = ecw._tensor_array([a, b])
    ys = (ctypes.c_void_p * 2)(256, 512)
    assert L.dec_gemv_group(None, arr, 2, 256, 1, ys, 1, None, 0) == 1
    assert L.dec_gemv_group(None, arr, 0, 256, 1, ys, 1, None, 0) == 1
    assert L.dec_gemv_group(None, arr, 9, 256, 1, ys, 1, None, 0) == 1
    n = ctypes.c_size_t()
    assert L.dec_gemv_group_workspace_size(arr, 2, 1, ctypes.byref(n)) == 0
    # one kernel serves a launch: codes per symbol and the lattice reconstruction
    # route must match too
    for pair in ((cases.small_cases()[1], _retile(cases.small_cases()[1], k=1)),
                 (cases.e8_case(4), cases.e8_case(5))):
        ts = [ecw.prepare(ecw.encode(c.lib_coding(), c.logical, c.scales)) for c in pair]
        for t in ts:
            t.device_blob = 256
        assert L.dec_gemv_group(None, ecw._tensor_array(ts), 2, 256, 1, ys, 1, None, 0) == 1
        assert "codes per symbol" in L.ecw_last_error().decode()


def _retile(case, k):
    import dataclasses
    return dataclasses.replace(case, k=k)


def test_probe_entry_points_reject_bad_arguments():
    L = ecw.lib()
    assert L.ecw_probe_stream_read(None, None, 16, None, 1) == 1
    assert L.ecw_probe_lds_lookup(None, 14, 8, 10, 1, 1, None) == 1
    assert L.ecw_probe_lds_lookup(None, 11, 6, 10, 1, 1, ctypes.c_void_p(16)) == 1
    p16 = ctypes.c_void_p(16)
    assert L.ecw_probe_tile_stream(None, None, 1 << 20, 1, 8, 4, 1, p16) == 1          # no buffer
    assert L.ecw_probe_tile_stream(None, p16, 1 << 20, 1, 8, 4, 3, p16) == 1           # 3 in flight
    assert L.ecw_probe_tile_stream(None, p16, 1 << 20, 1, 8, 17, 1, p16) == 1          # 17 waves per block
    assert L.ecw_probe_tile_stream(None, p16, 8 * 1024 - 1, 1, 8, 4, 1, p16) == 1      # buffer too short
    assert L.ecw_probe_tile_stream(None, ctypes.c_void_p(8), 1 << 20, 1, 8, 4, 1, p16) == 1   # misaligned


def test_bench_lattice_inputs_match_the_test_recipe():
    # bench.py generates the lattice workload with the library's quantiser (the
    # benchmark may not call the oracle); the tests generate it with the oracle's.
    # Both must give the same tensor, scales and activations.
    import bench
    v2, scales, x, step, bpw = bench.config5_inputs()
    v2o, so, xo = cases.config5()
    assert np.array_equal(v2, v2o)
    assert np.array_equal(scales.view(np.uint16), so.view(np.uint16))
    assert np.array_equal(x, xo)
    assert abs(bpw - 4.0) < 0.01


# ------------------------------------------------------------------ BF16 exponent pairs
def _pair_case(name):
    return [c for c in cases.small_cases() if c.name == name][0]


def test_bf16_pair_tables_match_oracle():
    from oracle import symbols
    for name in ("bf16_pairs_m12", "bf16_pairs_mixed_ragged"):
        case = _pair_case(name)
        t = ecw.build_tables(case.lib_coding(), case.logical)
        comp = P.encode(case.oracle_coding(), case.logical, case.scales)
        assert np.array_equal(np.array(list(t.pair_values)), comp.pair_values)
        _, _, esc = symbols.bf16_pair_split(case.logical, comp.pair_values)
        assert t.escapes == int(esc.sum()) > 0
        assert np.array_equal(t.count_array(), comp.counts)
        assert np.array_equal(t.freq_array(), comp.freq)


def test_bf16_pair_entry_payload_holds_both_rotated_exponents():
    # a8 = the symbol; h16 = rot(e0) | rot(e1) << 8 for the digits' exponents, so one
    # pair of byte permutes with the two raw bytes rebuilds both bf16 values
    case = _pair_case("bf16_pairs_m12")
    bl = blobfmt.parse(ecw.encode(case.lib_coding(), case.logical, case.scales))
    _, _, freq = blobfmt.tables(bl)
    pv = blobfmt.pair_values(bl)
    lut = blobfmt.lut(bl)[0]
    sym = np.repeat(np.arange(256), freq[0])
    assert np.array_equal(lut[:, 0] >> 24, sym)
    rot = lambda e: ((e >> 1) | (e << 7)) & 0xFF
    h = lut[:, 1] >> 16
    assert np.array_equal(h & 0xFF, rot(pv[sym & 15]))
    assert np.array_equal(h >> 8, rot(pv[sym >> 4]))


def test_bf16_pair_coding_limits_and_validation():
    L = ecw.lib()
    case = _pair_case("bf16_pairs_m12")
    # cols must be a multiple of 32; the record's 11-bit column caps the slice width
    for c in (ecw.Coding(ecw.BF16_EXP, 64, 48, 2, 0, 12, 64), ecw.Coding(ecw.BF16_EXP, 64, 4096, 2, 0, 12, 4096),
              ecw.Coding(ecw.BF16_EXP, 64, 64, 4, 0, 12, 64)):
        t = ecw.Tables()
        w = np.zeros((c.rows, c.cols), np.uint16)
        assert L.enc_build_tables(ctypes.byref(c), w.ctypes.data_as(ctypes.c_void_p), ctypes.byref(t)) == 2
    # digit 0 must stay exponent 0 (escaped weights are coded as +0.0)
    t = ecw.build_tables(case.lib_coding(), case.logical)
    t.pair_values[0] = 5
    with pytest.raises(ecw.EcwError):
        ecw.encode(case.lib_coding(), case.logical, None, t)
    base = ecw.encode(case.lib_coding(), case.logical, None)
    assert _prep_status(base) == 0
    bl = blobfmt.parse(base)
    off_t, n_t = bl.sec["tables"]
    assert n_t == 520 + 16
    b = base.copy()
    b[off_t + 520] = 7
    assert _prep_status(b) == 3
    # a tile too short to hold its correction stream's lane mask
    off_o, _ = bl.sec["offsets"]
    b = base.copy()
    offs = b[off_o: off_o + 8].view(np.uint32)
    offs[1] = offs[0] + 3
    assert _prep_status(b) == 3


def test_bf16_pairs_with_fewer_digits_escape_more():
    # tables may store fewer than 16 exponents (unused digits hold 0): every other
    # exponent is escaped, and the oracle still decodes the library's blob exactly
    case = _pair_case("bf16_pairs_m12")
    c = case.lib_coding()
    t = ecw.build_tables(c, case.logical)
    keep = [v for v in t.pair_values][:6]
    for d in range(6, 16):
        t.pair_values[d] = 0
    w = case.logical
    ex = (w.astype(np.int64) >> 7) & 0xFF
    # frequencies for the pair symbols the shortened table produces
    from oracle import coding, symbols
    sym, _, esc = symbols.bf16_pair_split(w, np.array(keep + [0] * 10))
    counts = coding.histogram(sym, 256)
    f = coding.normalise(counts, c.log2_m)
    for s_ in range(256):
        t.freq[0][s_] = int(f[s_])
    blob = ecw.encode(c, w, None, t)
    bl = blobfmt.parse(blob)
    comp = P.Components(case.oracle_coding(), 1, np.array([256]), np.array([0]), f[None, :],
                        bl.h["n_row_groups"], bl.h["n_slices"], bl.h["steps_full"], bl.h["steps_last"],
                        blobfmt.states(bl), blobfmt.offsets(bl), blobfmt.words(bl), bl.section("raw"), None,
                        pair_values=blobfmt.pair_values(bl))
    assert esc.sum() > 1000 and not np.isin(ex, keep).all()
    assert P.decode_symbols(comp)[1].all()
    assert np.array_equal(P.decode(comp), w)


# ------------------------------------------------------------------ INT quads over stored tuples
def test_quad_tables_match_oracle():
    from oracle import symbols
    for case in cases.quad_cases():
        t = ecw.build_tables(case.lib_coding(), case.logical)
        comp = P.encode(case.oracle_coding(), case.logical, case.scales)
        n = t.n_tuples
        assert n == comp.stored.size and t.alphabet[0] == n
        assert np.array_equal(np.array(t.tuples[:n]), comp.stored)
        assert np.array_equal(np.array(t.tuple_count[:n]), comp.counts[0, :n])
        assert np.array_equal(np.array(t.tuple_freq[:n]), comp.freq[0, :n])
        _, esc = symbols.quad_map(symbols.quad_tuples(case.logical), comp.stored)
        assert t.escapes == int(esc.sum())
        assert (t.escapes > 0) == (case.stored_tuples < 1000)


@pytest.mark.parametrize("name", ["quads_t64_m10_ragged", "quads_t2048_m12"])
def test_quad_entry_holds_state_update_and_fp16_codes(name):
    # lo = f | bias << 16; hi = the high bytes of the fp16 values of the symbol's four
    # codes (code i in byte i), all from the oracle's stored tuples and frequencies
    case = [c for c in cases.quad_cases() if c.name == name][0]
    bl = blobfmt.parse(ecw.encode(case.lib_coding(), case.logical, case.scales))
    comp = P.encode(case.oracle_coding(), case.logical, case.scales)
    n = comp.stored.size
    fq = comp.freq[0, :n].astype(np.int64)
    lut = blobfmt.lut(bl)[0].astype(np.int64)
    sym = np.repeat(np.arange(n), fq)
    cum = np.concatenate([[0], np.cumsum(fq)[:-1]])
    assert lut.shape[0] == sym.size
    assert np.array_equal(lut[:, 0] & 0xFFFF, fq[sym])
    assert np.array_equal(lut[:, 0] >> 16, np.arange(lut.shape[0]) - cum[sym])
    tup = comp.stored.astype(np.int64)[sym]
    for i in range(4):
        code = ((tup >> (4 * i)) & 15) - 8
        hb = code.astype(np.float16).view(np.uint16).astype(np.int64)
        assert np.all(hb & 0xFF == 0)
        assert np.array_equal((lut[:, 1] >> (8 * i)) & 0xFF, hb >> 8)


def test_group_geometry_is_the_launch_the_shape_defines():
    # 130 x 512 INT quads, 256-wide tiles, t = 2048, M = 2^12
    case = [c for c in cases.quad_cases() if c.name == "quads_t2048_m12"][0]
    t = ecw.prepare(ecw.encode(case.lib_coding(), case.logical, case.scales))
    t.waves_per_block, t.tiles_per_wave = 2, 1
    grid, block, lds16 = ecw.group_geometry([t], 1, ecw.DT_F16)
    # 3 row groups x 1 slice group (2 slices on 2 waves): 3 blocks, rounded up to 8
    assert (grid, block) == (8 * 2 * 64, 2 * 64)
    # the bf16 product adds the tuple-indexed table (8 bytes per stored tuple); the
    # fp16 product reads the codes from the decode entries (M x 8 bytes in both)
    _, _, lds_bf = ecw.group_geometry([t], 1, ecw.DT_BF16)
    assert lds_bf - lds16 == 8 * 2048 and lds16 > 8 * 4096
    t.waves_per_block = 1
    grid1, block1, _ = ecw.group_geometry([t], 4, ecw.DT_F16)
    assert (grid1, block1) == (8 * 64, 64)          # 3 row groups x 2 slice groups = 6 blocks
    u = ecw.prepare(ecw.encode(case.lib_coding(), case.logical, case.scales))
    u.waves_per_block = 2
    with pytest.raises(ecw.EcwError):
        ecw.group_geometry([t, u], 1, ecw.DT_F16)    # members must share waves per block
    with pytest.raises(ecw.EcwError):
        ecw.group_geometry([u], 5, ecw.DT_F16)


def test_quad_coding_limits_and_validation():
    L = ecw.lib()
    w = np.zeros((64, 128), np.int8)
    bad = [ecw.Coding(ecw.INT_CODES, 64, 128, 4, 4, 10, 64, stored_tuples=0),       # no table
           ecw.Coding(ecw.INT_CODES, 64, 128, 4, 4, 10, 64, stored_tuples=1025),    # more than M
           ecw.Coding(ecw.INT_CODES, 64, 128, 4, 4, 13, 64, stored_tuples=4097),    # more than 4096
           ecw.Coding(ecw.INT_CODES, 64, 128, 2, 4, 10, 64, stored_tuples=16),      # not a quad coding
           ecw.Coding(ecw.INT_CODES, 64, 4096, 4, 4, 12, 4096, stored_tuples=16)]   # 11-bit record column
    for c in bad:
        t = ecw.Tables()
        assert L.enc_build_tables(ctypes.byref(c), w.ctypes.data_as(ctypes.c_void_p), ctypes.byref(t)) != 0
    case = [c for c in cases.quad_cases() if c.name == "quads_t64_m10_ragged"][0]
    t = ecw.build_tables(case.lib_coding(), case.logical)
    t2 = ecw.build_tables(case.lib_coding(), case.logical)
    t2.tuples[1], t2.tuples[2] = t2.tuples[2], t2.tuples[1]          # not ascending
    with pytest.raises(ecw.EcwError):
        ecw.encode(case.lib_coding(), case.logical, case.scales, t2)
    t3 = ecw.build_tables(case.lib_coding(), case.logical)
    i0 = list(t3.tuples[:t3.n_tuples]).index(0x8888)
    t3.tuples[i0] = 0x8887 if i0 == 0 or t3.tuples[i0 - 1] < 0x8887 else 0x8889
    with pytest.raises(ecw.EcwError):
        ecw.encode(case.lib_coding(), case.logical, case.scales, t3)
    base = ecw.encode(case.lib_coding(), case.logical, case.scales, t)
    assert _prep_status(base) == 0
    bl = blobfmt.parse(base)
    off_t, n_t = bl.sec["tables"]
    assert n_t == 520 + 4 * 64
    n = t.n_tuples
    for mutate in (lambda b: b[off_t + 520: off_t + 524].view(np.uint16).__setitem__(slice(None), [5, 5]),
                   lambda b: b[off_t: off_t + 4].view(np.uint32).__setitem__(0, 65),         # n > stored_tuples
                   lambda b: b[off_t + 520 + 128: off_t + 522 + 128].view(np.uint16).__setitem__(0, 1)):
        b = base.copy()
        mutate(b)
        assert _prep_status(b) == 3
    # the header's stored-tuple count: required for quads, forbidden elsewhere
    b = base.copy()
    b[80:84] = np.array([0], np.uint32).view(np.uint8)          # header field after lut_entry_bytes
    assert _prep_status(b) == 3
    pair = cases.small_cases()[1]
    pb = ecw.encode(pair.lib_coding(), pair.logical, pair.scales)
    assert _prep_status(pb) == 0
    pb[80:84] = np.array([16], np.uint32).view(np.uint8)
    assert _prep_status(pb) == 3
    # fewer stored tuples than slots: the slots past them must stay zero
    c8 = ecw.Coding(ecw.INT_CODES, 64, 128, 4, 4, 10, 64, stored_tuples=64)
    w8 = np.zeros((64, 128), np.int8)
    w8[0, :4] = 1
    base = ecw.encode(c8, w8, np.ones(64, np.float16))
    bl = blobfmt.parse(base)
    off_t, _ = bl.sec["tables"]
    assert _prep_status(base) == 0 and int(base[off_t: off_t + 4].view(np.uint32)[0]) == 2
    b = base.copy()
    b[off_t + 520 + 2 * 63] = 1
    assert _prep_status(b) == 3


def test_counter_record_separates_launches_by_lds(tmp_path, monkeypatch):
    # two launches of one kernel template with the same grid and block size (the layer
    # set's gate/up and down can be) are told apart by their LDS size
    import csv
    import json
    import bench
    sig = "k_decode<1, 4, 4, 1, false, false>"
    lm = {"2": {"gate_up": [sig, 458752, 1024, 1000, 43008], "down": [sig, 458752, 1024, 2000, 38912]},
          "k": {"gate_up": ["k_decode<1, 4, 2, 1, false, false>", 917504, 256, 3000, 20480]}}
    assert bench.dispatch_launches(lm, f"void ecw::{sig}(unsigned int)", 458752, 1024, 43008) == [("2", "gate_up")]
    assert bench.dispatch_launches(lm, f"void ecw::{sig}(unsigned int)", 458752, 1024, 39424) == [("2", "down")]
    assert bench.dispatch_launches(lm, f"void ecw::{sig}(unsigned int)", 917504, 1024, 43008) == []
    d = tmp_path / "sq0"
    d.mkdir()
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "LDS_Block_Size", "VGPR_Count",
              "Counter_Name", "Counter_Value"]
    with open(d / "sq0_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for did, lds, valu in [(1, 43008, 100), (2, 38912, 40), (3, 43008, 120), (4, 38912, 60)]:
            for name, v in [("SQ_INSTS_VALU", valu), ("SQ_WAVES", 7168)]:
                w.writerow({"Dispatch_Id": did, "Kernel_Name": f"void ecw::{sig}(unsigned int)",
                            "Grid_Size": 458752, "Workgroup_Size": 1024, "LDS_Block_Size": lds, "VGPR_Count": 64,
                            "Counter_Name": name, "Counter_Value": v})
    lmp = tmp_path / "launch_map.json"
    lmp.write_text(json.dumps(lm))
    out = tmp_path / "record.txt"
    bench.write_counter_record(str(tmp_path), str(lmp), str(out), ["(test)"])
    rec = {k.strip(): v.strip() for k, v in (l.split("=", 1) for l in out.read_text().splitlines()
                                            if "=" in l and not l.startswith("#"))}
    assert float(rec["2.gate_up.SQ_INSTS_VALU"]) == 110.0 and float(rec["2.down.SQ_INSTS_VALU"]) == 50.0
    assert rec["2.gate_up.dispatches"] == "2" and "k.gate_up.SQ_INSTS_VALU" not in rec
    # the launch map entry of a real tensor carries the library's geometry
    case = [c for c in cases.quad_cases() if c.name == "quads_t2048_m12"][0]
    t = ecw.prepare(ecw.encode(case.lib_coding(), case.logical, case.scales))
    monkeypatch.setattr(bench, "LAUNCH_MAP", {})
    bench.note_launch("q", "w", [t], 1, False)
    assert bench.LAUNCH_MAP["q"]["w"] == [bench.kernel_sig(t.coding, 1, False),
                                          *ecw.group_geometry([t], 1, ecw.DT_F16)[:2],
                                          130 * 512 // 4, ecw.group_geometry([t], 1, ecw.DT_F16)[2]]


def test_counter_record_attributes_dispatches_by_order(tmp_path):
    # the profiler shows no LDS size (0) and the same kernel and grid for gate/up and
    # down; the run's dispatch log (one launch per fused dispatch in issue order)
    # tells them apart
    import csv
    import json
    import bench
    sig = "k_decode<1, 4, 4, 1, false, false>"
    d = tmp_path / "sq0"
    d.mkdir()
    lm = {"2": {"gate_up": [sig, 458752, 1024, 1000, 43008], "down": [sig, 458752, 1024, 2000, 38912]}}
    (d / "launch_map.json").write_text(json.dumps(lm))
    # issue order: gate_up, down, gate_up, gate_up (one per-launch graph), then a
    # kernel that is not a fused GEMV (a dequantising decode) in between
    (d / "launch_map.json.dispatches.json").write_text(json.dumps(
        {"owners": [[["2", "gate_up"]], [["2", "down"]]], "log": [0, 1, 0, 0]}))
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "LDS_Block_Size", "VGPR_Count",
              "Counter_Name", "Counter_Value"]
    with open(d / "sq0_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for did, name, valu in [(7, sig, 100), (9, sig, 40), (10, "k_decode<1, 4, 4, 1, true, true>", 5),
                                (12, sig, 120), (13, sig, 110)]:
            for cname, v in [("SQ_INSTS_VALU", valu), ("SQ_WAVES", 7168)]:
                w.writerow({"Dispatch_Id": did, "Kernel_Name": f"void ecw::{name}(unsigned int)",
                            "Grid_Size": 458752, "Workgroup_Size": 1024, "LDS_Block_Size": 0, "VGPR_Count": 64,
                            "Counter_Name": cname, "Counter_Value": v})
    out = tmp_path / "record.txt"
    bench.write_counter_record(str(tmp_path), str(d / "launch_map.json"), str(out), ["(test)"])
    text = out.read_text()
    rec = {k.strip(): v.strip() for k, v in (l.split("=", 1) for l in text.splitlines()
                                            if "=" in l and not l.startswith("#"))}
    assert float(rec["2.gate_up.SQ_INSTS_VALU"]) == 110.0 and rec["2.gate_up.dispatches"] == "3"
    assert float(rec["2.down.SQ_INSTS_VALU"]) == 40.0
    assert "attributed to launches by dispatch order" in text


def test_dispatch_log_records_each_launch(monkeypatch, tmp_path):
    # eager calls are logged in issue order under the launch key note_launch registered
    import json
    import torch
    import bench
    case = [c for c in cases.quad_cases() if c.name == "quads_t2048_m12"][0]
    t = ecw.prepare(ecw.encode(case.lib_coding(), case.logical, case.scales))
    calls = []
    monkeypatch.setattr(ecw, "gemv_group_raw", lambda ts, x, ys, ws, stream=None: calls.append(len(ts)))
    monkeypatch.setattr(ecw, "gemv_raw", lambda t, x, y, ws, stream=None: calls.append(1))
    monkeypatch.setattr(torch.cuda, "CUDAGraph", torch.cuda.CUDAGraph)
    monkeypatch.setattr(bench, "LAUNCH_KEYS", {})
    monkeypatch.setattr(bench, "LAUNCH_MAP", {})
    monkeypatch.setattr(bench, "DISPATCH_LOG", None)
    bench.note_launch("2", "w", [t], 1, False)
    bench.install_dispatch_log()
    x1 = torch.zeros((1, 512), dtype=torch.float16)
    x4 = torch.zeros((4, 512), dtype=torch.float16)
    ecw.gemv_group_raw([t], x1, [None], None)
    ecw.gemv_raw(t, x4, None, None)              # batch 4: another kernel, not registered
    ecw.gemv_raw(t, x1, None, None)
    assert calls == [1, 1, 1]
    bench.write_dispatch_log(str(tmp_path / "log.json"))
    lg = json.loads((tmp_path / "log.json").read_text())
    assert lg["log"] == [0, 1, 0] and lg["owners"] == [[["2", "w"]], []]


def test_quad_case_has_records_on_the_ring_mirror():
    # The fused product's correction rounds read a record's two halves from one ring
    # address; a record that starts on the ring's last word (of 512) takes its high
    # half from the mirror of the ring head.  With one tile per wave a wave's ring
    # position of word w is (w - the tile's chunk-aligned start) mod 512.  The model is
    # checked first: each tile's correction stream (a 4-word lane mask, then two words
    # per record) ends at the next tile's offset and its mask is the oracle's rows with
    # escapes.  Then the case the quad GEMV tests run at one tile per wave
    # (fp16 activations) must hold such records, so those tests cover the mirror read.
    from oracle import symbols as S
    case = [c for c in cases.quad_cases() if c.name == "quads_t64_m10_ragged"][0]
    assert case.x_dtype == "f16"
    bl = blobfmt.parse(ecw.encode(case.lib_coding(), case.logical, case.scales))
    offs, words = blobfmt.offsets(bl), blobfmt.words(bl)
    stored = blobfmt.quad_tables(bl)[0]
    _, esc = S.quad_map(S.quad_tuples(case.logical), np.asarray(stored))
    n, k = case.logical.shape
    tc, nsl, nrg = bl.h["tile_cols"], bl.h["n_slices"], bl.h["n_row_groups"]
    on_last_word = 0
    for rg in range(nrg):
        for sl in range(nsl):
            t = rg * nsl + sl
            e = esc[rg * 64:min(n, rg * 64 + 64), sl * tc:min(k, sl * tc + tc)]
            recs = int(e.sum())
            cs = int(offs[t + 1]) - (4 + 2 * recs)
            mask = sum(int(words[cs + i]) << (16 * i) for i in range(4))
            want = sum(1 << lane for lane in range(e.shape[0]) if e[lane].any())
            assert mask == want, (t, hex(mask), hex(want))
            gb = int(offs[t]) & ~255
            on_last_word += sum(1 for r in range(recs) if (cs + 4 + 2 * r - gb) % 512 == 511)
    assert on_last_word > 0
