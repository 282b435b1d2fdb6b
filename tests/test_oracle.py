"""Pins of the CPU oracle against facts outside itself (no GPU needed).

Each test names what fixes the expected value: a closed form, a brute-force
enumeration, a library routine (torch dtype casts, math.fsum), or a value printed
on the pages (tests/golden).
"""
import itertools
import math
import os

import numpy as np
import pytest

import ecw_inputs as E
from oracle import coding, e8, gemv, pipeline as P, rans, symbols

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([int(v) for v in line.split()])
    return rows


# ------------------------------------------------------------------ normaliser
def _compositions(total, parts):
    """All f in Z^parts with f >= 1 and sum f = total (stars and bars)."""
    cuts = np.array(list(itertools.combinations(range(1, total), parts - 1)), dtype=np.int64)
    edges = np.concatenate([np.zeros((len(cuts), 1), np.int64), cuts,
                            np.full((len(cuts), 1), total, np.int64)], axis=1)
    return np.diff(edges, axis=1)


@pytest.mark.parametrize("log2_m", [4, 5])
@pytest.mark.parametrize("seed", range(4))
def test_normaliser_is_optimal_by_enumeration(log2_m, seed):
    rng = np.random.default_rng([7, seed, log2_m])
    counts = rng.integers(1, 1000, 8) ** rng.integers(1, 3, 8)
    if seed == 3:
        counts[[2, 5]] = 0       # absent symbols keep f = 0
    f = coding.normalise(counts, log2_m)
    present = counts > 0
    assert f.sum() == 1 << log2_m
    assert np.all((f > 0) == present)
    comps = _compositions(1 << log2_m, int(present.sum()))
    c = counts[present].astype(np.float64)
    costs = (c[None, :] * (log2_m - np.log2(comps))).sum(axis=1)
    got = coding.cross_entropy_total_bits(counts, f, log2_m)
    assert got == pytest.approx(costs.min(), rel=1e-12, abs=1e-9)


def test_normaliser_corner_cases():
    assert list(coding.normalise(np.array([0, 5, 0]), 8)) == [0, 256, 0]
    assert list(coding.normalise(np.zeros(4, np.int64), 8)) == [0, 0, 0, 0]
    with pytest.raises(ValueError):
        coding.normalise(np.ones(300, np.int64), 8)
    # equal counts split evenly; ties go to the smallest index
    assert list(coding.normalise(np.array([3, 3, 3]), 4)) == [6, 5, 5]


def test_pair_alphabet_limits_match_page():
    for M, t_max in _golden("pair_alphabet_limits.txt"):
        m = M.bit_length() - 1
        assert coding.tuple_mode_legal(t_max, 2, m)
        assert not coding.tuple_mode_legal(t_max + 1, 2, m)


def test_entropy_closed_forms():
    assert coding.entropy_bits(np.array([1, 1, 1, 1])) == pytest.approx(2.0)
    assert coding.entropy_bits(np.array([5])) == 0.0
    p = np.array([0.5, 0.25, 0.125, 0.125])
    assert coding.entropy_bits(p * 8) == pytest.approx(1.75)


# ------------------------------------------------------------------ rANS codec
def _toy_tables(log2_m):
    M = 1 << log2_m
    uniform = np.full(8, M // 8)
    skew = np.array([M // 2, M // 4, M // 8, M // 16, M // 32, M // 64, M // 128, M // 128])
    spike = np.array([M - 7, 1, 1, 1, 1, 1, 1, 1])
    return {"uniform": uniform, "skew": skew, "spike": spike}


def _roundtrip(seqs, freq, log2_m, lanes_active):
    """seqs int [n, S]; pack lanes_active sequences per tile."""
    n, S = seqs.shape
    per = lanes_active
    T = -(-n // per)
    sym = np.zeros((T, 64, S), np.int64)
    act = np.zeros((T, 64), bool)
    for i in range(n):
        t, l = divmod(i, per)
        sym[t, l] = seqs[i]
        act[t, l] = True
    tbl = np.zeros_like(sym)
    fr = np.zeros((1, 256), np.int64)
    fr[0, :8] = freq
    st, words, cnt = rans.encode_tiles(sym, tbl, fr, log2_m, act)
    dec, ok = rans.decode_tiles(st, words, rans.offsets_from_counts(cnt), S, fr, log2_m, act)
    return sym, act, dec, ok, cnt


@pytest.mark.parametrize("log2_m", [8, 12])
@pytest.mark.parametrize("table", ["uniform", "skew", "spike"])
def test_rans_exhaustive_interleaved_roundtrip(log2_m, table):
    freq = _toy_tables(log2_m)[table]
    for S in range(1, 7):
        seqs = np.array(list(itertools.product(range(8), repeat=S)), dtype=np.int64)
        sym, act, dec, ok, _ = _roundtrip(seqs, freq, log2_m, 64)
        assert ok.all()
        assert np.array_equal(np.where(act[:, :, None], sym, 0), dec)


@pytest.mark.parametrize("table", ["uniform", "skew", "spike"])
def test_rans_exhaustive_single_lane_roundtrip_and_size_bound(table):
    log2_m = 12
    M = 1 << log2_m
    freq = _toy_tables(log2_m)[table]
    for S in range(1, 6):
        seqs = np.array(list(itertools.product(range(8), repeat=S)), dtype=np.int64)
        sym, act, dec, ok, cnt = _roundtrip(seqs, freq, log2_m, 1)
        assert ok.all()
        assert np.array_equal(dec[:, 0, :], seqs)
        # bound from the encode map: 16 * words <= sum log2(M/f) + n log2(1 + M/L)
        info = (log2_m - np.log2(freq[seqs])).sum(axis=1)
        assert np.all(16 * cnt <= info + S * math.log2(1 + M / rans.L) + 1e-9)


def test_rans_single_symbol_alphabet_reads_nothing():
    freq = np.zeros(8, np.int64)
    freq[3] = 1 << 10
    seqs = np.full((64, 50), 3)
    sym, act, dec, ok, cnt = _roundtrip(seqs, freq, 10, 64)
    assert ok.all() and cnt.sum() == 0 and np.all(dec == 3)


def test_rans_corrupt_stream_breaks_invariant():
    rng = np.random.default_rng(5)
    freq = _toy_tables(12)["skew"]
    seqs = rng.choice(8, size=(64, 40), p=freq / freq.sum())
    fr = np.zeros((1, 256), np.int64)
    fr[0, :8] = freq
    sym = seqs[None]
    st, words, cnt = rans.encode_tiles(sym, np.zeros_like(sym), fr, 12, np.ones((1, 64), bool))
    bad = st.copy()
    bad[0, 17] ^= 1 << 20
    dec, ok = rans.decode_tiles(bad, words, rans.offsets_from_counts(cnt), 40, fr, 12,
                                np.ones((1, 64), bool))
    assert not ok[0]


# ------------------------------------------------------------------ generators / size gate
def test_generator_entropies_match_closed_forms():
    t = E.config1()
    h = coding.entropy_bits(coding.histogram(t.codes.astype(np.int64) + 8, 16))
    assert h == pytest.approx(3.0615, abs=0.01)
    q = E.config2_tensor("k").codes
    h2 = coding.entropy_bits(coding.histogram(q.astype(np.int64) + 8, 16))
    assert h2 == pytest.approx(2.2, abs=0.01)


def test_size_gate_config1_words_within_one_percent_of_entropy():
    t = E.config1()
    c = P.Coding(P.INT_CODES, 1024, 1024, k=1, code_bits=4, log2_m=12, tile_cols=256)
    comp = P.encode(c, t.codes, t.scales)
    n = t.codes.size
    h = coding.entropy_bits(comp.counts[0])
    assert 16 * comp.words.size <= 1.01 * n * h
    assert np.array_equal(P.decode(comp), t.codes)


def test_size_gate_bf16_and_fp8_slabs():
    b = E.bf16_weights((256, 4096), np.random.default_rng([0, 3, 9]))
    c = P.Coding(P.BF16_EXP, 256, 4096, k=1, log2_m=12, tile_cols=512)
    comp = P.encode(c, b.bits)
    h = coding.entropy_bits(comp.counts[0])
    assert 2.4 < h < 2.7
    assert 16 * comp.words.size <= 1.01 * b.bits.size * h
    assert np.array_equal(P.decode(comp), b.bits)
    f = E.fp8_weights((256, 4096), np.random.default_rng([0, 4, 9]))
    c = P.Coding(P.FP8_E4M3, 256, 4096, k=1, log2_m=12, tile_cols=512)
    comp = P.encode(c, f.codes, f.scales)
    h = coding.entropy_bits(comp.counts[0])
    assert 16 * comp.words.size <= 1.01 * f.codes.size * h
    assert np.array_equal(P.decode(comp), f.codes)


def test_pair_mode_cross_entropy_gate():
    q = E.config2_tensor("k").codes[:256]
    c = P.Coding(P.INT_CODES, 256, 4096, k=2, code_bits=4, log2_m=11, tile_cols=256)
    comp = P.encode(c, q, np.ones(256, np.float16))
    xent = coding.cross_entropy_total_bits(comp.counts[0], comp.freq[0], 11)
    assert 16 * comp.words.size <= 1.01 * xent
    assert np.array_equal(P.decode(comp), q)


@pytest.mark.parametrize("shape,tile_cols,k", [((1, 64), 64, 1), ((65, 200), 64, 2),
                                               ((130, 96), 64, 1), ((64, 64), 64, 2)])
def test_ragged_shapes_roundtrip(shape, tile_cols, k):
    t = E.small_int_codes(shape[0], shape[1], 3)
    c = P.Coding(P.INT_CODES, shape[0], shape[1], k=k, code_bits=4, log2_m=10, tile_cols=tile_cols)
    comp = P.encode(c, t.codes, t.scales)
    _, ok = P.decode_symbols(comp)
    assert ok.all()
    assert np.array_equal(P.decode(comp), t.codes)


def test_quad_mode_two_bit_codes_roundtrip():
    rng = np.random.default_rng(11)
    q = rng.integers(-2, 2, (70, 256)).astype(np.int8)
    c = P.Coding(P.INT_CODES, 70, 256, k=4, code_bits=2, log2_m=10, tile_cols=128)
    comp = P.encode(c, q, np.ones(70, np.float16))
    assert np.array_equal(P.decode(comp), q)


def test_int_symbol_packing_low_digit_first():
    q = np.array([[-8, 7, 0, -1]], dtype=np.int8)
    s = symbols.int_codes_to_symbols(q, 4, 2)
    assert list(s[0]) == [0 | (15 << 4), 8 | (7 << 4)]
    assert np.array_equal(symbols.symbols_to_int_codes(s, 4, 2), q)


# ------------------------------------------------------------------ BF16 / E4M3 formats
def test_bf16_split_join_exhaustive_against_torch():
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ex, raw = symbols.bf16_split(bits)
    assert np.array_equal(symbols.bf16_join(ex, raw), bits)
    f32 = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float()
    u = f32.view(torch.int32).numpy().view(np.uint32)
    assert np.array_equal(ex, (u >> 23) & 0xFF)
    assert np.array_equal(raw >> 7, u >> 31)
    assert np.array_equal(raw & 0x7F, (u >> 16) & 0x7F)
    val = symbols.bf16_value(bits)
    ref = f32.double().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(val[fin], ref[fin])
    assert np.array_equal(np.isnan(val), np.isnan(ref))


def test_bf16_exponent_values_match_page():
    for e, lg in _golden("bf16_exponent_values.txt"):
        v = symbols.bf16_value(np.array([e << 7], np.uint16))[0]
        assert v == 2.0 ** lg


def test_e4m3_table_exhaustive_against_torch():
    import torch
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).float().double().numpy()
    val = symbols.e4m3_value(np.arange(256))
    fin = np.isfinite(ref)
    assert np.array_equal(val[fin], ref[fin])
    assert np.array_equal(np.isnan(val), np.isnan(ref))
    assert np.nanmax(val) == 448.0


def test_e4m3_rne_matches_torch_cast():
    import torch
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 0.05, 20000),
                        symbols.e4m3_value(np.arange(127)),
                        (symbols.e4m3_value(np.arange(126)) + symbols.e4m3_value(np.arange(1, 127))) / 2])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = symbols.e4m3_rne(v.astype(np.float32).astype(np.float64))
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ E8
def _brute_e8_min_dist(u):
    best = np.inf
    for c in (0, 1):
        base = np.floor(u - c / 2.0)
        for d in itertools.product(range(-1, 3), repeat=8):
            z = base + np.array(d)
            if int(z.sum()) % 2:
                continue
            dist = ((u - (z + c / 2.0)) ** 2).sum()
            best = min(best, dist)
    return best


def test_e8_nearest_point_matches_brute_force():
    rng = np.random.default_rng(21)
    u = rng.normal(0, 1.7, (12, 8))
    c, z = e8.nearest_e8(u)
    for i in range(u.shape[0]):
        assert int(z[i].sum()) % 2 == 0
        got = ((u[i] - (z[i] + c[i] / 2.0)) ** 2).sum()
        assert got == pytest.approx(_brute_e8_min_dist(u[i]), abs=1e-12)


def test_e8_fields_roundtrip_and_parity_saving():
    rng = np.random.default_rng(22)
    c, z = e8.nearest_e8(rng.normal(0, 2.5, (200000, 8)))
    f = e8.point_to_fields(c, z)
    c2, z2 = e8.fields_to_point(f)
    assert np.array_equal(c, c2) and np.array_equal(z, z2)
    v2 = e8.doubled_coords(c, z)
    c3, z3 = e8.doubled_to_point(v2)
    assert np.array_equal(c3, c) and np.array_equal(z3, z)
    # parity reduction (EntroPack A.3): coding m instead of z8 saves about one bit
    # per 8-weight block, 0.10-0.13 bits per weight on the page
    h = lambda a: coding.entropy_bits(np.unique(a, return_counts=True)[1])
    saving_bpp = (h(z[:, 7]) - h(f[:, 8])) / 8
    assert 0.10 <= saving_bpp <= 0.13


def test_e8_pipeline_roundtrip_with_17_tables():
    rng = np.random.default_rng(23)
    c, z = e8.nearest_e8(rng.normal(0, 3.0, (96 * 24, 8)))
    v2 = e8.doubled_coords(c, z).reshape(96, 192).astype(np.int8)
    cd = P.Coding(P.E8_LATTICE, 96, 192, k=8, log2_m=11, tile_cols=64, recon_dtype=P.DT_I8)
    comp = P.encode(cd, v2, np.ones(96, np.float16))
    assert comp.n_tables == 17
    assert np.array_equal(P.decode(comp), v2)


# ------------------------------------------------------------------ GEMV
def test_gemv_f64_matches_fsum_on_rectangular_shapes():
    rng = np.random.default_rng(31)
    w = rng.normal(0, 1, (7, 13))
    x = rng.normal(0, 1, (3, 13))
    y = gemv.gemv_f64(w, x)
    assert y.shape == (3, 7)
    for b in range(3):
        for r in range(7):
            assert y[b, r] == pytest.approx(math.fsum(w[r] * x[b]), rel=1e-13, abs=1e-13)
    ok, worst = gemv.check(y, w, x)
    assert ok and worst < 1e-9
    bad = y.copy()
    bad[1, 2] += 0.01 * gemv.abs_bound(w, x)[1, 2]
    assert not gemv.check(bad, w, x)[0]


def test_weight_values_definitions():
    c = P.Coding(P.INT_CODES, 2, 2, k=1)
    w = P.weight_values(c, np.array([[-8, 7], [1, 0]], np.int8), np.array([0.5, 2.0], np.float16))
    assert np.array_equal(w, [[-4.0, 3.5], [2.0, 0.0]])
    c = P.Coding(P.FP8_E4M3, 1, 2, k=1)
    w = P.weight_values(c, np.array([[0x38, 0xB8]], np.uint8), np.array([2.0], np.float16))
    assert np.array_equal(w, [[2.0, -2.0]])        # 0x38 = 1.0 in E4M3
    assert gemv.x_values(np.array([0x3F80], np.uint16), "bf16")[0] == 1.0


def test_e8_reconstruction_routes_by_hand():
    # EntroPack page, Sections 3.2 and A.3: the decoder hands out the lattice point
    # as INT8 or as FP8.  The logical tensor holds doubled coordinates 2v.  Values
    # below are worked by hand, not by the oracle's own formula.
    # INT8 route: the stored integer is 2v itself and the row scale applies to v,
    # so the weight is 2v * scale / 2.
    c = P.Coding(P.E8_LATTICE, 2, 8, k=8, recon_dtype=P.DT_I8)
    v2 = np.array([[3, -5, 1, 1, 1, 1, 1, 1],          # coset 1 (all odd)
                   [0, 2, -2, 4, 0, 0, 0, 0]], np.int8)    # coset 0 (all even)
    sc = np.array([0.5, 2.0], np.float16)
    w = P.weight_values(c, v2, sc)
    assert np.array_equal(w[0], [0.75, -1.25, 0.25, 0.25, 0.25, 0.25, 0.25, 0.25])
    assert np.array_equal(w[1], [0.0, 2.0, -2.0, 4.0, 0.0, 0.0, 0.0, 0.0])
    assert np.array_equal(P.reconstructed_dtype_tensor(c, v2), v2)
    # FP8 route: e4m3 of v, round to nearest with ties to the even significand.
    # In [8, 16) E4M3 steps by 1, in [16, 32) by 2, in [2, 4) by 0.25.
    #   v = 8.5  -> 8   (0x50: exponent 10, significand 000)  tie, even wins
    #   v = 9.5  -> 10  (0x52)                                 tie: 9 = 1.001b odd, 10 = 1.010b even
    #   v = 17   -> 16  (0x58)                                 tie between 16 and 18
    #   v = -8.5 -> -8  (0xD0);  v = -11.5 -> -12 (0xD4): 11 = 1.011b odd, 12 = 1.100b even
    #   v = 23.5 -> 24  (0x5C)                                 not a tie
    #   v = 0.5  -> 0.5 (0x30);  v = -2.5 -> -2.5 (0xC2)      exact
    c = P.Coding(P.E8_LATTICE, 1, 16, k=8, recon_dtype=P.DT_FP8)
    v2 = np.array([[17, 19, 34, -17, -23, 47, 1, -5, 0, 0, 0, 0, 0, 0, 0, 0]], np.int8)
    want_bytes = [0x50, 0x52, 0x58, 0xD0, 0xD4, 0x5C, 0x30, 0xC2] + [0] * 8
    assert list(P.reconstructed_dtype_tensor(c, v2)[0]) == want_bytes
    w = P.weight_values(c, v2, np.array([2.0], np.float16))
    assert np.array_equal(w[0], [16.0, 20.0, 32.0, -16.0, -24.0, 48.0, 1.0, -5.0] + [0.0] * 8)


# ------------------------------------------------------------------ BF16 exponent pairs
def test_bf16_pair_values_keep_zero_and_the_fifteen_most_frequent():
    # MINE page, Section 4.2 "Tuning t": the t most frequent codes, and always 0.
    counts = np.zeros(256, np.int64)
    counts[100:120] = np.arange(1, 21)          # exponent 100 + i occurs i + 1 times
    v = symbols.bf16_pair_values(counts)
    assert list(v) == [0] + list(range(105, 120))
    counts[104] = counts[105]                   # a tie for the last place: smaller exponent
    assert list(symbols.bf16_pair_values(counts)) == [0, 104] + list(range(106, 120))
    counts[:] = 0
    counts[0], counts[127], counts[126] = 500, 3, 1  # exponent 0 never takes a slot of its own
    assert list(symbols.bf16_pair_values(counts)) == [0, 126, 127] + [0] * 13


def test_bf16_pair_stream_worked_example():
    # One 64 x 64 tile of 1.0 (exponent 127) with 14 more exponents (110..123) twice
    # each in row 20 and three rare exponents (90, 91, 92) once each: those three are
    # the escapes.  Expected words written out by hand from the record layout:
    # weight bits | column << 16 | last << 27, a lane mask first, rounds of lanes.
    bits = np.full((64, 64), 0x3F80, np.uint16)
    for i, e in enumerate(range(110, 124)):
        bits[20, 2 * i] = bits[20, 2 * i + 1] = e << 7
    bits[3, 5] = 0x8000 | (90 << 7) | 0x15      # 0xAD15
    bits[3, 40] = (91 << 7) | 0x7F              # 0x2DFF
    bits[9, 0] = (92 << 7) | 0x01               # 0x2E01
    c = P.Coding(P.BF16_EXP, 64, 64, k=2, log2_m=10, tile_cols=64)
    comp = P.encode(c, bits)
    assert list(comp.pair_values) == [0] + list(range(110, 124)) + [127]
    tail = [0x0208, 0, 0, 0,                    # lanes 3 and 9 hold records
            0xAD15, 0x0005,                     # round 0, lane 3: column 5
            0x2E01, 0x0800,                     # round 0, lane 9: column 0, last
            0x2DFF, 0x0828]                     # round 1, lane 3: column 40, last
    assert [int(w) for w in comp.words[-10:]] == tail
    sym, ok = P.decode_symbols(comp)
    assert ok.all()
    assert sym[3, 2] == 15 | (0 << 4)           # 1.0 is digit 15; the escape is digit 0
    raw = P.raw_rows(comp)
    assert raw[3, 5] == 0 and raw[3, 40] == 0 and raw[9, 0] == 0
    assert np.array_equal(P.decode(comp), bits)


def _bf16_mixed(rows, cols, seed):
    """Gaussian bf16 weights plus zeros, negative zeros, subnormals, huge values and
    infinities, so that many exponents are escaped."""
    rng = np.random.default_rng([0, 310, seed])
    b = E.bf16_weights((rows, cols), rng).bits.copy()
    n = b.size
    flat = b.reshape(-1)
    idx = rng.choice(n, n // 50, replace=False)
    special = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0x7F80, 0xFF80, 0x4000, 0x3F80], np.uint16)
    flat[idx] = rng.choice(special, idx.size)
    idx = rng.choice(n, n // 100, replace=False)
    flat[idx] = rng.integers(0, 1 << 16, idx.size).astype(np.uint16)
    return b


@pytest.mark.parametrize("rows,cols,tc,m", [(70, 288, 128, 12), (64, 64, 64, 8), (130, 512, 256, 10)])
def test_bf16_pairs_roundtrip_with_escapes(rows, cols, tc, m):
    b = _bf16_mixed(rows, cols, rows + cols)
    c = P.Coding(P.BF16_EXP, rows, cols, k=2, log2_m=m, tile_cols=tc)
    comp = P.encode(c, b)
    _, ok = P.decode_symbols(comp)
    assert ok.all()
    assert np.array_equal(P.decode(comp), b)


def test_bf16_pairs_escape_count_and_stream_length():
    # every weight whose exponent is neither 0 nor stored is one record (two words);
    # each tile adds its 4-word mask
    b = _bf16_mixed(96, 256, 7)
    c = P.Coding(P.BF16_EXP, 96, 256, k=2, log2_m=12, tile_cols=128)
    comp = P.encode(c, b)
    ex = ((b.astype(np.int64) >> 7) & 0xFF)
    kept = set(int(v) for v in comp.pair_values) | {0}
    n_esc = int(sum(np.count_nonzero(ex == e) for e in range(256) if e not in kept))
    assert n_esc > 0
    _, _, corr = P._decode_all(comp)
    assert sum(len(r) for lanes in corr.values() for r in lanes) == n_esc
    T = comp.n_rg * comp.n_sl
    offs = comp.offsets
    # the ANS part of each tile is what a rANS decode of that tile reads
    ans = sum(int(offs[t + 1] - offs[t]) for t in range(T)) - 4 * T - 2 * n_esc
    assert ans >= 0
    assert 16 * ans <= 1.01 * coding.cross_entropy_total_bits(comp.counts[0], comp.freq[0], 12) + 16 * 64 * T


def test_bf16_pairs_size_matches_single_exponent_coding():
    # Gaussian weights: 29 or so exponents, the 15 most frequent cover all but ~1e-4
    # of the weights, so pairs code the exponent in about the single-symbol size
    b = E.bf16_weights((256, 2048), np.random.default_rng([0, 3, 10])).bits
    one = P.encode(P.Coding(P.BF16_EXP, 256, 2048, k=1, log2_m=12, tile_cols=512), b)
    two = P.encode(P.Coding(P.BF16_EXP, 256, 2048, k=2, log2_m=12, tile_cols=512), b)
    assert np.array_equal(P.decode(two), b)
    assert two.words.size < 1.01 * one.words.size
    h1 = coding.entropy_bits(one.counts[0])
    assert 16 * two.words.size <= 1.02 * b.size * h1


def test_bf16_pairs_corrupt_correction_stream_is_detected():
    bits = np.full((64, 64), 0x3F80, np.uint16)
    for i, e in enumerate(range(100, 116)):
        bits[i, 3] = e << 7                     # 16 rare exponents: one is escaped
    c = P.Coding(P.BF16_EXP, 64, 64, k=2, log2_m=10, tile_cols=64)
    comp = P.encode(c, bits)
    assert P.decode_symbols(comp)[1].all()
    bad = P.Components(**{**comp.__dict__, "words": comp.words.copy()})
    bad.words[-1] ^= 0x0800                     # clear the last flag
    assert not P.decode_symbols(bad)[1].any()
    bad = P.Components(**{**comp.__dict__, "words": comp.words.copy()})
    bad.words[-1] = (bad.words[-1] & 0xF800) | 64   # column outside the slice
    assert not P.decode_symbols(bad)[1].any()


def test_dequantized_rounds_to_nearest_even():
    # hand-rounded values.  fp16, scale 1 + 2^-10: 3 * scale = 3 + 1.5 * 2^-9 lies
    # half-way between 3 + 2^-9 (odd significand) and 3 + 2^-8 (even): 3 + 2^-8 =
    # 0x4202.  -7 * scale = -(7 + 1.75 * 2^-8) rounds to -(7 + 2^-7) = 0xC702.
    c = P.Coding(P.INT_CODES, 1, 2, k=1, code_bits=4)
    sc = np.array([1.0 + 2.0 ** -10], np.float16)
    assert list(P.dequantized(c, np.array([[3, -7]], np.int8), sc, "f16").ravel()) == [0x4202, 0xC702]
    # bf16, scale 1 + 2^-8: 1 * scale ties between 1 and 1 + 2^-7 -> 1.0 = 0x3F80;
    # 3 * scale = 3 + 0.75 * 2^-6 -> 3 + 2^-6 = 0x4041
    sc = np.array([1.0 + 2.0 ** -8], np.float16)
    assert list(P.dequantized(c, np.array([[1, 3]], np.int8), sc, "bf16").ravel()) == [0x3F80, 0x4041]
    # bf16 weights pass through unchanged
    b = P.dequantized(P.Coding(P.BF16_EXP, 1, 2), np.array([[0x3F81, 0xC2F7]], np.uint16), None, "bf16")
    assert list(b.ravel()) == [0x3F81, 0xC2F7]


# ------------------------------------------------------------------ quads of 4-bit codes
def test_quad_stored_keeps_the_most_frequent_and_zero():
    # MINE page, Section 4.1 "Escapes": the table keeps the most frequent symbols and
    # always the value escapes are coded as (here the tuple of four zero codes)
    counts = np.zeros(1 << 16, np.int64)
    counts[0x8888], counts[0x8889], counts[0x88A8], counts[0x1234], counts[0x0001] = 50, 9, 7, 7, 3
    assert list(symbols.quad_stored(counts, 3)) == [0x1234, 0x8888, 0x8889]     # tie: the smaller tuple
    assert list(symbols.quad_stored(counts, 9)) == [0x0001, 0x1234, 0x8888, 0x8889, 0x88A8]
    counts[0x8888] = 0                          # zero takes the last place when missing
    assert list(symbols.quad_stored(counts, 2)) == [0x8888, 0x8889]
    assert list(symbols.quad_stored(counts, 1)) == [0x8888]


def test_quad_map_is_the_fewest_escapes_by_enumeration():
    # against every stored tuple: the chosen one agrees with the tuple wherever it is
    # not a zero code, no stored tuple needs fewer escapes, and ties go to the first
    # set of zeroed positions in the order (count, mask)
    rng = np.random.default_rng([0, 4, 4])
    stored = np.unique(np.concatenate([[0x8888], rng.integers(0, 1 << 16, 40),
                                       0x8888 ^ (rng.integers(0, 16, 40) << (4 * rng.integers(0, 4, 40)))]))
    tup = np.concatenate([stored[:10], rng.integers(0, 1 << 16, 300),
                          0x8888 ^ (rng.integers(0, 16, 100) << (4 * rng.integers(0, 4, 100)))])
    ids, esc = symbols.quad_map(tup[None, :], stored)
    dig = lambda v: [(int(v) >> (4 * i)) & 15 for i in range(4)]
    for j, v in enumerate(tup):
        d = dig(v)
        best = None
        for s in stored:
            e = dig(s)
            if all(e[i] == d[i] or e[i] == 8 for i in range(4)):
                pos = [i for i in range(4) if e[i] != d[i]]
                key = (len(pos), sum(1 << i for i in pos))
                if best is None or key < best[0]:
                    best = (key, int(s), pos)
        assert stored[ids[0, j]] == best[1]
        assert [i for i in range(4) if esc[0, 4 * j + i]] == best[2]


def test_quad_stream_worked_example():
    # One 64 x 64 tile of zero codes with three stored tuples (zero, (1,0,0,0) ten
    # times, (0,2,0,0) five times) and three tuples outside the table.  Records
    # written out by hand: bf16 of the code | column << 16 | last << 27.
    q = np.zeros((64, 64), np.int8)
    q[0:10, 0] = 1                              # tuple 0x8889
    q[0:5, 5] = 2                               # tuple 0x88A8
    q[7, 8:10] = (1, 2)                         # 0x88A9: zeroing the 1 gives 0x88A8
    q[3, 63] = -3                               # 0x5888: only zero is reachable
    q[3, 12] = 7                                # 0x888F
    c = P.Coding(P.INT_CODES, 64, 64, k=4, code_bits=4, log2_m=8, tile_cols=64, stored_tuples=3)
    comp = P.encode(c, q)
    assert list(comp.stored) == [0x8888, 0x8889, 0x88A8]
    tail = [0x0088, 0, 0, 0,                    # lanes 3 and 7 hold records
            0x40E0, 0x000C,                     # round 0, lane 3: 7.0 at column 12
            0x3F80, 0x0808,                     # round 0, lane 7: 1.0 at column 8, last
            0xC040, 0x083F]                     # round 1, lane 3: -3.0 at column 63, last
    assert [int(w) for w in comp.words[-10:]] == tail
    sym, ok = P.decode_symbols(comp)
    assert ok.all()
    assert sym[7, 2] == 2 and sym[3, 15] == 0 and sym[3, 3] == 0 and sym[0, 0] == 1 and sym[0, 1] == 2
    assert np.array_equal(P.decode(comp), q)


@pytest.mark.parametrize("rows,cols,tc,m,t", [(130, 512, 256, 12, 2048), (70, 256, 128, 10, 64),
                                              (64, 64, 64, 8, 1), (65, 192, 64, 13, 4096)])
def test_quads_roundtrip_with_escapes(rows, cols, tc, m, t):
    q = E.laplace_codes((rows, cols), np.random.default_rng([0, 44, rows])).codes
    c = P.Coding(P.INT_CODES, rows, cols, k=4, code_bits=4, log2_m=m, tile_cols=tc, stored_tuples=t)
    comp = P.encode(c, q)
    assert comp.stored.size <= t and 0x8888 in comp.stored
    _, ok = P.decode_symbols(comp)
    assert ok.all()
    assert np.array_equal(P.decode(comp), q)


def test_quads_escape_count_and_size():
    # every code set to 0 by the mapping is one record (two words), each tile adds its
    # 4-word mask; the ANS part stays within the cross-entropy bound
    q = E.laplace_codes((128, 1024), np.random.default_rng([0, 45])).codes
    c = P.Coding(P.INT_CODES, 128, 1024, k=4, code_bits=4, log2_m=12, tile_cols=256, stored_tuples=1024)
    comp = P.encode(c, q)
    coded = symbols.quad_join(P.decode_symbols(comp)[0], comp.stored)
    n_esc = int(np.count_nonzero(coded != q))
    assert n_esc > 0 and np.all(coded[coded != q] == 0)
    _, _, corr = P._decode_all(comp)
    assert sum(len(r) for lanes in corr.values() for r in lanes) == n_esc
    T = comp.n_rg * comp.n_sl
    ans = int(comp.offsets[-1]) - 4 * T - 2 * n_esc
    ce = coding.cross_entropy_total_bits(comp.counts[0], comp.freq[0], 12)
    assert 16 * ans <= 1.01 * ce + 16 * 64 * T
    assert ce <= 16 * ans + 32 * 64 * T


def test_quads_need_one_to_m_stored_tuples():
    q = np.zeros((64, 64), np.int8)
    for t in (0, 257):
        with pytest.raises(ValueError):
            P.encode(P.Coding(P.INT_CODES, 64, 64, k=4, code_bits=4, log2_m=8, tile_cols=64, stored_tuples=t), q)
