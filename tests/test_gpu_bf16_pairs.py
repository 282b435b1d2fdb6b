"""GPU parity of BF16 exponent pairs with escaped weights, through the C ABI.

Pair symbols over the 16 stored exponents, escaped weights coded as +0.0 and
restored from each tile's correction stream (MINE page, Section 4.1 "Escapes"):
dec_materialize must return the logical tensor bit for bit, dec_gemv must stay
within |y - y_ref| <= 1e-3 * sum|w x| of the oracle's float64 product, at launch
shapes that put several tiles (so several correction streams) into one wave's word
stream, several row groups into one block, and a row group over several blocks.
"""
import numpy as np
import pytest
import torch

import entropy_coded_weight_amd as ecw
from oracle import gemv, pipeline as P
from tests import cases
from tests.test_gpu_parity import _x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(name):
    return [c for c in cases.small_cases() if c.name == name][0]


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 1), (4, 2, 2), (8, 1, 1), (1, 4, 3)])
@pytest.mark.parametrize("name", ["bf16_pairs_mixed_bf16x", "bf16_pairs_mixed_ragged"])
def test_bf16_pairs_launch_shapes(name, shape):
    W, R, P_ = shape
    print(f"[gpu] bf16 pairs {name} W={W} R={R} P={P_}", flush=True)
    case = _case(name)
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    ct = ecw.CompressedTensor(blob, waves_per_block=W, tiles_per_wave=R, row_groups_per_block=P_)
    wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
    for batch in (1, 4):
        xd, xv = _x(case, batch)
        y0 = ct.gemv(xd)
        y1 = ct.gemv(xd)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)
        ok, worst = gemv.check(y0.cpu().numpy(), wv, xv)
        assert ok, f"batch {batch}: worst error / bound = {worst}"


def _every_exponent(e_lo, e_hi):
    vals = [(s << 15) | (e << 7) | m for e in range(e_lo, e_hi) for s in (0, 1) for m in (0, 1, 0x55, 0x7F)]
    vals = np.array(vals, np.uint16)
    n = vals.size // 16
    return np.repeat(vals[: n * 16].reshape(n, 16), 4, axis=1)       # K = 64


def test_bf16_pairs_every_exponent_materialize():
    # 255 exponents, 16 stored: most weights are escaped, up to 64 records per row
    bits = _every_exponent(0, 255)
    c = ecw.Coding(ecw.BF16_EXP, bits.shape[0], 64, 2, 0, 9, 64)
    print(f"[gpu] bf16 pairs every exponent {bits.shape}", flush=True)
    ct = ecw.CompressedTensor(ecw.encode(c, bits))
    sym, w, st = ct.materialize()
    torch.cuda.synchronize()
    assert int(st.abs().sum()) == 0
    assert np.array_equal(w.cpu().numpy().view(np.uint16), bits)
    comp = P.encode(P.Coding(P.BF16_EXP, bits.shape[0], 64, k=2, log2_m=9, tile_cols=64), bits)
    ref_sym, ok = P.decode_symbols(comp)
    assert ok.all()
    assert np.array_equal(sym.cpu().numpy().view(np.uint16).astype(np.int64), ref_sym)


@pytest.mark.parametrize("xdt", ["bf16", "f16"])
def test_bf16_pairs_mostly_escaped_gemv(xdt):
    # exponents 90..159 (products and sums stay normal fp32): most weights escaped
    bits = _every_exponent(90, 160)
    n = bits.shape[0]
    case = cases.Case("every_exp", cases.BF16, n, 64, 2, 0, 9, 64, bits, None, xdt)
    ct = ecw.CompressedTensor(ecw.encode(case.lib_coding(), bits))
    wv = P.weight_values(case.oracle_coding(), bits)
    for batch in (1, 4):
        xd, xv = _x(case, batch)
        y = ct.gemv(xd)
        torch.cuda.synchronize()
        ok, worst = gemv.check(y.cpu().numpy(), wv, xv)
        assert ok, worst


def test_bf16_pairs_ignore_a_second_row_stream():
    # pair tensors decode one row-group stream per wave: asking for two gives the
    # same launch and the same bits
    case = _case("bf16_pairs_mixed_bf16x")
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    one = ecw.CompressedTensor(blob, waves_per_block=2, tiles_per_wave=1, streams_per_wave=1)
    two = ecw.CompressedTensor(blob, waves_per_block=2, tiles_per_wave=1, streams_per_wave=2)
    xd, _ = _x(case, 1)
    assert torch.equal(one.gemv(xd), two.gemv(xd))


@pytest.mark.parametrize("batch", [1, 4])
def test_bf16_pairs_grouped_launch(batch):
    specs = [(96, 11, 128, 1), (64, 12, 256, 1), (130, 10, 128, 2)]
    cts, cs = [], []
    for i, (n, m, tc, R) in enumerate(specs):
        bits = cases.bf16_mixed(n, 512, 40 + i)
        case = cases.Case(f"gp{i}", cases.BF16, n, 512, 2, 0, m, tc, bits, None, "bf16")
        cts.append(ecw.CompressedTensor(ecw.encode(case.lib_coding(), bits), waves_per_block=2, tiles_per_wave=R))
        cs.append(case)
    xd, xv = _x(cs[0], batch)
    ys = ecw.GemvGroup(cts).gemv(xd)
    torch.cuda.synchronize()
    for ct, case, y in zip(cts, cs, ys):
        assert torch.equal(y, ct.gemv(xd))
        wv = P.weight_values(case.oracle_coding(), case.logical)
        ok, worst = gemv.check(y.cpu().numpy(), wv, xv)
        assert ok, worst


def test_bf16_pairs_damaged_correction_stream_is_reported():
    # A cleared last-record flag makes the lane read on past its records; the rounds
    # stop after as many rounds as the slice has columns, every read stays inside the
    # wave's ring and every store inside the lane's row, and the tile reports that it
    # did not end on its word count.  The validator cannot see this (it does not
    # decode), so the decode must end on its own.
    bits = np.full((64, 64), 0x3F80, np.uint16)
    for i, e in enumerate(range(100, 116)):
        bits[i, 3] = e << 7                     # 16 rare exponents: one is escaped
    c = ecw.Coding(ecw.BF16_EXP, 64, 64, 2, 0, 10, 64)
    blob = ecw.encode(c, bits)
    from tests import blobfmt
    bl = blobfmt.parse(blob)
    off_w, _ = bl.sec["words"]
    n_words = int(blobfmt.offsets(bl)[-1])
    bad = blob.copy()
    hi = bad[off_w + 2 * (n_words - 1): off_w + 2 * n_words].view(np.uint16)
    assert hi[0] & 0x0800                       # the last record's flag
    hi[0] &= ~np.uint16(0x0800)
    ct = ecw.CompressedTensor(bad)
    _, w, st = ct.materialize()
    torch.cuda.synchronize()
    assert int(st.cpu().numpy()[0]) != 0
    ok = ecw.CompressedTensor(blob)
    _, w0, st0 = ok.materialize()
    torch.cuda.synchronize()
    assert int(st0.abs().sum()) == 0 and np.array_equal(w0.cpu().numpy().view(np.uint16), bits)
