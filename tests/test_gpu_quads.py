"""GPU parity of INT quads (four 4-bit codes per symbol over a table of stored
4-tuples, escaped codes in each tile's correction stream), through the C ABI.

MINE page, Section 4.1 "Escapes": codes outside the table are coded as 0 and
restored from the correction stream.  dec_materialize must return the logical codes
bit for bit and the oracle's symbols; dec_gemv must stay within
|y - y_ref| <= 1e-3 * sum|w x| of the oracle's float64 product, at launch shapes
that put several tiles (so several correction streams) into one wave's word stream,
several row groups into one block, and a row group over several blocks; a grouped
launch must equal separate launches; a damaged correction stream must be reported.
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
    return [c for c in cases.quad_cases() if c.name == name][0]


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 1), (4, 2, 2), (8, 1, 1), (1, 4, 3), (16, 1, 1)])
@pytest.mark.parametrize("name", ["quads_t64_m10_ragged", "quads_t512_m11_bf16x", "quads_t1_m8"])
def test_quads_launch_shapes(name, shape):
    W, R, P_ = shape
    print(f"[gpu] quads {name} W={W} R={R} P={P_}", flush=True)
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


@pytest.mark.parametrize("shape", [(1, 1, 1), (4, 2, 1), (8, 1, 2), (16, 1, 1), (2, 3, 2)])
@pytest.mark.parametrize("name", ["quads_t64_m10_ragged", "quads_t2048_m12", "quads_t1_m8_f16_two_streams",
                                  "quads_16_slices_m12"])
def test_quads_two_row_streams(name, shape):
    # fp16 activations: a wave decodes two adjacent row groups in lockstep, each with
    # its own word stream and its own correction rounds (every nonzero code escaped
    # in the t = 1 case); the same bits as one stream per wave, within the bound
    W, R, P_ = shape
    print(f"[gpu] quads two streams {name} W={W} R={R} P={P_}", flush=True)
    case = _case(name)
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    one = ecw.CompressedTensor(blob, waves_per_block=W, tiles_per_wave=R, row_groups_per_block=P_)
    two = ecw.CompressedTensor(blob, waves_per_block=W, tiles_per_wave=R, streams_per_wave=2,
                               row_groups_per_block=P_)
    wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
    for batch in (1, 4):
        xd, xv = _x(case, batch)
        y1 = one.gemv(xd)
        y2 = two.gemv(xd)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
        ok, worst = gemv.check(y2.cpu().numpy(), wv, xv)
        assert ok, f"batch {batch}: worst error / bound = {worst}"


def test_quads_symbols_are_the_oracle_symbols():
    for case in cases.quad_cases():
        print(f"[gpu] quads symbols {case.name}", flush=True)
        ct = ecw.CompressedTensor(ecw.encode(case.lib_coding(), case.logical, case.scales))
        sym, w, st = ct.materialize()
        torch.cuda.synchronize()
        assert int(st.abs().sum()) == 0
        assert np.array_equal(w.cpu().numpy(), case.logical)
        ref, ok = P.decode_symbols(P.encode(case.oracle_coding(), case.logical, case.scales))
        assert ok.all()
        assert np.array_equal(sym.cpu().numpy().view(np.uint16).astype(np.int64), ref)


@pytest.mark.parametrize("batch", [1, 4])
def test_quads_grouped_launch(batch):
    specs = [(96, 11, 128, 1, 512), (64, 12, 256, 1, 2048), (130, 10, 128, 2, 64)]
    cts, cs = [], []
    for i, (n, m, tc, R, t) in enumerate(specs):
        c = cases._int(f"gq{i}", n, 512, 4, 4, m, tc, seed=60 + i)
        c.stored_tuples = t
        cts.append(ecw.CompressedTensor(ecw.encode(c.lib_coding(), c.logical, c.scales), waves_per_block=2,
                                        tiles_per_wave=R))
        cs.append(c)
    xd, xv = _x(cs[0], batch)
    ys = ecw.GemvGroup(cts).gemv(xd)
    torch.cuda.synchronize()
    for ct, c, y in zip(cts, cs, ys):
        assert torch.equal(y, ct.gemv(xd))
        wv = P.weight_values(c.oracle_coding(), c.logical, c.scales)
        ok, worst = gemv.check(y.cpu().numpy(), wv, xv)
        assert ok, worst


def test_quads_every_code_escaped_in_one_row():
    # a single stored tuple (zero): every nonzero code of row 5 is a record, 128 per
    # tile, as many rounds as the slice has columns
    q = np.zeros((64, 256), np.int8)
    q[5] = np.tile(np.array([c for c in range(-8, 8) if c], np.int8), 18)[:256]
    q[5, ::16] = -8
    c = ecw.Coding(ecw.INT_CODES, 64, 256, 4, 4, 8, 128, stored_tuples=1)
    sc = np.full(64, 0.5, np.float16)
    ct = ecw.CompressedTensor(ecw.encode(c, q, sc))
    _, w, st = ct.materialize()
    torch.cuda.synchronize()
    assert int(st.abs().sum()) == 0 and np.array_equal(w.cpu().numpy(), q)
    case = cases.Case("all_esc", cases.INT, 64, 256, 4, 4, 8, 128, q, sc, "f16", stored_tuples=1)
    wv = P.weight_values(case.oracle_coding(), q, sc)
    for batch in (1, 4):
        xd, xv = _x(case, batch)
        y = ct.gemv(xd)
        torch.cuda.synchronize()
        ok, worst = gemv.check(y.cpu().numpy(), wv, xv)
        assert ok, worst


def test_quads_damaged_correction_stream_is_reported():
    # a cleared last-record flag: the lane reads on past its records; the rounds stop
    # after as many rounds as the slice has columns, every read stays in the ring and
    # every store in the lane's row, and the tile reports the mismatch
    q = np.zeros((64, 64), np.int8)
    q[3, 12] = 7                                # escaped (one stored tuple)
    c = ecw.Coding(ecw.INT_CODES, 64, 64, 4, 4, 8, 64, stored_tuples=1)
    sc = np.ones(64, np.float16)
    blob = ecw.encode(c, q, sc)
    from tests import blobfmt
    bl = blobfmt.parse(blob)
    off_w, _ = bl.sec["words"]
    n_words = int(blobfmt.offsets(bl)[-1])
    bad = blob.copy()
    hi = bad[off_w + 2 * (n_words - 1): off_w + 2 * n_words].view(np.uint16)
    assert hi[0] & 0x0800
    hi[0] &= ~np.uint16(0x0800)
    _, _, st = ecw.CompressedTensor(bad).materialize()
    torch.cuda.synchronize()
    assert int(st.cpu().numpy()[0]) != 0
    _, w0, st0 = ecw.CompressedTensor(blob).materialize()
    torch.cuda.synchronize()
    assert int(st0.abs().sum()) == 0 and np.array_equal(w0.cpu().numpy(), q)
