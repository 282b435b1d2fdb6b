"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

* decode parity (bit-exact): dec_materialize's symbols and weights equal the
  oracle's decode / the encoded logical tensor; every tile ends on its invariant.
* operator parity: dec_gemv within |y - y_ref| <= 1e-3 * sum|w x| per output, with
  y_ref the float64 product of the oracle's weight values.
"""
import numpy as np
import pytest
import torch

import entropy_coded_weight_amd as ecw
import ecw_inputs as E
from oracle import gemv, pipeline as P
from tests import cases

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _x(case, batch, seed=0):
    rng = np.random.default_rng([0, 900, seed, batch])
    xv = rng.standard_normal((batch, case.cols))
    if case.x_dtype == "f16":
        host = xv.astype(np.float16)
        dev = torch.from_numpy(host).cuda()
        return dev, gemv.x_values(host, "f16")
    import torch as T
    bits = T.from_numpy(xv.astype(np.float32)).to(T.bfloat16)
    host = bits.view(T.int16).numpy().view(np.uint16)
    return bits.cuda(), gemv.x_values(host, "bf16")


def _logical_view(case, w):
    a = w.cpu().numpy()
    if case.payload == cases.BF16:
        return a.view(np.uint16)
    return a


@pytest.mark.parametrize("case", cases.small_cases(), ids=lambda c: c.name)
def test_materialize_bit_exact(case):
    print(f"[gpu] materialize {case.name}", flush=True)
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    ct = ecw.CompressedTensor(blob)
    sym, w, st = ct.materialize()
    torch.cuda.synchronize()
    assert int(st.abs().sum()) == 0
    assert np.array_equal(_logical_view(case, w), case.logical)
    comp = P.encode(case.oracle_coding(), case.logical, case.scales)
    ref_sym, ok = P.decode_symbols(comp)
    assert ok.all()
    assert np.array_equal(sym.cpu().numpy().view(np.uint16).astype(np.int64), ref_sym)


@pytest.mark.parametrize("batch", [1, 2, 3, 4])
@pytest.mark.parametrize("case", cases.small_cases(), ids=lambda c: c.name)
def test_gemv_within_bound(case, batch):
    print(f"[gpu] gemv {case.name} batch={batch}", flush=True)
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    ct = ecw.CompressedTensor(blob)
    xd, xv = _x(case, batch)
    y = ct.gemv(xd)
    torch.cuda.synchronize()
    wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
    ok, worst = gemv.check(y.cpu().numpy(), wv, xv)
    assert ok, f"worst error / bound = {worst}"


@pytest.mark.parametrize("shape", [(1, 1), (2, 3), (3, 1), (8, 1), (16, 1), (4, 2), (1, 16)])
def test_launch_shapes_agree_and_reduction_is_deterministic(shape):
    W, R = shape
    print(f"[gpu] launch shape W={W} R={R}", flush=True)
    case = cases._int("shapes", 200, 2048, 2, 4, 11, 128, seed=9)
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    ct = ecw.CompressedTensor(blob, waves_per_block=W, tiles_per_wave=R)
    xd, xv = _x(case, 1)
    wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
    ys = []
    for _ in range(3):                       # counters must return to zero each call
        ys.append(ct.gemv(xd).cpu().numpy())
    for y in ys:
        ok, worst = gemv.check(y, wv, xv)
        assert ok, worst
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def test_fp8_every_code_value():
    # row r repeats E4M3 code r: y[r] = K * e4m3(r) * scale, so any mis-decoded
    # code (subnormals included) breaks its own row's bound
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n, K = codes.size, 64
    q = np.repeat(codes[:, None], K, axis=1)
    sc = np.full(n, 1.0, np.float16)
    c = ecw.Coding(ecw.FP8_E4M3, n, K, 1, 0, 9, 64)
    ct = ecw.CompressedTensor(ecw.encode(c, q, sc))
    xd = torch.ones((1, K), dtype=torch.bfloat16, device="cuda")
    y = ct.gemv(xd).cpu().numpy()[0]
    wv = P.weight_values(P.Coding(P.FP8_E4M3, n, K), q, sc)
    assert np.array_equal(y.astype(np.float64), wv.sum(axis=1))


def test_bf16_every_exponent_and_sign():
    # every finite bf16 exponent with both signs and a few mantissas
    vals = []
    for e in range(0, 255):
        for s in (0, 1):
            for m in (0, 1, 0x55, 0x7F):
                vals.append((s << 15) | (e << 7) | m)
    vals = np.array(vals, np.uint16)
    n = vals.size // 16
    bits = vals[: n * 16].reshape(n, 16)
    bits = np.repeat(bits, 4, axis=1)              # K = 64
    c = ecw.Coding(ecw.BF16_EXP, n, 64, 1, 0, 9, 64)
    ct = ecw.CompressedTensor(ecw.encode(c, bits))
    sym, w, st = ct.materialize()
    assert np.array_equal(w.cpu().numpy().view(np.uint16), bits)


def test_degenerate_shapes():
    # K == 0: y must be zero; N == 0: nothing happens
    c = ecw.Coding(ecw.INT_CODES, 70, 0, 1, 4, 10, 64)
    ct = ecw.CompressedTensor(ecw.encode(c, np.zeros((70, 0), np.int8), np.ones(70, np.float16)))
    y = torch.full((1, 70), 7.0, device="cuda")
    ecw.gemv_raw(ct.t, torch.zeros((1, 16), dtype=torch.float16, device="cuda")[:, :0].contiguous(), y, None)
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0
    c = ecw.Coding(ecw.INT_CODES, 0, 64, 1, 4, 10, 64)
    ct = ecw.CompressedTensor(ecw.encode(c, np.zeros((0, 64), np.int8), np.zeros(0, np.float16)))
    y = torch.empty((1, 0), device="cuda")
    ecw.gemv_raw(ct.t, torch.zeros((1, 64), dtype=torch.float16, device="cuda"), y, None)
    torch.cuda.synchronize()


@pytest.mark.parametrize("k", [2, 4])
@pytest.mark.parametrize("shape", [(16, 1), (4, 1)])
def test_graph_capture_replays_match_eager(shape, k):
    # the fused GEMV (when a row group spans blocks, with its in-kernel reduction
    # and arrival tickets; INT quads with their correction passes) is captured in a
    # HIP graph and replayed several times with eager work between
    W, R = shape
    case = cases._int("graph", 192, 4096, k, 4, 12, 128, seed=12)
    case.stored_tuples = 512 if k == 4 else 0
    ct = ecw.CompressedTensor(ecw.encode(case.lib_coding(), case.logical, case.scales),
                              waves_per_block=W, tiles_per_wave=R)
    xd, xv = _x(case, 1)
    y_eager = ct.gemv(xd).clone()
    y = torch.empty_like(y_eager)
    ws = ct.workspace(1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ecw.gemv_raw(ct.t, xd, y, ws)
    for i in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i} differs"
        ct.gemv(xd * 2.0)                  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("batch", [1, 4])
def test_grouped_launch_matches_separate_launches(batch):
    # q/k/v-like group: different rows, table sizes and tile widths, shared x
    specs = [(256, 11, 128, 1), (64, 12, 256, 1), (130, 10, 128, 2)]
    cts, cs = [], []
    for i, (n, m, tc, R) in enumerate(specs):
        case = cases._int(f"g{i}", n, 1024, 2, 4, m, tc, seed=20 + i)
        ct = ecw.CompressedTensor(ecw.encode(case.lib_coding(), case.logical, case.scales),
                                  waves_per_block=4, tiles_per_wave=R)
        cts.append(ct)
        cs.append(case)
    xd, xv = _x(cs[0], batch)
    ys = ecw.GemvGroup(cts).gemv(xd)
    torch.cuda.synchronize()
    for ct, case, y in zip(cts, cs, ys):
        y_sep = ct.gemv(xd)
        torch.cuda.synchronize()
        assert torch.equal(y, y_sep)
        wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
        ok, worst = gemv.check(y.cpu().numpy(), wv, xv)
        assert ok, worst


@pytest.mark.parametrize("W", [1, 4])
@pytest.mark.parametrize("batch", [1, 4])
def test_largest_group_matches_separate_launches(batch, W):
    # eight members, the most one launch takes: every member's first block reaches the
    # kernel as a preloaded argument of its own; with one-wave blocks every member's
    # row groups are split over blocks and finish through its own part of the
    # workspace
    print(f"[gpu] eight-member group batch={batch} W={W}", flush=True)
    specs = [(64, 11, 128), (130, 12, 256), (200, 10, 128), (70, 11, 256),
             (256, 12, 128), (96, 10, 256), (150, 11, 128), (65, 12, 128)]
    cts, cs = [], []
    for i, (n, m, tc) in enumerate(specs):
        case = cases._int(f"g8_{i}", n, 1024, 2, 4, m, tc, seed=70 + i)
        cts.append(ecw.CompressedTensor(ecw.encode(case.lib_coding(), case.logical, case.scales),
                                        waves_per_block=W, tiles_per_wave=1))
        cs.append(case)
    xd, xv = _x(cs[0], batch)
    ys = ecw.GemvGroup(cts).gemv(xd)
    torch.cuda.synchronize()
    for ct, case, y in zip(cts, cs, ys):
        assert torch.equal(y, ct.gemv(xd))
        ok, worst = gemv.check(y.cpu().numpy(), P.weight_values(case.oracle_coding(), case.logical, case.scales), xv)
        assert ok, worst


@pytest.mark.parametrize("case", cases.e8_cases(), ids=lambda c: c.name)
def test_e8_materialize_bit_exact(case):
    # symbols, reconstructed weights (INT8 2v or E4M3 bytes) and tile ends vs the oracle
    print(f"[gpu] e8 materialize {case.name}", flush=True)
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    ct = ecw.CompressedTensor(blob)
    sym, w, st = ct.materialize()
    torch.cuda.synchronize()
    assert int(st.abs().sum()) == 0
    want = P.reconstructed_dtype_tensor(case.oracle_coding(), case.logical)
    assert np.array_equal(w.cpu().numpy().view(want.dtype), want)
    comp = P.encode(case.oracle_coding(), case.logical, case.scales)
    ref_sym, ok = P.decode_symbols(comp)
    assert ok.all()
    assert np.array_equal(sym.cpu().numpy().view(np.uint16).astype(np.int64), ref_sym)


@pytest.mark.parametrize("batch", [1, 4])
@pytest.mark.parametrize("case", cases.e8_cases(), ids=lambda c: c.name)
def test_e8_gemv_within_bound(case, batch):
    print(f"[gpu] e8 gemv {case.name} batch={batch}", flush=True)
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    ct = ecw.CompressedTensor(blob)
    xd, xv = _x(case, batch)
    y = ct.gemv(xd)
    torch.cuda.synchronize()
    wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
    ok, worst = gemv.check(y.cpu().numpy(), wv, xv)
    assert ok, f"worst error / bound = {worst}"


@pytest.mark.parametrize("shape", [(4, 1, 1), (2, 2, 1), (8, 1, 2), (1, 3, 3), (16, 2, 1)])
@pytest.mark.parametrize("name", [c.name for c in cases.small_cases()])
def test_two_row_streams_per_wave_match_one(name, shape):
    # a wave decoding the tiles of two adjacent row groups in lockstep sums every row
    # in the same order as a one-stream wave: the same bits, within the bound
    W, R, P_ = shape
    print(f"[gpu] two row streams {name} W={W} R={R} P={P_}", flush=True)
    case = [c for c in cases.small_cases() if c.name == name][0]
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    one = ecw.CompressedTensor(blob, waves_per_block=W, tiles_per_wave=R, row_groups_per_block=P_)
    two = ecw.CompressedTensor(blob, waves_per_block=W, tiles_per_wave=R, streams_per_wave=2,
                               row_groups_per_block=P_)
    wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
    for batch in (1, 4):
        xd, xv = _x(case, batch)
        try:
            y1 = one.gemv(xd)
            y2 = two.gemv(xd)
        except ecw.EcwError as e:
            # a shape whose activation slice and rings exceed the CU's LDS is
            # rejected before any launch
            assert e.status == 2 and "LDS" in str(e), e   # ECW_E_UNSUPPORTED
            continue
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
        ok, worst = gemv.check(y2.cpu().numpy(), wv, xv)
        assert ok, worst


@pytest.mark.parametrize("batch", [1, 4])
def test_cross_block_reduction_is_stable(batch):
    # row groups split over 16 blocks of one wave: the last block of each row group
    # adds the published partial sums; 20 back-to-back calls must agree bit for bit
    # and stay within the bound
    print(f"[gpu] cross-block reduction batch={batch}", flush=True)
    case = cases._int("split", 320, 2048, 2, 4, 11, 128, seed=31)
    ct = ecw.CompressedTensor(ecw.encode(case.lib_coding(), case.logical, case.scales),
                              waves_per_block=1, tiles_per_wave=1)
    xd, xv = _x(case, batch)
    y0 = ct.gemv(xd).clone()
    wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
    ok, worst = gemv.check(y0.cpu().numpy(), wv, xv)
    assert ok, worst
    ys = [ct.gemv(xd) for _ in range(20)]
    torch.cuda.synchronize()
    for y in ys:
        assert torch.equal(y, y0)


@pytest.mark.parametrize("shape", [(4, 1, 2), (2, 2, 3), (8, 1, 5), (1, 1, 4)])
@pytest.mark.parametrize("name", ["pair_m11_ragged", "cfg1_gauss_k1_m12", "fp8_m12", "bf16_m12",
                                  "quads_t64_m10_ragged"])
def test_row_groups_per_block_match_one_per_block(name, shape):
    # a block decoding several row groups in sequence (staging once) gives the same
    # bits as one row group per block: same wave order, same block order
    W, R, P_ = shape
    print(f"[gpu] row groups per block {name} W={W} R={R} P={P_}", flush=True)
    case = [c for c in cases.small_cases() if c.name == name][0]
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    one = ecw.CompressedTensor(blob, waves_per_block=W, tiles_per_wave=R, row_groups_per_block=1)
    many = ecw.CompressedTensor(blob, waves_per_block=W, tiles_per_wave=R, row_groups_per_block=P_)
    wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
    for batch in (1, 4):
        xd, xv = _x(case, batch)
        y1 = one.gemv(xd)
        yp = many.gemv(xd)
        torch.cuda.synchronize()
        assert torch.equal(y1, yp)
        ok, worst = gemv.check(yp.cpu().numpy(), wv, xv)
        assert ok, worst


@pytest.mark.parametrize("batch", [1, 4])
@pytest.mark.parametrize("name", ["pair_m11_ragged", "cfg1_gauss_k1_m12", "bf16_m12", "fp8_m12",
                                  "quads_16_slices_m12"])
def test_split_row_groups_leave_tickets_at_zero(name, batch):
    # one-wave blocks split every row group over all its slices: the last block of
    # each row group adds the partials; afterwards every arrival ticket is zero again,
    # and other launch shapes with the same partition (two row-group streams per wave,
    # several row groups per block) on the same workspace give the same bits
    print(f"[gpu] tickets {name} batch={batch}", flush=True)
    case = [c for c in cases.small_cases() if c.name == name][0]
    blob = ecw.encode(case.lib_coding(), case.logical, case.scales)
    ct = ecw.CompressedTensor(blob, waves_per_block=1, tiles_per_wave=1)
    xd, xv = _x(case, batch)
    ws = ct.workspace(batch)
    assert ws is not None
    y = torch.empty((batch, case.rows), dtype=torch.float32, device="cuda")
    ys = []
    for shape in [(1, 1, 1, 1), (1, 1, 2, 1), (1, 1, 1, 3), (1, 1, 2, 2), (1, 1, 1, 1)]:
        ct.set_launch(*shape)
        assert ecw.workspace_size(ct.t, batch) <= ws.numel()
        ecw.gemv_raw(ct.t, xd, y, ws)
        torch.cuda.synchronize()
        n_rg = (case.rows + 63) // 64
        if ecw.workspace_size(ct.t, batch):
            assert int(ws[:4 * n_rg].view(torch.int32).abs().sum()) == 0
        ys.append(y.clone())
    wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
    for yy in ys:
        assert torch.equal(yy, ys[0])
    ok, worst = gemv.check(ys[0].cpu().numpy(), wv, xv)
    assert ok, worst


def test_group_workspace_zero_fill_precondition():
    # dec_gemv_group's workspace through the C ABI.  Zero-filled once, every call
    # leaves the tickets at zero.  A member's launch shape fixes the size of its part
    # of the workspace, so changing it moves the later members' tickets onto bytes
    # that held partial sums: used without a new zero fill, those row groups never see
    # their last arrival and their y is not written (the call still returns OK).
    # Zero-filled again, the group gives the bits of separate calls.
    print("[gpu] group workspace precondition", flush=True)
    a = cases._int("ga", 256, 2048, 2, 4, 11, 128, seed=51)
    b = cases._int("gb", 192, 2048, 2, 4, 11, 128, seed=52)
    cta = ecw.CompressedTensor(ecw.encode(a.lib_coding(), a.logical, a.scales), waves_per_block=1, tiles_per_wave=1)
    ctb = ecw.CompressedTensor(ecw.encode(b.lib_coding(), b.logical, b.scales), waves_per_block=1, tiles_per_wave=1)
    xd, xv = _x(a, 1)
    big = ecw.group_workspace_size([cta.t, ctb.t], 1)
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    ya = torch.full((1, a.rows), float("nan"), device="cuda")
    yb = torch.full((1, b.rows), float("nan"), device="cuda")
    ecw.gemv_group_raw([cta.t, ctb.t], xd, [ya, yb], ws)
    torch.cuda.synchronize()
    assert int(ws.view(torch.int32)[:a.rows // 64].abs().sum()) == 0     # a's tickets
    assert torch.equal(ya, cta.gemv(xd)) and torch.equal(yb, ctb.gemv(xd))
    # a now takes two tiles per wave: its part shrinks and b's tickets move
    cta.set_launch(1, 2)
    assert ecw.group_workspace_size([cta.t, ctb.t], 1) < big
    ya.fill_(float("nan"))
    yb.fill_(float("nan"))
    ecw.gemv_group_raw([cta.t, ctb.t], xd, [ya, yb], ws)         # stale workspace
    torch.cuda.synchronize()
    assert torch.equal(ya, cta.gemv(xd)), "a's tickets did not move"
    assert bool(torch.isnan(yb).any()), "b's row groups finished on stale tickets"
    ws.zero_()
    yb.fill_(float("nan"))
    ecw.gemv_group_raw([cta.t, ctb.t], xd, [ya, yb], ws)
    torch.cuda.synchronize()
    assert torch.equal(ya, cta.gemv(xd)) and torch.equal(yb, ctb.gemv(xd))
    for y, c in ((ya, a), (yb, b)):      # same cols: both read x
        ok, worst = gemv.check(y.cpu().numpy(), P.weight_values(c.oracle_coding(), c.logical, c.scales), xv)
        assert ok, worst
