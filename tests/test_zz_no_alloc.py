"""dec_gemv_noalloc: the allocation-free variant of dec_gemv, through the C ABI.

Its partial sums and arrival tickets live in the library's per-GPU scratch array
instead of a caller workspace.  It must give the same bits as dec_gemv with the same
launch shape (and so stay within |y - y_ref| <= 1e-3 * sum|w x| of the float64
product), on two calls in a row, the second with a smaller input and another launch
shape; a launch whose partial sums exceed the scratch is refused before launching.
"""
import ctypes

import numpy as np
import pytest
import torch

import ecw_inputs as E
import entropy_coded_weight_amd as ecw
from oracle import gemv, pipeline as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tensor(rows, cols, k, m, tc, W, R, seed, stored=0, batch=1):
    t = E.small_int_codes(rows, cols, seed=seed, batch=batch)
    c = ecw.Coding(ecw.INT_CODES, rows, cols, k, 4, m, tc, stored_tuples=stored)
    ct = ecw.CompressedTensor(ecw.encode(c, t.codes, t.scales), waves_per_block=W, tiles_per_wave=R)
    oc = P.Coding(P.INT_CODES, rows, cols, k=k, code_bits=4, log2_m=m, tile_cols=tc, stored_tuples=stored)
    return t, ct, oc


def _noalloc(ct, x, y):
    L = ecw.lib()
    st = L.dec_gemv_noalloc(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(ct.t),
                            x.data_ptr(), ecw.DT_F16, y.data_ptr(), x.shape[0])
    return st


def _with_workspace(ct, x):
    y = torch.empty((x.shape[0], ct.rows), dtype=torch.float32, device="cuda")
    n = ecw.workspace_size(ct.t, x.shape[0])
    ws = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    ecw.gemv_raw(ct.t, x, y, ws if n else None)
    return y


@pytest.mark.parametrize("batch", [1, 4])
def test_noalloc_matches_dec_gemv_on_two_calls(batch):
    # call 1: 512 x 4096 pairs, 64-wide tiles, 4 waves per block -> every row group is
    # split over 16 blocks (scratch partials and tickets in use)
    big, ct_big, oc_big = _tensor(512, 4096, 2, 11, 64, 4, 1, seed=41, batch=batch)
    # call 2: smaller, another launch shape and coding (quads, 3 blocks per row group)
    small, ct_small, oc_small = _tensor(200, 1536, 4, 12, 128, 4, 1, seed=42, stored=256, batch=batch)
    for t, ct, oc in ((big, ct_big, oc_big), (small, ct_small, oc_small)):
        assert ecw.workspace_size(ct.t, batch) > 0, "the case must use split row groups"
        print(f"[gpu] noalloc batch={batch} rows={oc.rows} cols={oc.cols} k={oc.k}", flush=True)
        x = torch.from_numpy(t.x).cuda()
        want = _with_workspace(ct, x)
        y = torch.full((batch, ct.rows), float("nan"), dtype=torch.float32, device="cuda")
        assert _noalloc(ct, x, y) == 0, ecw.lib().ecw_last_error()
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.cpu().numpy().view(np.uint32)), "bits differ from dec_gemv"
        ok, worst = gemv.check(got, P.weight_values(oc, t.codes, t.scales), gemv.x_values(t.x, "f16"))
        assert ok, f"worst error / bound = {worst}"
    # the first tensor again after the smaller one: the scratch holds no stale state
    x = torch.from_numpy(big.x).cuda()
    y = torch.empty((batch, ct_big.rows), dtype=torch.float32, device="cuda")
    assert _noalloc(ct_big, x, y) == 0
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), _with_workspace(ct_big, x).cpu().numpy().view(np.uint32))


def test_noalloc_refuses_launches_beyond_the_scratch():
    # 8192 x 4096 pairs at 64-wide tiles, one wave per block and batch 4: 128 row
    # groups x 64 blocks x 4 rows x 256 B = 8 MiB of partial sums, beyond the
    # scratch's (8 MiB - 64 KiB)
    t, ct, _ = _tensor(8192, 4096, 2, 11, 64, 1, 1, seed=43, batch=4)
    x = torch.from_numpy(t.x).cuda()
    y = torch.full((4, ct.rows), 7.0, dtype=torch.float32, device="cuda")
    st = _noalloc(ct, x, y)
    assert st == 2, "expected ECW_E_UNSUPPORTED"
    assert b"allocation-free" in ecw.lib().ecw_last_error()
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "nothing may be written on error"
