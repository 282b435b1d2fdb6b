"""GPU parity of the dequantising decode and the dense GEMM path, through the C ABI.

* dec_dequantize writes the real weight values rounded to nearest even into fp16
  or bf16: bit for bit the oracle's rounding of its float64 weight values, for every
  small case (INT codes 1/2/4 per symbol, BF16 one exponent or a pair with escapes,
  FP8, lattice fields on both reconstruction routes), ragged row groups and slices
  included (lattice slices ending on a partial 32-weight segment).
* CompressedTensor.gemm above four activation rows multiplies those dense weights
  with the library GEMM: within |y - y_ref| <= 1e-3 * sum|w x| of the float64
  product of the same rounded weights; up to four rows it is the fused decode-GEMV.
"""
import numpy as np
import pytest
import torch

import entropy_coded_weight_amd as ecw
from oracle import gemv, pipeline as P
from tests import cases

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dequant_cases():
    return cases.small_cases() + cases.e8_cases() + [cases.e8_case(4, rows=70, cols=200, m=10, tc=64, seed=7),
                                                     cases.e8_case(5, rows=64, cols=264, m=11, tc=128, seed=8)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", _dequant_cases(), ids=lambda c: c.name)
def test_dequantize_bit_exact(case, dtype):
    print(f"[gpu] dequantize {case.name} {dtype}", flush=True)
    ct = ecw.CompressedTensor(ecw.encode(case.lib_coding(), case.logical, case.scales))
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    out = torch.full((case.rows, case.cols), -1, dtype=torch.int16, device="cuda").view(tdt)
    ct.dequantize(tdt, out=out)
    torch.cuda.synchronize()
    want = P.dequantized(case.oracle_coding(), case.logical, case.scales, dtype)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_dequantize_rejects_bad_buffers():
    L = ecw.lib()
    c1 = cases.small_cases()[1]
    out = torch.empty((c1.rows, c1.cols), dtype=torch.float16, device="cuda")
    ct = ecw.CompressedTensor(ecw.encode(c1.lib_coding(), c1.logical, c1.scales))
    import ctypes
    assert L.dec_dequantize(None, ctypes.byref(ct.t), out.data_ptr() + 2, ecw.DT_F16) == 1   # misaligned
    assert L.dec_dequantize(None, ctypes.byref(ct.t), out.data_ptr(), ecw.DT_F32) == 1       # dtype


@pytest.mark.parametrize("batch", [5, 8, 33])
@pytest.mark.parametrize("name", ["pair_m11_ragged", "cfg1_gauss_k1_m12", "bf16_pairs_mixed_bf16x", "fp8_m12",
                                  "quad_int2"])
def test_gemm_above_four_rows(name, batch):
    print(f"[gpu] gemm {name} batch={batch}", flush=True)
    case = [c for c in cases.small_cases() if c.name == name][0]
    ct = ecw.CompressedTensor(ecw.encode(case.lib_coding(), case.logical, case.scales))
    rng = np.random.default_rng([0, 902, batch])
    xv = rng.standard_normal((batch, case.cols))
    tdt = torch.bfloat16 if case.x_dtype == "bf16" else torch.float16
    xd = torch.from_numpy(xv.astype(np.float32)).to(tdt).cuda()
    y = ct.gemm(xd)
    torch.cuda.synchronize()
    assert y.dtype == torch.float32 and y.shape == (batch, case.rows)
    wbits = P.dequantized(case.oracle_coding(), case.logical, case.scales, "bf16" if tdt == torch.bfloat16 else "f16")
    if tdt == torch.bfloat16:
        w16 = torch.from_numpy(wbits.view(np.int16)).view(torch.bfloat16).double().numpy()
    else:
        w16 = wbits.view(np.float16).astype(np.float64)
    x64 = xd.double().cpu().numpy()
    ok, worst = gemv.check(y.cpu().numpy(), w16, x64)
    assert ok, f"worst error / bound = {worst}"


def test_gemm_up_to_four_rows_is_the_fused_path():
    case = cases.small_cases()[1]
    ct = ecw.CompressedTensor(ecw.encode(case.lib_coding(), case.logical, case.scales))
    xd = torch.randn((3, case.cols), dtype=torch.float16, device="cuda")
    assert torch.equal(ct.gemm(xd), ct.gemv(xd))
