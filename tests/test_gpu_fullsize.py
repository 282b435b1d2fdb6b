"""GPU parity at the workloads' full sizes, through the C ABI.

For every tensor shape of the five workloads:
* decode parity: dec_materialize's weights over the WHOLE tensor equal the logical
  tensor bit for bit (for the lattice FP8 route: its E4M3 rounding), and every tile
  ends on its invariant;
* operator parity: dec_gemv (grouped as the benchmark groups it, in its launch
  configuration for the INT4 layer set) on EVERY row against a float64 product,
  |y - y_ref| <= 1e-3 * sum|w x| per output.
"""
import json
import os

import numpy as np
import pytest
import torch

import ecw_inputs as E
import entropy_coded_weight_amd as ecw
from oracle import gemv, pipeline as P, symbols as S
from tests import cases

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_all_rows(y, wv_of, xv, n, chunk=8192):
    """Every output of y [batch, n] against the float64 product, in row chunks;
    wv_of(r0, r1) gives the float64 weight values of rows [r0, r1)."""
    assert y.shape[1] == n
    worst = 0.0
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        ok, w = gemv.check(y[:, r0:r1], wv_of(r0, r1), xv)
        assert ok, f"rows [{r0}, {r1}): worst error / bound = {w}"
        worst = max(worst, w)
    return worst


def _materialize_equal(ct, want):
    _, w, st = ct.materialize(want_symbols=False)
    torch.cuda.synchronize()
    assert int(st.abs().sum()) == 0, "a tile did not end on its invariant"
    got = w.cpu().numpy()
    assert np.array_equal(got.view(want.dtype), want)


def test_config2_layer_set_at_the_benchmarked_launches():
    # the INT4 layer set, codings and launch shapes from the committed tune file,
    # grouped exactly as the benchmark launches it
    tune = json.load(open(os.path.join(ROOT, "entropy_coded_weight_amd", "tuned",
                                       "llama8b_int4_laplace_batch1.json")))["picks"]
    groups = [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
    for names in groups:
        print(f"[gpu] config 2 launch {'+'.join(names)}", flush=True)
        ts, cts = [], []
        for n in names:
            t = E.config2_tensor(n)
            p = tune[n]
            c = ecw.Coding(ecw.INT_CODES, *t.codes.shape, p["k"], 4, p["log2_m"], p["tile_cols"],
                           stored_tuples=p.get("stored_tuples", 0))
            cts.append(ecw.CompressedTensor(ecw.encode(c, t.codes, t.scales), waves_per_block=p["waves_per_block"],
                                            tiles_per_wave=p["tiles_per_wave"],
                                            streams_per_wave=p.get("streams_per_wave", 1),
                                            row_groups_per_block=p.get("row_groups_per_block", 1)))
            ts.append(t)
        x = torch.from_numpy(ts[0].x).cuda()
        ys = ecw.GemvGroup(cts).gemv(x)
        torch.cuda.synchronize()
        xv = gemv.x_values(ts[0].x, "f16")
        for t, ct, y in zip(ts, cts, ys):
            _check_all_rows(y.cpu().numpy(),
                            lambda r0, r1: t.codes[r0:r1].astype(np.float64)
                            * t.scales[r0:r1].astype(np.float64)[:, None], xv, t.codes.shape[0])
            _materialize_equal(ct, t.codes)


# (weights per symbol, log2 M, tile width, waves per block): one exponent per symbol,
# and exponent pairs in the codings and launch shapes the autotuner picked on MI355X
@pytest.mark.parametrize("name,k,m,tc,W", [("gate", 1, 12, 256, None), ("down", 1, 12, 256, None),
                                           ("gate", 2, 11, 128, 4), ("down", 2, 12, 128, 16)])
def test_config3_bf16_full(name, k, m, tc, W):
    print(f"[gpu] config 3 {name} k={k} m={m} tc={tc} W={W}", flush=True)
    t = E.config3_tensor(name)
    c = ecw.Coding(ecw.BF16_EXP, *t.bits.shape, k, 0, m, tc)
    ct = ecw.CompressedTensor(ecw.encode(c, t.bits), waves_per_block=W, tiles_per_wave=1 if W else None)
    x = torch.from_numpy(t.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y = ct.gemv(x).cpu().numpy()
    _check_all_rows(y, lambda r0, r1: S.bf16_value(t.bits[r0:r1]), gemv.x_values(t.x_bits, "bf16"),
                    t.bits.shape[0])
    _materialize_equal(ct, t.bits)


@pytest.mark.parametrize("name", ["q", "k", "o", "gate", "down", "lm_head"])
def test_config4_fp8_full_batch_1_and_4(name):
    print(f"[gpu] config 4 {name}", flush=True)
    t = E.config4_tensor(name, batch=4)
    n, K = t.codes.shape
    c = ecw.Coding(ecw.FP8_E4M3, n, K, 1, 0, 12, 256)
    ct = ecw.CompressedTensor(ecw.encode(c, t.codes, t.scales))

    def wv(r0, r1):
        return S.e4m3_value(t.codes[r0:r1]) * t.scales[r0:r1].astype(np.float64)[:, None]

    for batch in (1, 4):
        xb = t.x_bits[:batch]
        x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda().view(torch.bfloat16)
        y = ct.gemv(x).cpu().numpy()
        _check_all_rows(y, wv, gemv.x_values(xb, "bf16"), n)
    _materialize_equal(ct, t.codes)


@pytest.mark.parametrize("recon", [4, 5], ids=["int8", "fp8"])
def test_config5_e8_full(recon):
    print(f"[gpu] config 5 recon {recon}", flush=True)
    v2, scales, xh = cases.config5()
    n, K = v2.shape
    c = ecw.Coding(ecw.E8_LATTICE, n, K, 8, 0, 11, 128, recon)
    ct = ecw.CompressedTensor(ecw.encode(c, v2, scales))
    y = ct.gemv(torch.from_numpy(xh).cuda()).cpu().numpy()

    def wv(r0, r1):
        oc = P.Coding(P.E8_LATTICE, r1 - r0, K, k=8, log2_m=11, tile_cols=128, recon_dtype=recon)
        return P.weight_values(oc, v2[r0:r1], scales[r0:r1])

    _check_all_rows(y, wv, gemv.x_values(xh, "f16"), n)
    want = P.reconstructed_dtype_tensor(P.Coding(P.E8_LATTICE, n, K, k=8, log2_m=11, tile_cols=128,
                                                 recon_dtype=recon), v2)
    _materialize_equal(ct, want)


@pytest.mark.parametrize("which", ["int4_gate_f16", "bf16_gate_pairs_bf16"])
def test_dequantize_full_size(which):
    # the dense matrix the GEMM path reads, at full size in the benchmarked codings:
    # every weight bit for bit against the oracle's rounding; the GEMM at 16
    # activation rows, every output within the bound of the same dense weights
    print(f"[gpu] dequantize full size {which}", flush=True)
    if which.startswith("int4"):
        t = E.config2_tensor("gate")
        p = json.load(open(os.path.join(ROOT, "entropy_coded_weight_amd", "tuned",
                                        "llama8b_int4_laplace_batch1.json")))["picks"]["gate"]
        c = ecw.Coding(ecw.INT_CODES, *t.codes.shape, p["k"], 4, p["log2_m"], p["tile_cols"],
                       stored_tuples=p.get("stored_tuples", 0))
        logical, scales, tdt, dname = t.codes, t.scales, torch.float16, "f16"
        oc = P.Coding(P.INT_CODES, *t.codes.shape, k=p["k"], code_bits=4, log2_m=p["log2_m"],
                      tile_cols=p["tile_cols"])
    else:
        t = E.config3_tensor("gate")
        c = ecw.Coding(ecw.BF16_EXP, *t.bits.shape, 2, 0, 11, 128)
        logical, scales, tdt, dname = t.bits, None, torch.bfloat16, "bf16"
        oc = P.Coding(P.BF16_EXP, *t.bits.shape, k=2, log2_m=11, tile_cols=128)
    ct = ecw.CompressedTensor(ecw.encode(c, logical, scales))
    w = ct.dequantize(tdt)
    torch.cuda.synchronize()
    want = P.dequantized(oc, logical, scales, dname)
    got = w.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    x = torch.randn((16, logical.shape[1]), dtype=tdt, device="cuda")
    y = ct.gemm(x, w_buf=w)
    torch.cuda.synchronize()
    w16 = torch.from_numpy(want.view(np.int16)).view(tdt)
    _check_all_rows(y.cpu().numpy(), lambda r0, r1: w16[r0:r1].double().numpy(), x.double().cpu().numpy(),
                    logical.shape[0])
