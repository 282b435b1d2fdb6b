"""Benchmark: fused rANS decode + batch-1 GEMV over one Llama-3.1-8B-shaped layer set.

One step = one pass of the hot path over the seven linear layers of one transformer
block (q, k, v, o 4096x4096 / 1024x4096, gate/up 14336x4096, down 4096x14336), each
stored as 16-level Laplacian codes (2.2 bits of entropy) packed two per rANS symbol,
decoded and multiplied into y = W x at batch 1.  Launch order follows the block's
data flow: q, k, v, o, gate, up, down.  Blobs are rotated over >= 512 MiB of copies
(twice the 256 MiB Infinity Cache), so every step reads its weights from HBM.  Each
step is captured once per rotated copy as a HIP graph; the timed region replays them.

The other workloads are measured in the same run (secondary, under "configs"): the
1024x1024 Gaussian-code matrix, BF16 exponent coding of the gate / down shapes, and
one transformer layer of per-row FP8 E4M3 weights at batch 1 and 4 (optionally with
the 128256x4096 LM head).  Each picks its coding and launch shape with the
autotuner on this device, then is timed cold like the layer set.

Prints one JSON line (stdout).  Per-tensor details go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "µs per fused decode-GEMV layer + effective weight GB/s (% HBM peak), batch 1"
ORDER = ["q", "k", "v", "o", "gate", "up", "down"]
# launches of one decode step, in data-flow order; tensors of a launch share x
LAUNCHES = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gate_up", ["gate", "up"]), ("down", ["down"])]

# per-tensor coding: (k, log2_m, tile_cols, waves_per_block, tiles_per_wave,
# streams_per_wave, row_groups_per_block).  Used
# when no tune file exists; `--tune` measures every candidate on the device and
# writes TUNE_FILE, which later runs load.
DEFAULT_CODING = {"q": (2, 12, 128, 16, 1, 1, 1, 0), "k": (2, 12, 128, 16, 1, 1, 1, 0),
                  "v": (2, 12, 128, 16, 1, 1, 1, 0), "o": (2, 12, 128, 16, 1, 1, 1, 0),
                  "gate": (2, 12, 256, 16, 1, 1, 1, 0), "up": (2, 12, 256, 16, 1, 1, 1, 0),
                  "down": (2, 12, 256, 16, 1, 1, 1, 0)}
TUNE_FILE = os.path.join(ROOT, "entropy_coded_weight_amd", "tuned", "llama8b_int4_laplace_batch1.json")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_decode_llama8b_int4_gate_up_traffic.txt")


def load_coding(path: str):
    if not os.path.exists(path):
        return dict(DEFAULT_CODING), "defaults"
    with open(path) as f:
        d = json.load(f)
    coding = dict(DEFAULT_CODING)
    for n, p in d["picks"].items():
        coding[n] = (p["k"], p["log2_m"], p["tile_cols"], p["waves_per_block"], p["tiles_per_wave"],
                     p.get("streams_per_wave", 1), p.get("row_groups_per_block", 1), p.get("stored_tuples", 0))
    return coding, os.path.relpath(path, ROOT)


def run_tuner(path: str, batch: int):
    """Autotune every tensor of the layer set (k in {1, 2, 4} with quads over stored
    tuples, M in {2^10, 2^11, 2^12}, tile width in {64..512}, waves per block, tiles
    per wave, row streams per wave, row groups per block) and write the picks."""
    import torch
    import ecw_inputs as E
    from entropy_coded_weight_amd import autotune as A, INT_CODES
    cands, specs, xs = {}, {}, {}
    for name in ORDER:
        t = E.config2_tensor(name, layer=0, batch=batch)
        xs[name] = torch.from_numpy(t.x).cuda()
        specs[name] = (INT_CODES, t.codes, t.scales, 4)
        log(f"tuning {name} {t.codes.shape}")
        cands[name] = A.tune_tensor(INT_CODES, t.codes, t.scales, xs[name], code_bits=4, ks=(1, 2, 4), log=log)
    picks, fronts = {}, {}
    for ln, names in LAUNCHES:
        log(f"tuning launch {ln}")
        pts = []
        g = A.tune_group({n: specs[n] for n in names}, {n: cands[n] for n in names}, xs[names[0]], log=log,
                         points=pts)
        picks.update(g)
        # the launch's speed-size Pareto front over every timed grouping (MINE page, Section 4.2)
        fronts[ln] = [[round(u, 3), int(b), ch] for u, b, ch in A.pareto_front(pts)]
    table = {n: [dict(k=c.k, log2_m=c.log2_m, tile_cols=c.tile_cols, stored_tuples=c.stored_tuples,
                      stored_bytes=c.stored_bytes,
                      shapes={f"{w}x{r}x{ns}x{p}": round(us, 3) for (w, r, ns, p), us in c.shape_us.items()})
                 for c in cands[n]] for n in ORDER}
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"workload": "Llama-3.1-8B-shaped layer set, 16-level Laplacian codes (H=2.2 bits), "
                               f"fp16 row scales, fp16 x, batch {batch}",
                   "device": torch.cuda.get_device_name(0), "picks": picks, "fronts": fronts,
                   "candidates": table}, f, indent=1)
    log(f"wrote {path}")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_layer(batch: int, coding: dict):
    import ecw_inputs as E
    import entropy_coded_weight_amd as ecw
    layer = {}
    for name in ORDER:
        t = E.config2_tensor(name, layer=0, batch=batch)
        kk, m, tc, W, R, NS, RPB, T = coding[name]
        n, k = t.codes.shape
        c = ecw.Coding(ecw.INT_CODES, n, k, kk, 4, m, tc, stored_tuples=T)
        blob = ecw.encode(c, t.codes, t.scales)
        layer[name] = dict(tensor=t, coding=c, blob=blob, launch=(W, R, NS, RPB))
    return layer


def cpu_baseline(layer, target_s: float = 12.0):
    """Time the oracle (numpy decode + fp64 GEMV) on whole 64-row groups of every
    tensor until about target_s seconds of work, then scale to one full layer by
    symbol count.  The sampled rows are encoded by the oracle first (untimed)."""
    from threadpoolctl import threadpool_limits
    from oracle import gemv as G, pipeline as P
    done_syms, total_syms, t_used, rows_done = 0, 0, 0.0, 0
    for name in ORDER:
        total_syms += layer[name]["tensor"].codes.size // layer[name]["coding"].weights_per_symbol
    max_rg = max((layer[n]["tensor"].codes.shape[0] + 63) // 64 for n in ORDER)
    with threadpool_limits(limits=1):
        rg = 0
        while t_used < target_s and rg < max_rg:
            for name in ORDER:
                t = layer[name]["tensor"]
                n, K = t.codes.shape
                r0, r1 = rg * 64, min(rg * 64 + 64, n)
                if r0 >= n:
                    continue
                c = layer[name]["coding"]
                kk = c.weights_per_symbol
                ocd = P.Coding(P.INT_CODES, r1 - r0, K, k=kk, code_bits=4, log2_m=c.log2_m,
                               tile_cols=c.tile_cols, stored_tuples=c.stored_tuples)
                comp = P.encode(ocd, t.codes[r0:r1], t.scales[r0:r1])
                t0 = time.perf_counter()
                q = P.decode(comp)
                wv = P.weight_values(ocd, q, t.scales[r0:r1])
                G.gemv_f64(wv, G.x_values(t.x, "f16"))
                t_used += time.perf_counter() - t0
                done_syms += q.size // kk
                rows_done += r1 - r0
            rg += 1
    us_layer = t_used / done_syms * total_syms * 1e6
    return {"value": round(us_layer, 1), "unit": "us/layer", "cores": 1, "kind": "oracle",
            "sample": f"{rows_done} rows in whole 64-row groups of all 7 tensors ({done_syms} symbols, "
                      f"{t_used:.1f} s): numpy decode + float64 GEMV, BLAS limited to 1 thread, "
                      f"scaled to the full layer by symbol count"}


def check_rows(y: np.ndarray, w_rows: np.ndarray, x: np.ndarray) -> float:
    """Worst |y - y_ref| / (1e-3 * sum|w x|) over the given rows, y_ref in float64.
    y [batch, rows], w_rows float64 [rows, K], x float64 [batch, K]."""
    ref = x @ w_rows.T
    bound = 1e-3 * (np.abs(x) @ np.abs(w_rows).T)
    err = np.abs(y.astype(np.float64) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    return float(r.max())


def check_all(y: np.ndarray, wv_of, x: np.ndarray, chunk: int = 8192) -> float:
    """check_rows over EVERY row of y [batch, N], in row chunks; wv_of(r0, r1) gives
    the float64 weight values of rows [r0, r1)."""
    worst = 0.0
    for r0 in range(0, y.shape[1], chunk):
        r1 = min(y.shape[1], r0 + chunk)
        worst = max(worst, check_rows(y[:, r0:r1], wv_of(r0, r1), x))
    return worst


def fp8_values(t):
    """Row-chunk weight values of a per-row FP8 E4M3 tensor (E4M3 value * row scale)."""
    import torch
    return lambda r0, r1: torch.from_numpy(t.codes[r0:r1]).view(torch.float8_e4m3fn).double().numpy() \
        * t.scales[r0:r1].astype(np.float64)[:, None]


def int_values(t):
    """Row-chunk weight values of an INT-code tensor (code * fp16 row scale)."""
    return lambda r0, r1: t.codes[r0:r1].astype(np.float64) * t.scales[r0:r1].astype(np.float64)[:, None]


def time_cold(launches, batch: int, steps: int, cold_bytes: float):
    """Cold device timing of grouped launches (autotune.time_cold)."""
    from entropy_coded_weight_amd import autotune as A
    return A.time_cold(launches, batch, steps, cold_bytes)


def _plugin_bits(counts: np.ndarray) -> float:
    p = counts[counts > 0] / counts.sum()
    return float(-(p * np.log2(p)).sum())


def e8_bits_per_weight(v2: np.ndarray) -> float:
    """Plug-in entropy per weight of the lattice fields of doubled-coordinate blocks
    v2 [n, 8]: the coset, then the eight fields (z1..z7, m = floor(z8 / 2)) given the
    coset, each with its own histogram (the 17 coset-indexed tables)."""
    v2 = np.asarray(v2, dtype=np.int64).reshape(-1, 8)
    c = v2[:, 0] & 1
    z = (v2 - c[:, None]) // 2
    f = np.concatenate([z[:, :7], np.floor_divide(z[:, 7:8], 2)], axis=1)
    total = _plugin_bits(np.bincount(c, minlength=2)) * len(c)
    for cc in (0, 1):
        sel = f[c == cc]
        for j in range(8):
            if len(sel):
                total += _plugin_bits(np.bincount(sel[:, j] - sel[:, j].min())) * len(sel)
    return total / (8 * len(c))


def config5_inputs():
    """The lattice workload, generated with the library's E8 quantiser: w = N(0, 0.02^2)
    [3072, 12288]; rows divided by their RMS; the lattice step from 12 steps of
    geometric bisection on [1e-3, 8] so that the plug-in entropy of the block fields on
    2^18 sampled blocks is 4.0 bits per weight; v = nearest E8 point of u / s; fp16
    row scale = least-squares refit <w_r, v_r> / <v_r, v_r>.  Returns (2v int8
    [N, K], fp16 scales, fp16 x [1, K], step, bits per weight)."""
    import math
    import ecw_inputs as E
    import entropy_coded_weight_amd as ecw
    n, k = 3072, 12288
    rng = E.rng_for(5, 0, 0)
    w = E.normal_matrix((n, k), rng)
    x = rng.standard_normal((1, k)).astype(np.float16)
    rms = np.sqrt((w * w).mean(axis=1))
    u = (w / rms[:, None]).reshape(-1, 8)
    srng = np.random.default_rng([0, 5, n, k])
    sample = u[srng.choice(u.shape[0], 1 << 18, replace=False)]
    lo, hi = 1e-3, 8.0
    for _ in range(12):
        mid = math.sqrt(lo * hi)
        if e8_bits_per_weight(ecw.e8_nearest(sample / mid)) > 4.0:
            lo = mid
        else:
            hi = mid
    step = math.sqrt(lo * hi)
    v2 = np.empty(u.shape, np.int8)
    for b0 in range(0, u.shape[0], 1 << 18):
        v2[b0:b0 + (1 << 18)] = ecw.e8_nearest(u[b0:b0 + (1 << 18)] / step)
    v2 = v2.reshape(n, k)
    v = v2.astype(np.float64) / 2.0
    scales = ((w * v).sum(axis=1) / np.maximum((v * v).sum(axis=1), 1e-30)).astype(np.float16)
    return v2, scales, x, step, e8_bits_per_weight(ecw.e8_nearest(sample / step))


def secondary_configs(which: str, steps: int, cold_bytes: float, lm_head: bool):
    """Per-workload measurements besides the layer set: coding and launch shape
    picked by the autotuner on this device (warm), then timed cold; every row
    checked against float64."""
    import torch
    import ecw_inputs as E
    import entropy_coded_weight_amd as ecw
    from entropy_coded_weight_amd import autotune as A
    dev = torch.device("cuda:0")
    res = {}

    def tuned_blob(payload, w, scales, x, code_bits=0, ks=None, log2_ms=(10, 11, 12),
                   tile_cols=(128, 256, 512)):
        cands = A.tune_tensor(payload, w, scales, x, code_bits=code_bits, ks=ks, log2_ms=log2_ms,
                              tile_cols=tile_cols, reps=10)
        p = A.pick(cands)
        c = ecw.Coding(payload, w.shape[0], w.shape[1], p["k"], code_bits if payload == ecw.INT_CODES else 0,
                       p["log2_m"], p["tile_cols"], stored_tuples=p.get("stored_tuples", 0))
        shape = (p["waves_per_block"], p["tiles_per_wave"], p["streams_per_wave"], p["row_groups_per_block"])
        return ecw.encode(c, w, scales), shape, p

    def summary(launch_us, blobs_bytes, n_weights, unc_bytes, worst, picks, extra=None):
        t = sum(launch_us.values())
        d = {"us": round(t, 3), "per_launch_us": {k: round(v, 3) for k, v in launch_us.items()},
             "stored_bytes": int(blobs_bytes), "stored_bits_per_weight": round(blobs_bytes * 8 / n_weights, 4),
             "gbps_compressed": round(blobs_bytes / (t * 1e-6) / 1e9, 1),
             "hbm_frac": round(blobs_bytes / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
             "gbps_uncompressed_equiv": round(unc_bytes / (t * 1e-6) / 1e9, 1),
             "parity_worst_err_over_bound": worst, "codings": picks}
        if extra:
            d.update(extra)
        return d

    def stored(blob):
        t = ecw.prepare(blob)
        return t.bytes_words + t.bytes_raw + t.bytes_tile_meta + t.bytes_tables + t.bytes_scales

    if "1" in which:
        log("config 1: 1024x1024 Gaussian codes, one code per symbol, M = 2^12")
        t = E.config1()
        x = torch.from_numpy(t.x).to(dev)
        blob, shape, p = tuned_blob(ecw.INT_CODES, t.codes, t.scales, x, code_bits=4, ks=(1,), log2_ms=(12,),
                                    tile_cols=(64, 128, 256, 512))
        us, ys = time_cold([("w", [(blob, shape)], x)], 1, steps, cold_bytes)
        worst = check_all(ys["w"][0], int_values(t), t.x.astype(np.float64))
        n = t.codes.size
        res["1"] = summary(us, stored(blob), n, n * 0.5 + 1024 * 2, worst, {"w": p},
                           {"workload": "one 1024x1024 matrix of 16-level codes from a discretised Gaussian "
                                        "(sigma 2 levels, seed 0), fp16 row scales, fp16 x, batch 1"})

    if "3" in which:
        log("config 3: BF16 exponent coding, gate 14336x4096 and down 4096x14336")
        launches, picks, nbytes, nw, checks = [], {}, 0, 0, []
        for name in ("gate", "down"):
            t = E.config3_tensor(name)
            x = torch.from_numpy(t.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
            blob, shape, p = tuned_blob(ecw.BF16_EXP, t.bits, None, x, log2_ms=(10, 11, 12))
            launches.append((name, [(blob, shape)], x))
            picks[name] = p
            nbytes += stored(blob)
            nw += t.bits.size
            xv = torch.from_numpy(t.x_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
            checks.append((name, t.bits, xv))
        us, ys = time_cold(launches, 1, steps, cold_bytes)
        worst = max(check_all(ys[n][0], lambda r0, r1, b=b: torch.from_numpy(b[r0:r1].view(np.int16))
                              .view(torch.bfloat16).double().numpy(), xv) for n, b, xv in checks)
        res["3"] = summary(us, nbytes, nw, nw * 2, worst, picks,
                           {"workload": "BF16 N(0, 0.02^2) weights at 14336x4096 and 4096x14336, exponent "
                                        "byte rANS-coded, sign+mantissa byte raw, bf16 x, batch 1; "
                                        "two launches"})

    if "5" in which:
        log("config 5: E8 lattice fields, 3072x12288, INT8 and FP8 reconstruction")
        v2, scales, xh, step, bpw = config5_inputs()
        x = torch.from_numpy(xh).to(dev)
        n, K = v2.shape
        for recon, tag in ((ecw.DT_I8, "int8"), (ecw.DT_FP8_E4M3, "fp8")):
            # table size and tile width tuned like the other payloads: the 17 tables
            # take 4 bytes per slot in LDS, so M = 2^9 leaves room for two blocks per CU
            cand = []
            for m in (9, 10, 11):
                for tc in (64, 128, 256):
                    c = ecw.Coding(ecw.E8_LATTICE, n, K, 8, 0, m, tc, recon)
                    blob = ecw.encode(c, v2, scales)
                    ct = ecw.CompressedTensor(blob)
                    stream = torch.cuda.Stream()
                    with torch.cuda.stream(stream):
                        su = A._tune_launch(ct, x, [s for s in A.DEFAULT_SHAPES if s[2] == 1], 10, stream)
                    stream.synchronize()
                    us, shape = min((u, s) for s, u in su.items())
                    cand.append((us, stored(blob), m, tc, shape, blob))
            t_min = min(c_[0] for c_ in cand)
            _, _, m, tc, shape, blob = min((c_ for c_ in cand if c_[0] <= 1.02 * t_min), key=lambda c_: c_[1])
            us, ys = time_cold([("w", [(blob, shape)], x)], 1, steps, cold_bytes)
            def wv(r0, r1, recon=recon):
                vv = v2[r0:r1].astype(np.float64) / 2.0
                if recon != ecw.DT_I8:
                    vv = torch.from_numpy(vv.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
                return vv * scales[r0:r1].astype(np.float64)[:, None]
            worst = check_all(ys["w"][0], wv, xh.astype(np.float64))
            res[f"5_{tag}"] = summary(us, stored(blob), v2.size, v2.size + n * 2, worst,
                                      {"w": dict(k=8, log2_m=m, tile_cols=tc, waves_per_block=shape[0],
                                                 tiles_per_wave=shape[1], streams_per_wave=shape[2],
                                                 row_groups_per_block=shape[3])},
                                      {"workload": "3072x12288 N(0, 0.02^2) weights, row-RMS normalised, E8 "
                                                   f"lattice step {step:.4f} ({bpw:.3f} bits/weight plug-in "
                                                   "entropy), 9 fields per 8-weight block coded with 17 "
                                                   f"coset-indexed tables (M tuned), {tag} reconstruction, "
                                                   "fp16 row scales, fp16 x, batch 1"})

    if "p" in which:
        res["budget"] = budget_points(steps, cold_bytes)

    if "d" in which:
        res["dequant"] = dequant_gemm(steps, cold_bytes)

    if "4" in which:
        names = ["q", "k", "v", "o", "gate", "up", "down"] + (["lm_head"] if lm_head else [])
        groups = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gate_up", ["gate", "up"]), ("down", ["down"])]
        if lm_head:
            groups.append(("lm_head", ["lm_head"]))
        log("config 4: one transformer layer of per-row FP8 E4M3 weights" + (" + LM head" if lm_head else ""))
        ts = {n: E.config4_tensor(n, batch=4) for n in names}

        def x_of(n, batch):
            return torch.from_numpy(np.ascontiguousarray(ts[n].x_bits[:batch]).view(np.int16)) \
                .to(dev).view(torch.bfloat16)

        cands = {}
        for batch in (1, 4):
            picks, blobs = {}, {}
            for ln, ns in groups:
                x = x_of(ns[0], batch)
                for n in ns:
                    t = ts[n]
                    if batch == 1:
                        # M and tile width per tensor, tuned at batch 1
                        cands[n] = A.tune_tensor(ecw.FP8_E4M3, t.codes, t.scales, x, log2_ms=(11, 12),
                                                 tile_cols=(128, 256), reps=10)
                    else:
                        # the batch-1 coding, launch shapes re-tuned for batch 4
                        p1 = prev_picks[n]
                        cands[n] = A.tune_tensor(ecw.FP8_E4M3, t.codes, t.scales, x, log2_ms=(p1["log2_m"],),
                                                 tile_cols=(p1["tile_cols"],), reps=10)
                specs = {n: (ecw.FP8_E4M3, ts[n].codes, ts[n].scales, 0) for n in ns}
                g = A.tune_group(specs, {n: cands[n] for n in ns}, x, cold=False, reps=10)
                picks.update(g)
            launches, nbytes, nw = [], 0, 0
            for ln, ns in groups:
                members = []
                for n in ns:
                    p = picks[n]
                    t = ts[n]
                    c = ecw.Coding(ecw.FP8_E4M3, *t.codes.shape, 1, 0, p["log2_m"], p["tile_cols"])
                    blob = ecw.encode(c, t.codes, t.scales)
                    members.append((blob, (p["waves_per_block"], p["tiles_per_wave"], p["streams_per_wave"],
                                           p["row_groups_per_block"])))
                    nbytes += stored(blob)
                    nw += t.codes.size
                launches.append((ln, members, x_of(ns[0], batch)))
            prev_picks = picks
            us, ys = time_cold(launches, batch, steps, cold_bytes)
            worst = 0.0
            for ln, ns in groups:
                xv = x_of(ns[0], batch).double().cpu().numpy()
                for i, n in enumerate(ns):
                    t = ts[n]
                    worst = max(worst, check_all(ys[ln][i], fp8_values(t), xv))
            layer_us = sum(v for k, v in us.items() if k != "lm_head")
            extra = {"workload": "one Llama-3.1-8B-shaped layer (q,k,v,o,gate,up,down) of N(0, 0.02^2) "
                                 "weights quantised per row to FP8 E4M3 (fp16 row scale), byte symbols "
                                 f"rANS-coded, bf16 x, batch {batch}; launches q/k/v, o, gate/up, down"
                                 + (", LM head" if lm_head else ""),
                     "layer_us": round(layer_us, 3)}
            if lm_head:
                extra["step_us_32_layers_plus_head"] = round(32 * layer_us + us["lm_head"], 1)
            res[f"4_batch{batch}"] = summary(us, nbytes, nw, sum(ts[n].codes.size + ts[n].codes.shape[0] * 2
                                                                 for n in names), worst, picks, extra)
    return res


def budget_points(steps: int, cold_bytes: float):
    """The layer set under byte budgets: from the tune file's per-launch speed-size
    Pareto fronts, the fastest choice of one grouping per launch whose stored bytes fit
    the budget (exact multiple-choice knapsack), for the smallest feasible budget, the
    fastest choice's size and one midway; each choice is encoded, timed cold and
    checked like the headline, and its payload words are set against the
    cross-entropy lower bound of its tables (MINE page, Section 4.2)."""
    import torch
    import ecw_inputs as E
    import entropy_coded_weight_amd as ecw
    from entropy_coded_weight_amd import autotune as A
    tf = json.load(open(TUNE_FILE))
    if "fronts" not in tf:
        return None
    fr = {ln: [(u, b, ch) for u, b, ch in pts] for ln, pts in tf["fronts"].items()}
    lo = sum(min(b for _, b, _ in pts) for pts in fr.values())
    fastest = A.choose_under_budget(fr, 1 << 62)
    tensors = {}
    out = []
    for label, budget in (("smallest", lo), ("midway", (lo + fastest[1]) // 2), ("fastest", fastest[1])):
        u_pred, b_sel, choice = A.choose_under_budget(fr, budget)
        log(f"budget {label}: {budget / 1e6:.3f} MB -> predicted {u_pred:.2f} us, {b_sel / 1e6:.3f} MB")
        launches, words, bound, stored_b = [], 0, 0.0, 0
        checks, xhost = [], {}
        for ln, ch in choice.items():
            members = []
            for n, p in ch.items():
                if n not in tensors:
                    tensors[n] = E.config2_tensor(n)
                t = tensors[n]
                c = ecw.Coding(ecw.INT_CODES, *t.codes.shape, p["k"], 4, p["log2_m"], p["tile_cols"],
                               stored_tuples=p.get("stored_tuples", 0))
                tab = ecw.build_tables(c, t.codes)
                blob = ecw.encode(c, t.codes, t.scales, tab)
                tt = ecw.prepare(blob)
                words += tt.bytes_words
                stored_b += tt.bytes_words + tt.bytes_raw + tt.bytes_tile_meta + tt.bytes_tables + tt.bytes_scales
                bound += A.size_lower_bound_bytes(tab)
                members.append((blob, (p["waves_per_block"], p["tiles_per_wave"], p["streams_per_wave"],
                                       p["row_groups_per_block"])))
                checks.append((ln, len(members) - 1, n))
            xh = tensors[next(iter(ch))].x          # the launch's activations: its first member's
            launches.append((ln, members, torch.from_numpy(xh).cuda()))
            xhost[ln] = xh
        us, ys = time_cold(launches, 1, steps, cold_bytes)
        worst = 0.0
        for ln, i, n in checks:
            worst = max(worst, check_all(ys[ln][i], int_values(tensors[n]), xhost[ln].astype(np.float64)))
        out.append({"label": label, "budget_bytes": int(budget), "stored_bytes": int(stored_b),
                    "predicted_us_warm": round(u_pred, 3), "measured_us_cold": round(sum(us.values()), 3),
                    "per_launch_us": {k: round(v, 3) for k, v in us.items()},
                    "payload_words_bytes": int(words), "payload_lower_bound_bytes": int(bound),
                    "words_over_bound": round(words / bound, 5), "parity_worst_err_over_bound": worst,
                    "codings": {n: {k: p.get(k, 0) for k in ("k", "stored_tuples", "log2_m", "tile_cols", "waves_per_block",
                                                      "tiles_per_wave", "streams_per_wave",
                                                      "row_groups_per_block")}
                                for ch in choice.values() for n, p in ch.items()}})
        log(f"  measured {out[-1]['measured_us_cold']:.2f} us cold, words/bound {out[-1]['words_over_bound']:.4f}")
    return {"workload": "the INT4 layer set under byte budgets (one grouping per launch from the tune file's "
                        "Pareto fronts)", "front_points": {ln: len(p) for ln, p in fr.items()}, "points": out}


def dequant_gemm(steps: int, cold_bytes: float):
    """Products with more than four activation rows: the dequantising decode writes the
    dense fp16 / bf16 weights (HBM: the stored bytes read, 2 bytes per weight
    written), then the library GEMM (hipBLASLt through torch.mm, fp32 output) reads
    them.  Timed cold (copies rotated over >= cold_bytes), per call, for the INT4 gate
    tensor in its tune-file coding and the BF16 gate tensor as exponent pairs; the
    dense GEMM alone on resident weights is timed beside it.  Every dense weight is
    checked bit for bit against float64 values rounded in numpy."""
    import torch
    import ecw_inputs as E
    import entropy_coded_weight_amd as ecw
    coding, _ = load_coding(TUNE_FILE)
    out = {}
    t_int = E.config2_tensor("gate")
    t_bf = E.config3_tensor("gate")
    kk, m, tc, *_, T = coding["gate"]
    specs = [("int4_gate", ecw.Coding(ecw.INT_CODES, *t_int.codes.shape, kk, 4, m, tc, stored_tuples=T), t_int.codes,
              t_int.scales, torch.float16),
             ("bf16_gate", ecw.Coding(ecw.BF16_EXP, *t_bf.bits.shape, 2, 0, 11, 128), t_bf.bits, None, torch.bfloat16)]
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(reps):
                fn(r)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (3 * reps)

    for label, c, w, sc, tdt in specs:
        blob = ecw.encode(c, w, sc)
        t = ecw.prepare(blob)
        stored = t.bytes_words + t.bytes_raw + t.bytes_tile_meta + t.bytes_tables + t.bytes_scales
        n, k = w.shape
        copies = max(2, int(np.ceil(cold_bytes / (stored + 2 * n * k))))
        cts = [ecw.CompressedTensor(blob) for _ in range(copies)]
        dense = [torch.empty((n, k), dtype=tdt, device="cuda") for _ in range(copies)]
        us_deq = timed(lambda r: cts[r % copies].dequantize(tdt, out=dense[r % copies]), max(copies, steps // 4))
        got = dense[0].view(torch.int16).cpu().numpy().view(np.uint16)
        if label.startswith("int4"):
            want = (w.astype(np.float64) * sc.astype(np.float64)[:, None]).astype(np.float16).view(np.uint16)
        else:
            want = w
        exact = bool(np.array_equal(got, want))
        d = {"dequant_us": round(us_deq, 3), "stored_bytes": int(stored), "dense_bytes": int(2 * n * k),
             "dequant_gbps": round((stored + 2 * n * k) / (us_deq * 1e-6) / 1e9, 1),
             "dequant_hbm_frac": round((stored + 2 * n * k) / (us_deq * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
             "dense_bits_exact": exact, "gemm": {}}
        for batch in (16, 256):
            x = torch.randn((batch, k), dtype=tdt, device="cuda")
            us_mm = timed(lambda r: torch.mm(x, dense[r % copies].t(), out_dtype=torch.float32),
                          max(copies, steps // 4))
            us_all = timed(lambda r: cts[r % copies].gemm(x, w_buf=dense[r % copies]), max(copies, steps // 4))
            d["gemm"][f"batch{batch}"] = {"dequant_plus_gemm_us": round(us_all, 3), "gemm_only_us": round(us_mm, 3)}
        log(f"dequant {label}: {us_deq:.2f} us ({d['dequant_gbps']:.0f} GB/s, {100 * d['dequant_hbm_frac']:.1f}% "
            f"of HBM), exact={exact}; " + ", ".join(f"{b}: {v['dequant_plus_gemm_us']:.1f} us (GEMM alone "
                                                    f"{v['gemm_only_us']:.1f})" for b, v in d["gemm"].items()))
        out[label] = d
        del cts, dense
    out["workload"] = ("gate 14336x4096: INT4 Laplacian codes (tune-file coding) to fp16, BF16 exponent pairs "
                       "(M = 2^11, 128-wide tiles) to bf16; GEMM batch 16 and 256, fp32 output")
    return out


def summarize_rocprof(directory: str):
    """Print per-(kernel, grid size) averages from rocprofv3 CSV output under
    `directory`: kernel durations from *_kernel_trace.csv and counter values from
    *_counter_collection.csv (one line per kernel and counter)."""
    import csv
    import collections
    import glob
    for path in sorted(glob.glob(os.path.join(directory, "**", "*_kernel_trace.csv"), recursive=True)):
        d = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"].split("(")[0], int(r["Grid_Size_X"]))
            d[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print(f"# kernel durations from {os.path.relpath(path, directory)}")
        print(f"{'kernel':48s} {'grid':>8s} {'calls':>6s} {'avg_us':>9s} {'median_us':>9s} {'min_us':>8s}")
        for (k, g), v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
            v.sort()
            print(f"{k[:48]:48s} {g:8d} {len(v):6d} {sum(v) / len(v):9.2f} {v[len(v) // 2]:9.2f} {v[0]:8.2f}")
    for path in sorted(glob.glob(os.path.join(directory, "**", "*_counter_collection.csv"), recursive=True)):
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for r in csv.DictReader(open(path)):
            per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = (r["Kernel_Name"].split("(")[0], int(r["Grid_Size"]))
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for did, cs in per.items():
            for c, v in cs.items():
                agg[names[did]][c].append(v)
        print(f"# counters from {os.path.relpath(path, directory)} (mean per dispatch)")
        for (k, g), cs in sorted(agg.items()):
            for c, v in sorted(cs.items()):
                print(f"{k[:48]:48s} {g:8d} {c:24s} n={len(v):4d} {sum(v) / len(v):16.1f}")


def measured_traffic(path: str):
    """HBM bytes per launch of the dominant launch from a committed profile record,
    valid only while the kernel source and tune file hash to what was profiled."""
    import hashlib
    if not os.path.exists(path):
        return None
    rec = dict(l.split("=", 1) for l in open(path).read().split("\n") if "=" in l and not l.startswith("#"))
    rec = {k.strip(): v.strip() for k, v in rec.items()}
    def sha(p):
        return hashlib.sha256(open(os.path.join(ROOT, p), "rb").read()).hexdigest()
    if rec.get("kernel_sha256") != sha("entropy_coded_weight_amd/csrc/ecw_kernels.hip"):
        return None
    if rec.get("tune_sha256") != sha(os.path.relpath(TUNE_FILE, ROOT)):
        return None
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-bytes", type=float, default=512e6)
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="after timing, run N plain device copies of 64 MiB (a kernel of known "
                         "traffic that scales the profiler's FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--tune", action="store_true",
                    help="autotune every tensor on this device first and rewrite the tune file")
    ap.add_argument("--tune-file", default=TUNE_FILE)
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="print per-launch averages of rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--configs", default="1,3,4,5,p,d",
                    help="secondary workloads measured after the layer set (1: Gaussian codes, "
                         "3: BF16 exponent coding, 4: FP8 layer at batch 1 and 4, 5: E8 lattice "
                         "fields, INT8 and FP8 reconstruction, p: the layer set under byte budgets "
                         "from the tune file's Pareto fronts, d: dequantising decode + GEMM for "
                         "batches above 4); '' for none")
    ap.add_argument("--lm-head", action="store_true",
                    help="include the 128256x4096 LM head in workload 4 (its generation takes minutes)")
    ap.add_argument("--tensors", default=",".join(ORDER),
                    help="subset of the layer to run (profiling); the JSON line is only "
                         "meaningful for the full set")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the kernel measured here is one GPU's share; sharding over GPUs is not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import entropy_coded_weight_amd as ecw

    ORDER[:] = [n for n in ORDER if n in args.tensors.split(",")]
    global LAUNCHES
    LAUNCHES = [(ln, [n for n in names if n in ORDER]) for ln, names in LAUNCHES]
    LAUNCHES = [(ln, names) for ln, names in LAUNCHES if names]
    dev = torch.device("cuda:0")
    if args.tune:
        run_tuner(args.tune_file, args.batch)
    coding, coding_src = load_coding(args.tune_file)
    t_build = time.time()
    layer = build_layer(args.batch, coding)
    log(f"encoded layer set in {time.time() - t_build:.1f} s (codings: {coding_src})")
    stored = {}
    for name in ORDER:
        stored[name] = ecw.prepare(layer[name]["blob"]).blob_bytes
    layer_bytes = 0
    for name in ORDER:
        t = ecw.prepare(layer[name]["blob"])
        stored[name] = t.bytes_words + t.bytes_raw + t.bytes_tile_meta + t.bytes_tables + t.bytes_scales
        layer_bytes += stored[name]
    copies = max(2, int(np.ceil(args.cold_bytes / layer_bytes)))
    cts = []
    for _ in range(copies):
        c = {n: ecw.CompressedTensor(layer[n]["blob"]) for n in ORDER}
        for n in ORDER:
            c[n].set_launch(*layer[n]["launch"])
        cts.append(c)
    groups = [{ln: ecw.GemvGroup([c[n] for n in names]) for ln, names in LAUNCHES} for c in cts]
    xs, ys = {}, {}
    for ln, names in LAUNCHES:
        xs[ln] = torch.from_numpy(layer[names[0]]["tensor"].x).to(dev)
        for n in names:
            ys[n] = torch.empty((args.batch, layer[n]["tensor"].codes.shape[0]), dtype=torch.float32, device=dev)
    wss = [{ln: g[ln].workspace(args.batch) for ln, _ in LAUNCHES} for g in groups]

    def launch(i, ln, names):
        c = i % copies
        ecw.gemv_group_raw([cts[c][n].t for n in names], xs[ln], [ys[n] for n in names], wss[c][ln])

    def step(i):
        for ln, names in LAUNCHES:
            launch(i, ln, names)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # One HIP graph per rotated copy: each replay is one full step (all launches of
    # the layer set, in order), so the timed loop measures device time, not the
    # Python launch loop.
    graphs = []
    for c in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(c)
        graphs.append(g)
    for c in range(copies):
        graphs[c].replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        graphs[i % copies].replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps

    # Per-launch device time: a graph of that launch over all rotated copies, timed
    # with events on the launch stream around replays.
    avg_us = {}
    for ln, names in LAUNCHES:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(copies):
                launch(c, ln, names)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = max(1, args.steps // (4 * copies))
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        avg_us[ln] = e0.elapsed_time(e1) * 1e3 / (reps * copies)     # us per launch

    # parity on the timed blobs: every row of every tensor against float64, with the
    # activations its launch used
    worst = 0.0
    for ln, names in LAUNCHES:
        xv = layer[names[0]]["tensor"].x.astype(np.float64)
        for name in names:
            t = layer[name]["tensor"]
            wr = check_all(ys[name].cpu().numpy(), int_values(t), xv)
            worst = max(worst, wr)
            if not wr <= 1.0:
                log(f"PARITY FAILURE on {name}: worst err/bound {wr}")
                sys.exit(1)

    n_weights = sum(layer[n]["tensor"].codes.size for n in ORDER)
    us_layer = ms_step * 1e3
    gbs = layer_bytes / (us_layer * 1e-6) / 1e9
    unc_bytes = sum(layer[n]["tensor"].codes.size * 0.5 + layer[n]["tensor"].codes.shape[0] * 2 for n in ORDER)
    launch_bytes = {}
    for ln, names in LAUNCHES:
        launch_bytes[ln] = sum(stored[n] + layer[n]["tensor"].codes.shape[0] * 4 * args.batch for n in names) \
            + layer[names[0]]["tensor"].x.size * 2
    dom = max(avg_us, key=lambda ln: avg_us[ln])
    achieved = launch_bytes[dom] / (avg_us[dom] * 1e-6) / 1e9
    # measured HBM traffic of that launch (calibrated rocprofv3 FETCH_SIZE + WRITE_SIZE),
    # if the committed record still describes this kernel and these codings
    dom_names = dict(LAUNCHES)[dom]
    dom_label = (f"k_decode<INT4, {layer[dom_names[0]]['coding'].weights_per_symbol} codes/symbol>"
                 + f" (launch {dom}: {'+'.join(dom_names)})")
    rec = measured_traffic(TRAFFIC_FILE) if args.tune_file == TUNE_FILE and args.batch == 1 else None
    traffic = int(rec["traffic_bytes"]) if rec and rec.get("launch") == dom else None
    for n in ORDER:
        c = layer[n]["coding"]
        log(f"{n:5s} {layer[n]['tensor'].codes.shape} k={c.weights_per_symbol} t={c.stored_tuples} "
            f"m={c.log2_m} tc={c.tile_cols} "
            f"launch={layer[n]['launch']} stored={stored[n] / 1e6:.3f} MB")
    for ln, names in LAUNCHES:
        log(f"launch {ln:8s} avg={avg_us[ln]:.2f} us  {launch_bytes[ln] / (avg_us[ln] * 1e-6) / 1e9:.0f} GB/s")
    out = {
        "metric": METRIC, "value": round(us_layer, 3), "unit": "us/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "u32 decode + f32 accumulate", "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped layer set (q,k,v,o,gate,up,down) of 16-level "
                               "Laplacian codes (H=2.2 bits), autotuned codes per rANS symbol, fp16 row "
                               "scales, fp16 x, batch 1, cold cache; 4 launches per step "
                               "(q/k/v, o, gate/up, down)",
                   "batch": args.batch, "copies_rotated": copies, "codings_from": coding_src,
                   "codings": {n: dict(k=layer[n]["coding"].weights_per_symbol,
                                       stored_tuples=layer[n]["coding"].stored_tuples,
                                       log2_m=layer[n]["coding"].log2_m,
                                       tile_cols=layer[n]["coding"].tile_cols,
                                       waves_per_block=layer[n]["launch"][0],
                                       tiles_per_wave=layer[n]["launch"][1],
                                       streams_per_wave=layer[n]["launch"][2],
                                       row_groups_per_block=layer[n]["launch"][3]) for n in ORDER}},
        "stored_bytes_per_layer": int(layer_bytes),
        "stored_bits_per_weight": round(layer_bytes * 8 / n_weights, 4),
        "gbps_compressed": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "gbps_uncompressed_equiv": round(unc_bytes / (us_layer * 1e-6) / 1e9, 1),
        "per_launch_us": {ln: round(v, 3) for ln, v in avg_us.items()},
        "host_wall_s": round(host_s, 3),
        "parity_worst_err_over_bound": worst,
        "roofline": {"bound": "hbm", "kernel": dom_label,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": int(launch_bytes[dom]), "avg_launch_us": round(avg_us[dom], 3)},
    }
    # roofline probes on this device: achievable streaming-read rate (2 GiB buffer)
    # and dependent LDS table lookups (the decode's table reads), all CUs busy
    big = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    achievable = ecw.probe_stream_read(big)
    del big
    lut_rate = {f"m{m}_{eb}B": round(ecw.probe_lds_lookup(m, eb) / 1e9, 1) for m in (11, 12) for eb in (4, 8)}
    # the decode loop is bound by instruction issue, not HBM: the same launch against
    # the chip's VALU issue rate (256 CUs x 4 SIMDs, one wave64 VALU instruction per
    # SIMD every 4 clocks at 2.4 GHz), from the VALU instruction count rocprofv3
    # measured for this kernel and these codings
    if rec and rec.get("valu_instructions") and rec.get("launch") == dom:
        valu = float(rec["valu_instructions"])
        peak_g = 256 * 4 * 2.4e9 / 4 / 1e9
        out["issue_roofline"] = {"bound": "alu", "kernel": dom_label,
                                 "achieved": round(valu / (avg_us[dom] * 1e-6) / 1e9, 1), "peak": peak_g,
                                 "unit": "G wave64 VALU instructions/s",
                                 "frac": round(valu / (avg_us[dom] * 1e-6) / 1e9 / peak_g, 4),
                                 "valu_instructions_per_launch": int(valu)}
    out["probes"] = {"hbm_read_gbs": round(achievable, 1),
                     "hbm_read_frac_of_peak": round(achievable / HBM_PEAK_GBS, 4),
                     "dominant_launch_frac_of_achievable": round(achieved / achievable, 4),
                     "lds_lookups_g_per_s": lut_rate,
                     "decode_table_lookups_g_per_s": round(sum(layer[n]["tensor"].codes.size
                                                               // layer[n]["coding"].weights_per_symbol
                                                               for n in ORDER) / (us_layer * 1e-6) / 1e9, 1)}
    if args.calibrate_copy:
        src = torch.ones(64 << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.calibrate_copy):
            dst.copy_(src)
        torch.cuda.synchronize()
    if args.configs and args.tensors == ",".join(["q", "k", "v", "o", "gate", "up", "down"]):
        out["configs"] = secondary_configs(args.configs, args.steps, args.cold_bytes, args.lm_head)
        budget = out["configs"].pop("budget", None)
        deq = out["configs"].pop("dequant", None)
        if deq:
            out["dequant"] = deq
            if not all(v["dense_bits_exact"] for k, v in deq.items() if k != "workload"):
                log("PARITY FAILURE in the dequantising decode")
                sys.exit(1)
        if budget:
            out["budget"] = budget
            for pt in budget["points"]:
                if not pt["parity_worst_err_over_bound"] <= 1.0:
                    log(f"PARITY FAILURE in budget point {pt['label']}")
                    sys.exit(1)
        for k, v in out["configs"].items():
            log(f"config {k}: {v['us']:.2f} us, {v['gbps_compressed']:.0f} GB/s ({100 * v['hbm_frac']:.1f}% of HBM), "
                f"{v['stored_bits_per_weight']:.3f} bits/weight, parity {v['parity_worst_err_over_bound']:.3g}")
            if not v["parity_worst_err_over_bound"] <= 1.0:
                log(f"PARITY FAILURE in config {k}")
                sys.exit(1)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layer)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
