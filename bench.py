"""Benchmark: fused rANS decode + batch-1 GEMV over one Llama-3.1-8B-shaped layer set.

One step = one pass of the hot path over the seven linear layers of one transformer
block (q, k, v, o 4096x4096 / 1024x4096, gate/up 14336x4096, down 4096x14336), each
stored as 16-level Laplacian codes (2.2 bits of entropy), decoded and multiplied into
y = W x at batch 1, in the codings the tuner picked on MI355X (quads of codes over
stored 4-tuples for every tensor).  Launch order follows the block's data flow: q/k/v,
o, gate/up, down.  Blobs are rotated over >= 512 MB of copies (twice the 256 MiB
Infinity Cache), so every step reads its weights from HBM.  The steps of all rotated
copies are captured as one HIP graph, as a model's decode step holds its layers; the
timed region replays it (whole graphs, then single-step graphs for the remainder of
the K steps), and one graph per step is timed beside it (each step then also pays a
graph launch).  Timing also follows the MINE page's protocol (Section 4.2 "Tuning
Grid": median of 5 bursts of at least 400 us).

The other workloads are measured in the same run (under "configs"), in the codings
and launch shapes of a committed tune file (entropy_coded_weight_amd/tuned/): the
1024x1024 Gaussian-code matrix, BF16 exponent coding of the gate / down shapes, the
full 32-layer FP8 decode step with its 128256x4096 LM head at batch 1 and 4, and the
E8 lattice fields on both reconstruction routes.  The layer set with two codes per
symbol everywhere is timed beside the tuned one.

Prints one JSON line (stdout).  Per-tensor details go to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
N_CU, N_SIMD = 256, 1024
METRIC = "µs per fused decode-GEMV layer + effective weight GB/s (% HBM peak), batch 1"
ORDER = ["q", "k", "v", "o", "gate", "up", "down"]
# launches of one decode step, in data-flow order; tensors of a launch share x
LAUNCHES = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gate_up", ["gate", "up"]), ("down", ["down"])]

# per-tensor coding: (k, log2_m, tile_cols, waves_per_block, tiles_per_wave,
# streams_per_wave, row_groups_per_block, stored_tuples).  Used when no tune file
# exists; `--tune` measures every candidate on the device and writes TUNE_FILE.
DEFAULT_CODING = {"q": (2, 12, 128, 16, 1, 1, 1, 0), "k": (2, 12, 128, 16, 1, 1, 1, 0),
                  "v": (2, 12, 128, 16, 1, 1, 1, 0), "o": (2, 12, 128, 16, 1, 1, 1, 0),
                  "gate": (2, 12, 256, 16, 1, 1, 1, 0), "up": (2, 12, 256, 16, 1, 1, 1, 0),
                  "down": (2, 12, 256, 16, 1, 1, 1, 0)}
TUNED = os.path.join(ROOT, "entropy_coded_weight_amd", "tuned")
TUNE_FILE = os.path.join(TUNED, "llama8b_int4_laplace_batch1.json")
SECONDARY_TUNE_FILE = os.path.join(TUNED, "secondary_workloads.json")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_decode_llama8b_int4_gate_up_traffic.txt")
COUNTER_FILE = os.path.join(ROOT, "profiles", "k_decode_all_workloads_counters.txt")
KERNEL_SRC = "entropy_coded_weight_amd/csrc/ecw_kernels.hip"
# rocprofv3 counter passes for the per-workload counter record (at most 8 SQ
# counters per pass)
COUNTER_SETS = [
    "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS "
    "SQ_WAVE_CYCLES",
    "SQ_WAIT_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
    "SQ_INSTS_BRANCH SQ_ACTIVE_INST_SCA",
]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sha256(path: str) -> str:
    import hashlib
    return hashlib.sha256(open(os.path.join(ROOT, path), "rb").read()).hexdigest()


def pick_tuple(p: dict):
    return (p["k"], p["log2_m"], p["tile_cols"], p["waves_per_block"], p["tiles_per_wave"],
            p.get("streams_per_wave", 1), p.get("row_groups_per_block", 1), p.get("stored_tuples", 0))


def load_coding(path: str):
    if not os.path.exists(path):
        return dict(DEFAULT_CODING), "defaults"
    with open(path) as f:
        d = json.load(f)
    coding = dict(DEFAULT_CODING)
    for n, p in d["picks"].items():
        coding[n] = pick_tuple(p)
    return coding, os.path.relpath(path, ROOT)


def k2_coding(path: str):
    """The layer set with two codes per symbol everywhere: per launch, the common
    waves-per-block value whose members' fastest two-code candidates (as the tune
    file ranks them) sum to the least time; each member at its fastest two-code
    (M, tile width, launch shape) at that value."""
    with open(path) as f:
        cands = json.load(f)["candidates"]
    coding = {}
    for ln, names in LAUNCHES:
        best = None
        for W in (4, 8, 16):
            tot, ch = 0.0, {}
            for n in names:
                opts = []
                for c in cands[n]:
                    if c["k"] != 2:
                        continue
                    for key, us in c["shapes"].items():
                        w, r, ns, p = (int(v) for v in key.split("x"))
                        if w == W:
                            opts.append((us, c["stored_bytes"], (2, c["log2_m"], c["tile_cols"], w, r, ns, p, 0)))
                if not opts:
                    tot = math.inf
                    break
                us, _, cd = min(opts)
                tot += us
                ch[n] = cd
            if best is None or tot < best[0]:
                best = (tot, ch)
        coding.update(best[1])
    return coding


def run_tuner(path: str, batch: int):
    """Autotune every tensor of the layer set (k in {1, 2, 4} with quads over stored
    tuples, M in {2^10, 2^11, 2^12}, tile width in {64..512}, waves per block, tiles
    per wave, row streams per wave, row groups per block) and write the picks."""
    import torch
    import ecw_inputs as E
    from entropy_coded_weight_amd import autotune as A, INT_CODES
    cands, specs, xs, ts = {}, {}, {}, {}
    for name in ORDER:
        ts[name] = E.config2_tensor(name, layer=0, batch=batch)
    # stored tuples of the quad codings: the page's t search per launch (MINE page,
    # Section 4.2 "Tuning t"), at each table size; each tensor is then timed at the t
    # values of the search's first selections (the byte-optimal one and the next
    # rounds of <= 1% more bytes)
    quad_ts = {n: {} for n in ORDER}
    t_trace = {}
    for ln, names in LAUNCHES:
        for m in A.DEFAULT_LOG2_M:
            curves = {n: A.t_curve(ts[n].codes, ts[n].scales, m, 256) for n in names}
            sels = A.t_search(curves)[:4]
            t_trace.setdefault(ln, {})[str(m)] = sels
            for n in names:
                quad_ts[n][m] = tuple(sorted({s[n] for s in sels}))
        log(f"t search {ln}: " + "; ".join(f"M=2^{m}: {v}" for m, v in t_trace[ln].items()))
    for name in ORDER:
        t = ts[name]
        xs[name] = torch.from_numpy(t.x).cuda()
        specs[name] = (INT_CODES, t.codes, t.scales, 4)
        log(f"tuning {name} {t.codes.shape}")
        cands[name] = A.tune_tensor(INT_CODES, t.codes, t.scales, xs[name], code_bits=4, ks=(1, 2, 4), log=log,
                                    quad_ts=quad_ts[name])
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
                   "t_search": t_trace, "candidates": table}, f, indent=1)
    log(f"wrote {path}")


def build_layer(batch: int, coding: dict, tensors: dict | None = None):
    import ecw_inputs as E
    import entropy_coded_weight_amd as ecw
    layer = {}
    for name in ORDER:
        t = tensors[name] if tensors else E.config2_tensor(name, layer=0, batch=batch)
        kk, m, tc, W, R, NS, RPB, T = coding[name]
        n, k = t.codes.shape
        c = ecw.Coding(ecw.INT_CODES, n, k, kk, 4, m, tc, stored_tuples=T)
        blob = ecw.encode(c, t.codes, t.scales)
        layer[name] = dict(tensor=t, coding=c, blob=blob, launch=(W, R, NS, RPB))
    return layer


# ------------------------------------------------------------------ CPU baseline
def host_description():
    import platform
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [dict(api=i.get("internal_api"), threads=i.get("num_threads")) for i in threadpool_info()]
    except Exception:        # threadpoolctl missing: report nothing rather than guess
        blas = []
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "numpy": np.__version__, "blas": blas}


_CPU_SAMPLE = None


def _oracle_pass(idx):
    """Oracle decode + float64 GEMV of the sample items idx: (seconds, symbols)."""
    from oracle import gemv as G, pipeline as P
    done, t_used = 0, 0.0
    for i in idx:
        comp, ocd, scales, x = _CPU_SAMPLE[i]
        t0 = time.perf_counter()
        q = P.decode(comp)
        wv = P.weight_values(ocd, q, scales)
        G.gemv_f64(wv, G.x_values(x, "f16"))
        t_used += time.perf_counter() - t0
        done += q.size // ocd.k
    return t_used, done


def _worker_pass(idx):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        _, done = _oracle_pass(idx)
        return time.perf_counter() - t0, done


def cpu_baseline(layer, per_core_s: float = 1.5, max_workers: int = 16):
    """The oracle (numpy decode + float64 GEMV) on whole 64-row groups of the layer
    set, timed on the host: one core (BLAS limited to one thread) and all cores (one
    forked process per core over disjoint row groups, one BLAS thread each); one
    warm-up, then the median of 3 passes, scaled to one full layer by symbol count.
    The sampled row groups are encoded by the oracle first (untimed).  Runs before
    the GPU is touched, so the forked processes hold no device state."""
    global _CPU_SAMPLE
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    from oracle import pipeline as P
    total_syms = sum(layer[n]["tensor"].codes.size // layer[n]["coding"].weights_per_symbol for n in ORDER)
    workers = max(1, min(max_workers, os.cpu_count() or 1))

    def sample_items(n_items, start):
        items, rg = [], start
        while len(items) < n_items:
            name = ORDER[rg % len(ORDER)]
            t = layer[name]["tensor"]
            c = layer[name]["coding"]
            n, K = t.codes.shape
            r0 = ((rg // len(ORDER)) * 64) % n
            r1 = min(r0 + 64, n)
            ocd = P.Coding(P.INT_CODES, r1 - r0, K, k=c.weights_per_symbol, code_bits=4, log2_m=c.log2_m,
                           tile_cols=c.tile_cols, stored_tuples=c.stored_tuples)
            items.append((P.encode(ocd, t.codes[r0:r1], t.scales[r0:r1]), ocd, t.scales[r0:r1], t.x))
            rg += 1
        return items

    # size one core's sample to about per_core_s per pass
    _CPU_SAMPLE = sample_items(len(ORDER), 0)
    with threadpool_limits(limits=1):
        s1, _ = _oracle_pass(range(len(_CPU_SAMPLE)))
    n_items = max(len(ORDER), int(len(ORDER) * per_core_s / max(s1, 1e-3)))
    _CPU_SAMPLE = _CPU_SAMPLE + sample_items(workers * n_items - len(_CPU_SAMPLE), len(_CPU_SAMPLE))
    one_idx = list(range(n_items))
    with threadpool_limits(limits=1):
        runs = [_oracle_pass(one_idx) for _ in range(4)][1:]
    t1 = sorted(r[0] for r in runs)[1]
    syms1 = runs[0][1]
    shares = [list(range(w * n_items, (w + 1) * n_items)) for w in range(workers)]
    with mp.get_context("fork").Pool(workers) as pool:
        walls = []
        for _ in range(4):
            t0 = time.perf_counter()
            res = pool.map(_worker_pass, shares, chunksize=1)
            walls.append((time.perf_counter() - t0, sum(r[1] for r in res)))
    tn = sorted(w[0] for w in walls[1:])[1]
    symsn = walls[1][1]
    _CPU_SAMPLE = None
    us_one = t1 / syms1 * total_syms * 1e6
    us_all = tn / symsn * total_syms * 1e6
    return {"value": round(us_all, 1), "unit": "us/layer", "cores": workers, "kind": "oracle",
            "one_core_us_per_layer": round(us_one, 1),
            "host": host_description(),
            "sample": f"{workers} processes x {n_items} whole 64-row groups drawn round-robin from the 7 tensors "
                      f"({symsn} symbols per pass; one core: {n_items} groups, {syms1} symbols): numpy decode + "
                      f"float64 GEMV, one BLAS thread per process; one warm-up, median of 3 passes "
                      f"({tn:.2f} s all cores, {t1:.2f} s one core), scaled to the full layer by symbol count"}


# ------------------------------------------------------------------ parity
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


# ------------------------------------------------------------------ timing
def time_cold(launches, batch: int, steps: int, cold_bytes: float):
    """Cold device timing of grouped launches (autotune.time_cold: median of 5 bursts)."""
    from entropy_coded_weight_amd import autotune as A
    return A.time_cold(launches, batch, steps, cold_bytes)


def stored_of(t) -> int:
    return t.bytes_words + t.bytes_raw + t.bytes_tile_meta + t.bytes_tables + t.bytes_scales


def kernel_sig(c, batch: int, x_bf16: bool) -> str:
    """The fused kernel's template arguments for a coding (PAY, CB, KW, B, MAT, XBF)."""
    cb = c.code_bits if c.payload == 1 else (1 if c.payload == 4 and c.recon_dtype == 5 else 0)
    # the fused kernels are built per activation type only where they multiply packed
    # 16-bit pairs (INT with several codes per symbol, BF16); the others stage fp32
    xbf = x_bf16 and ((c.payload == 1 and c.weights_per_symbol >= 2) or c.payload == 2)
    return f"k_decode<{c.payload}, {cb}, {c.weights_per_symbol}, {1 if batch == 1 else 4}, false, " \
           f"{'true' if xbf else 'false'}>"


LAUNCH_MAP = {}      # row -> launch -> [kernel template, grid threads, block threads, symbols, LDS bytes]


def launch_symbols(ts) -> int:
    """rANS symbols a grouped launch decodes (E8: 9 per block of 8 weights)."""
    n = 0
    for t in ts:
        c = t.coding
        n += c.rows * (c.cols // 8 * 9 if c.payload == 4 else c.cols // max(1, c.weights_per_symbol))
    return n


LAUNCH_KEYS = {}     # launch key (launch_key) -> [(row, launch), ...] registered by note_launch
DISPATCH_LOG = None  # profiling runs: {"keys": [launch key, ...], "log": [key index per fused dispatch]}


def launch_key(ts, batch: int, x_bf16: bool):
    """What identifies a grouped launch: the kernel template, and each member's coding
    and launch shape."""
    return (kernel_sig(ts[0].coding, batch, x_bf16),
            tuple((t.coding.payload, t.coding.rows, t.coding.cols, t.coding.weights_per_symbol, t.coding.log2_m,
                   t.coding.tile_cols, t.coding.stored_tuples, t.coding.recon_dtype, t.waves_per_block,
                   t.tiles_per_wave, t.streams_per_wave, t.row_groups_per_block) for t in ts))


def note_launch(row: str, launch: str, ts, batch: int, x_bf16: bool):
    """Record how the profiler's dispatches of a launch are recognised: the kernel
    template and the grid, block and LDS sizes the library reports for it, and the
    launch key the dispatch log uses."""
    import entropy_coded_weight_amd as ecw
    grid, block, lds = ecw.group_geometry(ts, batch, ecw.DT_BF16 if x_bf16 else ecw.DT_F16)
    LAUNCH_MAP.setdefault(row, {})[launch] = [kernel_sig(ts[0].coding, batch, x_bf16), grid, block,
                                              launch_symbols(ts), lds]
    owners = LAUNCH_KEYS.setdefault(launch_key(ts, batch, x_bf16), [])
    if [row, launch] not in owners:
        owners.append([row, launch])


def install_dispatch_log():
    """Profiling runs: log the launch of every fused decode-GEMV dispatch in the order
    it reaches the GPU (eager calls, and each graph replay expanded into the launches
    its capture recorded).  Profiler records are then attributed to launches by
    dispatch order, which also separates launches of one kernel with the same grid."""
    global DISPATCH_LOG
    import torch
    import entropy_coded_weight_amd as ecw
    DISPATCH_LOG = {"keys": [], "ids": {}, "log": []}
    state = {"capture": None}

    def record(ts, x):
        if not any(t.coding.rows and t.n_tiles for t in ts):
            return                                   # no decode kernel (K = 0: a fill)
        key = launch_key(ts, x.shape[0], x.dtype == torch.bfloat16)
        i = DISPATCH_LOG["ids"].get(key)
        if i is None:
            i = DISPATCH_LOG["ids"][key] = len(DISPATCH_LOG["keys"])
            DISPATCH_LOG["keys"].append(key)
        (state["capture"] if state["capture"] is not None else DISPATCH_LOG["log"]).append(i)

    group_raw, single_raw = ecw.gemv_group_raw, ecw.gemv_raw

    def gemv_group_raw(ts, x, ys, workspace, stream=None):
        group_raw(ts, x, ys, workspace, stream)
        record(list(ts), x)

    def gemv_raw(t, x, y, workspace, stream=None):
        single_raw(t, x, y, workspace, stream)
        record([t], x)

    ecw.gemv_group_raw, ecw.gemv_raw = gemv_group_raw, gemv_raw

    class LoggedGraph(torch.cuda.CUDAGraph):
        def capture_begin(self, *a, **k):
            self._launches = []
            state["capture"] = self._launches
            return super().capture_begin(*a, **k)

        def capture_end(self):
            try:
                return super().capture_end()
            finally:
                state["capture"] = None

        def replay(self):
            super().replay()
            DISPATCH_LOG["log"].extend(getattr(self, "_launches", []))

    torch.cuda.CUDAGraph = LoggedGraph


def write_dispatch_log(path: str):
    """The dispatch log beside the launch map: per logged launch key its (row, launch)
    owners, then one key index per fused dispatch."""
    keys = [LAUNCH_KEYS.get(k, []) for k in DISPATCH_LOG["keys"]]
    with open(path, "w") as f:
        json.dump({"owners": keys, "log": DISPATCH_LOG["log"]}, f)


FUSED_KERNEL = re.compile(r"k_decode<\d+, \d+, \d+, \d+, false, (?:true|false)>")


def attribute_dispatches(rows: dict, lm: dict, log_path: str):
    """(row, launch) owners of every fused decode-GEMV dispatch of a profiler CSV.
    rows: Dispatch_Id -> (kernel name, grid, block, LDS).  With the run's dispatch log
    (same number of fused dispatches) the n-th dispatch belongs to the n-th logged
    launch; otherwise dispatches are matched by kernel, grid, block and LDS."""
    fused = sorted((d for d, r in rows.items() if FUSED_KERNEL.search(r[0])), key=int)
    if log_path and os.path.exists(log_path):
        lg = json.load(open(log_path))
        if len(lg["log"]) == len(fused):
            return {d: [tuple(o) for o in lg["owners"][i]] for d, i in zip(fused, lg["log"])}, "dispatch order"
        log(f"dispatch log {log_path}: {len(lg['log'])} launches against {len(fused)} fused dispatches; "
            "matching by kernel, grid and LDS")
    return {d: dispatch_launches(lm, *rows[d]) for d in fused}, "kernel, grid and LDS"


def dispatch_launches(lm: dict, kname: str, grid: int, wg: int, lds: int) -> list:
    """The (row, launch) pairs of the launch map a profiled dispatch belongs to: same
    kernel template, grid and block size; where several launches share those, the one
    whose LDS size is nearest the dispatch's (launches of every row that match equally
    well are all returned, so repeated workloads pool their dispatches)."""
    cands = [(row, ln, e[4] if len(e) > 4 else None) for row, launches in lm.items()
             for ln, e in launches.items() if e[1] == grid and e[2] == wg and e[0] in kname]
    if not cands:
        return []
    if any(c[2] is None for c in cands) or lds is None:
        return [(r, ln) for r, ln, _ in cands]
    best = min(abs(c[2] - lds) for c in cands)
    return [(r, ln) for r, ln, l in cands if abs(l - lds) == best]


def bytes_row(us: float, stored: int, unc: float) -> dict:
    """compressed and uncompressed-equivalent GB/s of a workload timed at `us`."""
    g = stored / (us * 1e-6) / 1e9
    gu = unc / (us * 1e-6) / 1e9
    return {"gbps_compressed": round(g, 1), "hbm_frac": round(g / HBM_PEAK_GBS, 4),
            "gbps_uncompressed_equiv": round(gu, 1), "uncompressed_equiv_frac": round(gu / HBM_PEAK_GBS, 4)}


# ------------------------------------------------------------------ the layer set (headline)
def time_layer_set(layer, batch: int, steps: int, warmup: int, cold_bytes: float, row: str, clock=None):
    """Cold timing of the layer set `layer` (grouped launches per LAUNCHES): K timed
    steps (the benchmark's contract), the step by the burst protocol, and each launch
    alone (a graph of that launch over all rotated copies, burst protocol).  Returns
    (results, ys of the last step, launch bytes)."""
    import torch
    import entropy_coded_weight_amd as ecw
    from entropy_coded_weight_amd import autotune as A
    dev = torch.device("cuda:0")
    stored, layer_bytes = {}, 0
    for name in ORDER:
        stored[name] = stored_of(ecw.prepare(layer[name]["blob"]))
        layer_bytes += stored[name]
    copies = max(2, int(np.ceil(cold_bytes / layer_bytes)))
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
            ys[n] = torch.empty((batch, layer[n]["tensor"].codes.shape[0]), dtype=torch.float32, device=dev)
        note_launch(row, ln, [cts[0][n].t for n in names], batch, False)
    wss = [{ln: g[ln].workspace(batch) for ln, _ in LAUNCHES} for g in groups]

    def launch(i, ln, names):
        c = i % copies
        ecw.gemv_group_raw([cts[c][n].t for n in names], xs[ln], [ys[n] for n in names], wss[c][ln])

    def step(i):
        for ln, names in LAUNCHES:
            launch(i, ln, names)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # the steps of all rotated copies in one HIP graph, as a model's decode step holds
    # its layers (one graph launch per `copies` layers); beside it one graph per step,
    # which adds a graph launch to every step
    stack = torch.cuda.CUDAGraph()
    with torch.cuda.graph(stack):
        for c in range(copies):
            step(c)
    graphs = []
    for c in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(c)
        graphs.append(g)
    stack.replay()
    for c in range(copies):
        graphs[c].replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(run):
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        t_start.record(stream)
        run()
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / steps, time.perf_counter() - h0

    def k_steps_stacked():
        # exactly `steps` steps: whole stacks, then single steps for the remainder
        for _ in range(steps // copies):
            stack.replay()
        for c in range(steps % copies):
            graphs[c].replay()

    def k_steps_single():
        for i in range(steps):
            graphs[i % copies].replay()

    ms_step, host_s = timed(k_steps_stacked)
    ms_single, _ = timed(k_steps_single)

    if clock is not None:
        clock.start()
    step_burst, bursts, reps = A.burst_us(stack.replay, stream)
    step_burst /= copies
    avg_us = {}
    for ln, names in LAUNCHES:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(copies):
                launch(c, ln, names)
        avg_us[ln] = A.burst_us(g.replay, stream)[0] / copies
    launch_bytes = {ln: sum(stored[n] + layer[n]["tensor"].codes.shape[0] * 4 * batch for n in names)
                    + layer[names[0]]["tensor"].x.size * 2 for ln, names in LAUNCHES}
    n_weights = sum(layer[n]["tensor"].codes.size for n in ORDER)
    unc = sum(layer[n]["tensor"].codes.size * 0.5 + layer[n]["tensor"].codes.shape[0] * 2 for n in ORDER)
    res = {"us_mean_of_timed_steps": round(ms_step * 1e3, 3), "us_median_of_bursts": round(step_burst, 3),
           "us_one_graph_per_step": round(ms_single * 1e3, 3), "steps_per_graph": copies,
           "bursts_us": [round(b / copies, 3) for b in bursts], "steps_per_burst": reps * copies,
           "per_launch_us": {ln: round(v, 3) for ln, v in avg_us.items()},
           "stored_bytes_per_layer": int(layer_bytes),
           "stored_bits_per_weight": round(layer_bytes * 8 / n_weights, 4),
           "copies_rotated": copies, "host_wall_s": round(host_s, 3)}
    res.update(bytes_row(ms_step * 1e3, layer_bytes, unc))
    return res, {n: ys[n].cpu().numpy() for n in ORDER}, launch_bytes


def layer_parity(layer, ys) -> float:
    worst = 0.0
    for ln, names in LAUNCHES:
        xv = layer[names[0]]["tensor"].x.astype(np.float64)
        for name in names:
            t = layer[name]["tensor"]
            wr = check_all(ys[name], int_values(t), xv)
            worst = max(worst, wr)
            if not wr <= 1.0:
                log(f"PARITY FAILURE on {name}: worst err/bound {wr}")
                sys.exit(1)
    return worst


def codings_json(layer):
    return {n: dict(k=layer[n]["coding"].weights_per_symbol, stored_tuples=layer[n]["coding"].stored_tuples,
                    log2_m=layer[n]["coding"].log2_m, tile_cols=layer[n]["coding"].tile_cols,
                    waves_per_block=layer[n]["launch"][0], tiles_per_wave=layer[n]["launch"][1],
                    streams_per_wave=layer[n]["launch"][2], row_groups_per_block=layer[n]["launch"][3])
            for n in ORDER}


# ------------------------------------------------------------------ the other workloads
def config5_shape_candidates():
    from entropy_coded_weight_amd import autotune as A
    return [s for s in A.DEFAULT_SHAPES if s[2] == 1]


def tune_secondary(which: str, path: str, cold_bytes: float):
    """Tune the other workloads on this device and write their codings and launch
    shapes to `path`: per tensor, codings ranked by warm timings (tune_tensor), then
    each launch's groupings timed cold (tune_group: rotated copies, median of 5
    bursts of >= 400 us), the fastest within 2% taking the fewest bytes."""
    import torch
    import ecw_inputs as E
    import entropy_coded_weight_amd as ecw
    from entropy_coded_weight_amd import autotune as A
    dev = torch.device("cuda:0")
    out = json.load(open(path)) if os.path.exists(path) else {}
    out["device"] = torch.cuda.get_device_name(0)
    out["timing"] = ("codings ranked warm, each launch's groupings timed cold: copies rotated over >= 512 MB, "
                     "graph replays, median of 5 bursts of >= 400 us")
    if "1" in which:
        log("tuning config 1")
        t = E.config1()
        x = torch.from_numpy(t.x).to(dev)
        c = A.tune_tensor(ecw.INT_CODES, t.codes, t.scales, x, code_bits=4, ks=(1,), log2_ms=(12,),
                          tile_cols=(64, 128, 256, 512), reps=10)
        out["1"] = A.tune_group({"w": (ecw.INT_CODES, t.codes, t.scales, 4)}, {"w": c}, x, top=6,
                                cold_bytes=cold_bytes, log=log)
    if "3" in which:
        out["3"] = {}
        for name in ("gate", "down"):
            log(f"tuning config 3 {name}")
            t = E.config3_tensor(name)
            x = torch.from_numpy(t.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
            c = A.tune_tensor(ecw.BF16_EXP, t.bits, None, x, log2_ms=(10, 11, 12), tile_cols=(64, 128, 256, 512),
                              reps=10)
            out["3"].update(A.tune_group({name: (ecw.BF16_EXP, t.bits, None, 0)}, {name: c}, x, top=6,
                                         cold_bytes=cold_bytes, log=log))
    if "5" in which:
        v2, scales, xh, step, bpw = config5_inputs()
        x = torch.from_numpy(xh).to(dev)
        n, K = v2.shape
        for recon, tag in ((ecw.DT_I8, "int8"), (ecw.DT_FP8_E4M3, "fp8")):
            log(f"tuning config 5 {tag}")
            cand = []
            # tile widths in whole 8-weight blocks: 9216 tiles at 64 columns are 1.125
            # rounds of the chip's 8192 wave slots; 72 and 80 columns fit one round
            for m in (9, 10, 11):
                for tc in (64, 72, 80, 96, 128):
                    c = ecw.Coding(ecw.E8_LATTICE, n, K, 8, 0, m, tc, recon)
                    blob = ecw.encode(c, v2, scales)
                    ct = ecw.CompressedTensor(blob)
                    stream = torch.cuda.Stream()
                    with torch.cuda.stream(stream):
                        su = A._tune_launch(ct, x, config5_shape_candidates(), 10, stream)
                    stream.synchronize()
                    for s, us in su.items():
                        cand.append((us, stored_of(ct.t), m, tc, s, blob))
            cand.sort(key=lambda c_: c_[0])
            timed = []
            for us_w, nb, m, tc, s, blob in cand[:8]:
                us = time_cold([("w", [(blob, s)], x)], 1, 0, cold_bytes)[0]["w"]
                timed.append((us, nb, m, tc, s))
                log(f"  m={m} tc={tc} shape={s} warm {us_w:.2f} cold {us:.2f} us, {nb / 1e6:.3f} MB")
            t_min = min(c_[0] for c_ in timed)
            us, nb, m, tc, s = min((c_ for c_ in timed if c_[0] <= 1.02 * t_min), key=lambda c_: c_[1])
            out[f"5_{tag}"] = {"w": dict(k=8, log2_m=m, tile_cols=tc, waves_per_block=s[0], tiles_per_wave=s[1],
                                         streams_per_wave=s[2], row_groups_per_block=s[3], us=round(us, 3),
                                         stored_bytes=nb, stored_tuples=0)}
    if "4" in which:
        names = ["q", "k", "v", "o", "gate", "up", "down", "lm_head"]
        groups = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gate_up", ["gate", "up"]), ("down", ["down"]),
                  ("lm_head", ["lm_head"])]
        ts = {n: E.config4_tensor(n, batch=4) for n in names}
        specs = {n: (ecw.FP8_E4M3, ts[n].codes, ts[n].scales, 0) for n in names}
        out["4"] = {}
        prev = None
        for batch in (1, 4):
            picks = {}
            for ln, ns in groups:
                x = torch.from_numpy(np.ascontiguousarray(ts[ns[0]].x_bits[:batch]).view(np.int16)).to(dev) \
                    .view(torch.bfloat16)
                cands = {}
                for n in ns:
                    log(f"tuning config 4 {n} batch {batch}")
                    if prev is None:
                        cands[n] = A.tune_tensor(ecw.FP8_E4M3, ts[n].codes, ts[n].scales, x, log2_ms=(11, 12),
                                                 tile_cols=(128, 256), reps=10)
                    else:
                        # the batch-1 coding; launch shapes tuned again for batch 4
                        p1 = prev[n]
                        cands[n] = A.tune_tensor(ecw.FP8_E4M3, ts[n].codes, ts[n].scales, x,
                                                 log2_ms=(p1["log2_m"],), tile_cols=(p1["tile_cols"],), reps=10)
                picks.update(A.tune_group({n: specs[n] for n in ns}, cands, x, top=4 if len(ns) == 1 else None,
                                          cold_bytes=cold_bytes, log=log))
            out["4"][f"batch{batch}"] = picks
            prev = picks
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    log(f"wrote {path}")


def secondary_configs(which: str, cold_bytes: float, sec: dict):
    """The other workloads in the codings and launch shapes of the committed tune file
    (warm-tuned in this run if the file has no entry), timed cold; every row of every
    output checked against float64."""
    import torch
    import ecw_inputs as E
    import entropy_coded_weight_amd as ecw
    from entropy_coded_weight_amd import autotune as A
    dev = torch.device("cuda:0")
    res = {}

    def coding_for(key, name, payload, w, scales, x, code_bits=0, **kw):
        p = sec.get(key, {}).get(name)
        src = os.path.relpath(SECONDARY_TUNE_FILE, ROOT)
        if p is None:
            cands = A.tune_tensor(payload, w, scales, x, code_bits=code_bits, reps=10, **kw)
            p = A.pick(cands)
            src = "warm tuning in this run (no tune-file entry)"
        c = ecw.Coding(payload, w.shape[0], w.shape[1], p["k"], code_bits if payload == ecw.INT_CODES else 0,
                       p["log2_m"], p["tile_cols"], stored_tuples=p.get("stored_tuples", 0))
        shape = (p["waves_per_block"], p["tiles_per_wave"], p.get("streams_per_wave", 1),
                 p.get("row_groups_per_block", 1))
        return ecw.encode(c, w, scales), shape, p, src

    def summary(launch_us, blobs_bytes, n_weights, unc_bytes, worst, picks, src, extra=None):
        t = sum(launch_us.values())
        d = {"us": round(t, 3), "per_launch_us": {k: round(v, 3) for k, v in launch_us.items()},
             "stored_bytes": int(blobs_bytes), "stored_bits_per_weight": round(blobs_bytes * 8 / n_weights, 4),
             "parity_worst_err_over_bound": worst, "codings": picks, "codings_from": src}
        d.update(bytes_row(t, blobs_bytes, unc_bytes))
        if extra:
            d.update(extra)
        return d

    def stored(blob):
        return stored_of(ecw.prepare(blob))

    def note(row, ln, blob, shape, batch, xbf):
        t = ecw.prepare(blob)
        t.waves_per_block, t.tiles_per_wave, t.streams_per_wave, t.row_groups_per_block = shape
        note_launch(row, ln, [t], batch, xbf)

    if "1" in which:
        log("config 1: 1024x1024 Gaussian codes, one code per symbol, M = 2^12")
        t = E.config1()
        x = torch.from_numpy(t.x).to(dev)
        blob, shape, p, src = coding_for("1", "w", ecw.INT_CODES, t.codes, t.scales, x, code_bits=4, ks=(1,),
                                         log2_ms=(12,), tile_cols=(64, 128, 256, 512))
        note("1", "w", blob, shape, 1, False)
        us, ys = time_cold([("w", [(blob, shape)], x)], 1, 0, cold_bytes)
        worst = check_all(ys["w"][0], int_values(t), t.x.astype(np.float64))
        n = t.codes.size
        res["1"] = summary(us, stored(blob), n, n * 0.5 + 1024 * 2, worst, {"w": p}, src,
                           {"workload": "one 1024x1024 matrix of 16-level codes from a discretised Gaussian "
                                        "(sigma 2 levels, seed 0), fp16 row scales, fp16 x, batch 1"})

    if "3" in which:
        log("config 3: BF16 exponent coding, gate 14336x4096 and down 4096x14336")
        launches, picks, nbytes, nw, checks, srcs = [], {}, 0, 0, [], set()
        for name in ("gate", "down"):
            t = E.config3_tensor(name)
            x = torch.from_numpy(t.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
            blob, shape, p, src = coding_for("3", name, ecw.BF16_EXP, t.bits, None, x, log2_ms=(10, 11, 12))
            note("3", name, blob, shape, 1, True)
            launches.append((name, [(blob, shape)], x))
            picks[name] = p
            srcs.add(src)
            nbytes += stored(blob)
            nw += t.bits.size
            xv = torch.from_numpy(t.x_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
            checks.append((name, t.bits, xv))
        us, ys = time_cold(launches, 1, 0, cold_bytes)
        worst = max(check_all(ys[n][0], lambda r0, r1, b=b: torch.from_numpy(b[r0:r1].view(np.int16))
                              .view(torch.bfloat16).double().numpy(), xv) for n, b, xv in checks)
        res["3"] = summary(us, nbytes, nw, nw * 2, worst, picks, "; ".join(sorted(srcs)),
                           {"workload": "BF16 N(0, 0.02^2) weights at 14336x4096 and 4096x14336, exponent "
                                        "byte rANS-coded, sign+mantissa byte raw, bf16 x, batch 1; "
                                        "two launches"})

    if "5" in which:
        log("config 5: E8 lattice fields, 3072x12288, INT8 and FP8 reconstruction")
        v2, scales, xh, step, bpw = config5_inputs()
        x = torch.from_numpy(xh).to(dev)
        n, K = v2.shape
        for recon, tag in ((ecw.DT_I8, "int8"), (ecw.DT_FP8_E4M3, "fp8")):
            p = sec.get(f"5_{tag}", {}).get("w")
            src = os.path.relpath(SECONDARY_TUNE_FILE, ROOT)
            if p is None:
                p = dict(k=8, log2_m=9, tile_cols=64, waves_per_block=16, tiles_per_wave=1, streams_per_wave=1,
                         row_groups_per_block=1)
                src = "default (no tune-file entry)"
            c = ecw.Coding(ecw.E8_LATTICE, n, K, 8, 0, p["log2_m"], p["tile_cols"], recon)
            blob = ecw.encode(c, v2, scales)
            shape = (p["waves_per_block"], p["tiles_per_wave"], p["streams_per_wave"], p["row_groups_per_block"])
            note(f"5_{tag}", "w", blob, shape, 1, False)
            us, ys = time_cold([("w", [(blob, shape)], x)], 1, 0, cold_bytes)

            def wv(r0, r1, recon=recon):
                vv = v2[r0:r1].astype(np.float64) / 2.0
                if recon != ecw.DT_I8:
                    vv = torch.from_numpy(vv.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
                return vv * scales[r0:r1].astype(np.float64)[:, None]
            worst = check_all(ys["w"][0], wv, xh.astype(np.float64))
            res[f"5_{tag}"] = summary(us, stored(blob), v2.size, v2.size + n * 2, worst, {"w": p}, src,
                                      {"workload": "3072x12288 N(0, 0.02^2) weights, row-RMS normalised, E8 "
                                                   f"lattice step {step:.4f} ({bpw:.3f} bits/weight plug-in "
                                                   "entropy), 9 fields per 8-weight block coded with 17 "
                                                   f"coset-indexed tables, {tag} reconstruction, fp16 row "
                                                   "scales, fp16 x, batch 1"})

    if "4" in which:
        res.update(config4_step(sec, cold_bytes))
    return res


def config4_step(sec: dict, cold_bytes: float, layers: int = 32):
    """The full decode step of an 8B-shaped model with FP8 E4M3 weights: 32 layers of
    7 linears (4 grouped launches each: q/k/v, o, gate/up, down) and the 128256x4096 LM
    head, captured as ONE HIP graph and replayed (burst protocol), at batch 1 and 4.
    The 32 layers are 32 distinct device copies of one layer's blobs (5.9 GB, far
    beyond the 256 MiB Infinity Cache, so every layer reads HBM).  Every row of every
    tensor's output (the last layer's and the LM head's) is checked against float64."""
    import torch
    import ecw_inputs as E
    import entropy_coded_weight_amd as ecw
    from entropy_coded_weight_amd import autotune as A
    dev = torch.device("cuda:0")
    names = ["q", "k", "v", "o", "gate", "up", "down", "lm_head"]
    groups = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gate_up", ["gate", "up"]), ("down", ["down"])]
    log("config 4: 32-layer FP8 decode step + LM head")
    t0 = time.time()
    ts = {n: E.config4_tensor(n, batch=4) for n in names}
    log(f"  generated in {time.time() - t0:.1f} s")
    tuned = sec.get("4")
    src = os.path.relpath(SECONDARY_TUNE_FILE, ROOT)
    if tuned is None:
        default = dict(k=1, log2_m=12, tile_cols=256, waves_per_block=16, tiles_per_wave=1, streams_per_wave=1,
                       row_groups_per_block=1)
        tuned = {"batch1": {n: default for n in names}, "batch4": {n: default for n in names}}
        src = "default (no tune-file entry)"
    blobs = {}
    for n in names:
        p = tuned["batch1"][n]
        c = ecw.Coding(ecw.FP8_E4M3, *ts[n].codes.shape, 1, 0, p["log2_m"], p["tile_cols"])
        blobs[n] = ecw.encode(c, ts[n].codes, ts[n].scales)
    step_bytes = layers * sum(stored_of(ecw.prepare(blobs[n])) for n in names[:7]) + stored_of(
        ecw.prepare(blobs["lm_head"]))
    n_weights = layers * sum(ts[n].codes.size for n in names[:7]) + ts["lm_head"].codes.size
    unc = layers * sum(ts[n].codes.size + ts[n].codes.shape[0] * 2 for n in names[:7]) + \
        ts["lm_head"].codes.size + ts["lm_head"].codes.shape[0] * 2
    t0 = time.time()
    copies = [{n: ecw.CompressedTensor(blobs[n]) for n in names[:7]} for _ in range(layers)]
    heads = [ecw.CompressedTensor(blobs["lm_head"]) for _ in range(2)]
    log(f"  {layers} layer copies + 2 LM head copies on the device in {time.time() - t0:.1f} s "
        f"({step_bytes / 1e9:.2f} GB stored per step)")
    stream = torch.cuda.current_stream()
    res = {}
    for batch in (1, 4):
        picks = tuned[f"batch{batch}"]
        for cp in copies:
            for n in names[:7]:
                cp[n].set_launch(*pick_tuple(picks[n])[3:7])
        for h in heads:
            h.set_launch(*pick_tuple(picks["lm_head"])[3:7])
        xs = {ln: torch.from_numpy(np.ascontiguousarray(ts[ns[0]].x_bits[:batch]).view(np.int16)).to(dev)
              .view(torch.bfloat16) for ln, ns in groups + [("lm_head", ["lm_head"])]}
        ys = {n: torch.empty((batch, ts[n].codes.shape[0]), dtype=torch.float32, device=dev) for n in names}
        wss = [{ln: ecw.GemvGroup([cp[n] for n in ns]).workspace(batch) for ln, ns in groups} for cp in copies]
        hws = [ecw.GemvGroup([h]).workspace(batch) for h in heads]
        row = f"4_batch{batch}"
        for ln, ns in groups:
            note_launch(row, ln, [copies[0][n].t for n in ns], batch, True)
        note_launch(row, "lm_head", [heads[0].t], batch, True)

        def head(i):
            ecw.gemv_group_raw([heads[i].t], xs["lm_head"], [ys["lm_head"]], hws[i])

        def step():
            for l_ in range(layers):
                for ln, ns in groups:
                    ecw.gemv_group_raw([copies[l_][n].t for n in ns], xs[ln], [ys[n] for n in ns], wss[l_][ln])
            head(0)

        step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        us_step, bursts, _ = A.burst_us(g.replay, stream)
        gh = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gh):
            head(0)
            head(1)
        us_head = A.burst_us(gh.replay, stream)[0] / 2
        gl = {}
        for ln, ns in groups:
            gg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gg):
                for l_ in range(layers):
                    ecw.gemv_group_raw([copies[l_][n].t for n in ns], xs[ln], [ys[n] for n in ns], wss[l_][ln])
            gl[ln] = A.burst_us(gg.replay, stream)[0] / layers
        # parity: the step graph's outputs (last layer, LM head), every row
        g.replay()
        torch.cuda.synchronize()
        xv = {ln: torch.from_numpy(np.ascontiguousarray(ts[ns[0]].x_bits[:batch]).view(np.int16))
              .view(torch.bfloat16).double().numpy() for ln, ns in groups + [("lm_head", ["lm_head"])]}
        worst = 0.0
        for ln, ns in groups + [("lm_head", ["lm_head"])]:
            for n in ns:
                worst = max(worst, check_all(ys[n].cpu().numpy(), fp8_values(ts[n]), xv[ln]))
        d = {"workload": f"full decode step of an 8B-shaped model, FP8 E4M3 weights: {layers} layers x 7 linears "
                         "(q,k,v,o,gate,up,down; N(0, 0.02^2) quantised per row, fp16 row scale, byte symbols "
                         "rANS-coded; 4 grouped launches per layer) + the 128256x4096 LM head, one HIP graph, bf16 "
                         f"x, batch {batch}; the layers are {layers} device copies of one layer's blobs",
             "step_us_32_layers_plus_head": round(us_step, 1), "bursts_us": [round(b, 1) for b in bursts],
             "lm_head_us": round(us_head, 3), "layer_us_from_step": round((us_step - us_head) / layers, 3),
             "per_launch_us": {**{ln: round(v, 3) for ln, v in gl.items()}, "lm_head": round(us_head, 3)},
             "stored_bytes_per_step": int(step_bytes),
             "stored_bits_per_weight": round(step_bytes * 8 / n_weights, 4),
             "parity_worst_err_over_bound": worst, "codings": picks, "codings_from": src}
        d.update(bytes_row(us_step, step_bytes, unc))
        log(f"  batch {batch}: step {us_step:.1f} us ({d['hbm_frac'] * 100:.1f}% of HBM), LM head {us_head:.1f} us, "
            f"parity {worst:.3g}")
        res[f"4_batch{batch}"] = d
        del g, gh, gl, wss, hws
    return res


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


def _lds_of(r: dict) -> int:
    """LDS bytes of a dispatch in a rocprofv3 CSV row (kernel traces name the column
    after the group segment, counter collections after the LDS block)."""
    for k in ("LDS_Block_Size", "Group_Segment_Size", "Lds_Size"):
        if r.get(k) not in (None, ""):
            return int(float(r[k]))
    return 0


def summarize_rocprof(directory: str):
    """Print per-(kernel, grid size, LDS size) averages from rocprofv3 CSV output under
    `directory`: kernel durations from *_kernel_trace.csv and counter values from
    *_counter_collection.csv (one line per kernel and counter).  Where the run that
    made a CSV left its launch map and dispatch log beside it (--launch-map), the same
    figures follow per launch (row.launch) of the fused decode-GEMV."""
    import csv
    import collections
    import glob

    def by_launch(path, rows):
        lmp = os.path.join(os.path.dirname(path), "launch_map.json")
        if not os.path.exists(lmp):
            return None, None
        return attribute_dispatches(rows, json.load(open(lmp)), lmp + ".dispatches.json")

    for path in sorted(glob.glob(os.path.join(directory, "**", "*_kernel_trace.csv"), recursive=True)):
        d = collections.defaultdict(list)
        rows, dur = {}, {}
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"].split("(")[0], int(r["Grid_Size_X"]), _lds_of(r))
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            d[key].append(us)
            rows[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]), _lds_of(r))
            dur[r["Dispatch_Id"]] = us
        print(f"# kernel durations from {os.path.relpath(path, directory)}")
        print(f"{'kernel':48s} {'grid':>8s} {'lds':>7s} {'calls':>6s} {'avg_us':>9s} {'median_us':>9s} {'min_us':>8s}")
        for (k, g, lds), v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
            v.sort()
            print(f"{k[:48]:48s} {g:8d} {lds:7d} {len(v):6d} {sum(v) / len(v):9.2f} {v[len(v) // 2]:9.2f} "
                  f"{v[0]:8.2f}")
        att, how = by_launch(path, rows)
        if att:
            pl = collections.defaultdict(list)
            for did, owners in att.items():
                for o in owners:
                    pl[".".join(o)].append(dur[did])
            print(f"# per launch (dispatches attributed by {how})")
            print(f"{'launch':24s} {'calls':>6s} {'avg_us':>9s} {'median_us':>9s} {'min_us':>8s}")
            for ln, v in sorted(pl.items()):
                v.sort()
                print(f"{ln:24s} {len(v):6d} {sum(v) / len(v):9.2f} {v[len(v) // 2]:9.2f} {v[0]:8.2f}")
    for path in sorted(glob.glob(os.path.join(directory, "**", "*_counter_collection.csv"), recursive=True)):
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        names, rows = {}, {}
        for r in csv.DictReader(open(path)):
            per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = (r["Kernel_Name"].split("(")[0], int(r["Grid_Size"]), _lds_of(r))
            rows[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["Workgroup_Size"]), _lds_of(r))
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for did, cs in per.items():
            for c, v in cs.items():
                agg[names[did]][c].append(v)
        print(f"# counters from {os.path.relpath(path, directory)} (mean per dispatch)")
        for (k, g, lds), cs in sorted(agg.items()):
            for c, v in sorted(cs.items()):
                print(f"{k[:48]:48s} {g:8d} {lds:7d} {c:24s} n={len(v):4d} {sum(v) / len(v):16.1f}")
        att, how = by_launch(path, rows)
        if att:
            pl = collections.defaultdict(lambda: collections.defaultdict(list))
            for did, owners in att.items():
                for o in owners:
                    for c, v in per[did].items():
                        pl[".".join(o)][c].append(v)
            print(f"# per launch (dispatches attributed by {how}; mean per dispatch)")
            for ln, cs in sorted(pl.items()):
                for c, v in sorted(cs.items()):
                    print(f"{ln:24s} {c:24s} n={len(v):4d} {sum(v) / len(v):16.1f}")




# ------------------------------------------------------------------ counter records
def write_counter_record(directory: str, launch_map_path: str, out_path: str, commands: list):
    """From rocprofv3 counter-collection CSVs under `directory` and the launch map a
    bench run wrote, the mean counters per dispatch of every (workload, launch), as a
    key = value record hashed to the kernel source and tune files (bench.py uses it
    only while they still hash to these values)."""
    import collections
    import csv
    import glob
    lm = json.load(open(launch_map_path))
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    owners, how = {}, set()
    for path in sorted(glob.glob(os.path.join(directory, "**", "*_counter_collection.csv"), recursive=True)):
        rows = {}
        for r in csv.DictReader(open(path)):
            key = (path, r["Dispatch_Id"])
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
            rows[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["Workgroup_Size"]), _lds_of(r))
            per[key]["VGPR_Count"] = float(r["VGPR_Count"])
        # each profiled run leaves its own launch map and dispatch log beside its CSVs
        local = os.path.join(os.path.dirname(path), "launch_map.json")
        lmp = local if os.path.exists(local) else launch_map_path
        att, h = attribute_dispatches(rows, json.load(open(lmp)), lmp + ".dispatches.json")
        how.add(h)
        for did, o in att.items():
            owners[(path, did)] = o
    lines = ["# Mean SQ counters per dispatch of every launch of every workload bench.py measures, MI355X.",
             "# Read by bench.py (VALU, LDS and bank-conflict fractions per launch, priced at the clock measured",
             "# in the same bench run); valid only while the kernel source and tune files hash to the values below.",
             "#", "# Commands (repository root on the GPU host; cd /tmp && export TMPDIR=/tmp first):"]
    lines += [f"#   {c}" for c in commands]
    lines += [f"# dispatches attributed to launches by {' and '.join(sorted(how))}",
              f"kernel_sha256 = {sha256(KERNEL_SRC)}",
              f"tune_sha256 = {sha256(os.path.relpath(TUNE_FILE, ROOT))}",
              f"secondary_tune_sha256 = {sha256(os.path.relpath(SECONDARY_TUNE_FILE, ROOT))}"]
    table = ["| workload | launch | kernel | waves | VALU / wave-step | SALU / wave-step | LDS / wave-step | "
             "bank-conflict share of LDS-active cycles | dependency waits / wave cycles |",
             "|---|---|---|---|---|---|---|---|---|"]
    for row, launches in lm.items():
        for ln, (sig, grid, wg, nsym, *_) in launches.items():
            agg = collections.defaultdict(list)
            for key, cs in per.items():
                if (row, ln) in owners.get(key, ()):
                    for c, v in cs.items():
                        agg[c].append(v)
            if not agg:
                lines.append(f"# {row}.{ln}: no dispatch of {sig} with grid {grid}")
                continue
            lines.append(f"{row}.{ln}.kernel = {sig}")
            lines.append(f"{row}.{ln}.grid = {grid}")
            lines.append(f"{row}.{ln}.symbols = {nsym}")
            mean = {c: sum(v) / len(v) for c, v in agg.items()}
            for c in sorted(mean):
                lines.append(f"{row}.{ln}.{c} = {mean[c]:.1f}")
            lines.append(f"{row}.{ln}.dispatches = {max(len(v) for v in agg.values())}")
            ws = nsym / 64.0          # wave-steps: one symbol per lane
            g = lambda c: mean.get(c, float("nan"))     # noqa: E731
            table.append(f"| {row} | {ln} | `{sig}` | {int(g('SQ_WAVES'))} | {g('SQ_INSTS_VALU') / ws:.1f} | "
                         f"{g('SQ_INSTS_SALU') / ws:.1f} | {g('SQ_INSTS_LDS') / ws:.2f} | "
                         f"{g('SQ_LDS_BANK_CONFLICT') / g('SQ_LDS_IDX_ACTIVE'):.2f} | "
                         f"{g('SQ_WAIT_ANY') / g('SQ_WAVE_CYCLES'):.2f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    md = os.path.splitext(out_path)[0] + ".md"
    with open(md, "w") as f:
        f.write("# SQ counters of every launch of every workload (k_decode), MI355X\n\n"
                f"Derived from `{os.path.relpath(out_path, ROOT)}` (mean per dispatch; the commands that made it "
                "are in its header).\nA wave-step is one decode step of one wave (64 lanes, one rANS symbol each). "
                "Workload rows: 2 = the INT4 layer set in its tuned codings, k = the same with two codes per "
                "symbol, 1 = the 1024x1024 Gaussian codes, 3 = BF16 exponent pairs, 4_batchB = the FP8 decode "
                "step, 5_int8 / 5_fp8 = the E8 lattice fields.  bench.py turns the same record into VALU and LDS "
                "fractions of each launch's measured time at the measured clock.\n\n" + "\n".join(table) + "\n")
    log(f"wrote {out_path} and {md}")


def read_counter_record(path: str):
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_sha256") != sha256(KERNEL_SRC):
        return None
    if rec.get("tune_sha256") != sha256(os.path.relpath(TUNE_FILE, ROOT)):
        return None
    if os.path.exists(SECONDARY_TUNE_FILE) and \
            rec.get("secondary_tune_sha256") != sha256(os.path.relpath(SECONDARY_TUNE_FILE, ROOT)):
        return None
    return rec


def counter_fractions(rec, row: str, launch_us: dict, mhz: float):
    """Per launch of a workload: VALU issue fraction (wave64 VALU instructions x 4
    clocks over 1024 SIMDs x clock x time), LDS-active fraction (LDS indexed-access
    cycles over 256 CUs x clock x time), the bank-conflict share of the LDS-active
    cycles, and dependency waits per wave cycle; plus their time-weighted means."""
    if not rec or not mhz:
        return None
    out, wsum = {}, {}
    for ln, us in launch_us.items():
        pre = f"{row}.{ln}."
        if pre + "SQ_INSTS_VALU" not in rec:
            continue
        cyc = mhz * 1e6 * us * 1e-6
        g = lambda c: float(rec[pre + c]) if pre + c in rec else None   # noqa: E731
        d = {"valu_frac": round(g("SQ_INSTS_VALU") * 4 / (N_SIMD * cyc), 4)}
        if g("SQ_LDS_IDX_ACTIVE"):
            d["lds_active_frac"] = round(g("SQ_LDS_IDX_ACTIVE") / (N_CU * cyc), 4)
            d["lds_bank_conflict_share"] = round(g("SQ_LDS_BANK_CONFLICT") / g("SQ_LDS_IDX_ACTIVE"), 4)
        if g("SQ_WAIT_ANY") and g("SQ_WAVE_CYCLES"):
            d["wait_any_per_wave_cycle"] = round(g("SQ_WAIT_ANY") / g("SQ_WAVE_CYCLES"), 4)
        if g("SQ_WAIT_INST_LDS") and g("SQ_WAIT_INST_ANY"):
            d["lds_share_of_issue_waits"] = round(g("SQ_WAIT_INST_LDS") / g("SQ_WAIT_INST_ANY"), 4)
        d["valu_instructions"] = int(g("SQ_INSTS_VALU"))
        out[ln] = d
        for k, v in d.items():
            if k != "valu_instructions":
                wsum.setdefault(k, [0.0, 0.0])
                wsum[k][0] += v * us
                wsum[k][1] += us
    if not out:
        return None
    out["time_weighted"] = {k: round(a / b, 4) for k, (a, b) in wsum.items()}
    return out


def measured_traffic(path: str):
    """HBM bytes per launch of the dominant launch from a committed profile record,
    valid only while the kernel source and tune file hash to what was profiled."""
    if not os.path.exists(path):
        return None
    rec = dict(l.split("=", 1) for l in open(path).read().split("\n") if "=" in l and not l.startswith("#"))
    rec = {k.strip(): v.strip() for k, v in rec.items()}
    if rec.get("kernel_sha256") != sha256(KERNEL_SRC):
        return None
    if rec.get("tune_sha256") != sha256(os.path.relpath(TUNE_FILE, ROOT)):
        return None
    return rec


# ------------------------------------------------------------------ main
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
                    help="autotune every tensor of the layer set on this device first and rewrite the tune file")
    ap.add_argument("--tune-file", default=TUNE_FILE)
    ap.add_argument("--tune-configs", default="",
                    help="tune these other workloads (1,3,4,5) on this device first and write --secondary-file")
    ap.add_argument("--secondary-file", default=SECONDARY_TUNE_FILE)
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="print per-launch averages of rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--write-counter-record", metavar="DIR",
                    help="write the counter record from rocprofv3 counter CSVs under DIR and the launch map "
                         "(--launch-map) of the profiled run, and exit")
    ap.add_argument("--launch-map", metavar="PATH",
                    help="write (or, with --write-counter-record, read) the kernel template, grid and LDS of "
                         "every launch of the run, and beside it (PATH.dispatches.json) the launch of every fused "
                         "decode-GEMV dispatch in issue order, for attributing profiler records")
    ap.add_argument("--configs", default="1,3,4,5,k,p,d",
                    help="workloads measured after the layer set (1: Gaussian codes, 3: BF16 exponent coding, "
                         "4: 32-layer FP8 step + LM head at batch 1 and 4, 5: E8 lattice fields, INT8 and FP8 "
                         "reconstruction, k: the layer set with two codes per symbol, p: the layer set under byte "
                         "budgets from the tune file's Pareto fronts, d: dequantising decode + GEMM for batches "
                         "above 4); '' for none")
    ap.add_argument("--tensors", default=",".join(ORDER),
                    help="subset of the layer to run (profiling); the JSON line is only "
                         "meaningful for the full set")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    if args.write_counter_record:
        write_counter_record(args.write_counter_record, args.launch_map, COUNTER_FILE,
                             [f"rocprofv3 --pmc {s} --output-format csv -d $R/gpurun_out/<dir>/sq{i} -o sq{i} -- "
                              f"python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline --configs 1,3,4,5,k "
                              f"--launch-map $R/gpurun_out/<dir>/sq{i}/launch_map.json"
                              for i, s in enumerate(COUNTER_SETS)]
                             + ["python3 bench.py --write-counter-record gpurun_out/<dir> --launch-map "
                                "gpurun_out/<dir>/sq0/launch_map.json"])
        return
    if args.launch_map:
        install_dispatch_log()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the kernel measured here is one GPU's share; sharding over GPUs is not built)", file=sys.stderr)
        sys.exit(2)

    import entropy_coded_weight_amd as ecw

    full_set = args.tensors == ",".join(ORDER)
    ORDER[:] = [n for n in ORDER if n in args.tensors.split(",")]
    global LAUNCHES
    LAUNCHES = [(ln, [n for n in names if n in ORDER]) for ln, names in LAUNCHES]
    LAUNCHES = [(ln, names) for ln, names in LAUNCHES if names]
    coding, coding_src = load_coding(args.tune_file)
    t_build = time.time()
    layer = build_layer(args.batch, coding)
    log(f"encoded layer set in {time.time() - t_build:.1f} s (codings: {coding_src})")
    # the CPU baseline runs before anything touches the GPU (its worker processes are forked)
    cpu = None
    if not args.no_cpu_baseline and full_set:
        t0 = time.time()
        cpu = cpu_baseline(layer)
        log(f"cpu baseline in {time.time() - t0:.1f} s: {cpu['value']:.0f} us/layer on {cpu['cores']} cores, "
            f"{cpu['one_core_us_per_layer']:.0f} on one")

    import torch
    if args.tune:
        run_tuner(args.tune_file, args.batch)
        coding, coding_src = load_coding(args.tune_file)
        layer = build_layer(args.batch, coding, {n: layer[n]["tensor"] for n in ORDER})
    if args.tune_configs:
        tune_secondary(args.tune_configs, args.secondary_file, args.cold_bytes)
    sec = json.load(open(args.secondary_file)) if os.path.exists(args.secondary_file) else {}

    clock = ecw.ClockProbe(duration_us=4000)
    res, ys, launch_bytes = time_layer_set(layer, args.batch, args.steps, args.warmup, args.cold_bytes, "2",
                                           clock)
    mhz = clock.mhz()
    worst = layer_parity(layer, ys)
    avg_us = res["per_launch_us"]
    for n in ORDER:
        c = layer[n]["coding"]
        log(f"{n:5s} {layer[n]['tensor'].codes.shape} k={c.weights_per_symbol} t={c.stored_tuples} "
            f"m={c.log2_m} tc={c.tile_cols} launch={layer[n]['launch']}")
    for ln, _ in LAUNCHES:
        log(f"launch {ln:8s} {avg_us[ln]:.2f} us  {launch_bytes[ln] / (avg_us[ln] * 1e-6) / 1e9:.0f} GB/s")
    log(f"layer: {res['us_mean_of_timed_steps']:.2f} us (timed steps), {res['us_median_of_bursts']:.2f} us "
        f"(median of 5 bursts), {res['us_one_graph_per_step']:.2f} us (one graph per step), clock {mhz:.0f} MHz")
    us_layer = res["us_mean_of_timed_steps"]
    dom = max(avg_us, key=lambda ln: avg_us[ln])
    achieved = launch_bytes[dom] / (avg_us[dom] * 1e-6) / 1e9
    dom_names = dict(LAUNCHES)[dom]
    dom_label = (f"k_decode<INT4, {layer[dom_names[0]]['coding'].weights_per_symbol} codes/symbol>"
                 + f" (launch {dom}: {'+'.join(dom_names)})")
    rec = measured_traffic(TRAFFIC_FILE) if args.tune_file == TUNE_FILE and args.batch == 1 else None
    traffic = int(rec["traffic_bytes"]) if rec and rec.get("launch") == dom else None
    out = {
        "metric": METRIC, "value": round(us_layer, 3), "unit": "us/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us_layer / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "u32 decode + f32 accumulate", "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped layer set (q,k,v,o,gate,up,down) of 16-level "
                               "Laplacian codes (H=2.2 bits), autotuned codes per rANS symbol, fp16 row "
                               "scales, fp16 x, batch 1, cold cache; 4 launches per step "
                               "(q/k/v, o, gate/up, down)",
                   "batch": args.batch, "copies_rotated": res["copies_rotated"], "codings_from": coding_src,
                   "codings": codings_json(layer)},
        "us_per_layer_median_of_5_bursts": res["us_median_of_bursts"], "bursts_us": res["bursts_us"],
        "steps_per_graph": res["steps_per_graph"], "us_per_layer_one_graph_per_step": res["us_one_graph_per_step"],
        "stored_bytes_per_layer": res["stored_bytes_per_layer"],
        "stored_bits_per_weight": res["stored_bits_per_weight"],
        "gbps_compressed": res["gbps_compressed"], "hbm_frac": res["hbm_frac"],
        "gbps_uncompressed_equiv": res["gbps_uncompressed_equiv"],
        "uncompressed_equiv_frac": res["uncompressed_equiv_frac"],
        "per_launch_us": avg_us, "host_wall_s": res["host_wall_s"],
        "parity_worst_err_over_bound": worst,
        "sclk_mhz_measured": round(mhz, 1),
        "roofline": {"bound": "hbm", "kernel": dom_label,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": int(launch_bytes[dom]), "avg_launch_us": round(avg_us[dom], 3)},
    }
    # the same launch against the VALU issue rate (256 CUs x 4 SIMDs, one wave64 VALU
    # instruction per SIMD every 4 clocks) at the clock measured during the bursts
    crec = read_counter_record(COUNTER_FILE) if args.tune_file == TUNE_FILE and args.batch == 1 else None
    valu = None
    if crec and f"2.{dom}.SQ_INSTS_VALU" in crec:
        valu = float(crec[f"2.{dom}.SQ_INSTS_VALU"])
    elif rec and rec.get("valu_instructions") and rec.get("launch") == dom:
        valu = float(rec["valu_instructions"])
    if valu:
        peak_g = N_SIMD * mhz * 1e6 / 4 / 1e9
        out["issue_roofline"] = {"bound": "alu", "kernel": dom_label,
                                 "achieved": round(valu / (avg_us[dom] * 1e-6) / 1e9, 1), "peak": round(peak_g, 1),
                                 "unit": "G wave64 VALU instructions/s", "clock_mhz": round(mhz, 1),
                                 "frac": round(valu / (avg_us[dom] * 1e-6) / 1e9 / peak_g, 4),
                                 "valu_instructions_per_launch": int(valu)}
    cf = counter_fractions(crec, "2", avg_us, mhz)
    if cf:
        out["counters"] = cf
    configs = args.configs.split(",") if args.configs else []
    if "k" in configs and full_set and args.tune_file == TUNE_FILE and os.path.exists(TUNE_FILE):
        k2 = k2_coding(TUNE_FILE)
        layer2 = build_layer(args.batch, k2, {n: layer[n]["tensor"] for n in ORDER})
        res2, ys2, _ = time_layer_set(layer2, args.batch, max(20, args.steps // 4), 2, args.cold_bytes, "k")
        res2["parity_worst_err_over_bound"] = layer_parity(layer2, ys2)
        res2["codings"] = codings_json(layer2)
        res2["workload"] = ("the same layer set with two codes per rANS symbol everywhere (each launch at the "
                            "fastest two-code candidates of the tune file); timed like the headline")
        c2 = counter_fractions(crec, "k", res2["per_launch_us"], mhz)
        if c2:
            res2["counters"] = c2
        out["layer_two_codes_per_symbol"] = res2
        log(f"layer, two codes per symbol: {res2['us_mean_of_timed_steps']:.2f} us, "
            f"{res2['stored_bits_per_weight']:.3f} bits/weight, {100 * res2['hbm_frac']:.1f}% of HBM")
    # roofline probes on this device: achievable streaming-read rate (2 GiB buffer)
    # and dependent LDS table lookups (the decode's table reads), all CUs busy
    dev = torch.device("cuda:0")
    big = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    achievable = ecw.probe_stream_read(big)
    # the same read, one launch of the dominant launch's size (each rep another, cold
    # region): what a launch of that many bytes can reach at all
    at_size = ecw.probe_stream_read(big, region_bytes=int(launch_bytes[dom]))
    # per-wave streams shaped like the decode's plane reads (7168 waves, as the gate/up
    # launch and the BF16 launches run): 2 KiB and 8 KiB per wave, 1 or 2 KiB in flight
    tiles = {f"{kib}KiB_x7168_inflight{inf}": round(ecw.probe_tile_stream(big, kib, 7168, 16, inf), 1)
             for kib in (2, 8) for inf in (1, 2)}
    del big
    lut_rate = {f"m{m}_{eb}B": round(ecw.probe_lds_lookup(m, eb) / 1e9, 1) for m in (11, 12) for eb in (4, 8, 16)}
    out["probes"] = {"hbm_read_gbs": round(achievable, 1),
                     "hbm_read_frac_of_peak": round(achievable / HBM_PEAK_GBS, 4),
                     "dominant_launch_frac_of_achievable": round(achieved / achievable, 4),
                     "hbm_read_gbs_one_launch_of_dominant_size": round(at_size, 1),
                     "dominant_launch_frac_of_achievable_at_its_size": round(achieved / at_size, 4),
                     "tile_stream_gbs": tiles,
                     "lds_lookups_g_per_s": lut_rate}
    if args.calibrate_copy:
        src = torch.ones(64 << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.calibrate_copy):
            dst.copy_(src)
        torch.cuda.synchronize()
    if full_set and [c for c in configs if c in "1345pd"]:
        which = ",".join(c for c in configs if c in "1345")
        out["configs"] = secondary_configs(which, args.cold_bytes, sec) if which else {}
        for k, v in out["configs"].items():
            lus = v["per_launch_us"]
            cfk = counter_fractions(crec, k, lus, mhz)
            if cfk:
                v["counters"] = cfk
            log(f"config {k}: {v.get('step_us_32_layers_plus_head', v.get('us'))} us, "
                f"{v['gbps_compressed']:.0f} GB/s ({100 * v['hbm_frac']:.1f}% of HBM), "
                f"{v['stored_bits_per_weight']:.3f} bits/weight, parity {v['parity_worst_err_over_bound']:.3g}")
            if not v["parity_worst_err_over_bound"] <= 1.0:
                log(f"PARITY FAILURE in config {k}")
                sys.exit(1)
        if "p" in configs:
            budget = budget_points(args.steps, args.cold_bytes)
            if budget:
                out["budget"] = budget
                for pt in budget["points"]:
                    if not pt["parity_worst_err_over_bound"] <= 1.0:
                        log(f"PARITY FAILURE in budget point {pt['label']}")
                        sys.exit(1)
        if "d" in configs:
            deq = dequant_gemm(args.steps, args.cold_bytes)
            out["dequant"] = deq
            if not all(v["dense_bits_exact"] for k, v in deq.items() if k != "workload"):
                log("PARITY FAILURE in the dequantising decode")
                sys.exit(1)
    if args.launch_map:
        with open(args.launch_map, "w") as f:
            json.dump(LAUNCH_MAP, f, indent=1)
        write_dispatch_log(args.launch_map + ".dispatches.json")
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
