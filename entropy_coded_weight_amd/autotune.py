"""Per-tensor autotuner: weights per symbol, table size, tile width and launch shape.

The coding axes (weights per symbol k, table size M = 2^m, tile width) change the
stored blob, so each candidate is encoded on the host through the C ABI.  The launch
axes (waves per block, tiles per wave) are timed on the device by the library's
dec_tune_launch, which replays each shape as a captured HIP graph.  The fastest
candidate wins; when two are within `tie` of each other the smaller blob wins.  This
is the per-tensor tuning the MINE page describes (Section 4.2: tile width, table
size and symbol packing chosen per tensor by measurement, with the cross-entropy
size as the tie-breaker).

Tensors that share a launch (q/k/v, gate/up) must agree on waves per block;
tune_group times the real grouped launch for combinations of each member's best
single-tensor candidates at each common value.

For INT quads the number t of stored tuples follows the page's search (Section 4.2,
"Tuning t"; t_curve, t_search): from each tensor's byte-optimal t, the t that saves
the most escapes per added byte is raised until the launch's bytes grow by more than
1%, and each such selection becomes a candidate.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass, field

import torch

from . import (INT_CODES, BF16_EXP, FP8_E4M3, Coding, CompressedTensor, EcwError, encode, lib,
               workspace_size, _check, DT_F16, DT_BF16)

DEFAULT_LOG2_M = (10, 11, 12)
DEFAULT_TILE_COLS = (64, 128, 256, 512)
# (waves per block, tiles per wave, streams per wave, row groups per block)
DEFAULT_SHAPES = tuple((w, r, ns, p) for w in (4, 8, 16) for r in (1, 2, 4) for ns in (1, 2) for p in (1, 2))


@dataclass
class Candidate:
    k: int
    log2_m: int
    tile_cols: int
    stored_bytes: int
    shape_us: dict = field(default_factory=dict)     # (W, R, S, P) -> us per call (launchable shapes)
    stored_tuples: int = 0                           # INT quads: tuples the table stores

    def best(self, waves=None):
        items = [(us, s) for s, us in self.shape_us.items() if waves is None or s[0] == waves]
        return min(items) if items else (float("inf"), None)


def legal_ks(payload: int, code_bits: int, ks=None):
    if payload == INT_CODES:
        # 4-bit codes also come in quads over a table of stored tuples (with escapes)
        out = [k for k in (1, 2, 4) if code_bits * k <= 8 or (code_bits == 4 and k == 4)]
    elif payload == BF16_EXP:
        out = [1, 2]          # exponent pairs, with escapes outside the 16 stored exponents
    else:
        out = [1]
    return tuple(k for k in out if ks is None or k in ks)


def stored_tuples_for(log2_m: int) -> tuple:
    """Tuple counts t an INT quad table may store (MINE page, Section 4.2 "Tuning t":
    more stored tuples mean fewer escapes but coarser frequencies): a quarter, half
    and three quarters of the table slots, at most 4096.  On 2.2-bit Laplacian codes
    at M = 2^12, half the slots escape about 0.5% of the codes."""
    M = 1 << log2_m
    return tuple(sorted({min(4096, M // 4), min(4096, M // 2), min(4096, 3 * M // 4)}))


def t_grid(log2_m: int, steps: int = 32) -> tuple:
    """Stored-tuple counts the t search walks over: M / steps apart, up to min(M, 4096)
    (the page increments t one value at a time; M / 32 apart keeps the table builds
    of a large tensor few)."""
    M = 1 << log2_m
    d = max(1, M // steps)
    return tuple(range(d, min(M, 4096) + 1, d))


def t_search(curves: dict, growth: float = 0.01, max_rounds: int = 64):
    """The MINE page's search over the number t of stored values (Section 4.2
    "Tuning t"), per section and jointly for the sections of one launch.
    curves[name] = [(t, bytes, escapes), ...] ascending in t: the size bound (table
    cross-entropy plus the 4-byte records) and the escape count of each t.  Start
    from each section's byte-optimal t; then repeatedly increment the t of the
    section with the most escapes saved per additional byte (a size that does not
    grow counts as infinitely good) until one more increment would grow the launch's
    transfer size by more than `growth` over the round's start, or every t is at its
    cap; record that selection and start the next round from it.  Returns the
    selections [{name: t}], the byte-optimal one first."""
    pos = {n: min(range(len(c)), key=lambda i: (c[i][1], c[i][0])) for n, c in curves.items()}
    total = lambda: sum(curves[n][pos[n]][1] for n in curves)   # noqa: E731
    out = [{n: curves[n][pos[n]][0] for n in curves}]
    for _ in range(max_rounds):
        base = total()
        moved = False
        while True:
            best, best_r = None, -1.0
            for n, c in curves.items():
                i = pos[n]
                if i + 1 >= len(c):
                    continue
                db = c[i + 1][1] - c[i][1]
                de = c[i][2] - c[i + 1][2]
                r = math.inf if db <= 0 else de / db
                if r > best_r or (r == best_r and best is not None and n < best):
                    best, best_r = n, r
            if best is None:
                break
            i = pos[best]
            if total() + (curves[best][i + 1][1] - curves[best][i][1]) > base * (1.0 + growth):
                break
            pos[best] = i + 1
            moved = True
        if not moved:
            # even one increment exceeds the growth allowance: take the best one anyway
            # (the round's selection is then that single step), or stop at the caps
            cand = [(n, pos[n]) for n in curves if pos[n] + 1 < len(curves[n])]
            if not cand:
                break
            def ratio(n):
                c, i = curves[n], pos[n]
                db = c[i + 1][1] - c[i][1]
                return math.inf if db <= 0 else (c[i][2] - c[i + 1][2]) / db
            n = max(cand, key=lambda v: (ratio(v[0]), v[0]))[0]
            pos[n] += 1
        sel = {n: curves[n][pos[n]][0] for n in curves}
        if sel != out[-1]:
            out.append(sel)
        if all(pos[n] + 1 >= len(curves[n]) for n in curves):
            break
    return out


def t_curve(w, scales, log2_m: int, tile_cols: int, ts=None):
    """(t, size bound in bytes, escapes) of INT quads of 4-bit codes over t stored
    tuples, for each t of the grid: one table build each (enc_build_tables)."""
    from . import build_tables
    out = []
    for t in (ts or t_grid(log2_m)):
        c = Coding(INT_CODES, w.shape[0], w.shape[1], 4, 4, log2_m, tile_cols, stored_tuples=t)
        tab = build_tables(c, w)
        out.append((t, size_lower_bound_bytes(tab), int(tab.escapes)))
    return out


def coding_candidates(payload, rows, cols, code_bits=0, ks=None, log2_ms=DEFAULT_LOG2_M,
                      tile_cols=DEFAULT_TILE_COLS, quad_ts=None):
    """Every (k, m, tile width, stored tuples) the format accepts for this tensor
    (stored tuples: INT quads of 4-bit codes, else 0; quad_ts[m] overrides the
    stored-tuple counts tried at table size 2^m, e.g. with the t search's values)."""
    for k in legal_ks(payload, code_bits, ks):
        quads = payload == INT_CODES and code_bits == 4 and k == 4
        for m in log2_ms:
            for tc in tile_cols:
                if tc % 64 or tc % (8 * k) or tc > max(64, ((cols + 63) // 64) * 64):
                    continue
                if payload == BF16_EXP and k == 2 and (cols % 32 or tc > 2048):
                    continue
                if quads and (cols % 64 or tc > 2048):
                    continue
                ts = (quad_ts.get(m, stored_tuples_for(m)) if quad_ts else stored_tuples_for(m)) if quads else (0,)
                for t in ts:
                    yield k, m, tc, t


def _tune_launch(ct: CompressedTensor, x: torch.Tensor, shapes, reps: int, stream: torch.cuda.Stream):
    batch = x.shape[0]
    ws_need = 0
    for w, r, ns, rpb in shapes:
        ct.set_launch(w, r, ns, rpb)
        ws_need = max(ws_need, workspace_size(ct.t, batch))
    ws = torch.zeros(max(ws_need, 1), dtype=torch.uint8, device=x.device)
    y = torch.empty((batch, ct.rows), dtype=torch.float32, device=x.device)
    flat = (ctypes.c_uint32 * (4 * len(shapes)))(*[v for s in shapes for v in s])
    us = (ctypes.c_float * len(shapes))()
    xd = DT_F16 if x.dtype == torch.float16 else DT_BF16
    _check(lib().dec_tune_launch(ctypes.c_void_p(stream.cuda_stream), ctypes.byref(ct.t), x.data_ptr(), xd,
                                 y.data_ptr(), batch, ws.data_ptr(), ws.numel(), flat, len(shapes), reps, us),
           "dec_tune_launch")
    return {tuple(s): float(u) for s, u in zip(shapes, us) if u >= 0}


def tune_tensor(payload: int, w, scales, x: torch.Tensor, code_bits: int = 0, ks=None,
                log2_ms=DEFAULT_LOG2_M, tile_cols=DEFAULT_TILE_COLS, shapes=DEFAULT_SHAPES,
                reps: int = 20, log=None, quad_ts=None):
    """Search the codings of one logical tensor `w` (host array as enc_encode takes it)
    with activations `x` (device [batch, cols]).  Returns the list of Candidates."""
    rows, cols = w.shape
    # two row streams per wave exist for INT codes and FP8 only (INT quads: with fp16
    # activations only): elsewhere a shape asking for two runs as one and would only
    # be timed twice
    one_stream = tuple(s for s in shapes if s[2] == 1)
    if payload not in (INT_CODES, FP8_E4M3):
        shapes = one_stream
    quad_shapes = shapes if x.dtype == torch.float16 else one_stream
    stream = torch.cuda.Stream()
    out = []
    for k, m, tc, t in coding_candidates(payload, rows, cols, code_bits, ks, log2_ms, tile_cols, quad_ts):
        c = Coding(payload, rows, cols, k, code_bits if payload == INT_CODES else 0, m, tc, stored_tuples=t)
        try:
            blob = encode(c, w, scales)
        except EcwError:
            continue          # e.g. more distinct symbols than table slots
        ct = CompressedTensor(blob)
        cand = Candidate(k, m, tc, ct.stored_bytes(), stored_tuples=t)
        with torch.cuda.stream(stream):
            cand.shape_us = _tune_launch(ct, x, quad_shapes if t else shapes, reps, stream)
        stream.synchronize()
        if log:
            us, s = cand.best()
            log(f"  k={k} m={m} tc={tc:4d} t={t:4d} stored={cand.stored_bytes / 1e6:8.3f} MB best {s} {us:8.2f} us")
        out.append(cand)
        del ct
    return out


def pick(cands, waves=None, tie: float = 0.02):
    """Fastest candidate (optionally restricted to one waves-per-block value); within
    `tie` of the fastest, the smallest blob."""
    scored = [(c.best(waves), c) for c in cands]
    scored = [(us, s, c) for (us, s), c in scored if s is not None]
    if not scored:
        return None
    t_min = min(us for us, _, _ in scored)
    near = [(c.stored_bytes, us, s, c) for us, s, c in scored if us <= t_min * (1 + tie)]
    near.sort(key=lambda v: (v[0], v[1]))
    _, us, s, c = near[0]
    return dict(k=c.k, log2_m=c.log2_m, tile_cols=c.tile_cols, waves_per_block=s[0], tiles_per_wave=s[1],
                streams_per_wave=s[2], row_groups_per_block=s[3], us=us, stored_bytes=c.stored_bytes,
                stored_tuples=c.stored_tuples)


def time_group(cts, x: torch.Tensor, reps: int = 20, stream: torch.cuda.Stream | None = None) -> float:
    """Microseconds per grouped launch of CompressedTensors `cts` (current launch
    shapes), timed natively as a captured graph (dec_time_group)."""
    from . import GemvGroup, _tensor_array
    stream = stream or torch.cuda.Stream()
    grp = GemvGroup(cts)
    ys = [torch.empty((x.shape[0], c.rows), dtype=torch.float32, device=x.device) for c in cts]
    ws = grp.workspace(x.shape[0])
    yarr = (ctypes.c_void_p * len(ys))(*[y.data_ptr() for y in ys])
    us = ctypes.c_float(0)
    xd = DT_F16 if x.dtype == torch.float16 else DT_BF16
    # the workspace's zero fill (and x) were enqueued on the current stream: the timed
    # launches on `stream` must not start before them
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        _check(lib().dec_time_group(ctypes.c_void_p(stream.cuda_stream), _tensor_array([c.t for c in cts]),
                                    len(cts), x.data_ptr(), xd, yarr, x.shape[0],
                                    ws.data_ptr() if ws is not None else None,
                                    ws.numel() if ws is not None else 0, reps, ctypes.byref(us)),
               "dec_time_group")
    stream.synchronize()
    return us.value


def burst_us(replay, stream, bursts: int = 5, min_burst_us: float = 400.0):
    """Device microseconds per call of `replay` (a graph replay), by the MINE page's
    timing protocol (Section 4.2 "Tuning Grid"): one warm-up call, then `bursts`
    bursts, each repeating the call until it lasts at least min_burst_us; the median
    burst's time per call.  Returns (us per call, [us per call of each burst], calls
    per burst)."""
    replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    replay()
    e1.record(stream)
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1) * 1e3, 1e-3)
    reps = max(1, int(math.ceil(min_burst_us / one)))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(bursts + 1)]
    evs[0].record(stream)
    for b in range(bursts):
        for _ in range(reps):
            replay()
        evs[b + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[b].elapsed_time(evs[b + 1]) * 1e3 / reps for b in range(bursts)]
    return float(sorted(per)[len(per) // 2]), per, reps


def time_cold(launches, batch: int, steps: int = 0, cold_bytes: float = 512e6):
    """Device microseconds per launch, cold: every launch is a group of compressed
    tensors sharing x; blobs are rotated over >= cold_bytes of device copies, and
    each launch is captured as one graph over all copies and timed by burst_us (median
    of 5 bursts of >= 400 us; `steps` is not used).
    launches: [(name, [(blob, (W, R, S, P)), ...], x_dev)].  Returns
    ({name: us}, {name: [y of the last copy per tensor]})."""
    from . import CompressedTensor, GemvGroup, gemv_group_raw, prepare
    total = sum(prepare(b).blob_bytes for _, members, _ in launches for b, _ in members)
    copies = max(2, int(math.ceil(cold_bytes / max(total, 1))))
    stream = torch.cuda.current_stream()
    us, outs = {}, {}
    for name, members, x in launches:
        groups, wss = [], []
        for _ in range(copies):
            cts = []
            for blob, shape in members:
                ct = CompressedTensor(blob)
                ct.set_launch(*shape)
                cts.append(ct)
            g = GemvGroup(cts)
            groups.append(g)
            wss.append(g.workspace(batch))
        ys = [torch.empty((batch, ct.rows), dtype=torch.float32, device=x.device) for ct in groups[0].tensors]
        for c in range(copies):
            gemv_group_raw([ct.t for ct in groups[c].tensors], x, ys, wss[c])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(copies):
                gemv_group_raw([ct.t for ct in groups[c].tensors], x, ys, wss[c])
        us[name] = burst_us(g.replay, stream)[0] / copies
        outs[name] = [y.cpu().numpy() for y in ys]
        del g, groups, wss
    return us, outs


def _ranked(cands, waves, top):
    """The `top` fastest (candidate, shape) pairs at a given waves per block."""
    items = []
    for c in cands:
        for s, us in c.shape_us.items():
            if s[0] == waves:
                items.append((us, c.stored_bytes, id(c), c, s))
    items.sort(key=lambda v: (v[0], v[1]))
    out, seen = [], set()
    for us, _, cid, c, s in items:
        if cid not in seen:
            seen.add(cid)
            out.append((c, s))
        if len(out) == top:
            break
    return out


def tune_group(specs: dict, cands_by_name: dict, x: torch.Tensor, top: int | None = None,
               tie: float = 0.02, log=None, points: list | None = None, cold: bool = True,
               cold_bytes: float = 512e6, cold_steps: int = 200, reps: int = 20):
    """Tensors sharing one launch (same activations) must share waves per block and
    codes per symbol.  For each common (waves per block, codes per symbol), every
    combination of each member's `top` fastest single-tensor candidates at that
    value (timed warm by tune_tensor), and every launch shape all members can take
    (each with its fastest coding at that shape), is timed as the real grouped launch
    and cold (time_cold over cold_bytes of rotated copies); the fastest group wins
    (ties within `tie`: fewer stored bytes).  A launch of one tensor is searched the
    same way.  cold=False: groups are timed warm (time_group, `reps` graph replays of
    one copy) and a one-tensor launch takes its fastest warm candidate (a quicker
    search for secondary workloads).
    specs[name] = (payload, w, scales, code_bits) re-encodes a candidate.  By default
    `top` keeps the number of timed combinations near 16 per waves-per-block value.
    points: if given, every timed group is appended as (us, stored bytes, picks), the
    material of the launch's speed-size Pareto front."""
    import itertools
    names = list(cands_by_name)
    if top is None:
        top = {1: 16, 2: 4, 3: 2}.get(len(names), 1)
    if len(names) == 1 and not cold:
        if points is not None:
            points.extend((us, nbytes, {names[0]: p}) for us, nbytes, p in tensor_points(cands_by_name[names[0]]))
        return {names[0]: pick(cands_by_name[names[0]], tie=tie)}
    waves = sorted({s[0] for n in names for c in cands_by_name[n] for s in c.shape_us})
    blobs = {}
    stream = torch.cuda.Stream()

    def blob_for(name, c):
        key = (name, c.k, c.log2_m, c.tile_cols, c.stored_tuples)
        if key not in blobs:
            payload, w, scales, cb = specs[name]
            coding = Coding(payload, w.shape[0], w.shape[1], c.k, cb if payload == INT_CODES else 0,
                            c.log2_m, c.tile_cols, stored_tuples=c.stored_tuples)
            blobs[key] = encode(coding, w, scales)
        return blobs[key]

    results = []
    # one launch runs one kernel: its members share the codes per symbol
    ks = sorted(set.intersection(*[{c.k for c in cands_by_name[n]} for n in names]))
    for w, k in itertools.product(waves, ks):
        of_k = {n: [c for c in cands_by_name[n] if c.k == k] for n in names}
        ranked = [_ranked(of_k[n], w, top) for n in names]
        if any(not r for r in ranked):
            continue
        combos = list(itertools.product(*ranked))
        # A group holds more tiles than any member alone, so its best shape may be one
        # no member ranks high alone (e.g. more tiles per wave, to keep every wave of
        # the launch resident at once): also try each shape common to all members,
        # each member with its fastest coding at that shape.
        shapes = set.intersection(*[{s for c in of_k[n] for s in c.shape_us if s[0] == w} for n in names])
        for shape in sorted(shapes):
            combo = []
            for n in names:
                best = min(((c.shape_us[shape], c.stored_bytes, id(c), c) for c in of_k[n]
                            if shape in c.shape_us), default=None)
                combo.append((best[3], shape))
            combo = tuple(combo)
            if combo not in combos:
                combos.append(combo)
        for combo in combos:
            # timed cold, as the launch runs when serving: the members' blobs rotated
            # over >= cold_bytes of device copies (MINE page, Section 4.2: cold-cache
            # measurements, the kernel reproduced until the cache is filled twice)
            members = [(blob_for(n, c), s) for n, (c, s) in zip(names, combo)]
            if cold:
                us = time_cold([("g", members, x)], x.shape[0], cold_steps, cold_bytes)[0]["g"]
            else:
                cts = [CompressedTensor(b, waves_per_block=s[0], tiles_per_wave=s[1], streams_per_wave=s[2],
                                        row_groups_per_block=s[3]) for b, s in members]
                us = time_group(cts, x, reps, stream)
                del cts
            nbytes = sum(c.stored_bytes for c, _ in combo)
            results.append((us, nbytes, combo))
            if points is not None:
                points.append((us, nbytes, {n: _pick_dict(c, s, us) for n, (c, s) in zip(names, combo)}))
            if log:
                log(f"  group W={w}: " + ", ".join(f"{n}:k={c.k},m={c.log2_m},tc={c.tile_cols},R={s[1]},S={s[2]},P={s[3]}"
                                                   for n, (c, s) in zip(names, combo)) + f" -> {us:.2f} us")
    if not results:
        return None
    t_min = min(r[0] for r in results)
    near = sorted([r for r in results if r[0] <= t_min * (1 + tie)], key=lambda r: (r[1], r[0]))
    us, _, combo = near[0]
    return {n: _pick_dict(c, s, us) for n, (c, s) in zip(names, combo)}


def _pick_dict(c: Candidate, s, us: float) -> dict:
    return dict(k=c.k, log2_m=c.log2_m, tile_cols=c.tile_cols, waves_per_block=s[0], tiles_per_wave=s[1],
                streams_per_wave=s[2], row_groups_per_block=s[3], us=round(us, 3), stored_bytes=c.stored_bytes,
                stored_tuples=c.stored_tuples)


# ------------------------------------------------------------------ speed-size trade-off
# MINE page, Section 4.2: the tuner keeps the speed-size Pareto front of every
# section's codings, so that the fastest coding under a memory constraint can be
# chosen later (smaller codings may decode more slowly), and the cross-entropy of a
# table against the histogram is a lower bound on the coded size.

def pareto_front(points):
    """The points (us, bytes, payload) that no other point dominates (no slower and no
    larger, and better in one), sorted by bytes ascending (so us descending).  Of
    equal points the first is kept."""
    out = []
    for p in sorted(points, key=lambda p: (p[1], p[0])):
        if not out or p[0] < out[-1][0]:
            out.append(p)
    return out


def tensor_points(cands):
    """(us, bytes, pick) of every timed (coding, launch shape) of one tensor."""
    return [(us, c.stored_bytes, _pick_dict(c, s, us)) for c in cands for s, us in c.shape_us.items()]


def choose_under_budget(fronts: dict, budget: int):
    """One point per item (fronts[name] = [(us, bytes, payload)]) minimising the summed
    time with summed bytes <= budget: the multiple-choice knapsack, solved exactly by
    merging the items' fronts one at a time and keeping only the Pareto front of the
    partial sums (a dominated partial choice is never part of an optimum that its
    dominator cannot match).  Returns (us, bytes, {name: payload}) or None if no
    choice fits."""
    partial = [(0.0, 0, {})]
    for name, pts in fronts.items():
        merged = [(u + pu, b + pb, {**ch, name: pp}) for u, b, ch in partial for pu, pb, pp in pts
                  if b + pb <= budget]
        partial = pareto_front(merged)
        if not partial:
            return None
    return min(partial, key=lambda p: (p[0], p[1]))


def size_lower_bound_bytes(tables) -> float:
    """Cross-entropy bound of a coding's payload words: sum over symbols of
    count * log2(M / f) bits, from the histogram and frequencies of its tables; with
    escapes (BF16 pairs, INT quads) plus their 4-byte records (MINE page, Section 4.2
    "Tuning t")."""
    import math
    if tables.n_tuples:
        M = sum(int(f) for f in tables.tuple_freq[:tables.n_tuples])
        bits = sum(int(n) * (math.log2(M) - math.log2(int(f)))
                   for n, f in zip(tables.tuple_count[:tables.n_tuples], tables.tuple_freq[:tables.n_tuples]) if n)
        return bits / 8.0 + 4.0 * tables.escapes
    total = 4.0 * 8.0 * tables.escapes
    M = sum(int(f) for f in tables.freq[0])
    for t in range(tables.n_tables):
        m_t = sum(int(f) for f in tables.freq[t]) or M
        for s in range(256):
            n = int(tables.count[t][s])
            if n:
                total += n * (math.log2(m_t) - math.log2(int(tables.freq[t][s])))
    return total / 8.0
