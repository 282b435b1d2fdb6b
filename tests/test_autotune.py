"""Autotuner: candidate enumeration and selection rules (CPU), device timing (GPU)."""
import ctypes

import numpy as np
import pytest
import torch

import entropy_coded_weight_amd as ecw
from entropy_coded_weight_amd import autotune as A
from tests import cases


def test_candidates_respect_the_format():
    got = list(A.coding_candidates(ecw.INT_CODES, 256, 1024, code_bits=4))
    # 16-level codes: one or two per symbol, or quads over a table of stored tuples
    # (a quarter, half or three quarters of the table's slots); tile widths must be
    # multiples of 64 and of 8k
    assert {k for k, _, _, _ in got} == {1, 2, 4}
    assert all(tc % 64 == 0 for _, _, tc, _ in got)
    assert all(t in ((1 << m) // 4, (1 << m) // 2, 3 * (1 << m) // 4) if k == 4 else t == 0 for k, m, _, t in got)
    assert len(got) == 2 * 3 * 4 + 3 * 3 * 4
    got2 = list(A.coding_candidates(ecw.INT_CODES, 64, 256, code_bits=2, log2_ms=(10,), tile_cols=(64, 128)))
    assert {k for k, _, _, _ in got2} == {1, 2, 4} and all(t == 0 for *_, t in got2)
    # tiles wider than the (64-rounded) row are pointless
    assert all(tc <= 256 for _, _, tc, _ in got2)
    # quads: cols a multiple of 64, slices up to 2048 (the record's column field)
    assert not [c for c in A.coding_candidates(ecw.INT_CODES, 64, 4096, code_bits=4, ks=(4,), tile_cols=(4096,))]
    assert A.stored_tuples_for(13) == (2048, 4096) and A.stored_tuples_for(12) == (1024, 2048, 3072)
    # BF16: one exponent per symbol, or a pair (cols a multiple of 32, slices up to 2048)
    assert list(A.coding_candidates(ecw.BF16_EXP, 64, 512, log2_ms=(12,), tile_cols=(256,))) == [(1, 12, 256, 0),
                                                                                                (2, 12, 256, 0)]
    assert list(A.coding_candidates(ecw.BF16_EXP, 64, 528, log2_ms=(12,), tile_cols=(256,))) == [(1, 12, 256, 0)]
    assert list(A.coding_candidates(ecw.FP8_E4M3, 64, 512, log2_ms=(12,), tile_cols=(256,))) == [(1, 12, 256, 0)]


def _cand(k, m, tc, nbytes, shapes):
    c = A.Candidate(k, m, tc, nbytes)
    c.shape_us = shapes
    return c


def test_pick_prefers_speed_then_size_within_tie():
    a = _cand(2, 12, 128, 1000, {(16, 1, 1, 1): 10.0, (8, 1, 1, 1): 12.0})
    b = _cand(2, 11, 128, 900, {(16, 1, 1, 1): 10.1})          # within 2%, smaller: wins
    c = _cand(2, 10, 128, 500, {(16, 1, 1, 1): 11.0})          # 10% slower: loses despite size
    p = A.pick([a, b, c])
    assert (p["log2_m"], p["waves_per_block"], p["stored_bytes"]) == (11, 16, 900)
    p8 = A.pick([a, b, c], waves=8)
    assert (p8["log2_m"], p8["waves_per_block"]) == (12, 8)
    assert A.pick([_cand(2, 12, 64, 1, {})]) is None


def test_ranked_takes_the_fastest_shapes_per_candidate():
    a = _cand(2, 12, 128, 1, {(16, 1, 1, 1): 10.0, (16, 2, 1, 1): 9.0, (8, 1, 1, 1): 11.0})
    b = _cand(2, 11, 128, 1, {(16, 1, 1, 1): 9.5})
    r = A._ranked([a, b], 16, 2)
    assert [(c.log2_m, s) for c, s in r] == [(12, (16, 2, 1, 1)), (11, (16, 1, 1, 1))]
    assert A._ranked([a, b], 4, 2) == []


def test_tune_rejects_null_stream_without_launching():
    case = cases.small_cases()[1]
    ct = ecw.prepare(ecw.encode(case.lib_coding(), case.logical, case.scales))
    us = (ctypes.c_float * 1)()
    shapes = (ctypes.c_uint32 * 4)(4, 1, 1, 1)
    st = ecw.lib().dec_tune_launch(None, ctypes.byref(ct), None, ecw.DT_F16, None, 1, None, 0, shapes, 1, 5, us)
    assert st == 1   # ECW_E_INVALID_ARG


@pytest.mark.gpu
def test_device_tuning_picks_a_shape_that_stays_correct():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oracle import gemv, pipeline as P
    case = cases._int("tune", 256, 2048, 2, 4, 11, 128, seed=21)
    rng = np.random.default_rng([0, 901])
    xh = rng.standard_normal((1, case.cols)).astype(np.float16)
    x = torch.from_numpy(xh).cuda()
    cands = A.tune_tensor(ecw.INT_CODES, case.logical, case.scales, x, code_bits=4, ks=(2,),
                          log2_ms=(11, 12), tile_cols=(128, 256), shapes=((4, 1, 1, 1), (8, 1, 1, 2), (16, 2, 2, 1)), reps=5)
    assert len(cands) == 4 and all(c.shape_us for c in cands)
    # a two-member group of the same tensor shares one waves-per-block value
    g = A.tune_group({"a": (ecw.INT_CODES, case.logical, case.scales, 4),
                      "b": (ecw.INT_CODES, case.logical, case.scales, 4)}, {"a": cands, "b": cands}, x,
                     top=1, cold_bytes=32e6, cold_steps=40)
    assert g["a"]["waves_per_block"] == g["b"]["waves_per_block"]
    p = A.pick(cands)
    c = ecw.Coding(ecw.INT_CODES, case.rows, case.cols, p["k"], 4, p["log2_m"], p["tile_cols"])
    ct = ecw.CompressedTensor(ecw.encode(c, case.logical, case.scales), waves_per_block=p["waves_per_block"],
                              tiles_per_wave=p["tiles_per_wave"], streams_per_wave=p["streams_per_wave"],
                              row_groups_per_block=p["row_groups_per_block"])
    y = ct.gemv(x).cpu().numpy()
    wv = P.weight_values(case.oracle_coding(), case.logical, case.scales)
    ok, worst = gemv.check(y, wv, gemv.x_values(xh, "f16"))
    assert ok, worst


# ------------------------------------------------------------------ speed-size trade-off
def _dominated(p, q):
    return q[0] <= p[0] and q[1] <= p[1] and (q[0] < p[0] or q[1] < p[1])


@pytest.mark.parametrize("seed", range(6))
def test_pareto_front_is_the_set_of_undominated_points(seed):
    rng = np.random.default_rng([0, 77, seed])
    pts = [(float(rng.integers(1, 20)), int(rng.integers(1, 20)), i) for i in range(40)]
    front = A.pareto_front(pts)
    undominated = {(u, b) for u, b, _ in pts if not any(_dominated((u, b), (qu, qb)) for qu, qb, _ in pts)}
    assert {(u, b) for u, b, _ in front} == undominated
    assert len(front) == len(undominated)                     # one point per (us, bytes)
    assert all(front[i][1] < front[i + 1][1] and front[i][0] > front[i + 1][0] for i in range(len(front) - 1))


@pytest.mark.parametrize("seed", range(8))
def test_budget_choice_is_the_exact_knapsack_optimum(seed):
    import itertools
    rng = np.random.default_rng([0, 78, seed])
    fronts = {f"t{i}": [(float(rng.uniform(1, 10)), int(rng.integers(1, 30)), j) for j in range(int(rng.integers(1, 6)))]
              for i in range(4)}
    lo = sum(min(b for _, b, _ in pts) for pts in fronts.values())
    hi = sum(max(b for _, b, _ in pts) for pts in fronts.values())
    for budget in (lo - 1, lo, (lo + hi) // 2, hi):
        best = None
        for combo in itertools.product(*fronts.values()):
            b = sum(p[1] for p in combo)
            u = sum(p[0] for p in combo)
            if b <= budget and (best is None or u < best):
                best = u
        got = A.choose_under_budget(fronts, budget)
        if best is None:
            assert got is None
        else:
            assert got[0] == pytest.approx(best, abs=1e-9) and got[1] <= budget
            assert sum(fronts[n][[p[2] for p in fronts[n]].index(ch)][1] for n, ch in got[2].items()) == got[1]


def test_size_lower_bound_is_the_tables_cross_entropy():
    from oracle import coding as OC, pipeline as P
    # with escapes (MINE page, Section 4.2 "Tuning t"): plus 4 bytes per record
    names = ("bf16_pairs_m12", "bf16_pairs_mixed_ragged", "quads_t2048_m12", "quads_t64_m10_ragged")
    escaped = 0
    for case in cases.small_cases()[:3] + [c for c in cases.small_cases() if c.name in names]:
        t = ecw.build_tables(case.lib_coding(), case.logical)
        lb = A.size_lower_bound_bytes(t)
        comp = P.encode(case.oracle_coding(), case.logical, case.scales)
        _, _, corr = P._decode_all(comp)
        n_rec = sum(len(r) for lanes in corr.values() for r in lanes)
        assert n_rec == t.escapes
        escaped += n_rec
        assert lb == pytest.approx(OC.cross_entropy_total_bits(comp.counts[0], comp.freq[0], case.log2_m) / 8
                                   + 4 * n_rec, rel=1e-12)
        # the final states carry the last bits of information: the bound holds for the
        # words plus the tile metadata
        tt = ecw.prepare(ecw.encode(case.lib_coding(), case.logical, case.scales, t))
        assert lb <= tt.bytes_words + tt.bytes_tile_meta
    assert escaped > 0


# ------------------------------------------------------------------ the t search
def _brute_best(curves, start, budget):
    """Fewest total escapes over every selection with each section at or above its
    start index and total bytes within budget (exhaustive)."""
    import itertools
    names = sorted(curves)
    best = None
    for idx in itertools.product(*[range(start[n], len(curves[n])) for n in names]):
        b = sum(curves[n][i][1] for n, i in zip(names, idx))
        if b > budget:
            continue
        e = sum(curves[n][i][2] for n, i in zip(names, idx))
        if best is None or e < best:
            best = e
    return best


def test_t_search_matches_brute_force_on_unit_steps():
    # MINE page, Section 4.2 "Tuning t": from the byte-optimal t, increment the t with
    # the most escapes saved per additional byte until the transfer would grow by more
    # than 1%.  With every increment costing the same bytes and savings that shrink
    # with t, the greedy choice is optimal: each round's selection has the fewest
    # escapes of all selections (from the round's start) within the round's budget.
    rng = np.random.default_rng(7)
    for trial in range(40):
        curves = {}
        for n in ("gate", "up", "down")[: 1 + trial % 3]:
            steps = int(rng.integers(3, 7))
            saved = np.sort(rng.integers(1, 400, steps))[::-1]          # shrinking savings
            esc = [int(5000 + saved.sum())]
            for sv in saved:
                esc.append(esc[-1] - int(sv))
            base_bytes = float(rng.integers(80_000, 120_000))
            # a few increments that shrink the size first (the byte-optimal start is
            # past them), then equal steps of 250 bytes
            lead = int(rng.integers(0, 3))
            sizes = [base_bytes + 100 * (lead - i) for i in range(lead)] + \
                    [base_bytes + 250 * i for i in range(steps + 1 - lead)]
            curves[n] = [(64 * (i + 1), sizes[i], esc[i]) for i in range(steps + 1)]
        sels = A.t_search(curves)
        start = {n: min(range(len(c)), key=lambda i: (c[i][1], c[i][0])) for n, c in curves.items()}
        assert sels[0] == {n: curves[n][start[n]][0] for n in curves}   # the byte-optimal start
        pos = dict(start)
        for sel in sels[1:]:
            new = {n: [t for t, _, _ in curves[n]].index(sel[n]) for n in curves}
            base = sum(curves[n][pos[n]][1] for n in curves)
            got_b = sum(curves[n][new[n]][1] for n in curves)
            got_e = sum(curves[n][new[n]][2] for n in curves)
            assert all(new[n] >= pos[n] for n in curves)
            if got_b <= base * 1.01:
                assert got_e == _brute_best(curves, pos, base * 1.01)
            else:
                # no increment fits the allowance: the round takes exactly one step
                assert sum(new[n] - pos[n] for n in curves) == 1
            pos = new


def test_t_curve_escapes_match_the_oracle():
    # the size/escape curve the t search walks: the library's escape count for each t
    # equals the number of codes the oracle's stored-tuple mapping sets to 0
    from oracle import symbols as S
    case = cases._int("tq", 128, 512, 4, 4, 10, 128, seed=61)
    q = case.logical
    tup = S.quad_tuples(q)
    counts = np.bincount(tup.ravel(), minlength=1 << 16)
    for t, nbytes, esc in A.t_curve(q, case.scales, 10, 128, ts=(1, 16, 128, 512, 1024)):
        stored = S.quad_stored(counts, t)
        ids, _ = S.quad_map(tup, stored)
        coded = S.quad_join(ids, stored)
        assert esc == int(np.count_nonzero(coded != q)), t
        assert nbytes >= 4 * esc
