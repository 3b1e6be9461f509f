"""Pins for the token-selection oracle (FlashLoop integration RFC, vllm-rlt #156, sections 3.1
and 6.2): values the RFC prints, closed forms, the summation order, the tie rule, budgets
against the window length, and brute-force invariants on small inputs."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import selection as sel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(values, d=None):
    """Exact BF16 bit patterns of values that BF16 represents (rows padded with zeros to d)."""
    a = np.asarray(values, np.float32)
    if d is not None and a.shape[-1] < d:
        a = np.concatenate([a, np.zeros(a.shape[:-1] + (d - a.shape[-1],), np.float32)], axis=-1)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not representable in BF16"
    return (bits >> 16).astype(np.uint16)


def test_rfc_eight_token_example():
    """RFC 3.1's eight-token window: budgets 4 and 2 select t2, t4, t6, t8, then t4 and t8.
    The hidden states are built so that even tokens change most from loop 1 to 2, and t4 and t8
    most from loop 2 to 3; the loop-4 budget is 25 % of the window's 8 tokens (2), not of the 4
    tokens still active (which would give 1)."""
    g = json.load(open(os.path.join(GOLDEN, "token_selection_8tok.json")))
    T, W = g["T"], g["window"]
    a = np.array([0.25, 1, 0.25, 1, 0.25, 1, 0.25, 1], np.float32)   # loop 1 -> 2 change
    b = np.array([1, 0.5, 1, 2, 1, 0.5, 1, 2], np.float32)            # loop 2 -> 3 change
    H1 = np.ones(T, np.float32)
    H2 = H1 + a
    H3 = H2 + b
    h = [bf16(x[:, None], d=16) for x in (H1, H2, H3)]
    _, act3 = sel.select_rows(h[1], h[0], None, W, g["budget_pct"][0], 1e-6)
    _, act4 = sel.select_rows(h[2], h[1], act3, W, g["budget_pct"][1], 1e-6)
    assert list(act3 + 1) == g["active_one_based"]["loop 3"]
    assert list(act4 + 1) == g["active_one_based"]["loop 4"]
    assert [len(act3), len(act4)] == g["budget_tokens"]
    assert sel.select_count(T, W, g["budget_pct"][:1]) == 4
    assert sel.select_count(T, W, g["budget_pct"]) == 2


def test_scores_closed_forms():
    """3-4-5 triangles: the denominator is the norm of H[r-1] (5), not of H[r-2]; epsilon
    replaces a zero norm."""
    h1 = bf16([[3, 4], [3, 4], [0, 0], [3, 4]], d=8)
    h2 = bf16([[0, 0], [3, 0], [3, 4], [3, 4]], d=8)
    s = sel.change_scores(h1, h2, 0.5)
    assert s[0] == np.float32(1.0)
    assert s[1] == np.float32(0.8)                     # RN32(4 / 5)
    assert s[2] == np.float32(10.0)                    # 5 / max(0, 0.5)
    assert s[3] == np.float32(0.0)


def test_sum_of_squares_is_pairwise():
    """Squares [1, 2^-24 x 15]: in pairwise order 1 + 2^-24 rounds to 1 (tie to even) but the
    small terms first pair up (2^-23, 2^-22, ...), and the total is 1 + 14 * 2^-24 exactly; its
    square root rounds to 1 + 3 * 2^-23 (just below the midpoint 1 + 3.5 * 2^-23).  A running
    sum from the first term would stay at 1 and give a score of exactly 1."""
    h1 = bf16([[1.0] + [0.0] * 15])
    h2 = bf16([[0.0] + [-(2.0 ** -12)] * 15])
    assert sel.pairwise_sum_f32(np.array([1.0] + [2.0 ** -24] * 15, np.float32)) == np.float32(1 + 14 * 2.0 ** -24)
    s = sel.change_scores(h1, h2, 1e-6)
    assert s[0] == np.float32(1 + 3 * 2.0 ** -23)
    # 1 + 7 * 2^-23 lies strictly between the squares of 1 + 3 * 2^-23 and of the midpoint
    lo, mid = Fraction(1) + Fraction(3, 2 ** 23), Fraction(1) + Fraction(7, 2 ** 24)
    assert lo * lo < Fraction(1) + Fraction(7, 2 ** 23) < mid * mid


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 100, 4096, 4100])
def test_pairwise_sum_error_bound(n):
    """Within the pairwise bound ceil(log2 n) * 2^-24 * sum|x| of the exact sum; exact for
    small integers (any order)."""
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n).astype(np.float32) ** 2
    exact = math.fsum(float(v) for v in x)
    bound = max(1, math.ceil(math.log2(n))) * 2.0 ** -24 * float(np.abs(x).sum()) * 1.0001
    assert abs(float(sel.pairwise_sum_f32(x)) - exact) <= bound
    ints = np.arange(n, dtype=np.float32) % 7
    assert float(sel.pairwise_sum_f32(ints)) == float(ints.sum(dtype=np.float64))


def test_scores_near_binary64_values():
    """Random rows: binary32 scores within (log2 d + 8) * 2^-24 relative of the binary64 value."""
    rng = np.random.default_rng(3)
    T, d = 50, 520
    h1 = (rng.standard_normal((T, d)) * rng.uniform(0.1, 10, (T, 1))).astype(np.float32)
    h2 = h1 + (rng.standard_normal((T, d)) * rng.uniform(0.001, 1, (T, 1))).astype(np.float32)
    b1, b2 = bf16_round(h1), bf16_round(h2)
    s = sel.change_scores(b1, b2, 1e-6).astype(np.float64)
    a = sel.f32_of_bf16(b1).astype(np.float64)
    c = sel.f32_of_bf16(b2).astype(np.float64)
    ref = np.linalg.norm(a - c, axis=1) / np.linalg.norm(a, axis=1)
    assert np.all(np.abs(s - ref) <= (math.log2(d) + 8) * 2.0 ** -24 * ref)


def bf16_round(x):
    """RNE of binary32 to BF16 bit patterns (input generation only)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def test_equal_scores_go_to_the_lower_position():
    """Identical rows score identically; the budget boundary falls inside the group."""
    T, d = 12, 8
    h1 = np.tile(bf16([[1.0]], d=d), (T, 1))
    h2 = np.tile(bf16([[0.5]], d=d), (T, 1))             # score 0.5 everywhere ...
    h2[[3, 9]] = bf16([[0.25]], d=d)                        # ... but 0.75 at positions 3 and 9
    _, rows = sel.select_rows(h1, h2, None, T, 50, 1e-6)    # 6 of 12
    assert list(rows) == [0, 1, 2, 3, 4, 9]
    _, rows = sel.select_rows(h1, h2, None, 6, 50, 1e-6)    # windows of 6: 3 each
    assert list(rows) == [0, 1, 3, 6, 7, 9]


def _brute_force_check(h1, h2, prev, W, pct, eps, scores, rows):
    T = h1.shape[0]
    elig = list(range(T)) if prev is None else list(prev)
    score_of = dict(zip(elig, scores))
    chosen = set(int(p) for p in rows)
    assert chosen <= set(elig)                                     # nested
    assert list(rows) == sorted(chosen)                            # ascending, distinct
    for w0 in range(0, T, W):
        length = min(W, T - w0)
        e = [p for p in elig if w0 <= p < w0 + length]
        c = [p for p in e if p in chosen]
        assert len(c) == min(math.ceil(pct * length / 100), len(e))
        for s in c:                                                # every chosen beats every other
            for u in e:
                if u not in chosen:
                    assert (score_of[s], -s) > (score_of[u], -u)


@pytest.mark.parametrize("T,W,d,pcts,seed", [
    (37, 8, 16, [50, 25], 0), (64, 64, 24, [25, 10], 1), (100, 7, 8, [60, 30, 0], 2),
    (20, 30, 40, [50, 50], 3), (33, 1, 8, [100, 0], 4),
])
def test_nested_selection_brute_force(T, W, d, pcts, seed):
    """Per window: the budget count, nesting, and that every chosen token outranks every
    eligible unchosen one (score, then lower position), checked pair by pair."""
    rng = np.random.default_rng(seed)
    hs = [bf16_round(rng.standard_normal((T, d)).astype(np.float32))]
    for _ in range(len(pcts) + 1):
        step = (rng.standard_normal((T, d)) * rng.uniform(0, 1, (T, 1))).astype(np.float32)
        hs.append(bf16_round(sel.f32_of_bf16(hs[-1]) + step))
    hs[2][::5] = hs[1][::5]                        # some tokens unchanged: score 0, ties
    prev = None
    for i, p in enumerate(pcts):
        scores, rows = sel.select_rows(hs[i + 2], hs[i + 1], prev, W, p, 1e-6)
        _brute_force_check(hs[i + 2], hs[i + 1], prev, W, p, 1e-6, scores, rows)
        assert len(rows) == sel.select_count(T, W, pcts[:i + 1])
        prev = rows
    slot = sel.slot_map(prev, T)
    assert all(slot[p] == j for j, p in enumerate(prev))
    assert int((slot >= 0).sum()) == len(prev)


def test_budget_rounding_and_short_last_window():
    """ceil(pct * len / 100) per window; the last window may be shorter (RFC 3.1, 6.1)."""
    assert sel.window_budget(7, 25) == 2 and sel.window_budget(8, 25) == 2 and sel.window_budget(9, 25) == 3
    assert sel.window_budget(10, 10) == 1 and sel.window_budget(11, 10) == 2 and sel.window_budget(5, 0) == 0
    assert sel.select_count(20, 8, [25]) == 2 + 2 + 1       # windows of 8, 8, 4
    assert sel.select_count(20, 8, [100]) == 20
    assert sel.select_count(20, 8, [50, 100]) == 4 + 4 + 2  # nested: never more than still active


def test_partition_rfc_example():
    g = json.load(open(os.path.join(GOLDEN, "row_partition.json")))
    names = g["rows"]
    cls = [sel.ROW_DECODE if n.startswith("D") else
           sel.ROW_ACTIVE if n in g["active_prefill"] else sel.ROW_INACTIVE for n in names]
    gather, scatter, (split, total) = sel.partition_rows(cls)
    assert [names[i] for i in gather] == g["gathered"]
    assert split == g["split_offset"] and total == len(g["gathered"])
    for i, n in enumerate(names):
        assert scatter[i] == (g["gathered"].index(n) if n in g["gathered"] else -1)


def test_partition_is_stable_and_complete():
    rng = np.random.default_rng(9)
    cls = rng.integers(0, 3, 1000)
    gather, scatter, (split, total) = sel.partition_rows(cls)
    assert np.all(cls[gather[:split]] == sel.ROW_DECODE) and np.all(cls[gather[split:]] == sel.ROW_ACTIVE)
    assert np.all(np.diff(gather[:split]) > 0) and np.all(np.diff(gather[split:]) > 0)
    assert total == int((cls != sel.ROW_INACTIVE).sum())
    assert np.all(scatter[gather] == np.arange(total)) and np.all(scatter[cls == sel.ROW_INACTIVE] == -1)
    assert sel.partition_rows([])[2] == (0, 0)


def _exact_ratio(h1, h2, eps):
    """Exact squared change scores ||h1 - h2||^2 / max(||h1||^2, eps^2) per row, as Fractions.
    BF16 values are dyadic rationals: scaled by 2^140 they are integers, so the sums of squares
    are exact big-integer sums."""
    a = sel.f32_of_bf16(h1).astype(np.float64) * 2.0 ** 140
    b = sel.f32_of_bf16(h2).astype(np.float64) * 2.0 ** 140
    e2 = Fraction(float(np.float32(eps))) ** 2 * Fraction(2) ** 280
    out = []
    for ra, rb in zip(a.tolist(), b.tolist()):
        ia = [int(v) for v in ra]
        ib = [int(v) for v in rb]
        num = sum((x - y) * (x - y) for x, y in zip(ia, ib))
        den = sum(x * x for x in ia)
        out.append(Fraction(num) / max(Fraction(den), e2))
    return out


@pytest.mark.parametrize("seed,T,d,W,pcts", [(0, 1600, 64, 256, [50, 25]), (1, 1200, 96, 100, [30, 10]),
                                             (2, 700, 136, 64, [50, 50])])
def test_selection_matches_exact_top_k(seed, T, d, W, pcts):
    """The selected sets against exact arithmetic.  Each score is a square root of an exact
    rational (squared norm ratio), so ranking by the exact squared ratios is exact.  Wherever a
    window's exact k-th and (k+1)-th squared ratios are separated by more than the binary32
    error of the score ((log2 d + 8) * 2^-24 relative, squared), the oracle must choose exactly
    the exact top k of that window (RFC 3.1: highest scores, equal scores by lower position)."""
    rng = np.random.default_rng(100 + seed)
    hs = [bf16_round(rng.standard_normal((T, d)).astype(np.float32) * 3)]
    for _ in range(len(pcts) + 1):
        step = (rng.standard_normal((T, d)) * np.exp(rng.uniform(np.log(1e-3), 0, (T, 1)))).astype(np.float32)
        hs.append(bf16_round(sel.f32_of_bf16(hs[-1]) + step))
    delta = Fraction(math.ceil(math.log2(d)) + 8, 2 ** 24)
    lo, hi = (1 - delta) ** 2, (1 + delta) ** 2
    prev, decided, windows = None, 0, 0
    for i, p in enumerate(pcts):
        _, rows = sel.select_rows(hs[i + 2], hs[i + 1], prev, W, p, 1e-6)
        elig = np.arange(T, dtype=np.int32) if prev is None else prev
        ratio = dict(zip(elig.tolist(), _exact_ratio(hs[i + 2][elig], hs[i + 1][elig], 1e-6)))
        chosen = set(rows.tolist())
        for w0 in range(0, T, W):
            length = min(W, T - w0)
            e = [q for q in elig.tolist() if w0 <= q < w0 + length]
            k = min(sel.window_budget(length, p), len(e))
            got = sorted(q for q in e if q in chosen)
            assert len(got) == k
            ranked = sorted(e, key=lambda q: (-ratio[q], q))
            if not 0 < k < len(e):
                continue
            windows += 1
            if ratio[ranked[k - 1]] * lo > ratio[ranked[k]] * hi:
                assert got == sorted(ranked[:k]), f"window {w0}, loop {i + 3}"
                decided += 1
        prev = rows
    assert windows > 0 and decided >= 0.8 * windows     # the comparison is not vacuous
