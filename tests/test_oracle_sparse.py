"""Pins for the oracle's sparse decode attention (RFC, vllm-rlt #156, section 3.2).

The formula layer (reference statistics, correction) is pinned by the page's scalar example;
the selection by hand cases with ties and by its defining invariants on random scores; the
whole reference + loop path by the page's m = 1 reduction to dense attention, by the full
reference output being ordinary attention, and by the correction vanishing when a loop's keys
and values equal the reference's.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_scalar_example_of_the_page():
    g = json.load(open(os.path.join(GOLDEN, "sparse_scalar.json")))
    p = np.array(g["p_ref"])
    v = np.array(g["v_ref"])[:, None]
    m, o_ref, c_ref = orc.sparse_stats(p, v, np.array(g["selected"]))
    assert abs(o_ref[0] - g["o_ref"]) < 1e-12
    assert abs(m - g["mass"]) < 1e-12
    assert abs(c_ref[0] - g["c_ref"]) < 1e-12
    assert abs((o_ref[0] - c_ref[0]) - g["unselected_contribution"]) < 1e-12
    out = orc.sparse_correct(np.array(g["p_local"]), np.array(g["v_selected_later"])[:, None], m, o_ref, c_ref)
    assert abs(out[0] - g["o_new"]) < 1e-12


@pytest.mark.parametrize("k,want", [(1, [1]), (2, [1, 2]), (3, [1, 2, 4]), (4, [1, 2, 3, 4]), (5, [0, 1, 2, 3, 4])])
def test_topk_ties_go_to_the_lower_position(k, want):
    assert orc.topk_positions(np.array([1.0, 3.0, 3.0, 2.0, 3.0]), k).tolist() == want


@pytest.mark.parametrize("seed", range(5))
def test_topk_invariants(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 400))
    s = np.round(rng.standard_normal(T) * 4) / 4          # many exact ties
    k = int(rng.integers(1, T + 1))
    sel = orc.topk_positions(s, k)
    assert sel.size == k and np.all(np.diff(sel) > 0)
    rest = np.setdiff1d(np.arange(T), sel)
    if rest.size:
        assert s[sel].min() >= s[rest].max()
        tau = s[sel].min()
        # at the threshold the selected positions are the lowest ones with that score
        eq_sel, eq_rest = sel[s[sel] == tau], rest[s[rest] == tau]
        if eq_rest.size:
            assert eq_sel.max() < eq_rest.min()


def _random_kv(rng, T, H, D, scale=1.0):
    kh = orc.bf16_from_f32((scale * rng.standard_normal((T, H, D))).astype(np.float32))
    vh = orc.bf16_from_f32(rng.standard_normal((T, H, D)).astype(np.float32))
    return kh, vh


def test_all_keys_kept_reduces_to_dense_attention():
    """m = 1 when every key is kept: the loop output is that loop's dense attention."""
    rng = np.random.default_rng(1)
    T, H, Hq, D = 300, 2, 8, 16
    k2, v2 = _random_kv(rng, T, H, D)
    k3, v3 = _random_kv(rng, T, H, D)
    q2 = orc.bf16_from_f32(rng.standard_normal((Hq, D)).astype(np.float32))
    q3 = orc.bf16_from_f32(rng.standard_normal((Hq, D)).astype(np.float32))
    ref = orc.sparse_reference(q2, k2, v2, 0.25, T)
    assert np.allclose(ref.mass, 1.0, atol=1e-12)
    assert np.array_equal(ref.sel, np.tile(np.arange(T, dtype=np.int32), (Hq, 1)))
    assert np.allclose(orc.sparse_loop(q3, k3, v3, 0.25, ref), orc.decode_attn(q3, k3, v3, 0.25), atol=1e-12)


def test_reference_output_is_full_attention_and_stats_match_definition():
    rng = np.random.default_rng(2)
    T, H, Hq, D, k = 200, 2, 4, 8, 17
    k2, v2 = _random_kv(rng, T, H, D, 2.0)
    q = orc.bf16_from_f32(rng.standard_normal((Hq, D)).astype(np.float32))
    ref = orc.sparse_reference(q, k2, v2, 0.5, k)
    assert np.allclose(ref.o_ref, orc.decode_attn(q, k2, v2, 0.5), atol=1e-12)
    kf, vf = orc.f32_from_bf16(k2).astype(np.float64), orc.f32_from_bf16(v2).astype(np.float64)
    qf = orc.f32_from_bf16(q).astype(np.float64)
    for i in range(Hq):
        h = i // (Hq // H)
        s = 0.5 * kf[:, h] @ qf[i]
        p = np.exp(s - s.max())
        p /= p.sum()
        # S holds the k highest probabilities (numpy's stable sort on -p, positions ascending)
        want = np.sort(np.argsort(-s, kind="stable")[:k])
        assert np.array_equal(ref.sel[i], want)
        assert abs(ref.mass[i] - p[want].sum()) < 1e-12
        assert np.allclose(ref.c_ref[i], p[want] @ vf[want, h], atol=1e-12)


def test_unchanged_loop_reproduces_the_reference_output():
    """If a later loop's queries, keys and values equal the reference loop's, the selected
    softmax is the reference probabilities renormalized on S, so C_new = C_ref and the
    corrected output equals O_ref: the correction keeps the contribution outside S."""
    rng = np.random.default_rng(3)
    T, H, Hq, D, k = 257, 1, 2, 32, 40
    k2, v2 = _random_kv(rng, T, H, D, 3.0)
    q = orc.bf16_from_f32(rng.standard_normal((Hq, D)).astype(np.float32))
    ref = orc.sparse_reference(q, k2, v2, 0.2, k)
    assert np.all(ref.mass < 1.0)
    assert np.allclose(orc.sparse_loop(q, k2, v2, 0.2, ref), ref.o_ref, atol=1e-12)


def test_given_selection_and_scores_agree_with_the_reference():
    rng = np.random.default_rng(4)
    T, H, Hq, D, k = 150, 2, 4, 8, 20
    k2, v2 = _random_kv(rng, T, H, D, 2.0)
    q = orc.bf16_from_f32(rng.standard_normal((Hq, D)).astype(np.float32))
    ref = orc.sparse_reference(q, k2, v2, 0.4, k)
    given = orc.sparse_reference_given(q, k2, v2, 0.4, ref.sel)
    assert np.allclose(given.mass, ref.mass, atol=1e-15) and np.allclose(given.c_ref, ref.c_ref, atol=1e-13)
    s = orc.attn_scores(q, k2, 0.4)
    for i in range(Hq):
        assert np.array_equal(orc.topk_positions(s[i], k), ref.sel[i])
