"""Pins for the CPU oracle: checks that do not route through the oracle's own formulas.

Each test ties the oracle to something fixed outside it: an independent library
conversion (torch BF16, numpy binary16), a value the pages state (tests/golden/*.json,
each with its citation), brute force over all 16 codes, a closed form, or an invariant of
the method (error bound, lossless grid, inheritance, K/V grouping duality).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16(vals):
    """BF16 bits of binary32 values via torch's conversion (independent of the oracle)."""
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32(bits):
    return orc.f32_from_bf16(bits)


def params_split(p):
    p = np.asarray(p, np.uint32)
    m = (p & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    s = (p >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    return m, s


def unpack_codes(codes):
    c = np.asarray(codes, np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = c & 0xF
    out[..., 1::2] = c >> 4
    return out


# --------------------------------------------------------------------------- conversions

def _random_patterns(n, seed):
    g = np.random.default_rng(seed)
    u = g.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    # structured patterns at every rounding boundary of BF16: each upper half with the
    # lower half just below, at and above the midpoint, plus 0 and all-ones
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    s = (hi[:, None] | lows[None, :]).ravel()
    return np.concatenate([u, s])


def test_bf16_conversion_matches_torch():
    u = _random_patterns(1 << 21, 1)
    x = u.view(np.float32)
    finite = np.isfinite(x)
    ours = orc.bf16_from_f32(x[finite])
    ref = torch.from_numpy(x[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_conversion_matches_numpy():
    u = _random_patterns(1 << 21, 2)
    x = u.view(np.float32)
    # add every binary16 midpoint and its binary32 neighbours (tie cases and near-ties)
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    a = h.view(np.float16).astype(np.float64)
    b = np.append(a[1:], 65536.0)
    mid = ((a + b) / 2).astype(np.float32)
    extra = np.concatenate([mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0)),
                            -mid])
    x = np.concatenate([x, extra])
    x = x[np.isfinite(x)]
    ours = orc.f16_from_f32(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_widening_exhaustive():
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    ours = orc.f32_from_f16(h)
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok].view(np.uint32), ref[ok].view(np.uint32))
    assert np.all(np.isnan(ours[~ok]))


def test_bf16_subset_of_f16_band():
    """Every BF16 value with 2^-17 <= |x| <= 65280 is exact in binary16, so the FP16 minimum
    of a group on that band equals its BF16 minimum bit for bit."""
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    x = f32(b)
    band = np.isfinite(x) & (np.abs(x) >= 2.0**-17) & (np.abs(x) <= 65280)
    back = orc.f32_from_f16(orc.f16_from_f32(x[band]))
    assert band.sum() > 8000
    assert np.array_equal(back.view(np.uint32), x[band].view(np.uint32))


# --------------------------------------------------------------------------- golden values

def test_rounding_ties_golden():
    g = golden("rounding_ties.json")
    vals = np.zeros(64, np.float32)
    vals[: len(g["values"])] = g["values"]
    # V: one group along the 64 channels of one row
    x = bf16(vals).reshape(1, 1, 64)
    codes, params = orc.quantize(orc.V, x)
    c = unpack_codes(codes).ravel()
    assert list(c[: len(g["values"])]) == g["expected_codes"]
    m, s = params_split(params)
    assert m.ravel()[0] == g["expected_min"] and s.ravel()[0] == g["expected_scale"]
    # K: the same values down 64 rows of one channel give the same codes
    xk = bf16(vals).reshape(64, 1, 1).repeat(2, axis=2)
    ck, pk = orc.quantize(orc.K, xk)
    assert list(unpack_codes(ck)[: len(g["values"]), 0, 0]) == g["expected_codes"]
    assert list(unpack_codes(ck)[: len(g["values"]), 0, 1]) == g["expected_codes"]


def test_nibble_order_golden():
    g = golden("nibble_order.json")
    codes = np.array(g["codes"], np.float32)
    # integer-valued groups are on the grid min=0, scale=1 once 0 and 15 are present
    vals = np.zeros(64, np.float32)
    vals[: len(codes)] = codes
    vals[62], vals[63] = 0.0, 15.0
    packed, _ = orc.quantize(orc.V, bf16(vals).reshape(1, 1, 64))
    assert list(packed.ravel()[: len(g["expected_bytes"])]) == g["expected_bytes"]
    assert packed.ravel()[31] == 0xF0


def test_storage_closed_forms_golden():
    g = golden("storage.json")
    H, D, n = 8, 128, 4096
    for kind in (orc.K, orc.V):
        bits = 8 * (orc.codes_bytes(H, D, n) + orc.params_bytes(kind, H, D, n)) / (n * H * D)
        assert bits == g["bits_per_element"]
    # V at D = 96 pays a second (half) group per row: 4 + 64/96 bits
    assert 8 * (orc.codes_bytes(1, 96, 10) + orc.params_bytes(orc.V, 1, 96, 10)) / 960 == pytest.approx(4 + 64 / 96)
    ratio = (4 * 16) / (sum(g["retention"]) * 4)
    assert abs(ratio - g["payload_ratio"]) <= g["payload_ratio_tolerance"]
    # the same ratio from the oracle's stream sizes on a dense-vs-retained chain (codes only)
    N = 1000 * 64
    codes_bits = sum(8 * orc.codes_bytes(1, 64, int(round(1000 * r))) for r in g["retention"])
    assert abs(4 * N * 16 / codes_bits - g["payload_ratio"]) <= g["payload_ratio_tolerance"]


def test_actual_stream_bytes_match_closed_forms():
    g = np.random.default_rng(5)
    for kind in (orc.K, orc.V):
        for (n, H, D) in [(1, 1, 64), (65, 3, 96), (130, 2, 32), (64, 1, 200)]:
            x = bf16(g.standard_normal((n, H, D)))
            codes, params = orc.quantize(kind, x)
            assert codes.nbytes == orc.codes_bytes(H, D, n) == n * H * D // 2
            assert params.nbytes == orc.params_bytes(kind, H, D, n)
            ng = math.ceil(n / 64) * H * D if kind == orc.K else n * H * math.ceil(D / 64)
            assert params.nbytes == 4 * ng


def test_predecessor_golden():
    g = golden("predecessor.json")
    D = 64
    x1 = np.zeros(D, np.float32)
    x1[1] = 15.0
    x1[5] = g["x1"]
    X1 = bf16(x1).reshape(1, 1, D)
    base, recon = orc.encode_base(orc.V, X1)
    assert f32(recon)[0, 0, 5] == g["x1_hat"]
    x2 = f32(recon).ravel().copy()
    x2[5] = g["x2"]
    x2[9] = f32(recon).ravel()[9] + 15 * g["residual"]   # residual group max: scale = residual
    X2 = bf16(x2).reshape(1, 1, D)
    res = orc.encode_residual(orc.V, X2, None, recon)
    m, s = params_split(res.params)
    assert s.ravel()[0] == g["residual"] and m.ravel()[0] == 0.0
    assert unpack_codes(res.codes).ravel()[5] == 1          # residual 0.125 = 1 * scale
    assert f32(recon)[0, 0, 5] == g["x2"]                   # reconstructed exactly
    # subtracting the uncompressed source would have stored the raw difference instead
    assert g["x2"] - g["x1"] == g["raw_difference"] != g["residual"]


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(6))
def test_codes_minimize_distance_brute_force(seed):
    """Each code is the grid point min16 + scale16*k (k in 0..15) nearest to x, except where
    two grid points are equally near up to binary32 rounding of (x - min)/scale."""
    g = np.random.default_rng(seed)
    scale_pick = [1e-3, 0.05, 1.0, 37.0][seed % 4]
    for kind, shape in ((orc.V, (5, 3, 64 + 24)), (orc.K, (64 + 40, 2, 8))):
        x = bf16(g.standard_normal(shape) * scale_pick + g.standard_normal() * scale_pick)
        codes, params = orc.quantize(kind, x)
        c = unpack_codes(codes).astype(np.int64)
        xv = f32(x).astype(np.float64)
        if kind == orc.V:
            p = np.repeat(params, 64, axis=2)[:, :, : shape[2]]
        else:
            p = np.repeat(params, 64, axis=0)[: shape[0]]
        m, s = params_split(p)
        grid = m[..., None] + s[..., None] * np.arange(16)
        dist = np.abs(xv[..., None] - grid)
        best = dist.min(axis=-1)
        chosen = np.take_along_axis(dist, c[..., None], axis=-1)[..., 0]
        near_tie = np.sort(dist, axis=-1)[..., 1] - best <= 1e-5 * s
        assert np.all((chosen == best) | near_tie)
        assert near_tie.mean() < 0.01


def test_params_from_group_extremes():
    """min16 is the group minimum (exact on the binary16 band) and scale16 is within one
    binary16 rounding of (max - min)/15 computed exactly."""
    g = np.random.default_rng(11)
    x = bf16(g.standard_normal((4, 4, 128)) * 3)
    xv = f32(x).astype(np.float64)
    _, params = orc.quantize(orc.V, x)
    m, s = params_split(params)
    grp = xv.reshape(4, 4, 2, 64)
    assert np.array_equal(m, grp.min(axis=-1))
    exact = (grp.max(axis=-1) - grp.min(axis=-1)) / 15
    assert np.all(np.abs(s - exact) <= exact * 2.0**-11 * 1.0001)
    _, pk = orc.quantize(orc.K, x.transpose(2, 1, 0).copy())   # 128 rows, channels = old rows
    mk, _ = params_split(pk)
    assert np.array_equal(mk[0], xv[:, :, :64].min(axis=-1).T)
    assert np.array_equal(mk[1], xv[:, :, 64:].min(axis=-1).T)


def test_error_bound_every_element():
    """|x - x_hat| <= scale16/2 plus the BF16 rounding of x_hat, on each workload's value
    distributions (normal, heavy-tailed with channel multipliers, small deltas)."""
    g = np.random.default_rng(3)
    dists = [g.standard_normal((300, 4, 96)),
             g.standard_t(3, size=(300, 4, 96)) * np.exp(g.uniform(np.log(0.1), np.log(10), (1, 4, 96))),
             g.standard_normal((300, 4, 96)) * 0.05]
    for y in dists:
        x = bf16(y)
        xv = f32(x).astype(np.float64)
        for kind in (orc.K, orc.V):
            base, recon = orc.encode_base(kind, x)
            xh = f32(recon).astype(np.float64)
            if kind == orc.V:
                p = np.repeat(base.params, 64, axis=2)[:, :, :96]
            else:
                p = np.repeat(base.params, 64, axis=0)[:300]
            _, s = params_split(p)
            ulp_bf16 = np.exp2(np.floor(np.log2(np.maximum(np.abs(xh), 1e-30))) - 7)
            err = np.abs(xv - xh)
            assert np.all(err <= s * (0.5 + 2.0**-18) + ulp_bf16 / 2 + 1e-30)
            # and the bound is tight: some element sits near half a step away
            assert np.max(err / np.maximum(s, 1e-30)) > 0.45


# --------------------------------------------------------------------------- special cases

def test_lossless_grid_and_constant_groups():
    g = np.random.default_rng(4)
    k = g.integers(0, 16, size=(64, 2, 64)).astype(np.float32)
    r = np.arange(64)
    k[r, :, r] = 0                        # every row and every column holds a 0 and a 15,
    k[r, :, (r + 1) % 64] = 15            # so every K and V group spans exactly [0, 15]
    off, step = 0.75, 0.25
    y = off + step * k
    x = bf16(y)
    for kind in (orc.K, orc.V):
        base, recon = orc.encode_base(kind, x)
        assert np.array_equal(recon, x)
        assert np.array_equal(unpack_codes(base.codes), k.astype(np.uint8))
    c = bf16(np.full((70, 1, 64), -2.5, np.float32))
    for kind in (orc.K, orc.V):
        base, recon = orc.encode_base(kind, c)
        assert np.all(base.codes == 0)
        assert np.array_equal(recon, c)
        _, s = params_split(base.params)
        assert np.all(s == 0)
    # zero residuals make constant groups: X_hat[r] == X_hat[r-1]
    x1 = bf16(g.standard_normal((100, 2, 64)))
    _, recon = orc.encode_base(orc.K, x1)
    before = recon.copy()
    res = orc.encode_residual(orc.K, before.copy(), None, recon)
    assert np.array_equal(recon, before) and np.all(res.codes == 0)


def test_signed_zero_total_order():
    """-0 sorts below +0: a group of {-0, +0} stores min -0 and scale +0.  It decodes to
    min + scale*0 = -0 + +0, which IEEE addition rounds to +0 for every element."""
    x = bf16(np.zeros(64, np.float32)).reshape(1, 1, 64).copy()
    x[0, 0, 7] = 0x8000
    codes, params = orc.quantize(orc.V, x)
    assert int(params.ravel()[0]) == 0x00008000
    deq = orc.dequantize(orc.V, codes, params, 64)
    assert np.all(deq == 0x0000)


def test_length_one_and_partial_tail_groups():
    g = np.random.default_rng(6)
    for n in (1, 65, 127, 129):
        x = bf16(g.standard_normal((n, 1, 32)))
        base, recon = orc.encode_base(orc.K, x)
        assert base.params.shape == (math.ceil(n / 64), 1, 32)
        if n % 64 == 1:
            # a single-row tail group is constant: exact
            assert np.array_equal(recon[-1], x[-1])
    x = bf16(g.standard_normal((3, 2, 96)))
    base, recon = orc.encode_base(orc.V, x)
    assert base.params.shape == (3, 2, 2)
    # the tail group of 32 channels takes its extremes from its own 32 values only
    m, _ = params_split(base.params)
    assert np.array_equal(m[:, :, 1], f32(x)[:, :, 64:].astype(np.float64).min(axis=-1))


def test_group_boundary_locality():
    """Perturbing one element changes only its own group's params and codes."""
    g = np.random.default_rng(8)
    x = bf16(g.standard_normal((130, 2, 96)))
    for kind in (orc.K, orc.V):
        c0, p0 = orc.quantize(kind, x)
        for (r, h, ch) in [(0, 0, 0), (63, 1, 95), (64, 0, 63), (129, 1, 64)]:
            y = x.copy()
            y[r, h, ch] = bf16([100.0])[0]
            c1, p1 = orc.quantize(kind, y)
            gi = (r // 64, h, ch) if kind == orc.K else (r, h, ch // 64)
            diff = np.argwhere(p0 != p1)
            assert [tuple(d) for d in diff] == [gi]
            cu0, cu1 = unpack_codes(c0), unpack_codes(c1)
            changed = np.argwhere(cu0 != cu1)
            for (rr, hh, cc) in changed:
                if kind == orc.K:
                    assert rr // 64 == r // 64 and hh == h and cc == ch
                else:
                    assert rr == r and hh == h and cc // 64 == ch // 64


def test_k_v_grouping_duality():
    """K groups run down rows of a channel; V groups along channels of a row.  So the K
    encoding of a [64, 1, D] tensor is the V encoding of its transpose [D, 1, 64]."""
    g = np.random.default_rng(9)
    x = bf16(g.standard_normal((64, 1, 48)))
    ck, pk = orc.quantize(orc.K, x)
    xt = x.transpose(2, 1, 0).copy()
    cv, pv = orc.quantize(orc.V, xt)
    assert np.array_equal(pk[0, 0, :], pv[:, 0, 0])
    assert np.array_equal(unpack_codes(ck)[:, 0, :], unpack_codes(cv)[:, 0, :].T)


def test_nonfinite_and_overflow_rejected():
    x = bf16(np.ones((64, 1, 64), np.float32))
    x[3, 0, 5] = bf16([np.inf])[0]
    for kind in (orc.K, orc.V):
        with pytest.raises(orc.OracleError) as e:
            orc.quantize(kind, x)
        assert e.value.code == orc.E_NONFINITE
    y = bf16(np.full((64, 1, 64), 1e6, np.float32))
    for kind in (orc.K, orc.V):
        with pytest.raises(orc.OracleError) as e:
            orc.quantize(kind, y)
        assert e.value.code == orc.E_RANGE
    z = bf16(np.zeros((64, 1, 64), np.float32))
    z[0, 0, 0] = bf16([-1e6])[0]
    z[0, 0, 1] = bf16([1e6])[0]          # range/15 overflows binary16
    with pytest.raises(orc.OracleError):
        orc.quantize(orc.V, z)


# --------------------------------------------------------------------------- residual chains

def _grid_chain_8tok():
    """8 tokens, loops 1-4, V kind, every residual on a power-of-two grid so each loop is
    reconstructed exactly and each position's value names the loop it resolved to."""
    fx = golden("inheritance_8tok.json")
    T, D = fx["T"], 64
    act = {int(k): np.array(v, np.int32) for k, v in fx["active"].items()}
    base = np.zeros((T, 1, D), np.float32)
    base[:, 0, 1] = 15.0
    xs_full = [base]
    for r in (2, 3, 4):
        y = xs_full[-1].copy()
        y[:, 0, 0] += 16.0 ** (r - 1)        # loop r adds 16^(r-1) at channel 0
        y[:, 0, 1] += 16.0 ** (r - 1)        # keep each residual group on a grid
        xs_full.append(y)
    return fx, act, [bf16(v) for v in xs_full]


def test_inheritance_8tok_golden():
    fx, act, xs = _grid_chain_8tok()
    T = fx["T"]
    rows = [None, None, act[3], act[4]]
    inputs = [xs[0], xs[1], xs[2][act[3]], xs[3][act[4]]]
    chain, recon = orc.encode_chain(orc.V, inputs, rows)
    depth_value = {d: f32(xs[d - 1])[0, 0, 0] for d in (1, 2, 3, 4)}
    out3 = orc.reconstruct(orc.V, chain[:3], T, 1, 64)
    got3 = [next(d for d, v in depth_value.items() if v == f32(out3)[t, 0, 0]) for t in range(T)]
    assert got3 == fx["loop3_logical_depth"]
    out4 = orc.reconstruct(orc.V, chain, T, 1, 64)
    got4 = [next(d for d, v in depth_value.items() if v == f32(out4)[t, 0, 0]) for t in range(T)]
    assert got4 == fx["loop4_logical_depth"]
    for name, depth in fx["resolution_examples"].items():
        assert got4[int(name[1:]) - 1] == depth
    assert np.array_equal(out4, recon)


def test_absent_is_not_code_zero():
    """A stored residual of code 0 decodes to its minimum (here 0.5) and changes the value;
    an absent position keeps its predecessor bit for bit."""
    T, D = 4, 64
    x1 = bf16(np.zeros((T, 1, D), np.float32))
    _, recon = orc.encode_base(orc.V, x1)
    x2 = bf16(np.full((1, 1, D), 0.5, np.float32))
    res = orc.encode_residual(orc.V, x2, np.array([2], np.int32), recon)
    assert np.all(unpack_codes(res.codes) == 0)
    assert np.all(f32(recon)[2] == 0.5)
    assert np.array_equal(recon[[0, 1, 3]], x1[[0, 1, 3]])


def test_dense_equals_sparse_full_and_uses_predecessor():
    g = np.random.default_rng(12)
    T, H, D = 200, 2, 96
    x1 = bf16(g.standard_normal((T, H, D)))
    x2 = bf16(f32(x1) + 0.1 * g.standard_normal((T, H, D)).astype(np.float32))
    for kind in (orc.K, orc.V):
        _, ra = orc.encode_base(kind, x1)
        rb = ra.copy()
        sa = orc.encode_residual(kind, x2, None, ra)
        sb = orc.encode_residual(kind, x2, np.arange(T, dtype=np.int32), rb)
        assert np.array_equal(sa.codes, sb.codes) and np.array_equal(sa.params, sb.params)
        assert np.array_equal(ra, rb)
        # the stored residual is against X_hat[1]: decoding it and adding reproduces X_hat[2]
        _, r1 = orc.encode_base(kind, x1)
        dh = orc.dequantize(kind, sa.codes, sa.params, D)
        tsum = (torch.from_numpy(f32(r1)) .to(torch.float32) + torch.from_numpy(f32(dh))).to(torch.bfloat16)
        assert np.array_equal(tsum.view(torch.int16).numpy().view(np.uint16), ra)


def test_error_does_not_compound_across_loops():
    """Each loop's reconstruction error is bounded by that loop's own residual scale, not by
    the sum of earlier errors (the effect of subtracting the reconstructed predecessor)."""
    g = np.random.default_rng(13)
    T, H, D = 256, 2, 64
    y = g.standard_normal((T, H, D)).astype(np.float32)
    xs = []
    for r in range(6):
        if r:
            y = y + 0.05 * g.standard_normal((T, H, D)).astype(np.float32)
        xs.append(bf16(y))
    for kind in (orc.K, orc.V):
        _, recon = orc.encode_base(kind, xs[0])
        for r in range(1, 6):
            prev = f32(recon).astype(np.float64)
            st = orc.encode_residual(kind, xs[r], None, recon)
            if kind == orc.V:
                p = np.repeat(st.params, 64, axis=2)
            else:
                p = np.repeat(st.params, 64, axis=0)[:T]
            _, s = params_split(p)
            xv = f32(xs[r]).astype(np.float64)
            xh = f32(recon).astype(np.float64)

            def ulp(a):
                return np.exp2(np.floor(np.log2(np.maximum(np.abs(a), 1e-30))) - 7)
            # quantization (s/2) + BF16 rounding of the residual and of its decoded value
            # (each at most half an ulp of |x - prev| + s) + BF16 rounding of the sum
            err = np.abs(xv - xh)
            assert np.all(err <= 0.5 * s * (1 + 2.0**-10) + ulp(np.abs(xv - prev) + s) + 0.5 * ulp(xh))


def test_reconstruct_matches_encode_chain_sparse():
    g = np.random.default_rng(14)
    T, H, D = 300, 3, 96
    sets = [None, None, np.sort(g.choice(T, 150, replace=False)).astype(np.int32)]
    sets.append(np.sort(g.choice(sets[2], 40, replace=False)).astype(np.int32))
    y = g.standard_normal((T, H, D)).astype(np.float32)
    full = []
    for r in range(4):
        if r:
            y = y + 0.1 * g.standard_normal((T, H, D)).astype(np.float32)
        full.append(bf16(y))
    inputs = [full[0], full[1], full[2][sets[2]], full[3][sets[3]]]
    for kind in (orc.K, orc.V):
        chain, recon = orc.encode_chain(kind, inputs, sets)
        assert np.array_equal(orc.reconstruct(kind, chain, T, H, D), recon)
        # positions outside loop 4's set keep loop 3's value; outside loop 3's keep loop 2's
        c3, r3 = orc.encode_chain(kind, inputs[:3], sets[:3])
        absent4 = np.setdiff1d(np.arange(T), sets[3])
        assert np.array_equal(recon[absent4], r3[absent4])
        assert chain[2].params.shape[0] == math.ceil(150 / 64) if kind == orc.K else True


def test_f32_params_variant_agrees_when_params_exact():
    """The upstream convention (codes from binary32 params) coincides with the FP16-param
    rule whenever the params round to binary16 exactly, and disagrees rarely otherwise."""
    g = np.random.default_rng(15)
    k = g.integers(0, 16, size=(64, 2, 64)).astype(np.float32)
    k[0], k[1] = 0, 15
    x = bf16(-3.0 + 0.5 * k)
    for kind in (orc.K, orc.V):
        assert all(np.array_equal(a, b) for a, b in zip(orc.quantize(kind, x), orc.quantize(kind, x, True)))
    y = bf16(g.standard_normal((512, 4, 128)))
    a, _ = orc.quantize(orc.V, y)
    b, _ = orc.quantize(orc.V, y, True)
    frac = np.mean(unpack_codes(a) != unpack_codes(b))
    assert 0 < frac < 0.01


# --------------------------------------------------------------------------- attention

def test_decode_attention_matches_torch_float64():
    g = np.random.default_rng(16)
    Hq, Hkv, D, T = 8, 2, 64, 200
    q = bf16(g.standard_normal((Hq, D)))
    k = bf16(g.standard_normal((T, Hkv, D)))
    v = bf16(g.standard_normal((T, Hkv, D)))
    scale = 1 / math.sqrt(D)
    out = orc.decode_attn(q, k, v, scale)
    qt = torch.from_numpy(f32(q)).double().reshape(Hkv, Hq // Hkv, 1, D)
    kt = torch.from_numpy(f32(k)).double().permute(1, 0, 2).unsqueeze(1).contiguous()
    vt = torch.from_numpy(f32(v)).double().permute(1, 0, 2).unsqueeze(1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    assert np.allclose(out, ref.reshape(Hq, D).numpy(), rtol=1e-12, atol=1e-12)
    # one token: the output is that token's value row; zero query: the mean of the values
    one = orc.decode_attn(q, k[:1], v[:1], scale)
    assert np.array_equal(one, np.repeat(f32(v[0]).astype(np.float64), Hq // Hkv, axis=0))
    zq = bf16(np.zeros((Hq, D), np.float32))
    mean = orc.decode_attn(zq, k, v, scale)
    assert np.allclose(mean, np.repeat(f32(v).astype(np.float64).mean(axis=0), Hq // Hkv, axis=0), rtol=1e-12)


def test_tile_index_definition():
    """tile_index[t] counts the rows before position 64t; spot values checked by hand."""
    rows = np.array([0, 5, 63, 64, 200, 511], np.int32)
    ti = orc.tile_index(rows, 600)
    assert list(ti) == [0, 3, 4, 4, 5, 5, 5, 5, 6, 6, 6]
    assert list(orc.tile_index(np.array([], np.int32), 130)) == [0, 0, 0, 0]
    g = np.random.default_rng(20)
    r = np.sort(g.choice(5000, 777, replace=False)).astype(np.int32)
    assert np.array_equal(orc.tile_index(r, 5000), np.searchsorted(r, 64 * np.arange(-(-5000 // 64) + 1)))
