"""Pins for the oracle's page-local K groups and rolling-tail rule.

Page-local (tile) K groups follow the PR #166 review, item 3 "Group ownership vs 16-token
pages": no K group may merge rows of different logical 64-token groups, so a page's
metadata stays with it.  The rolling tail follows the RFC (vllm-rlt #156), section 3.3, last
paragraph: at least 64 recent tokens stay in BF16 and whole 64-token groups are flushed, so
64 to 127 tokens remain after a step.

Each test ties the oracle to something outside its own tile code: a hand-derived fixture,
the already pinned compact-row quantizer applied to one tile's rows, the dense special case,
locality and append invariants that hold only for tile-local groups, or the pages' stated
tail bounds.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(vals):
    return orc.bf16_from_f32(np.asarray(vals, np.float32))


def _hex(a):
    return np.array([[int(v, 16) for v in r] for r in a], np.uint32)


def _unpack(codes):
    c = np.asarray(codes, np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = c & 0xF
    out[..., 1::2] = c >> 4
    return out


def _chain_inputs(rng, T, H, D, fracs):
    """Loop 1 dense, then nested random active sets of the given fractions."""
    y = rng.standard_normal((T, H, D)).astype(np.float32)
    xs, rows, prev = [orc.bf16_from_f32(y)], [None], np.arange(T, dtype=np.int32)
    for f in fracs:
        y = y + (0.1 * rng.standard_normal((T, H, D))).astype(np.float32)
        xb = orc.bf16_from_f32(y)
        if f is None:
            xs.append(xb)
            rows.append(None)
            continue
        prev = np.sort(rng.choice(prev, size=int(round(f * T)), replace=False)).astype(np.int32)
        xs.append(np.ascontiguousarray(xb[prev]))
        rows.append(prev)
    return xs, rows


# --------------------------------------------------------------------------- fixture

def test_golden_page_local_k_groups():
    g = json.load(open(os.path.join(GOLDEN, "page_local_k.json")))
    T, H, D = g["T"], g["H"], g["D"]
    rows = np.array(g["rows"], np.int32)
    x = _bits(g["x"]).reshape(len(rows), H, D)
    # tile groups, through the residual encoder against a zero predecessor
    recon = np.zeros((T, H, D), np.uint16)
    st = orc.encode_residual(orc.K, x, rows, recon, k_tiles=True)
    assert np.array_equal(st.params.reshape(-1, D), _hex(g["tile_groups"]["params"]))
    assert np.array_equal(_unpack(st.codes).reshape(-1, D), np.array(g["tile_groups"]["codes"]))
    assert np.array_equal(recon[rows].reshape(-1, D), _bits(g["tile_groups"]["recon_rows"]))
    # compact-row groups of the same loop
    recon = np.zeros((T, H, D), np.uint16)
    st = orc.encode_residual(orc.K, x, rows, recon, k_tiles=False)
    assert np.array_equal(st.params.reshape(-1, D), _hex(g["row_groups"]["params"]))
    assert np.array_equal(_unpack(st.codes).reshape(-1, D), np.array(g["row_groups"]["codes"]))


# --------------------------------------------------------------------------- reductions

@pytest.mark.parametrize("T", [64, 200, 257])
def test_dense_tile_groups_are_row_groups(T):
    """A dense stream's tile t holds compact rows 64t..64t+63, its compact-row group t."""
    rng = np.random.default_rng(T)
    xs, rows = _chain_inputs(rng, T, 2, 16, [None, None])
    a, ra = orc.encode_chain(orc.K, xs, rows, k_tiles=True)
    b, rb = orc.encode_chain(orc.K, xs, rows, k_tiles=False)
    assert np.array_equal(ra, rb)
    for sa, sb in zip(a, b):
        assert np.array_equal(sa.codes, sb.codes) and np.array_equal(sa.params, sb.params)


@pytest.mark.parametrize("seed", range(4))
def test_tile_group_is_one_standalone_group(seed):
    """Each tile's rows, quantized alone by the (separately pinned) compact-row quantizer,
    form a single group of at most 64 rows: its codes and params must be the tile group's."""
    rng = np.random.default_rng(100 + seed)
    T, H, D = int(rng.integers(65, 400)), 2, 16
    n = int(rng.integers(1, T))
    rows = np.sort(rng.choice(T, size=n, replace=False)).astype(np.int32)
    x = orc.bf16_from_f32(rng.standard_normal((n, H, D)).astype(np.float32))
    codes, params = orc.quantize_k_tiles(x, rows, T)
    assert params.shape == ((T + 63) // 64, H, D)
    for t in range(params.shape[0]):
        sel = np.nonzero(rows // 64 == t)[0]
        if sel.size == 0:
            assert not params[t].any(), "an empty tile's params are 0"
            continue
        c1, p1 = orc.quantize(orc.K, x[sel])
        assert p1.shape[0] == 1
        assert np.array_equal(params[t], p1[0])
        assert np.array_equal(_unpack(codes[sel]), _unpack(c1))
    # and the dequantizer reads each row's tile parameters
    xh = orc.dequantize_k_tiles(codes, params, rows, T, D)
    for t in range(params.shape[0]):
        sel = np.nonzero(rows // 64 == t)[0]
        if sel.size:
            assert np.array_equal(xh[sel], orc.dequantize(orc.K, codes[sel], params[t:t + 1], D))


def test_tile_group_error_bound():
    """|x - x_hat| <= scale/2 (plus the BF16 rounding of the decoded value) for every element,
    with the scale of the element's own tile group."""
    rng = np.random.default_rng(7)
    T, H, D, n = 700, 3, 32, 300
    rows = np.sort(rng.choice(T, size=n, replace=False)).astype(np.int32)
    x = orc.bf16_from_f32((rng.standard_normal((n, H, D)) * 3).astype(np.float32))
    codes, params = orc.quantize_k_tiles(x, rows, T)
    xh = orc.f32_from_bf16(orc.dequantize_k_tiles(codes, params, rows, T, D)).astype(np.float64)
    xf = orc.f32_from_bf16(x).astype(np.float64)
    p = params[rows // 64]
    m = (p & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    s = (p >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    # FP16 rounding of min and scale shifts the grid by at most half an FP16 ulp of each; the
    # decoded value's BF16 rounding adds half a BF16 ulp
    bound = s / 2 + np.abs(m) * 2.0**-11 + 15 * s * 2.0**-11 + np.abs(xh) * 2.0**-8 + 1e-30
    assert np.all(np.abs(xf - xh) <= bound)


# --------------------------------------------------------------------------- locality

def _encode(xs, rows, k_tiles):
    return orc.encode_chain(orc.K, xs, rows, k_tiles=k_tiles)


def test_page_locality_of_tile_groups():
    """Changing the tokens of one tile changes no other tile's K codes or params, at any
    loop; with compact-row groups the change reaches other tiles (the review's concern)."""
    rng = np.random.default_rng(11)
    T, H, D = 512, 2, 16
    xs, rows = _chain_inputs(rng, T, H, D, [None, 0.45, 0.2])
    victim = 3
    xs2 = [x.copy() for x in xs]
    for l, (x, r) in enumerate(zip(xs2, rows)):
        pos = np.arange(T) if r is None else r
        sel = np.nonzero(pos // 64 == victim)[0]
        x[sel] = orc.bf16_from_f32(orc.f32_from_bf16(x[sel]) * 4.0 + 1.0)
    for k_tiles in (True, False):
        a, _ = _encode(xs, rows, k_tiles)
        b, _ = _encode(xs2, rows, k_tiles)
        spread = False
        for l, (sa, sb) in enumerate(zip(a, b)):
            pos = np.arange(T) if sa.rows is None else sa.rows
            other = pos // 64 != victim
            if k_tiles:
                keep = np.arange(sa.params.shape[0]) != victim
                assert np.array_equal(sa.params[keep], sb.params[keep]), f"loop {l} params"
                assert np.array_equal(sa.codes[other], sb.codes[other]), f"loop {l} codes"
            else:
                spread |= not np.array_equal(sa.codes[other], sb.codes[other])
        if not k_tiles:
            assert spread, "compact-row groups should mix tiles in this case"


def _stitch(parts, starts):
    """Concatenate per-window chains (positions relative to each window's start) into one."""
    out = []
    for l in range(len(parts[0][0])):
        dense = parts[0][0][l].rows is None
        streams = [chain[l] for chain, _ in parts]
        rows = None if dense else np.concatenate([s.rows + p0 for s, p0 in zip(streams, starts)]).astype(np.int32)
        out.append(orc.Stream(sum(s.n_rows for s in streams), rows,
                              np.concatenate([s.codes for s in streams]),
                              np.concatenate([s.params for s in streams])))
    return out


@pytest.mark.parametrize("k_tiles", [True, False])
def test_append_of_whole_tiles_equals_one_shot(k_tiles):
    """Encoding positions [0, 192) and then [192, 448) as separate windows and appending
    gives exactly the streams of encoding [0, 448) at once when K groups are tile-local
    (the rolling tail flushes whole 64-token groups); compact-row groups do not have this
    property once a compact loop's row count is not a multiple of 64."""
    rng = np.random.default_rng(21)
    T, H, D, P1 = 448, 2, 16, 192
    xs, rows = _chain_inputs(rng, T, H, D, [None, 0.5, 0.25])
    one, rone = orc.encode_chain(orc.K, xs, rows, k_tiles=k_tiles)
    parts = []
    for lo, hi in ((0, P1), (P1, T)):
        wx, wr = [], []
        for x, r in zip(xs, rows):
            if r is None:
                wx.append(x[lo:hi])
                wr.append(None)
            else:
                sel = (r >= lo) & (r < hi)
                wx.append(x[sel])
                wr.append((r[sel] - lo).astype(np.int32))
        parts.append(orc.encode_chain(orc.K, wx, wr, k_tiles=k_tiles))
    stitched = _stitch(parts, [0, P1])
    recon = np.concatenate([r for _, r in parts])
    same = np.array_equal(recon, rone) and all(
        np.array_equal(a.codes, b.codes) and np.array_equal(a.params, b.params) and
        (a.rows is None or np.array_equal(a.rows, b.rows)) for a, b in zip(stitched, one))
    if k_tiles:
        assert same
        # and the stitched chain reconstructs like the one-shot chain
        assert np.array_equal(orc.reconstruct(orc.K, stitched, T, H, D, k_tiles=True), rone)
    else:
        assert not same


def test_tile_chain_reconstruct_equals_inplace():
    rng = np.random.default_rng(5)
    T, H, D = 1000, 2, 96
    xs, rows = _chain_inputs(rng, T, H, D, [None, 0.5, 0.25])
    chain, recon = orc.encode_chain(orc.K, xs, rows, k_tiles=True)
    assert np.array_equal(orc.reconstruct(orc.K, chain, T, H, D, k_tiles=True), recon)
    # V ignores the K grouping
    cv, rv = orc.encode_chain(orc.V, xs, rows, k_tiles=True)
    cw, rw = orc.encode_chain(orc.V, xs, rows, k_tiles=False)
    assert np.array_equal(rv, rw)


def test_tile_params_storage_accounts_for_padding():
    """RFC section 7.4: small residual streams pay for partially filled groups.  A tile-
    grouped K stream stores one parameter row per tile whatever its occupancy."""
    H, D, T = 8, 128, 32768
    assert orc.k_tile_params_bytes(H, D, T) == 4 * (T // 64) * H * D
    # a 25 % loop: 8192 rows; compact-row groups need 128 parameter rows, tile groups 512
    assert orc.params_bytes(orc.K, H, D, 8192) == 4 * 128 * H * D
    assert orc.k_tile_params_bytes(H, D, T) == 4 * orc.params_bytes(orc.K, H, D, 8192)


# --------------------------------------------------------------------------- rolling tail

def test_rolling_prefix_small_cases():
    # fewer than 128 tokens: nothing can be flushed while keeping 64
    for n in range(0, 128):
        assert orc.rolling_prefix(n) == 0
    assert orc.rolling_prefix(128) == 64
    assert orc.rolling_prefix(191) == 64
    assert orc.rolling_prefix(192) == 128


@pytest.mark.parametrize("seed", range(3))
def test_rolling_tail_bounds_over_steps(seed):
    """Simulated decode: a prompt, then steps of 1 token (sometimes a chunk).  After every
    step the packed prefix is whole 64-token groups, never shrinks, leaves at least 64 tokens
    in the tail once 64 exist, holds 64-127 tokens in the tail once 128 exist, and no further
    group could be flushed without breaking the 64-token minimum."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 600))
    last = 0
    for _ in range(2000):
        n += 1 if rng.random() < 0.9 else int(rng.integers(2, 300))
        p = orc.rolling_prefix(n)
        tail = n - p
        assert p % 64 == 0 and p >= last
        assert tail >= min(n, 64)
        if n >= 128:
            assert 64 <= tail <= 127
        assert n - (p + 64) < 64
        last = p
