"""Pins for the NVFP4 oracle (vllm-rlt PR #166, review item 2; the chain of the RFC, vllm-rlt
#156, section 3.3): the E2M1 and E4M3 grids from their bit-level definitions, nearest-even
ties worked by hand, saturation, the storage cost the review states, symmetry, the review's
remark on outlier channels, round trips and the chain's self-consistency."""
import numpy as np
import pytest
import torch

from oracle import fp4
from oracle import oracle as orc


def test_e2m1_grid_from_the_bit_layout():
    """E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal."""
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        v = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert fp4.e2m1_value(np.array([code]))[0] == (-v if s else v)
    assert sorted(set(np.abs(fp4.e2m1_value(np.arange(16))))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


@pytest.mark.parametrize("y,v", [
    (0.25, 0.0), (0.2500001, 0.5), (0.75, 1.0), (1.25, 1.0), (1.2500001, 1.5), (1.75, 2.0), (2.5, 2.0),
    (2.5000002, 3.0), (3.5, 4.0), (5.0, 4.0), (5.0000005, 6.0), (6.0, 6.0), (7.0, 6.0), (1e30, 6.0),
    (0.1, 0.0), (-0.75, -1.0), (-5.0, -4.0), (-100.0, -6.0),
])
def test_e2m1_nearest_even(y, v):
    """Ties go to the even mantissa: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2,
    3.5 -> 4, 5 -> 4; magnitudes past 6 saturate."""
    y32 = np.float32(y)
    assert fp4.e2m1_value(fp4.e2m1_code(np.array([y32])))[0] == v


def test_e2m1_negative_values_that_round_to_zero_keep_the_sign():
    c = fp4.e2m1_code(np.array([np.float32(-0.1), np.float32(0.1), np.float32(-0.0)]))
    assert list(c) == [8, 0, 8]


def test_e4m3_grid_from_the_bit_layout():
    """E4M3 without infinities: bytes 0x00..0x7E are the 127 non-negative finite values (0x7F
    is NaN); exponent bias 7, exponent 0 subnormal: min 2^-9, min normal 2^-6, max 448."""
    vals = fp4.e4m3_value(np.arange(0x7F))
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        want = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        assert vals[b] == want
    assert np.all(np.diff(vals) > 0)
    assert vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6 and vals[-1] == 448.0
    assert np.array_equal(fp4.e4m3_bits(vals), np.arange(0x7F, dtype=np.uint8))


@pytest.mark.parametrize("v,want", [
    (448.0, 448.0), (449.0, 448.0), (464.0, 448.0), (1e6, 448.0),        # saturation
    (1.0625, 1.0), (1.1875, 1.25), (1.0625001, 1.125),                   # ties at 1 + 1/16, 1 + 3/16
    (2.0 ** -10, 0.0), (1.5 * 2.0 ** -9, 2.0 * 2.0 ** -9), (2.5 * 2.0 ** -9, 2.0 * 2.0 ** -9),  # subnormals
    (0.0, 0.0), (2.0 ** -6 * 1.0625, 2.0 ** -6),
])
def test_e4m3_nearest_even_and_saturation(v, want):
    assert fp4.e4m3_round(np.array([np.float32(v)]))[0] == want


def test_storage_is_about_four_and_a_half_bits():
    """The review: E2M1 plus one E4M3 scale per 16 elements (and one FP32 per tensor) is about
    4.5 bits per element, the same as INT4 with 64-element groups and FP16 min and scale."""
    assert abs(fp4.stream_bits_per_element(8, 128, 32768) - 4.5) < 1e-5
    assert 4 + 32 / 64 == 4.5


def test_symmetric_no_zero_point():
    """Negating the input flips every nonzero code's sign bit and nothing else."""
    rng = np.random.default_rng(0)
    x = fp4.f32_of_bf16(fp4.bf16_of_f32(rng.standard_normal((5, 2, 32)).astype(np.float32)))
    c1, s1, g1, _, d1 = fp4.encode_values(x)
    c2, s2, g2, _, d2 = fp4.encode_values(-x)
    assert np.array_equal(s1, s2) and g1 == g2
    assert np.array_equal(c1 ^ 0x88, c2)
    assert np.array_equal(d1, -d2)


def test_grid_block_round_trips_exactly():
    """A block holding the E2M1 grid times a power of two decodes back to its BF16 values."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6, 6], np.float32)
    for k in (-20, -3, 0, 5, 30):
        x = (grid * np.float32(2.0 ** k)).reshape(1, 1, 16)
        codes, scales, s_g, amax, dec = fp4.encode_values(x)
        assert np.array_equal(fp4.bf16_of_f32(dec), fp4.bf16_of_f32(x))


def test_error_bound_on_random_blocks():
    """|x - x_hat| <= bs * (half the E2M1 step at |x / bs|, or the excess past 6) + one binary32
    rounding, block by block."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 4, 64)) * np.exp(rng.uniform(-3, 3, (64, 4, 1)))).astype(np.float32)
    x = fp4.f32_of_bf16(fp4.bf16_of_f32(x))
    codes, scales, s_g, amax, dec = fp4.encode_values(x)
    bs = (fp4.e4m3_value(scales).astype(np.float32) * s_g).astype(np.float32)
    bsx = np.repeat(bs, 16, axis=-1).astype(np.float64)
    y = np.abs(x / bsx)
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    allowed = bsx * np.maximum(step / 2, y - 6) + 2.0 ** -23 * np.abs(x)
    assert np.all(np.abs(x.astype(np.float64) - dec) <= allowed * (1 + 1e-6))
    # the scale makes the block's largest magnitude land near the top of the grid
    assert np.all(np.abs(x).reshape(64, 4, 4, 16).max(-1) / bs <= 6 * 1.07)


def test_outlier_channel_costs_its_block_precision():
    """The review: a 16-channel block with an outlier channel loses precision on the other 15."""
    base = np.linspace(-1, 1, 16).astype(np.float32)
    x = np.stack([base, base.copy()]).reshape(1, 2, 16)
    x[0, 1, 3] = 96.0                                     # outlier in the second block
    x = fp4.f32_of_bf16(fp4.bf16_of_f32(x))
    *_, dec = fp4.encode_values(x)
    others = [i for i in range(16) if i != 3]
    clean = np.abs(dec[0, 0, others] - x[0, 0, others]).max()
    hit = np.abs(dec[0, 1, others] - x[0, 1, others]).max()
    assert hit > 10 * clean


def test_stream_scale_uses_the_whole_range():
    """s_g = amax / 2688: the block holding amax gets the E4M3 scale 448."""
    rng = np.random.default_rng(2)
    x = fp4.f32_of_bf16(fp4.bf16_of_f32(rng.standard_normal((10, 3, 48)).astype(np.float32)))
    codes, scales, s_g, amax, _ = fp4.encode_values(x)
    assert amax == np.abs(x).max() and s_g == np.float32(amax) / np.float32(2688)
    blk = np.abs(x).reshape(10, 3, 3, 16).max(-1)
    assert fp4.e4m3_value(scales[blk == amax]).max() == 448.0
    z = np.zeros((2, 1, 16), np.float32)
    codes, scales, s_g, amax, dec = fp4.encode_values(z)
    assert s_g == 1 and amax == 0 and not codes.any() and not scales.any() and not dec.any()


@pytest.mark.parametrize("int4_base", [False, True])
def test_chain_reconstructs_from_stored_bytes(int4_base):
    """Base (NVFP4, or INT4 from the INT4 oracle) plus NVFP4 residuals, dense and compact, and an
    unchanged loop: the reconstruction from the stored streams equals the encoder's running
    X_hat bit for bit."""
    rng = np.random.default_rng(3)
    T, H, D = 200, 3, 64
    y = rng.standard_normal((T, H, D)).astype(np.float32)
    xs, rows = [fp4.bf16_of_f32(y)], [None]
    prev = np.arange(T, dtype=np.int32)
    for n in [None, 100, 37]:                       # loop 2 dense, loops 3-4 nested compact sets
        y = y + (0.05 * rng.standard_normal((T, H, D))).astype(np.float32)
        if n is not None:
            prev = np.sort(rng.choice(prev, n, replace=False)).astype(np.int32)
        sel = None if n is None else prev
        xb = fp4.bf16_of_f32(y)
        xs.append(xb if sel is None else xb[sel])
        rows.append(sel)
    if int4_base:
        _, recon = orc.encode_base(orc.K, xs[0])
    else:
        _, recon = fp4.encode_base(xs[0])
    base = recon.copy()
    streams = [fp4.encode_residual(x, r, recon) for x, r in zip(xs[1:], rows[1:])]
    assert np.array_equal(fp4.apply_residuals(base, streams), recon)
    # a loop equal to the reconstruction encodes zeros and changes no value (a -0 in the base
    # becomes +0: -0 + +0 = +0 in IEEE arithmetic)
    before = recon.copy()
    s = fp4.encode_residual(recon.copy(), None, recon)
    assert s.amax == 0 and np.array_equal(fp4.f32_of_bf16(recon), fp4.f32_of_bf16(before))


def test_e2m1_code_against_brute_force():
    """Each code is the grid value nearest to y (ties to the even magnitude index, i.e. the even
    mantissa bit), searched over all 16 codes; magnitudes past 6 land on 6; values that round to
    zero keep their sign."""
    rng = np.random.default_rng(4)
    grid = fp4.E2M1_VALUES
    mids = (grid[1:] + grid[:-1]) / 2
    y = np.concatenate([rng.uniform(-9, 9, 20000), mids, -mids, grid, -grid, [7.0, -7.0, 1e9]])
    y = y.astype(np.float32).astype(np.float64)
    got = fp4.e2m1_code(y)
    vals = fp4.e2m1_value(np.arange(16))
    for yi, ci in zip(y, got):
        d = np.abs(vals - yi)
        best = np.flatnonzero(d == d.min())
        mags = {int(b) & 7 for b in best}
        mag = min(mags) if len(mags) == 1 else [m for m in mags if m % 2 == 0][0]
        assert int(ci) & 7 == mag, yi
        assert (int(ci) >> 3) == (1 if np.signbit(yi) else 0), yi


# ----------------------------------------------------------------------------- MXFP4

def test_e8m0_grid_from_the_bit_layout():
    """E8M0 is a bare biased exponent: byte b is 2^(b - 127), b = 0 .. 254."""
    b = np.arange(255)
    v = fp4.e8m0_value(b)
    assert v[127] == 1.0 and v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127
    assert np.all(v[1:] / v[:-1] == 2.0)


@pytest.mark.parametrize("amax,byte", [
    (1.0, 125),            # floor(log2 1) = 0  -> X = 2^-2
    (6.0, 127),            # floor(log2 6) = 2  -> X = 1: the block's largest value is 6 X
    (7.0, 127),            # still X = 1: 7 clips to 6
    (8.0, 128),            # floor(log2 8) = 3  -> X = 2
    (0.75, 124),           # floor(log2 0.75) = -1 -> X = 2^-3
    (3.999, 126),          # floor(log2 3.999) = 1 -> X = 2^-1: 3.999 / X = 7.998 clips to 6
    (0.0, 0),              # a block of zeros: the smallest scale
    (2.0 ** -130, 0),      # -132 clamps to -127
    (1.5 * 2.0 ** 127, 252),
])
def test_mx_shared_exponent(amax, byte):
    """OCP MX v1.0: X = 2^(floor(log2 amax) - 2), clamped to E8M0's range."""
    assert int(fp4.mx_scale_bits(np.array([amax]))[0]) == byte


def test_mx_worked_block():
    """One block worked by hand: amax 7 gives X = 1; 7 and -6.5 clip to +-6, 0.25, 0.75, 2.5
    and 5 are ties that go to the even mantissa (0, 1, 2, 4), -0.3 (BF16 -0.30078125) is nearer
    -0.5 than -0; the same block times 2^-10 gives X = 2^-10 and the same codes."""
    vals = [7.0, 1.0, -0.3, 0.25, 0.75, 2.5, 5.0, -6.5]
    want_codes = [7, 2, 9, 0, 2, 4, 6, 15]
    want_dec = [6.0, 1.0, -0.5, 0.0, 1.0, 2.0, 4.0, -6.0]
    for k in (0, -10):
        x = np.zeros((1, 1, 32), np.float32)
        x[0, 0, :8] = np.array(vals, np.float32) * np.float32(2.0 ** k)
        x = fp4.f32_of_bf16(fp4.bf16_of_f32(x))
        codes, scales, dec = fp4.mx_encode_values(x)
        assert int(scales[0, 0, 0]) == 127 + k
        c4 = np.empty(32, np.uint8)
        c4[0::2], c4[1::2] = codes[0, 0] & 15, codes[0, 0] >> 4
        assert list(c4[:8]) == want_codes and not c4[8:].any()
        assert list(dec[0, 0, :8]) == [v * 2.0 ** k for v in want_dec] and not dec[0, 0, 8:].any()


def test_mx_storage_is_four_and_a_quarter_bits():
    assert fp4.mx_stream_bits_per_element(8, 128, 32768) == 4.25


def test_mx_error_bound_and_clipping():
    """|x - x_hat| <= X * (half the E2M1 step at |x / X|) when |x / X| <= 6; above 6 the value
    clips to 6 X and the error is below 2 X.  Every block's amax lies in [4 X, 8 X)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 4, 64)) * np.exp(rng.uniform(-6, 6, (64, 4, 1)))).astype(np.float32)
    x = fp4.f32_of_bf16(fp4.bf16_of_f32(x))
    codes, scales, dec = fp4.mx_encode_values(x)
    X = np.repeat(fp4.e8m0_value(scales), 32, axis=-1)
    y = np.abs(x / X)
    amax = np.abs(x).reshape(64, 4, 2, 32).max(-1) / fp4.e8m0_value(scales)
    assert np.all((amax >= 4) & (amax < 8))
    err = np.abs(x.astype(np.float64) - dec)
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    inside = y <= 6
    assert np.all(err[inside] <= X[inside] * step[inside] / 2)
    assert np.all(err[~inside] == (y[~inside] - 6) * X[~inside]) and np.all(err[~inside] < 2 * X[~inside])
    assert (~inside).any()                                          # clipping does occur


def test_mx_symmetric_and_grid_round_trip():
    rng = np.random.default_rng(6)
    x = fp4.f32_of_bf16(fp4.bf16_of_f32(rng.standard_normal((5, 2, 64)).astype(np.float32)))
    c1, s1, d1 = fp4.mx_encode_values(x)
    c2, s2, d2 = fp4.mx_encode_values(-x)
    assert np.array_equal(s1, s2) and np.array_equal(c1 ^ 0x88, c2) and np.array_equal(d1, -d2)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6, 6], np.float32)
    for k in (-120, -3, 0, 5, 100):
        g = np.tile(grid, 2).reshape(1, 1, 32) * np.float32(2.0 ** k)
        *_, dec = fp4.mx_encode_values(g)
        assert np.array_equal(dec, g)


def test_mx_block_is_32_channels():
    """An outlier changes the scale of its own 32-channel block only."""
    x = np.tile(np.linspace(-1, 1, 32).astype(np.float32), 3).reshape(1, 1, 96)
    x = fp4.f32_of_bf16(fp4.bf16_of_f32(x))
    _, s0, d0 = fp4.mx_encode_values(x)
    x[0, 0, 40] = 96.0
    _, s1, d1 = fp4.mx_encode_values(x)
    assert list(s0[0, 0] != s1[0, 0]) == [False, True, False]
    assert np.array_equal(d0[0, 0, :32], d1[0, 0, :32]) and np.array_equal(d0[0, 0, 64:], d1[0, 0, 64:])


@pytest.mark.parametrize("int4_base", [False, True])
def test_mx_chain_reconstructs_from_stored_bytes(int4_base):
    rng = np.random.default_rng(7)
    T, H, D = 200, 3, 64
    y = rng.standard_normal((T, H, D)).astype(np.float32)
    xs, rows = [fp4.bf16_of_f32(y)], [None]
    prev = np.arange(T, dtype=np.int32)
    for n in [None, 100, 37]:
        y = y + (0.05 * rng.standard_normal((T, H, D))).astype(np.float32)
        if n is not None:
            prev = np.sort(rng.choice(prev, n, replace=False)).astype(np.int32)
        sel = None if n is None else prev
        xb = fp4.bf16_of_f32(y)
        xs.append(xb if sel is None else xb[sel])
        rows.append(sel)
    if int4_base:
        _, recon = orc.encode_base(orc.V, xs[0])
    else:
        base, recon = fp4.encode_base(xs[0], mx=True)
        assert isinstance(base, fp4.MxStream)
        assert np.array_equal(fp4.bf16_of_f32(fp4.mx_decode_stream(base)), recon)
    start = recon.copy()
    streams = [fp4.encode_residual(x, r, recon, mx=True) for x, r in zip(xs[1:], rows[1:])]
    assert all(isinstance(s, fp4.MxStream) for s in streams)
    assert np.array_equal(fp4.apply_residuals(start, streams), recon)
    # an MXFP4 residual step is closer to X_r than the base alone
    x4 = fp4.f32_of_bf16(xs[-1])
    assert np.abs(fp4.f32_of_bf16(recon[rows[-1]]) - x4).mean() < np.abs(fp4.f32_of_bf16(start[rows[-1]]) - x4).mean()


def test_bf16_of_f32_matches_torch():
    """The FP4 oracle's own BF16 rounding (residuals and reconstructions of every FP4 chain)
    against torch's BF16 cast, an independent implementation: 2M random binary32 patterns plus,
    for every BF16 upper half, the lower halves just below, at and above the rounding midpoint."""
    g = np.random.default_rng(17)
    u = g.integers(0, 2**32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    x = np.concatenate([u, (hi[:, None] | lows[None, :]).ravel()]).view(np.float32)
    # finite inputs whose rounding stays finite (the oracle's precondition)
    x = x[np.isfinite(x) & (np.abs(x) < np.float32(3.3895313e38))]
    ours = fp4.bf16_of_f32(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_round_matches_torch_float8():
    """e4m3_round against torch's float8_e4m3fn cast (round to nearest even) below the
    saturation point, over every E4M3 midpoint and its binary32 neighbours and random values
    spanning the subnormal and normal ranges."""
    vals = fp4.e4m3_value(np.arange(0x7F))
    mid = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    g = np.random.default_rng(5)
    rnd = np.exp(g.uniform(np.log(2.0 ** -12), np.log(447.0), 200000)).astype(np.float32)
    x = np.concatenate([vals.astype(np.float32), mid, np.nextafter(mid, np.float32(0)),
                        np.nextafter(mid, np.float32(np.inf)), rnd])
    ours = fp4.e4m3_round(x)
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(ours, ref)
