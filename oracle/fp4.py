"""Oracle of the FP4 variants of the packed-KV codec: E2M1 element codes with NVFP4 scales (one
E4M3 scale per 16 consecutive channels and one binary32 scale per stream) or MXFP4 scales (one
E8M0 power-of-two scale per 32 consecutive channels); a base loop and residual loops, which may
also follow an INT4 base.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and its binding)
never imports this module, and this module never imports the product.

What it follows: vllm-rlt pull request #166, the review's second item ("Before the NVFP4 hot
path"): NVFP4 is E2M1 codes with one E4M3 scale per 16 elements and one FP32 scale per tensor,
about 4.5 bits per element like INT4 with 64-element groups; it is symmetric (no zero point);
an INT4 base with NVFP4 residuals is an option; the oracle rounds E2M1 to nearest-even and
rounds the E4M3 scales.  The residual chain is the RFC's (vllm-rlt issue #156, section 3.3).
E2M1 (2 exponent bits, bias 1, 1 mantissa bit) holds +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}; E4M3
(4 exponent bits, bias 7, 3 mantissa bits, no infinities) holds 0, 2^-9 .. 448.

Readings taken where the review leaves a step open:
- blocks run along the channels of one (row, head) for K and V alike (16 channels);
- the stream's scale is s_g = RN32(amax / 2688), 2688 = 6 * 448, over the magnitudes it
  encodes (X for a base loop, the BF16 residuals for a residual loop), or 1 when amax is 0,
  so that the largest block scale reaches the top of E4M3;
- a block's scale is E4M3(RN32(amax_b / RN32(6 * s_g))), rounded to nearest-even and
  saturated at 448; its binary32 value bs = RN32(e4m3 * s_g) both divides (encode) and
  multiplies (decode);
- code = E2M1 nearest-even of RN32(x / bs), saturated at 6; a value that rounds to zero keeps
  its sign; a block whose scale is 0 has all codes +0;
- decode = bf16(RN32(e2m1 * bs)); a residual is rounded to BF16 before it is encoded and the
  reconstruction adds the decoded BF16 residual in binary32, rounded to BF16 (as the INT4 chain);
- stored stream: codes [n, H, D/2] (low nibble = even channel), then a params buffer of a
  16-byte header (s_g, amax, two zero words) followed by the block scales [n, H, D/16].

MXFP4 is not defined on the pages: the review names NVFP4, and MX-scaled FP4 appears there only
in the name of an instruction.  It is taken from the OCP Microscaling Formats (MX)
specification, version 1.0, section 6 (the MXFP4 element and scale types and the conversion of a
block of 32 values):
- a block is 32 consecutive channels of one (row, head), for K and V alike;
- its scale is the E8M0 value X = 2^e with e = floor(log2(amax_b)) - 2 (2 = the exponent of
  E2M1's largest power of two), clamped to E8M0's range [-127, 127]; a block of zeros takes
  e = -127;
- code = E2M1 nearest-even of x / X (exact, X is a power of two), saturated at 6 (amax_b / X
  lies in [4, 8), so values above 6 X are clipped, as the specification's conversion does); a
  value that rounds to zero keeps its sign;
- decode = bf16(e2m1 * X) (exact); the residual chain is the same as above;
- stored stream: codes [n, H, D/2] as above, params = the E8M0 bytes [n, H, D/32] (no header);
  4.25 bits per element.
Inputs are finite.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

BLOCK = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
HEADER_BYTES = 16
MX_BLOCK = 32
E2M1_EMAX = 2          # E2M1's largest power of two is 2^2 (its largest value 6 = 1.5 * 2^2)


def f32_of_bf16(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_of_f32(x: np.ndarray) -> np.ndarray:
    """Round binary32 to BF16, nearest-even (finite inputs); returns bit patterns."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------- element formats

def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Nearest-even E4M3 value of non-negative v (binary64 result), saturated at 448."""
    v = np.asarray(v, np.float64)
    out = np.empty_like(v)
    sat = v >= E4M3_MAX
    sub = v < 2.0 ** -6
    out[sub] = np.rint(v[sub] * 512.0) / 512.0                   # subnormal grid 2^-9
    nrm = ~sat & ~sub
    _, k = np.frexp(v[nrm])                                         # v = f * 2^k, f in [0.5, 1)
    ulp = np.ldexp(1.0, k - 1 - 3)
    out[nrm] = np.rint(v[nrm] / ulp) * ulp
    out[sat] = E4M3_MAX
    return np.minimum(out, E4M3_MAX)


def e4m3_bits(value: np.ndarray) -> np.ndarray:
    """Byte of an E4M3 grid value (non-negative)."""
    value = np.asarray(value, np.float64)
    bits = np.zeros(value.shape, np.uint8)
    sub = (value > 0) & (value < 2.0 ** -6)
    bits[sub] = (value[sub] * 512.0).astype(np.uint8)
    nrm = value >= 2.0 ** -6
    f, k = np.frexp(value[nrm])
    e = k - 1                                                       # value = (1 + m/8) 2^e
    bits[nrm] = ((e + 7) << 3 | np.rint((value[nrm] / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)).astype(np.uint8)
    return bits


def e4m3_value(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, np.int64)
    e, m = (b >> 3) & 15, b & 7
    return np.where(e == 0, m / 512.0, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))


def e2m1_code(y: np.ndarray) -> np.ndarray:
    """4-bit E2M1 code (sign in bit 3) of the nearest-even value of y, saturated at 6."""
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = np.minimum(np.rint(a / step) * step, E2M1_MAX)
    mag = np.searchsorted(E2M1_VALUES, q).astype(np.uint8)
    return mag | (np.signbit(y).astype(np.uint8) << 3)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code, np.int64)
    v = E2M1_VALUES[c & 7]
    return np.where(c & 8, -v, v)


# ----------------------------------------------------------------------------- one stream

@dataclass
class Fp4Stream:
    codes: np.ndarray            # uint8 [n, H, D/2]
    scales: np.ndarray           # uint8 [n, H, D/16], E4M3
    s_g: np.float32
    amax: np.float32
    rows: Optional[np.ndarray]   # ascending positions, or None (dense)

    @property
    def n_rows(self) -> int:
        return self.codes.shape[0]

    def params_bytes(self) -> np.ndarray:
        """The stored params buffer: header (s_g, amax, 0, 0) then the block scales."""
        head = np.array([self.s_g, self.amax, 0, 0], np.float32).view(np.uint8)
        return np.concatenate([head, self.scales.reshape(-1)])


def stream_scale(amax: np.float32) -> np.float32:
    return np.float32(1.0) if amax == 0 else np.float32(amax) / np.float32(2688.0)


def encode_values(v: np.ndarray):
    """Encode binary32 values [n, H, D] (BF16-representable) as one stream; returns
    (codes, scales, s_g, amax, decoded binary32 values)."""
    v = np.asarray(v, np.float32)
    n, H, D = v.shape
    blk = v.reshape(n, H, D // BLOCK, BLOCK)
    amax = np.float32(np.abs(v).max()) if v.size else np.float32(0)
    s_g = stream_scale(amax)
    amax_b = np.abs(blk).max(axis=-1)                               # exact
    sb32 = amax_b / (np.float32(6.0) * s_g)                          # binary32 quotient
    e4 = e4m3_round(sb32.astype(np.float32))
    scales = e4m3_bits(e4)
    bs = (e4.astype(np.float32) * s_g).astype(np.float32)            # binary32 product
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(bs[..., None] > 0, blk / bs[..., None], np.float32(0)).astype(np.float32)
    codes4 = e2m1_code(y)
    codes4 = np.where(bs[..., None] > 0, codes4, np.uint8(0)).astype(np.uint8)
    dec = (e2m1_value(codes4).astype(np.float32) * bs[..., None]).astype(np.float32)
    codes4 = codes4.reshape(n, H, D)
    codes = (codes4[..., 0::2] | (codes4[..., 1::2] << 4)).astype(np.uint8)
    return codes, scales, s_g, amax, dec.reshape(n, H, D)


def decode_stream(s: Fp4Stream) -> np.ndarray:
    """Binary32 values [n, H, D] of a stream (from its stored bytes only)."""
    n, H, half = s.codes.shape
    D = 2 * half
    c4 = np.empty((n, H, D), np.uint8)
    c4[..., 0::2] = s.codes & 15
    c4[..., 1::2] = s.codes >> 4
    bs = (e4m3_value(s.scales).astype(np.float32) * np.float32(s.s_g)).astype(np.float32)
    v = e2m1_value(c4).astype(np.float32).reshape(n, H, D // BLOCK, BLOCK) * bs[..., None]
    return v.astype(np.float32).reshape(n, H, D)


# ----------------------------------------------------------------------------- MXFP4 streams

def e8m0_value(bits: np.ndarray) -> np.ndarray:
    """E8M0: an unsigned biased exponent, byte b -> 2^(b - 127) (0xFF, NaN, is never written)."""
    return np.ldexp(1.0, np.asarray(bits, np.int64) - 127)


def mx_scale_bits(amax_b: np.ndarray) -> np.ndarray:
    """E8M0 byte of a block's shared scale: floor(log2(amax_b)) - 2, clamped to [-127, 127],
    plus the bias 127; -127 for a block of zeros."""
    a = np.asarray(amax_b, np.float64)
    _, k = np.frexp(a)                                              # a = f * 2^k, f in [0.5, 1)
    e = np.where(a > 0, k - 1 - E2M1_EMAX, -127)
    return (np.clip(e, -127, 127) + 127).astype(np.uint8)


@dataclass
class MxStream:
    codes: np.ndarray            # uint8 [n, H, D/2]
    scales: np.ndarray           # uint8 [n, H, D/32], E8M0
    rows: Optional[np.ndarray]   # ascending positions, or None (dense)

    @property
    def n_rows(self) -> int:
        return self.codes.shape[0]

    def params_bytes(self) -> np.ndarray:
        """The stored params buffer: the block scales."""
        return self.scales.reshape(-1).copy()


def mx_encode_values(v: np.ndarray):
    """Encode binary32 values [n, H, D] (BF16-representable) as one MXFP4 stream; returns
    (codes, scales, decoded binary32 values)."""
    v = np.asarray(v, np.float32)
    n, H, D = v.shape
    blk = v.reshape(n, H, D // MX_BLOCK, MX_BLOCK).astype(np.float64)
    scales = mx_scale_bits(np.abs(blk).max(axis=-1)) if v.size else np.zeros((n, H, D // MX_BLOCK), np.uint8)
    X = e8m0_value(scales)[..., None]
    codes4 = e2m1_code(blk / X)                                     # exact quotient
    dec = (e2m1_value(codes4) * X).astype(np.float32)               # exact product
    codes4 = codes4.reshape(n, H, D)
    codes = (codes4[..., 0::2] | (codes4[..., 1::2] << 4)).astype(np.uint8)
    return codes, scales, dec.reshape(n, H, D)


def mx_decode_stream(s: MxStream) -> np.ndarray:
    """Binary32 values [n, H, D] of an MXFP4 stream (from its stored bytes only)."""
    n, H, half = s.codes.shape
    D = 2 * half
    c4 = np.empty((n, H, D), np.uint8)
    c4[..., 0::2] = s.codes & 15
    c4[..., 1::2] = s.codes >> 4
    X = e8m0_value(s.scales)[..., None]
    v = e2m1_value(c4).reshape(n, H, D // MX_BLOCK, MX_BLOCK) * X
    return v.astype(np.float32).reshape(n, H, D)


def mx_stream_bits_per_element(H: int, D: int, n: int) -> float:
    """Stored bits per encoded element: 4 for the code and 8 per 32 for the block scale."""
    return (n * H * D / 2 + n * H * D / MX_BLOCK) * 8 / (n * H * D)


# ----------------------------------------------------------------------------- chains

def encode_base(x: np.ndarray, mx: bool = False):
    """Loop 1 as an NVFP4 (or, with mx, MXFP4) stream: x BF16 [T, H, D] -> (stream, X_hat_1
    BF16)."""
    if mx:
        codes, scales, dec = mx_encode_values(f32_of_bf16(x))
        return MxStream(codes, scales, None), bf16_of_f32(dec)
    codes, scales, s_g, amax, dec = encode_values(f32_of_bf16(x))
    return Fp4Stream(codes, scales, s_g, amax, None), bf16_of_f32(dec)


def encode_residual(x_rows: np.ndarray, rows: Optional[np.ndarray], recon: np.ndarray, mx: bool = False):
    """Loop r >= 2 as an NVFP4 (or MXFP4) residual against recon = X_hat_{r-1} (BF16 [T, H, D],
    updated in place to X_hat_r).  x_rows: BF16 [n, H, D] at the ascending positions rows
    (None = dense)."""
    idx = np.arange(recon.shape[0]) if rows is None else np.asarray(rows, np.int64)
    prev = f32_of_bf16(recon[idx])
    delta = f32_of_bf16(bf16_of_f32(f32_of_bf16(x_rows) - prev))    # residual rounded to BF16
    keep = None if rows is None else np.asarray(rows, np.int32)
    if mx:
        codes, scales, dec = mx_encode_values(delta)
        stream = MxStream(codes, scales, keep)
    else:
        codes, scales, s_g, amax, dec = encode_values(delta)
        stream = Fp4Stream(codes, scales, s_g, amax, keep)
    dhat = f32_of_bf16(bf16_of_f32(dec))
    recon[idx] = bf16_of_f32(prev + dhat)
    return stream


def apply_residuals(base_recon: np.ndarray, residuals: list) -> np.ndarray:
    """X_hat after the residual streams, from the base loop's reconstruction and the streams'
    stored bytes only."""
    out = base_recon.copy()
    for s in residuals:
        if s.n_rows == 0:
            continue
        idx = np.arange(out.shape[0]) if s.rows is None else s.rows.astype(np.int64)
        vals = mx_decode_stream(s) if isinstance(s, MxStream) else decode_stream(s)
        dhat = f32_of_bf16(bf16_of_f32(vals))
        out[idx] = bf16_of_f32(f32_of_bf16(out[idx]) + dhat)
    return out


def stream_bits_per_element(H: int, D: int, n: int) -> float:
    """Stored bits per encoded element: 4 for the code, 8 per 16 for the block scale, and the
    16-byte header spread over the stream."""
    return (n * H * D / 2 + n * H * D / BLOCK + HEADER_BYTES) * 8 / (n * H * D)
