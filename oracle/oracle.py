"""Python driver for the scalar C oracle of the FlashLoop packed-KV codec.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and its
binding) never imports this module, and this module never imports the product.

The arithmetic lives in ``flk_oracle.c``; this file only marshals numpy arrays.  The
method it checks is described in the FlashLoop integration RFC (vllm-rlt issue #156),
section 3.3, and in vllm-rlt pull request #166 ("Purpose" and the review's format notes).

Array conventions: BF16 tensors are numpy ``uint16`` arrays of bit patterns shaped
``[rows, H, D]``; codes are ``uint8`` ``[rows, H, D//2]``; params are ``uint32`` (FP16
minimum in the low half, FP16 scale in the high half), ``[ceil(rows/64), H, D]`` for K,
``[ceil(T/64), H, D]`` for K with tile (page-local) groups and ``[rows, H, ceil(D/64)]``
for V; ``rows`` are ascending ``int32`` positions or ``None``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flk_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

K, V = 0, 1
GROUP = 64

OK, E_NONFINITE, E_RANGE, E_ARG = 0, 1, 2, 3


class OracleError(RuntimeError):
    """Raised when the oracle rejects its input (non-finite values, FP16 overflow, shape)."""

    def __init__(self, code: int, what: str):
        names = {E_NONFINITE: "non-finite input", E_RANGE: "FP16 parameter overflow",
                 E_ARG: "bad argument"}
        super().__init__(f"{what}: {names.get(code, code)}")
        self.code = code


def build(force: bool = False) -> str:
    """Compile the oracle with plain gcc (IEEE binary32, no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
            "-frounding-math", "-fexcess-precision=standard", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i = ctypes.c_int
        sz = ctypes.c_size_t
        L = _lib
        L.orc_bf16_from_f32.restype = ctypes.c_uint16
        L.orc_bf16_from_f32.argtypes = [ctypes.c_float]
        L.orc_f16_from_f32.restype = ctypes.c_uint16
        L.orc_f16_from_f32.argtypes = [ctypes.c_float]
        L.orc_f32_from_f16.restype = ctypes.c_float
        L.orc_f32_from_f16.argtypes = [ctypes.c_uint16]
        L.orc_f32_from_bf16.restype = ctypes.c_float
        L.orc_f32_from_bf16.argtypes = [ctypes.c_uint16]
        for name in ("orc_bf16_from_f32_array", "orc_f16_from_f32_array", "orc_f32_from_f16_array"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [P, P, sz]
        L.orc_num_groups.restype = sz
        L.orc_num_groups.argtypes = [i, i, i, i]
        L.orc_codes_bytes.restype = sz
        L.orc_codes_bytes.argtypes = [i, i, i]
        L.orc_params_bytes.restype = sz
        L.orc_params_bytes.argtypes = [i, i, i, i]
        L.orc_rows_bytes.restype = sz
        L.orc_rows_bytes.argtypes = [i, i]
        L.orc_quantize.restype = i
        L.orc_quantize.argtypes = [i, i, i, i, P, P, P, i]
        L.orc_dequantize.restype = i
        L.orc_dequantize.argtypes = [i, i, i, i, P, P, P]
        L.orc_encode_base.restype = i
        L.orc_encode_base.argtypes = [i, i, i, i, P, P, P, P, i, i]
        L.orc_encode_residual.restype = i
        L.orc_encode_residual.argtypes = [i, i, i, i, i, P, P, P, P, P, i, i]
        L.orc_reconstruct.restype = i
        L.orc_reconstruct.argtypes = [i, i, i, i, i, P, P, P, P, P, i]
        L.orc_quantize_k_tiles.restype = i
        L.orc_quantize_k_tiles.argtypes = [i, i, i, i, P, P, P, P, i]
        L.orc_dequantize_k_tiles.restype = i
        L.orc_dequantize_k_tiles.argtypes = [i, i, i, i, P, P, P, P]
        L.orc_k_tile_params_bytes.restype = sz
        L.orc_k_tile_params_bytes.argtypes = [i, i, i]
        L.orc_tile_index.restype = i
        L.orc_tile_index.argtypes = [P, i, i, P]
        L.orc_decode_attn.restype = i
        L.orc_decode_attn.argtypes = [i, i, i, i, P, P, P, ctypes.c_double, P]
        L.orc_sparse_reference.restype = i
        L.orc_sparse_reference.argtypes = [i, i, i, i, P, P, P, ctypes.c_double, i, P, P, P, P]
        L.orc_sparse_loop.restype = i
        L.orc_sparse_loop.argtypes = [i, i, i, i, P, P, P, ctypes.c_double, i, P, P, P, P, P]
        L.orc_sparse_stats.restype = i
        L.orc_sparse_stats.argtypes = [i, i, P, P, i, P, P, P, P]
        L.orc_sparse_correct.restype = i
        L.orc_sparse_correct.argtypes = [i, i, P, P, ctypes.c_double, P, P, P]
        L.orc_topk_positions.restype = i
        L.orc_topk_positions.argtypes = [i, P, i, P]
        L.orc_attn_scores.restype = i
        L.orc_attn_scores.argtypes = [i, i, i, i, P, P, ctypes.c_double, P]
        L.orc_sparse_reference_given.restype = i
        L.orc_sparse_reference_given.argtypes = [i, i, i, i, P, P, P, ctypes.c_double, i, P, P, P, P]
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------- conversions

def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_from_f32_array(_p(x), _p(out), x.size)
    return out


def f16_from_f32(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f16_from_f32_array(_p(x), _p(out), x.size)
    return out


def f32_from_f16(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_f32_from_f16_array(_p(h), _p(out), h.size)
    return out


def f32_from_bf16(b: np.ndarray) -> np.ndarray:
    """Widening is exact: a BF16 pattern is the upper half of a binary32 pattern."""
    return (_c(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- sizes

def num_groups(kind: int, H: int, D: int, n: int) -> int:
    return int(lib().orc_num_groups(kind, H, D, n))


def codes_bytes(H: int, D: int, n: int) -> int:
    return int(lib().orc_codes_bytes(H, D, n))


def params_bytes(kind: int, H: int, D: int, n: int) -> int:
    return int(lib().orc_params_bytes(kind, H, D, n))


def rows_bytes(n: int, sparse: bool) -> int:
    return int(lib().orc_rows_bytes(n, 1 if sparse else 0))


def params_shape(kind: int, H: int, D: int, n: int, T: Optional[int] = None, k_tiles: bool = False):
    """K with tile groups has one parameter row per 64-position tile of the T positions."""
    if kind == K and k_tiles:
        return ((T + GROUP - 1) // GROUP, H, D)
    return ((n + GROUP - 1) // GROUP, H, D) if kind == K else (n, H, (D + GROUP - 1) // GROUP)


def k_tile_params_bytes(H: int, D: int, T: int) -> int:
    return int(lib().orc_k_tile_params_bytes(H, D, T))


# ----------------------------------------------------------------------------- codec

@dataclass
class Stream:
    """One encoded loop of one tensor: n compact rows (rows None = dense), codes, params."""
    n_rows: int
    rows: Optional[np.ndarray]
    codes: np.ndarray
    params: np.ndarray

    def nbytes(self) -> int:
        return self.codes.nbytes + self.params.nbytes + (0 if self.rows is None else self.rows.nbytes)


def _check(st: int, what: str):
    if st != OK:
        raise OracleError(st, what)


def quantize(kind: int, x: np.ndarray, f32_params: bool = False):
    x = _c(x, np.uint16)
    n, H, D = x.shape
    codes = np.zeros((n, H, D // 2), np.uint8)
    params = np.zeros(params_shape(kind, H, D, n), np.uint32)
    _check(lib().orc_quantize(kind, H, D, n, _p(x), _p(codes), _p(params), int(f32_params)), "quantize")
    return codes, params


def dequantize(kind: int, codes: np.ndarray, params: np.ndarray, D: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    params = _c(params, np.uint32)
    n, H = codes.shape[0], codes.shape[1]
    out = np.zeros((n, H, D), np.uint16)
    _check(lib().orc_dequantize(kind, H, D, n, _p(codes), _p(params), _p(out)), "dequantize")
    return out


def quantize_k_tiles(x: np.ndarray, rows: Optional[np.ndarray], T: int, f32_params: bool = False):
    """K rows x [n, H, D] at positions rows (None = 0..n-1) with tile groups: one group per
    (64-position tile, head, channel).  Returns codes [n, H, D//2], params [ceil(T/64), H, D]."""
    x = _c(x, np.uint16)
    n, H, D = x.shape
    rows_c = None if rows is None else _c(rows, np.int32)
    codes = np.zeros((n, H, D // 2), np.uint8)
    params = np.zeros(params_shape(K, H, D, n, T, True), np.uint32)
    _check(lib().orc_quantize_k_tiles(H, D, T, n, _p(rows_c), _p(x), _p(codes), _p(params), int(f32_params)),
           "quantize_k_tiles")
    return codes, params


def dequantize_k_tiles(codes: np.ndarray, params: np.ndarray, rows: Optional[np.ndarray], T: int,
                       D: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    params = _c(params, np.uint32)
    n, H = codes.shape[0], codes.shape[1]
    rows_c = None if rows is None else _c(rows, np.int32)
    out = np.zeros((n, H, D), np.uint16)
    _check(lib().orc_dequantize_k_tiles(H, D, T, n, _p(rows_c), _p(codes), _p(params), _p(out)),
           "dequantize_k_tiles")
    return out


def encode_base(kind: int, x: np.ndarray, f32_params: bool = False, k_tiles: bool = False):
    """Returns (Stream, recon) with recon = X_hat[1] as BF16 bits."""
    x = _c(x, np.uint16)
    T, H, D = x.shape
    codes = np.zeros((T, H, D // 2), np.uint8)
    params = np.zeros(params_shape(kind, H, D, T, T, k_tiles), np.uint32)
    recon = np.zeros_like(x)
    _check(lib().orc_encode_base(kind, H, D, T, _p(x), _p(codes), _p(params), _p(recon), int(f32_params),
                                 int(k_tiles)), "encode_base")
    return Stream(T, None, codes, params), recon


def encode_residual(kind: int, x_rows: np.ndarray, rows: Optional[np.ndarray], recon: np.ndarray,
                    f32_params: bool = False, k_tiles: bool = False) -> Stream:
    """Encode one residual loop; `recon` (X_hat[r-1]) is updated in place to X_hat[r]."""
    x_rows = _c(x_rows, np.uint16)
    assert recon.dtype == np.uint16 and recon.flags.c_contiguous
    n, H, D = x_rows.shape
    T = recon.shape[0]
    rows_c = None if rows is None else _c(rows, np.int32)
    codes = np.zeros((n, H, D // 2), np.uint8)
    params = np.zeros(params_shape(kind, H, D, n, T, k_tiles), np.uint32)
    _check(lib().orc_encode_residual(kind, H, D, T, n, _p(rows_c), _p(x_rows), _p(recon), _p(codes),
                                     _p(params), int(f32_params), int(k_tiles)), "encode_residual")
    return Stream(n, rows_c, codes, params)


def reconstruct(kind: int, chain: Sequence[Stream], T: int, H: int, D: int, k_tiles: bool = False) -> np.ndarray:
    n_loops = len(chain)
    n_rows = np.array([s.n_rows for s in chain], np.int32)
    keep = [(s.rows, _c(s.codes, np.uint8), _c(s.params, np.uint32)) for s in chain]
    P = ctypes.c_void_p
    rows_arr = (P * n_loops)(*[(_p(r).value if r is not None else None) for r, _, _ in keep])
    codes_arr = (P * n_loops)(*[_p(c).value for _, c, _ in keep])
    params_arr = (P * n_loops)(*[_p(p).value for _, _, p in keep])
    out = np.zeros((T, H, D), np.uint16)
    _check(lib().orc_reconstruct(kind, H, D, T, n_loops, _p(n_rows), rows_arr, codes_arr, params_arr,
                                 _p(out), int(k_tiles)), "reconstruct")
    return out


def encode_chain(kind: int, xs: Sequence[np.ndarray], rows_list: Sequence[Optional[np.ndarray]],
                 f32_params: bool = False, k_tiles: bool = False):
    """Encode a full loop chain.  xs[0] is X[1] over all T rows; xs[r] (r >= 1) holds X[r+1]
    at the positions rows_list[r] (all T rows when that entry is None).  Returns the list of
    Streams and the final in-place reconstruction X_hat[R]."""
    base, recon = encode_base(kind, xs[0], f32_params, k_tiles)
    chain: List[Stream] = [base]
    for x, rows in zip(xs[1:], rows_list[1:]):
        chain.append(encode_residual(kind, x, rows, recon, f32_params, k_tiles))
    return chain, recon


def tile_index(rows: np.ndarray, T: int) -> np.ndarray:
    """out[t] = number of rows < 64*t for t = 0 .. ceil(T/64)."""
    rows = _c(rows, np.int32)
    out = np.zeros((T + GROUP - 1) // GROUP + 1, np.int32)
    _check(lib().orc_tile_index(_p(rows), rows.size, T, _p(out)), "tile_index")
    return out


def decode_attn(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Binary64 softmax attention of BF16 queries [Hq, D] over BF16 K/V [T, Hkv, D]."""
    q = _c(q, np.uint16)
    khat = _c(khat, np.uint16)
    vhat = _c(vhat, np.uint16)
    Hq, D = q.shape
    T, Hkv, _ = khat.shape
    out = np.zeros((Hq, D), np.float64)
    _check(lib().orc_decode_attn(Hq, Hkv, D, T, _p(q), _p(khat), _p(vhat), float(softmax_scale), _p(out)),
           "decode_attn")
    return out


# ----------------------------------------------------------------------------- rolling tail

def rolling_prefix(n_tokens: int) -> int:
    """Positions a rolling cache of n_tokens holds packed; the rest stay in the BF16 tail.

    RFC section 3.3 (last paragraph): the rolling tail keeps at least 64 recent tokens and
    flushes whole 64-token groups, so after a step it holds 64 to 127 tokens.  Written as the
    rule itself: the packed prefix is the largest whole number of 64-token groups that still
    leaves 64 tokens in the tail (none while fewer than 128 tokens exist)."""
    prefix = 0
    while n_tokens - (prefix + GROUP) >= GROUP:
        prefix += GROUP
    return prefix


def decode_attn_rolling(q: np.ndarray, khat_prefix: np.ndarray, vhat_prefix: np.ndarray,
                        k_tail: np.ndarray, v_tail: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Attention of one query over a rolling cache: the packed prefix's reconstruction
    followed by the BF16 tail (RFC section 3.3: the recent BF16 tail stays part of the
    cache).  Plain concatenation of the two token ranges, then textbook attention."""
    khat = np.concatenate([khat_prefix, k_tail], axis=0)
    vhat = np.concatenate([vhat_prefix, v_tail], axis=0)
    return decode_attn(q, khat, vhat, softmax_scale)


# ----------------------------------------------------------------------------- sparse decode attention

@dataclass
class SparseRef:
    """Reference-loop state per query head (RFC section 3.2): selected positions (ascending),
    their reference mass, the full reference output and the selected keys' contribution."""
    sel: np.ndarray      # int32 [Hq, k]
    mass: np.ndarray     # float64 [Hq]
    o_ref: np.ndarray    # float64 [Hq, D]
    c_ref: np.ndarray    # float64 [Hq, D]


def sparse_reference(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray, softmax_scale: float, k: int) -> SparseRef:
    q, khat, vhat = _c(q, np.uint16), _c(khat, np.uint16), _c(vhat, np.uint16)
    Hq, D = q.shape
    T, Hkv, _ = khat.shape
    sel = np.zeros((Hq, k), np.int32)
    mass = np.zeros(Hq, np.float64)
    o_ref = np.zeros((Hq, D), np.float64)
    c_ref = np.zeros((Hq, D), np.float64)
    _check(lib().orc_sparse_reference(Hq, Hkv, D, T, _p(q), _p(khat), _p(vhat), float(softmax_scale), k, _p(sel),
                                      _p(mass), _p(o_ref), _p(c_ref)), "sparse_reference")
    return SparseRef(sel, mass, o_ref, c_ref)


def sparse_loop(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray, softmax_scale: float, ref: SparseRef) -> np.ndarray:
    q, khat, vhat = _c(q, np.uint16), _c(khat, np.uint16), _c(vhat, np.uint16)
    Hq, D = q.shape
    T, Hkv, _ = khat.shape
    k = ref.sel.shape[1]
    out = np.zeros((Hq, D), np.float64)
    _check(lib().orc_sparse_loop(Hq, Hkv, D, T, _p(q), _p(khat), _p(vhat), float(softmax_scale), k,
                                 _p(_c(ref.sel, np.int32)), _p(_c(ref.mass, np.float64)),
                                 _p(_c(ref.o_ref, np.float64)), _p(_c(ref.c_ref, np.float64)), _p(out)), "sparse_loop")
    return out


def sparse_stats(p: np.ndarray, v: np.ndarray, sel: np.ndarray):
    """(m, O_ref, C_ref) of one head from its reference probabilities p [T] and values v [T, D]."""
    p, v, sel = _c(p, np.float64), _c(v, np.float64), _c(sel, np.int32)
    T, D = v.shape
    m = np.zeros(1, np.float64)
    o_ref, c_ref = np.zeros(D, np.float64), np.zeros(D, np.float64)
    _check(lib().orc_sparse_stats(T, D, _p(p), _p(v), sel.size, _p(sel), _p(m), _p(o_ref), _p(c_ref)), "sparse_stats")
    return float(m[0]), o_ref, c_ref


def sparse_correct(p_local: np.ndarray, v_sel: np.ndarray, m: float, o_ref: np.ndarray, c_ref: np.ndarray):
    p_local, v_sel = _c(p_local, np.float64), _c(v_sel, np.float64)
    k, D = v_sel.shape
    out = np.zeros(D, np.float64)
    _check(lib().orc_sparse_correct(k, D, _p(p_local), _p(v_sel), float(m), _p(_c(o_ref, np.float64)),
                                    _p(_c(c_ref, np.float64)), _p(out)), "sparse_correct")
    return out


def topk_positions(scores: np.ndarray, k: int) -> np.ndarray:
    scores = _c(scores, np.float64)
    sel = np.zeros(k, np.int32)
    _check(lib().orc_topk_positions(scores.size, _p(scores), k, _p(sel)), "topk_positions")
    return sel


def attn_scores(q: np.ndarray, khat: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Binary64 scaled scores [Hq, T] of BF16 queries [Hq, D] against BF16 keys [T, Hkv, D]."""
    q, khat = _c(q, np.uint16), _c(khat, np.uint16)
    Hq, D = q.shape
    T, Hkv, _ = khat.shape
    out = np.zeros((Hq, T), np.float64)
    _check(lib().orc_attn_scores(Hq, Hkv, D, T, _p(q), _p(khat), float(softmax_scale), _p(out)), "attn_scores")
    return out


def sparse_reference_given(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray, softmax_scale: float,
                           sel: np.ndarray) -> SparseRef:
    """The reference statistics for the selection sel [Hq, k] (made elsewhere)."""
    q, khat, vhat = _c(q, np.uint16), _c(khat, np.uint16), _c(vhat, np.uint16)
    sel = _c(sel, np.int32)
    Hq, D = q.shape
    T, Hkv, _ = khat.shape
    k = sel.shape[1]
    mass = np.zeros(Hq, np.float64)
    o_ref = np.zeros((Hq, D), np.float64)
    c_ref = np.zeros((Hq, D), np.float64)
    _check(lib().orc_sparse_reference_given(Hq, Hkv, D, T, _p(q), _p(khat), _p(vhat), float(softmax_scale), k,
                                            _p(sel), _p(mass), _p(o_ref), _p(c_ref)), "sparse_reference_given")
    return SparseRef(sel, mass, o_ref, c_ref)
