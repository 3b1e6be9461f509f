"""ctypes binding of libflk.so, the gfx950 packed-KV codec (include/flk.h).

Argument marshalling only: every step of the codec runs in the HIP kernels behind the C ABI.
torch supplies device memory and the current stream.  There is no CPU fallback: if the
library is missing or cannot load, every call raises.

Tensors: BF16 data are torch.bfloat16 [rows, H, D] (contiguous, on the GPU); codes are
torch.uint8 [n, H, D//2]; params torch.int32 (FP16 min | FP16 scale << 16, bit pattern),
shaped [ceil(n/64), H, D] for K, [ceil(T/64), H, D] for K with tile (page-local) groups and
[n, H, ceil(D/64)] for V; rows are torch.int32 [n] ascending positions or None (dense).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflk.so")

K, V = 0, 1
KGROUP_ROWS, KGROUP_TILE = 0, 1
GROUP = 64
MAX_LOOPS = 8
DEV_NONFINITE, DEV_RANGE, DEV_ROWS = 1, 2, 4


class FlkError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = _lib.flk_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint16), ("format", ctypes.c_uint8), ("kind", ctypes.c_uint8),
                ("group", ctypes.c_uint16), ("param_dtype", ctypes.c_uint8), ("nibble_order", ctypes.c_uint8),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("k_grouping", ctypes.c_uint8),
                ("reserved", ctypes.c_uint8 * 3)]


class StreamC(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int32), ("reserved", ctypes.c_int32), ("rows", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("params", ctypes.c_void_p), ("tile_start", ctypes.c_void_p)]


class UnitC(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_void_p), ("recon", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("params", ctypes.c_void_p), ("tile_start", ctypes.c_void_p),
                ("n_rows", ctypes.c_int32), ("T", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class AppendUnitC(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_void_p), ("recon", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("params", ctypes.c_void_p), ("tile_start", ctypes.c_void_p),
                ("n_rows", ctypes.c_int32), ("p0", ctypes.c_int32), ("n_pos", ctypes.c_int32),
                ("rows_before", ctypes.c_int32), ("kind", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ReconUnitC(ctypes.Structure):
    _fields_ = [("chain", ctypes.POINTER(StreamC)), ("out", ctypes.c_void_p), ("T", ctypes.c_int32),
                ("n_loops", ctypes.c_int32), ("kind", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libflk.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m quantized_kv_cache_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(Desc)
        S = ctypes.POINTER(StreamC)
        L.flk_desc_init.restype = None
        L.flk_desc_init.argtypes = [D, ctypes.c_int, i32, i32]
        L.flk_desc_check.restype = ctypes.c_int
        L.flk_desc_check.argtypes = [D]
        L.flk_codes_bytes.restype = sz
        L.flk_codes_bytes.argtypes = [D, i32]
        L.flk_params_bytes.restype = sz
        L.flk_params_bytes.argtypes = [D, i32, i32]
        L.flk_stream_bytes.restype = sz
        L.flk_stream_bytes.argtypes = [D, i32, i32, ctypes.c_int]
        L.flk_rolling_prefix.restype = i32
        L.flk_rolling_prefix.argtypes = [i32]
        L.flk_append_base.restype = ctypes.c_int
        L.flk_append_base.argtypes = [D, P, i32, i32, P, P, P, P, P]
        L.flk_append_residual.restype = ctypes.c_int
        L.flk_append_residual.argtypes = [D, P, P, i32, i32, i32, i32, P, P, P, P, P, P]
        L.flk_decode_attn_rolling.restype = ctypes.c_int
        L.flk_decode_attn_rolling.argtypes = [D, D, i32, P, i32, S, S, i32, P, P, i32, ctypes.c_float, P, P, sz, P]
        L.flk_rows_bytes.restype = sz
        L.flk_rows_bytes.argtypes = [i32, ctypes.c_int]
        L.flk_tile_index_bytes.restype = sz
        L.flk_tile_index_bytes.argtypes = [i32]
        L.flk_attn_workspace_bytes.restype = sz
        L.flk_attn_workspace_bytes.argtypes = [D, i32, i32]
        L.flk_status_string.restype = ctypes.c_char_p
        L.flk_status_string.argtypes = [ctypes.c_int]
        L.flk_abi_version.restype = ctypes.c_int
        L.flk_abi_version.argtypes = []
        L.flk_encode_base.restype = ctypes.c_int
        L.flk_encode_base.argtypes = [D, P, i32, P, P, P, P, P]
        L.flk_encode_residual.restype = ctypes.c_int
        L.flk_encode_residual.argtypes = [D, P, P, i32, i32, P, P, P, P, P, P]
        L.flk_reconstruct.restype = ctypes.c_int
        L.flk_reconstruct.argtypes = [D, i32, S, i32, P, P]
        U = ctypes.POINTER(UnitC)
        for name in ("flk_encode_base_batch", "flk_encode_residual_batch"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [D, D, U, i32, P, P]
        for name in ("flk_append_base_batch", "flk_append_residual_batch"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [D, D, ctypes.POINTER(AppendUnitC), i32, P, P]
        L.flk_reconstruct_batch.restype = ctypes.c_int
        L.flk_reconstruct_batch.argtypes = [D, D, ctypes.POINTER(ReconUnitC), i32, P]
        L.flk_sparse_workspace_bytes.restype = sz
        L.flk_sparse_workspace_bytes.argtypes = [D, i32, i32, i32, i32]
        L.flk_sparse_attn_reference.restype = ctypes.c_int
        L.flk_sparse_attn_reference.argtypes = [D, D, i32, P, i32, S, S, i32, i32, ctypes.c_float, P, P, P, P, P, P,
                                                sz, P]
        L.flk_sparse_attn_loop.restype = ctypes.c_int
        L.flk_sparse_attn_loop.argtypes = [D, D, i32, P, i32, S, S, i32, i32, ctypes.c_float, P, P, P, P, P, P, sz, P]
        L.flk_sparse_attn_reference_mixed.restype = ctypes.c_int
        L.flk_sparse_attn_reference_mixed.argtypes = [D, D, D, D, i32, P, i32, S, S, i32, i32, ctypes.c_float, P, P,
                                                      P, P, P, P, sz, P]
        L.flk_sparse_attn_loop_mixed.restype = ctypes.c_int
        L.flk_sparse_attn_loop_mixed.argtypes = [D, D, D, D, i32, P, i32, S, S, i32, i32, ctypes.c_float, P, P, P, P,
                                                 P, P, sz, P]
        for name in ("flk_desc_init_nvfp4", "flk_desc_init_mxfp4"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [D, ctypes.c_int, i32, i32]
        L.flk_reconstruct_mixed.restype = ctypes.c_int
        L.flk_reconstruct_mixed.argtypes = [D, D, i32, S, i32, P, P]
        L.flk_decode_attn_mixed.restype = ctypes.c_int
        L.flk_decode_attn_mixed.argtypes = [D, D, D, D, i32, P, i32, S, S, i32, ctypes.c_float, P, P, sz, P]
        L.flk_select_count.restype = i32
        L.flk_select_count.argtypes = [i32, i32, P, i32]
        L.flk_select_workspace_bytes.restype = sz
        L.flk_select_workspace_bytes.argtypes = [i32, i32]
        L.flk_select_rows.restype = ctypes.c_int
        L.flk_select_rows.argtypes = [P, P, i32, i32, P, i32, i32, i32, ctypes.c_float, P, P, i32, P, P, sz, P, P]
        L.flk_partition_rows.restype = ctypes.c_int
        L.flk_partition_rows.argtypes = [P, i32, P, P, P, P, P]
        L.flk_decode_attn_packed.restype = ctypes.c_int
        L.flk_decode_attn_packed.argtypes = [D, D, i32, P, i32, S, S, i32, ctypes.c_float, P, P, sz, P]
        L.flk_decode_attn_packed_noalloc.restype = ctypes.c_int
        L.flk_decode_attn_packed_noalloc.argtypes = [D, D, i32, P, i32, S, S, i32, ctypes.c_float, P, P]
        _lib = L
    return _lib


INT4, NVFP4, MXFP4 = "int4", "nvfp4", "mxfp4"
FORMATS = (INT4, NVFP4, MXFP4)


def _fmt(nvfp4: bool, fmt: Optional[str]) -> str:
    """The stream format from the nvfp4 flag or the format name (int4, nvfp4, mxfp4)."""
    if fmt is None:
        return NVFP4 if nvfp4 else INT4
    if fmt not in FORMATS or (nvfp4 and fmt != NVFP4):
        raise ValueError(f"unknown or conflicting stream format {fmt!r} (nvfp4={nvfp4})")
    return fmt


def desc(kind: int, H: int, D: int, k_tiles: bool = False, nvfp4: bool = False, fmt: Optional[str] = None) -> Desc:
    """k_tiles: K groups per 64-position tile (page-local) instead of per 64 compact rows;
    fmt (or nvfp4=True): NVFP4 (E2M1 codes, E4M3 scales per 16 channels, one FP32 stream
    scale) or MXFP4 (E2M1 codes, E8M0 scales per 32 channels) instead of INT4."""
    f = _fmt(nvfp4, fmt)
    d = Desc()
    if f != INT4:
        init = lib().flk_desc_init_nvfp4 if f == NVFP4 else lib().flk_desc_init_mxfp4
        init(ctypes.byref(d), kind, H, D)
        return d
    lib().flk_desc_init(ctypes.byref(d), kind, H, D)
    d.k_grouping = KGROUP_TILE if k_tiles else KGROUP_ROWS
    return d


def _check(st: int, what: str):
    if st != 0:
        raise FlkError(st, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected a contiguous {dtype} GPU tensor, got {t.dtype} {tuple(t.shape)}")


# ----------------------------------------------------------------------------- sizes

def codes_bytes(kind: int, H: int, D: int, n: int) -> int:
    return int(lib().flk_codes_bytes(ctypes.byref(desc(kind, H, D)), n))


def params_bytes(kind: int, H: int, D: int, n: int, T: int = 0, k_tiles: bool = False, nvfp4: bool = False,
                 fmt: Optional[str] = None) -> int:
    return int(lib().flk_params_bytes(ctypes.byref(desc(kind, H, D, k_tiles, nvfp4, fmt)), n, T))


def stream_bytes(kind: int, H: int, D: int, n: int, T: int, sparse: bool, k_tiles: bool = False,
                 nvfp4: bool = False, fmt: Optional[str] = None) -> int:
    return int(lib().flk_stream_bytes(ctypes.byref(desc(kind, H, D, k_tiles, nvfp4, fmt)), n, T,
                                      1 if sparse else 0))


def rolling_prefix(n_tokens: int) -> int:
    return int(lib().flk_rolling_prefix(n_tokens))


def rows_bytes(n: int, sparse: bool) -> int:
    return int(lib().flk_rows_bytes(n, 1 if sparse else 0))


def tile_index_bytes(T: int) -> int:
    return int(lib().flk_tile_index_bytes(T))


def attn_workspace_bytes(H: int, D: int, T: int, n_q_heads: int) -> int:
    return int(lib().flk_attn_workspace_bytes(ctypes.byref(desc(K, H, D)), T, n_q_heads))


def params_shape(kind: int, H: int, D: int, n: int, T: int = 0, k_tiles: bool = False):
    if kind == K and k_tiles:
        return ((T + GROUP - 1) // GROUP, H, D)
    return ((n + GROUP - 1) // GROUP, H, D) if kind == K else (n, H, (D + GROUP - 1) // GROUP)


@dataclass
class Packed:
    """Device buffers of one encoded loop (caller-owned torch tensors).  Compact loops also
    carry tile_start, the inverse map per 64 positions that flk_encode_residual writes.
    k_tiles marks K streams with tile (page-local) groups; it and fmt select the descriptor."""
    n_rows: int
    rows: Optional[torch.Tensor]
    codes: torch.Tensor
    params: torch.Tensor
    tile_start: Optional[torch.Tensor] = None
    k_tiles: bool = False
    fmt: str = INT4

    @property
    def nvfp4(self) -> bool:
        return self.fmt == NVFP4

    @staticmethod
    def empty(kind: int, H: int, D: int, n: int, rows: Optional[torch.Tensor] = None, T: int = 0,
              tile_start: Optional[torch.Tensor] = None, device="cuda", k_tiles: bool = False,
              compact: Optional[bool] = None, nvfp4: bool = False, fmt: Optional[str] = None) -> "Packed":
        """compact: the stream has a tile index (default: when rows is given).  fmt (or
        nvfp4=True): an NVFP4 stream (params: a 16-byte header, then one E4M3 byte per 16
        elements) or an MXFP4 stream (params: one E8M0 byte per 32 elements)."""
        f = _fmt(nvfp4, fmt)
        if k_tiles and kind == K and T < 1:
            raise ValueError("tile-grouped K needs T to size its params")
        if f != INT4 and k_tiles:
            raise ValueError("FP4 blocks run along channels; there are no tile groups")
        compact = rows is not None if compact is None else compact
        codes = torch.empty((n, H, D // 2), dtype=torch.uint8, device=device)
        if f != INT4:
            params = torch.empty((params_bytes(kind, H, D, n, fmt=f) + 3) // 4, dtype=torch.int32, device=device)
        else:
            params = torch.empty(params_shape(kind, H, D, n, T, k_tiles), dtype=torch.int32, device=device)
        if compact and tile_start is None:
            if T < 1:
                raise ValueError("a compact loop needs T to size its tile index")
            tile_start = torch.empty(tile_index_bytes(T) // 4, dtype=torch.int32, device=device)
        return Packed(n, rows, codes, params, tile_start if compact else None, k_tiles and kind == K, f)

    def c(self) -> StreamC:
        return StreamC(self.n_rows, 0, None if self.rows is None else self.rows.data_ptr(),
                       self.codes.data_ptr(), self.params.data_ptr(),
                       None if self.tile_start is None else self.tile_start.data_ptr())

    def nbytes(self) -> int:
        return self.codes.numel() + 4 * self.params.numel() + (0 if self.rows is None else 4 * self.rows.numel())


# ----------------------------------------------------------------------------- codec calls

def encode_base(kind: int, x: torch.Tensor, out: Packed, recon: torch.Tensor,
                status: Optional[torch.Tensor] = None, stream=None) -> None:
    _need(x, torch.bfloat16, "x")
    _need(recon, torch.bfloat16, "recon")
    T, H, D = x.shape
    _check(lib().flk_encode_base(ctypes.byref(desc(kind, H, D, out.k_tiles, fmt=out.fmt)), _ptr(x), T, _ptr(out.codes),
                                 _ptr(out.params), _ptr(recon), _ptr(status), _stream(stream)),
           "flk_encode_base")


def encode_residual(kind: int, x_rows: torch.Tensor, rows: Optional[torch.Tensor], recon: torch.Tensor,
                    out: Packed, status: Optional[torch.Tensor] = None, stream=None) -> None:
    _need(x_rows, torch.bfloat16, "x_rows")
    _need(recon, torch.bfloat16, "recon")
    if rows is not None:
        _need(rows, torch.int32, "rows")
    n, H, D = x_rows.shape
    T = recon.shape[0]
    _check(lib().flk_encode_residual(ctypes.byref(desc(kind, H, D, out.k_tiles, fmt=out.fmt)), _ptr(x_rows), _ptr(rows), n, T,
                                     _ptr(recon), _ptr(out.codes), _ptr(out.params), _ptr(out.tile_start),
                                     _ptr(status), _stream(stream)),
           "flk_encode_residual")


def _chain(chain: Sequence[Packed]):
    arr = (StreamC * len(chain))(*[p.c() for p in chain])
    return arr


def reconstruct(kind: int, chain: Sequence[Packed], out: torch.Tensor, stream=None) -> None:
    """X_hat of the chain; an INT4 or FP4 base, INT4 or FP4 residual loops (one format for all
    of them)."""
    _need(out, torch.bfloat16, "out")
    T, H, D = out.shape
    arr = _chain(chain)
    bf, rf = _chain_formats(chain)
    if bf == INT4 and rf == INT4:
        _check(lib().flk_reconstruct(ctypes.byref(desc(kind, H, D, chain[0].k_tiles)), T, arr, len(chain), _ptr(out),
                                     _stream(stream)), "flk_reconstruct")
        return
    _check(lib().flk_reconstruct_mixed(ctypes.byref(desc(kind, H, D, chain[0].k_tiles, fmt=bf)),
                                       ctypes.byref(desc(kind, H, D, fmt=rf)), T, arr, len(chain), _ptr(out),
                                       _stream(stream)), "flk_reconstruct_mixed")


def decode_attn_packed(q: torch.Tensor, k_chain: Sequence[Packed], v_chain: Sequence[Packed], T: int,
                       H: int, softmax_scale: float, out: torch.Tensor, workspace: torch.Tensor,
                       stream=None) -> None:
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    Hq, D = q.shape
    ka, va = _chain(k_chain), _chain(v_chain)
    _check(lib().flk_decode_attn_packed(ctypes.byref(desc(K, H, D, k_chain[0].k_tiles)), ctypes.byref(desc(V, H, D)),
                                        T, _ptr(q),
                                        Hq, ka, va, len(k_chain), float(softmax_scale), _ptr(out),
                                        _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(stream)), "flk_decode_attn_packed")


def decode_attn_packed_noalloc(q: torch.Tensor, k_chain: Sequence[Packed], v_chain: Sequence[Packed], T: int,
                               H: int, softmax_scale: float, out: torch.Tensor, stream=None) -> None:
    """decode_attn_packed with the library's per-device scratch array instead of a workspace."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    Hq, D = q.shape
    ka, va = _chain(k_chain), _chain(v_chain)
    _check(lib().flk_decode_attn_packed_noalloc(ctypes.byref(desc(K, H, D, k_chain[0].k_tiles)),
                                                ctypes.byref(desc(V, H, D)), T, _ptr(q), Hq, ka, va, len(k_chain),
                                                float(softmax_scale), _ptr(out), _stream(stream)),
           "flk_decode_attn_packed_noalloc")


def _chain_formats(chain: Sequence[Packed]):
    """(base format, residual format) of a chain; one format for all its residual loops."""
    base = chain[0].fmt
    resid = {p.fmt for p in chain[1:]}
    if len(resid) > 1:
        raise ValueError("the residual loops of one chain share one format")
    return base, (resid.pop() if resid else base)


def decode_attn_mixed(q: torch.Tensor, k_chain: Sequence[Packed], v_chain: Sequence[Packed], T: int,
                      H: int, softmax_scale: float, out: torch.Tensor, workspace: torch.Tensor,
                      stream=None) -> None:
    """Decode attention over chains of INT4 and FP4 streams (formats taken from the streams)."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    Hq, D = q.shape
    kb, kr = _chain_formats(k_chain)
    vb, vr = _chain_formats(v_chain)
    ka, va = _chain(k_chain), _chain(v_chain)
    _check(lib().flk_decode_attn_mixed(ctypes.byref(desc(K, H, D, k_chain[0].k_tiles, fmt=kb)),
                                       ctypes.byref(desc(K, H, D, fmt=kr)), ctypes.byref(desc(V, H, D, fmt=vb)),
                                       ctypes.byref(desc(V, H, D, fmt=vr)), T, _ptr(q), Hq, ka, va, len(k_chain),
                                       float(softmax_scale), _ptr(out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)),
           "flk_decode_attn_mixed")


# ----------------------------------------------------------------------------- rolling tail

def append_base(kind: int, x: torch.Tensor, p0: int, out: Packed, recon: torch.Tensor,
                status: Optional[torch.Tensor] = None, stream=None) -> None:
    """Encode loop 1 of positions [p0, p0 + len(x)) into the stream `out` (its full buffers);
    recon [len(x), H, D] receives the window's X_hat[1]."""
    _need(x, torch.bfloat16, "x")
    _need(recon, torch.bfloat16, "recon")
    n_pos, H, D = x.shape
    _check(lib().flk_append_base(ctypes.byref(desc(kind, H, D, out.k_tiles)), _ptr(x), p0, n_pos, _ptr(out.codes),
                                 _ptr(out.params), _ptr(recon), _ptr(status), _stream(stream)), "flk_append_base")


def append_residual(kind: int, x_rows: Optional[torch.Tensor], rows: Optional[torch.Tensor], n_rows: int, p0: int,
                    n_pos: int, rows_before: int, recon: torch.Tensor, out: Packed,
                    status: Optional[torch.Tensor] = None, stream=None) -> None:
    """Encode loop r >= 2 of positions [p0, p0 + n_pos) and append it to `out`.  rows: the
    window's entries of the stream's rows (absolute positions), None for a dense loop;
    recon [n_pos, H, D]: the window's X_hat[r-1], updated to X_hat[r]."""
    _need(recon, torch.bfloat16, "recon")
    if x_rows is not None:
        _need(x_rows, torch.bfloat16, "x_rows")
    if rows is not None:
        _need(rows, torch.int32, "rows")
    H, D = recon.shape[1], recon.shape[2]
    _check(lib().flk_append_residual(ctypes.byref(desc(kind, H, D, out.k_tiles)), _ptr(x_rows), _ptr(rows), n_rows,
                                     p0, n_pos, rows_before, _ptr(recon), _ptr(out.codes), _ptr(out.params),
                                     _ptr(out.tile_start), _ptr(status), _stream(stream)), "flk_append_residual")


def decode_attn_rolling(q: torch.Tensor, k_chain: Sequence[Packed], v_chain: Sequence[Packed], T: int, H: int,
                        k_tail: Optional[torch.Tensor], v_tail: Optional[torch.Tensor], softmax_scale: float,
                        out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """Attention over packed positions [0, T) plus the BF16 tail [tail_len, H, D]."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    tail_len = 0
    if k_tail is not None:
        _need(k_tail, torch.bfloat16, "k_tail")
        _need(v_tail, torch.bfloat16, "v_tail")
        tail_len = k_tail.shape[0]
    Hq, D = q.shape
    kt = bool(k_chain) and k_chain[0].k_tiles
    ka, va = _chain(k_chain), _chain(v_chain)
    _check(lib().flk_decode_attn_rolling(ctypes.byref(desc(K, H, D, kt)), ctypes.byref(desc(V, H, D)), T, _ptr(q),
                                         Hq, ka, va, len(k_chain), _ptr(k_tail), _ptr(v_tail), tail_len,
                                         float(softmax_scale), _ptr(out), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)),
           "flk_decode_attn_rolling")


# ----------------------------------------------------------------------------- batched calls

def _k_tiles(flags) -> bool:
    """One K descriptor covers every K unit of a batched call, so their groupings must agree."""
    flags = set(flags)
    if len(flags) > 1:
        raise ValueError("the K units of one batched call must share their K grouping")
    return bool(flags and flags.pop())

def _unit(kind: int, x: Optional[torch.Tensor], rows: Optional[torch.Tensor], recon: torch.Tensor,
          out: "Packed") -> UnitC:
    if x is not None:
        _need(x, torch.bfloat16, "x")
    _need(recon, torch.bfloat16, "recon")
    if rows is not None:
        _need(rows, torch.int32, "rows")
    n = out.n_rows
    return UnitC(None if x is None else x.data_ptr(), None if rows is None else rows.data_ptr(), recon.data_ptr(),
                 out.codes.data_ptr(), out.params.data_ptr(),
                 None if out.tile_start is None else out.tile_start.data_ptr(), n, recon.shape[0], kind, 0)


def encode_base_batch(items, H: int, D: int, status: Optional[torch.Tensor] = None, stream=None) -> None:
    """items: (kind, x [T, H, D], recon [T, H, D], out Packed) per tensor; one call for all."""
    units = [_unit(kind, x, None, recon, out) for kind, x, recon, out in items]
    arr = (UnitC * max(1, len(units)))(*units)
    kt = _k_tiles(out.k_tiles for kind, _, _, out in items if kind == K)
    _check(lib().flk_encode_base_batch(ctypes.byref(desc(K, H, D, kt)), ctypes.byref(desc(V, H, D)), arr, len(units),
                                       _ptr(status), _stream(stream)), "flk_encode_base_batch")


def encode_residual_batch(items, H: int, D: int, status: Optional[torch.Tensor] = None, stream=None) -> None:
    """items: (kind, x_rows [n, H, D], rows or None, recon [T, H, D], out Packed) per tensor."""
    units = [_unit(kind, x, rows, recon, out) for kind, x, rows, recon, out in items]
    arr = (UnitC * max(1, len(units)))(*units)
    kt = _k_tiles(out.k_tiles for kind, _, _, _, out in items if kind == K)
    _check(lib().flk_encode_residual_batch(ctypes.byref(desc(K, H, D, kt)), ctypes.byref(desc(V, H, D)), arr,
                                           len(units), _ptr(status), _stream(stream)), "flk_encode_residual_batch")


def reconstruct_batch(items, H: int, D: int, stream=None) -> None:
    """items: (kind, chain [Packed, ...], out [T, H, D]) per tensor."""
    keep, units = [], []
    for kind, chain, out in items:
        _need(out, torch.bfloat16, "out")
        arr = _chain(chain)
        keep.append(arr)
        units.append(ReconUnitC(ctypes.cast(arr, ctypes.POINTER(StreamC)), out.data_ptr(), out.shape[0], len(chain),
                                kind, 0))
    tab = (ReconUnitC * max(1, len(units)))(*units)
    kt = _k_tiles(chain[0].k_tiles for kind, chain, _ in items if kind == K)
    _check(lib().flk_reconstruct_batch(ctypes.byref(desc(K, H, D, kt)), ctypes.byref(desc(V, H, D)), tab, len(units),
                                       _stream(stream)), "flk_reconstruct_batch")



def _append_unit(kind, x, rows, n_rows, p0, n_pos, rows_before, recon, out: "Packed") -> AppendUnitC:
    _need(recon, torch.bfloat16, "recon")
    if x is not None:
        _need(x, torch.bfloat16, "x")
    if rows is not None:
        _need(rows, torch.int32, "rows")
    return AppendUnitC(None if x is None else x.data_ptr(), None if rows is None else rows.data_ptr(),
                       recon.data_ptr(), out.codes.data_ptr(), out.params.data_ptr(),
                       None if out.tile_start is None else out.tile_start.data_ptr(),
                       n_rows, p0, n_pos, rows_before, kind, 0)


def append_base_batch(items, H: int, D: int, status: Optional[torch.Tensor] = None, stream=None) -> None:
    """items: (kind, x [n_pos, H, D], p0, recon [n_pos, H, D], out Packed) per tensor."""
    units = [_append_unit(kind, x, None, x.shape[0], p0, x.shape[0], p0, recon, out)
             for kind, x, p0, recon, out in items]
    arr = (AppendUnitC * max(1, len(units)))(*units)
    kt = _k_tiles(out.k_tiles for kind, _, _, _, out in items if kind == K)
    _check(lib().flk_append_base_batch(ctypes.byref(desc(K, H, D, kt)), ctypes.byref(desc(V, H, D)), arr,
                                       len(units), _ptr(status), _stream(stream)), "flk_append_base_batch")


def append_residual_batch(items, H: int, D: int, status: Optional[torch.Tensor] = None, stream=None) -> None:
    """items: (kind, x_rows or None, rows or None, n_rows, p0, n_pos, rows_before, recon, out Packed)."""
    units = [_append_unit(*it) for it in items]
    arr = (AppendUnitC * max(1, len(units)))(*units)
    kt = _k_tiles(it[-1].k_tiles for it in items if it[0] == K)
    _check(lib().flk_append_residual_batch(ctypes.byref(desc(K, H, D, kt)), ctypes.byref(desc(V, H, D)), arr,
                                           len(units), _ptr(status), _stream(stream)), "flk_append_residual_batch")


# ----------------------------------------------------------------------------- sparse decode attention

def sparse_workspace_bytes(H: int, D: int, T: int, n_q_heads: int, k: int, n_loops: int) -> int:
    return int(lib().flk_sparse_workspace_bytes(ctypes.byref(desc(K, H, D)), T, n_q_heads, k, n_loops))


@dataclass
class SparseState:
    """Reference-loop state per query head (device tensors): S [Hq, k] int32 ascending
    positions, mass [Hq], o_ref and c_ref [Hq, D] float32."""
    sel: torch.Tensor
    mass: torch.Tensor
    o_ref: torch.Tensor
    c_ref: torch.Tensor

    @staticmethod
    def empty(n_q_heads: int, D: int, k: int, device="cuda") -> "SparseState":
        return SparseState(torch.empty((n_q_heads, k), dtype=torch.int32, device=device),
                           torch.empty(n_q_heads, dtype=torch.float32, device=device),
                           torch.empty((n_q_heads, D), dtype=torch.float32, device=device),
                           torch.empty((n_q_heads, D), dtype=torch.float32, device=device))


def _mixed_descs(k_chain: Sequence[Packed], v_chain: Sequence[Packed], H: int, D: int):
    """The four descriptors of the *_mixed calls, or None when both chains are INT4 throughout."""
    kb, kr = _chain_formats(k_chain)
    vb, vr = _chain_formats(v_chain)
    if {kb, kr, vb, vr} == {INT4}:
        return None
    return [desc(K, H, D, k_chain[0].k_tiles, fmt=kb), desc(K, H, D, fmt=kr), desc(V, H, D, fmt=vb),
            desc(V, H, D, fmt=vr)]


def sparse_attn_reference(q: torch.Tensor, k_chain: Sequence[Packed], v_chain: Sequence[Packed], T: int, H: int,
                          k: int, softmax_scale: float, out: torch.Tensor, state: SparseState,
                          workspace: torch.Tensor, stream=None) -> None:
    """The reference loop over INT4 chains, or (flk_sparse_attn_reference_mixed) chains with FP4
    streams; formats taken from the streams."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    Hq, D = q.shape
    ka, va = _chain(k_chain), _chain(v_chain)
    mixed = _mixed_descs(k_chain, v_chain, H, D)
    if mixed is not None:
        _check(lib().flk_sparse_attn_reference_mixed(*[ctypes.byref(d) for d in mixed], T, _ptr(q), Hq, ka, va,
                                                     len(k_chain), k, float(softmax_scale), _ptr(out),
                                                     _ptr(state.sel), _ptr(state.mass), _ptr(state.o_ref),
                                                     _ptr(state.c_ref), _ptr(workspace),
                                                     workspace.numel() * workspace.element_size(), _stream(stream)),
               "flk_sparse_attn_reference_mixed")
        return
    _check(lib().flk_sparse_attn_reference(ctypes.byref(desc(K, H, D, k_chain[0].k_tiles)), ctypes.byref(desc(V, H, D)),
                                           T, _ptr(q), Hq, ka, va, len(k_chain), k, float(softmax_scale), _ptr(out),
                                           _ptr(state.sel), _ptr(state.mass), _ptr(state.o_ref), _ptr(state.c_ref),
                                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _stream(stream)), "flk_sparse_attn_reference")


def sparse_attn_loop(q: torch.Tensor, k_chain: Sequence[Packed], v_chain: Sequence[Packed], T: int, H: int, k: int,
                     softmax_scale: float, state: SparseState, out: torch.Tensor, workspace: torch.Tensor,
                     stream=None) -> None:
    """A later loop over INT4 chains, or (flk_sparse_attn_loop_mixed) chains with FP4 streams."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    Hq, D = q.shape
    ka, va = _chain(k_chain), _chain(v_chain)
    mixed = _mixed_descs(k_chain, v_chain, H, D)
    if mixed is not None:
        _check(lib().flk_sparse_attn_loop_mixed(*[ctypes.byref(d) for d in mixed], T, _ptr(q), Hq, ka, va,
                                                len(k_chain), k, float(softmax_scale), _ptr(state.sel),
                                                _ptr(state.mass), _ptr(state.o_ref), _ptr(state.c_ref), _ptr(out),
                                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                _stream(stream)), "flk_sparse_attn_loop_mixed")
        return
    _check(lib().flk_sparse_attn_loop(ctypes.byref(desc(K, H, D, k_chain[0].k_tiles)), ctypes.byref(desc(V, H, D)), T,
                                      _ptr(q), Hq, ka, va, len(k_chain), k, float(softmax_scale), _ptr(state.sel),
                                      _ptr(state.mass), _ptr(state.o_ref), _ptr(state.c_ref), _ptr(out),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "flk_sparse_attn_loop")


# ----------------------------------------------------------------------------- token selection

ROW_INACTIVE, ROW_ACTIVE, ROW_DECODE = 0, 1, 2


def select_count(T: int, window: int, pcts: Sequence[int]) -> int:
    """Active tokens after the budgets pcts (percent) are applied in turn to a dense loop's
    selection windows."""
    arr = (ctypes.c_int32 * max(1, len(pcts)))(*pcts)
    n = int(lib().flk_select_count(T, window, arr, len(pcts)))
    if n < 0:
        raise ValueError(f"select_count: bad arguments T={T} window={window} pcts={list(pcts)}")
    return n


def select_workspace_bytes(T: int, window: int) -> int:
    return int(lib().flk_select_workspace_bytes(T, window))


def select_rows(h_prev: torch.Tensor, h_prev2: torch.Tensor, rows_prev: Optional[torch.Tensor], window: int,
                pct: int, eps: float, scores: Optional[torch.Tensor], rows_out: torch.Tensor,
                workspace: torch.Tensor, slot: Optional[torch.Tensor] = None,
                status: Optional[torch.Tensor] = None, stream=None) -> None:
    """Loop r's active positions (rows_out, ascending) from H[r-1] = h_prev and H[r-2] = h_prev2
    (BF16 [T, d]) and loop r-1's active positions (None = all); scores gets the change score of
    each eligible token when 0 < pct < 100; slot (optional, int32 [T]) the index of each position
    in rows_out or -1."""
    _need(h_prev, torch.bfloat16, "h_prev")
    _need(h_prev2, torch.bfloat16, "h_prev2")
    _need(rows_out, torch.int32, "rows_out")
    T, d = h_prev.shape
    if tuple(h_prev2.shape) != (T, d):
        raise ValueError("h_prev2: shape differs from h_prev")
    n_prev = T if rows_prev is None else rows_prev.numel()
    if rows_prev is not None:
        _need(rows_prev, torch.int32, "rows_prev")
    if scores is not None:
        _need(scores, torch.float32, "scores")
        if scores.numel() < n_prev:
            raise ValueError("scores: fewer entries than eligible tokens")
    if slot is not None:
        _need(slot, torch.int32, "slot")
        if slot.numel() < T:
            raise ValueError("slot: fewer than T entries")
    _check(lib().flk_select_rows(_ptr(h_prev), _ptr(h_prev2), T, d, _ptr(rows_prev), n_prev, window, pct,
                                 float(eps), _ptr(scores), _ptr(rows_out), rows_out.numel(), _ptr(slot),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(status),
                                 _stream(stream)), "flk_select_rows")


def partition_rows(cls: torch.Tensor, gather: torch.Tensor, scatter: torch.Tensor, counts: torch.Tensor,
                   status: Optional[torch.Tensor] = None, stream=None) -> None:
    """Decode rows, then active prefill rows, each in order (gather); the position of every row
    in gather or -1 (scatter); counts = [decode rows, gathered rows]."""
    _need(cls, torch.uint8, "cls")
    for t, name in ((gather, "gather"), (scatter, "scatter"), (counts, "counts")):
        _need(t, torch.int32, name)
    n = cls.numel()
    if gather.numel() < n or scatter.numel() < n or counts.numel() < 2:
        raise ValueError("partition_rows: output buffers too small")
    _check(lib().flk_partition_rows(_ptr(cls), n, _ptr(gather), _ptr(scatter), _ptr(counts), _ptr(status),
                                    _stream(stream)), "flk_partition_rows")
