"""Shared helpers for the GPU tests: run one tensor's loop chain through the HIP library and
through the oracle on the same seeded inputs, and compare what each wrote."""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

from oracle import oracle as orc
from quantized_kv_cache_amd import flk


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev_rows(r: Optional[np.ndarray]) -> Optional[torch.Tensor]:
    return None if r is None else torch.from_numpy(np.ascontiguousarray(r, dtype=np.int32)).cuda()


class GpuChain:
    """Encodes xs (xs[0] = X[1] over T rows, xs[r] = X[r+1] at rows[r]) on the GPU and keeps
    a copy of the reconstruction after every loop."""

    def __init__(self, kind: int, xs: Sequence[np.ndarray], rows: Sequence[Optional[np.ndarray]],
                 status: Optional[torch.Tensor] = None, k_tiles: bool = False, fmt: str = "int4",
                 base_fmt: Optional[str] = None):
        """fmt: the residual loops' stream format; base_fmt: the base loop's (default fmt)."""
        T, H, D = xs[0].shape
        self.kind, self.T, self.H, self.D = kind, T, H, D
        self.recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
        self.packed: List[flk.Packed] = []
        self.recons: List[np.ndarray] = []
        for loop, (x, r) in enumerate(zip(xs, rows)):
            xd = to_dev_bf16(x)
            rd = to_dev_rows(r)
            f = (base_fmt or fmt) if loop == 0 else fmt
            p = flk.Packed.empty(kind, H, D, x.shape[0], rd, T=T, k_tiles=k_tiles, fmt=f)
            if loop == 0:
                flk.encode_base(kind, xd, p, self.recon, status)
            else:
                flk.encode_residual(kind, xd, rd, self.recon, p, status)
            self.packed.append(p)
            self.recons.append(to_host_u16(self.recon))
        torch.cuda.synchronize()

    def reconstruct(self, depth: Optional[int] = None) -> np.ndarray:
        depth = len(self.packed) if depth is None else depth
        out = torch.empty((self.T, self.H, self.D), dtype=torch.bfloat16, device="cuda")
        flk.reconstruct(self.kind, self.packed[:depth], out)
        torch.cuda.synchronize()
        return to_host_u16(out)

    def host_stream(self, loop: int):
        p = self.packed[loop]
        return p.codes.cpu().numpy(), p.params.cpu().numpy().view(np.uint32)


class OracleChain:
    def __init__(self, kind: int, xs: Sequence[np.ndarray], rows: Sequence[Optional[np.ndarray]],
                 k_tiles: bool = False):
        T, H, D = xs[0].shape
        self.kind, self.T, self.H, self.D, self.k_tiles = kind, T, H, D, k_tiles
        base, recon = orc.encode_base(kind, xs[0], k_tiles=k_tiles)
        self.streams = [base]
        self.recons = [recon.copy()]
        for x, r in zip(xs[1:], rows[1:]):
            self.streams.append(orc.encode_residual(kind, x, r, recon, k_tiles=k_tiles))
            self.recons.append(recon.copy())

    def reconstruct(self, depth: Optional[int] = None) -> np.ndarray:
        depth = len(self.streams) if depth is None else depth
        return orc.reconstruct(self.kind, self.streams[:depth], self.T, self.H, self.D, k_tiles=self.k_tiles)


def assert_same(got: np.ndarray, want: np.ndarray, what: str):
    if got.shape != want.shape:
        raise AssertionError(f"{what}: shape {got.shape} != {want.shape}")
    bad = np.argwhere(got != want)
    if len(bad):
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {got.size} differ; first at {i}: "
                             f"got {got[i]:#x} want {want[i]:#x}")


def compare_chains(g: GpuChain, o: OracleChain, head_slice: Optional[slice] = None, tag: str = ""):
    """Bit-exact comparison of codes, params and per-loop reconstructions (optionally on a
    head slice of the GPU result against an oracle run on that slice)."""
    hs = head_slice if head_slice is not None else slice(None)
    for loop in range(len(o.streams)):
        assert_same(g.recons[loop][:, hs], o.recons[loop], f"{tag} recon loop {loop + 1}")
        if o.streams[loop].n_rows == 0:
            continue                         # an empty loop writes nothing
        codes, params = g.host_stream(loop)
        assert_same(codes[:, hs], o.streams[loop].codes, f"{tag} codes loop {loop + 1}")
        assert_same(params[:, hs], o.streams[loop].params, f"{tag} params loop {loop + 1}")
        r = o.streams[loop].rows
        if r is not None and len(r):
            got = g.packed[loop].tile_start.cpu().numpy()
            assert np.array_equal(got, orc.tile_index(r, g.T)), f"{tag} tile index loop {loop + 1}"

