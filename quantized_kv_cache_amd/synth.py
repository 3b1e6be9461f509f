"""Seeded synthetic K/V loop trajectories for the packed-KV codec workloads.

This module only draws inputs: it holds none of the codec's arithmetic, and both the
HIP path's tests/benchmark and the CPU oracle consume what it returns.

Recipe (the same for every workload):
  * one numpy Generator per purpose, seeded with
    SeedSequence([0, workload_id, request, layer, tensor(K=0, V=1), loop, purpose]);
  * a binary32 trajectory Y[1] ~ dist, Y[r] = Y[r-1] + N(0, sigma_delta) for every token,
    and the BF16 inputs X[r] = bf16(Y[r]) (round-to-nearest-even, via torch's conversion);
  * loops 1 and 2 are dense; a later loop with a budget below 100% keeps the top
    ceil(p * T / 100) positions of fresh uniform binary32 scores drawn over the previous
    loop's active set, higher score first and equal scores broken by the lower position,
    so the active sets are nested; the kept positions are stored in ascending order.
    (The FlashLoop RFC, section 3.1, selects by FP32 scores with nested sets and
    position tie-breaks; random scores stand in for the model's hidden-state scores.)

Workloads (sizes fixed by the benchmark definition):
  1 tiny           K,V [256, 2, 64], 4 dense loops, Y1 ~ N(0,1), sigma 0.1
  2 partial_sparse K,V [1000, 8, 96], loops 3/4 keep 500/250 rows, N(0,1), sigma 0.1
  3 long_prompt    K,V [32768, 8, 128], budgets 100/100/50/25%; K ~ Student-t(3) times a
                   per-(head, channel) multiplier exp(U(ln 0.1, ln 10)); V ~ N(0,1); sigma 0.05
  4 batched        64 requests x 24 layers, lengths U{512..8192}, H 16, D 128, budgets as 3
  5 decode_attn    T 131072, Hkv 8, Hq 32, D 128, budgets as 3; q ~ N(0,1) BF16

Hidden states for token selection (hidden_states): H[1] = a per-token magnitude exp(U(ln 0.5,
ln 2)) times N(0,1) per element; H[r] = H[r-1] + s[t, r] * N(0,1) per element, with a change
size s[t, r] = exp(U(ln 0.01, ln 1)) per (token, loop), so that change scores spread over two
decades; every H[r] is rounded to BF16.  The long-prompt selection workload uses T = 32768 and
a hidden width d = 4096 (32 query heads x 128, the decode workload's attention width),
windows of 2048 tokens and budgets 50 % then 25 %.

Inputs too large to draw on the host (device_trajectory, the largest tensor the library
accepts): the same trajectory recipe with Y[1] ~ N(0,1), drawn on the device by torch's
generator in row chunks, chunk c of every loop from one generator seeded seed * 2^20 + c.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

K_TENSOR, V_TENSOR = 0, 1
P_VALUES, P_DELTA, P_SCORES, P_MULT, P_QUERY, P_LENGTHS, P_HIDDEN, P_HSTEP = range(8)


def rng(workload: int, request: int, layer: int, tensor: int, loop: int, purpose: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, workload, request, layer, tensor, loop, purpose]))


def to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """Round binary32 to BF16 (nearest-even) and return the 16-bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def select_nested(scores: np.ndarray, prev: np.ndarray, k: int) -> np.ndarray:
    """Top-k of `scores` over the candidate positions `prev`, ties to the lower position;
    returned in ascending position order."""
    cand = np.asarray(prev, dtype=np.int64)
    s = scores[cand]
    order = np.lexsort((cand, -s.astype(np.float64)))
    return np.sort(cand[order[:k]]).astype(np.int32)


def budget_rows(pct: int, length: int) -> int:
    return int(math.ceil(pct * length / 100))


@dataclass
class Workload:
    name: str
    wid: int
    T: int
    H: int
    D: int
    budgets: Sequence[int]             # per loop, percent of T (loop 1 must be 100)
    sigma: float
    k_dist: str = "normal"             # "normal" or "student_t3_mult"
    v_dist: str = "normal"
    Hq: int = 0                        # decode-attention workload only

    @property
    def n_loops(self) -> int:
        return len(self.budgets)


WORKLOADS = {
    1: Workload("tiny", 1, 256, 2, 64, (100, 100, 100, 100), 0.1),
    2: Workload("partial_sparse", 2, 1000, 8, 96, (100, 100, 50, 25), 0.1),
    3: Workload("long_prompt", 3, 32768, 8, 128, (100, 100, 50, 25), 0.05, "student_t3_mult"),
    4: Workload("batched", 4, 0, 16, 128, (100, 100, 50, 25), 0.05, "student_t3_mult"),
    5: Workload("decode_attn", 5, 131072, 8, 128, (100, 100, 50, 25), 0.05, "student_t3_mult", Hq=32),
}


@dataclass
class Chain:
    """Inputs for one tensor's loop chain.  xs[0] = X[1] over all T rows; xs[r] = X[r+1] at
    rows[r] (all rows when rows[r] is None).  full[r] is X[r+1] over all T rows."""
    tensor: int
    T: int
    H: int
    D: int
    xs: List[np.ndarray] = field(default_factory=list)
    rows: List[Optional[np.ndarray]] = field(default_factory=list)


def active_sets(w: Workload, T: int, request: int = 0, layer: int = 0, tensor: int = 0):
    """Nested active sets per loop (None = dense)."""
    out: List[Optional[np.ndarray]] = []
    prev = np.arange(T, dtype=np.int32)
    for loop, pct in enumerate(w.budgets):
        if pct >= 100 and len(prev) == T:
            out.append(None)
            continue
        k = budget_rows(pct, T)
        scores = rng(w.wid, request, layer, tensor, loop, P_SCORES).random(T, dtype=np.float32)
        prev = select_nested(scores, prev, k)
        out.append(prev)
    return out


def k_multipliers(w: Workload, H: int, D: int, layer: int = 0) -> np.ndarray:
    g = rng(w.wid, 0, layer, K_TENSOR, 0, P_MULT)
    return np.exp(g.uniform(math.log(0.1), math.log(10.0), size=(H, D))).astype(np.float32)


def make_chain(w: Workload, tensor: int, T: Optional[int] = None, H: Optional[int] = None,
               request: int = 0, layer: int = 0, sets=None, head_slice: Optional[slice] = None) -> Chain:
    """Draw one tensor's 4-loop trajectory.  `sets` may pass precomputed active sets so K and
    V of one unit share them (token sparsity selects tokens, not tensors).  `head_slice`
    returns only some heads (the draw itself is over all heads, so values match)."""
    T = w.T if T is None else T
    H = w.H if H is None else H
    D = w.D
    if sets is None:
        sets = active_sets(w, T, request, layer, 0)
    dist = w.k_dist if tensor == K_TENSOR else w.v_dist
    g = rng(w.wid, request, layer, tensor, 0, P_VALUES)
    if dist == "normal":
        y = g.standard_normal((T, H, D), dtype=np.float32)
    else:
        y = g.standard_t(3, size=(T, H, D)).astype(np.float32)
        y *= k_multipliers(w, H, D, layer)[None]
    c = Chain(tensor, T, H, D)
    hs = head_slice if head_slice is not None else slice(None)
    for loop in range(w.n_loops):
        if loop > 0:
            d = rng(w.wid, request, layer, tensor, loop, P_DELTA).standard_normal((T, H, D), dtype=np.float32)
            d *= np.float32(w.sigma)
            y += d
        xb = to_bf16_bits(y[:, hs, :])
        rows = sets[loop]
        c.xs.append(xb if rows is None else np.ascontiguousarray(xb[rows]))
        c.rows.append(rows)
    return c


def make_query(w: Workload) -> np.ndarray:
    g = rng(w.wid, 0, 0, 0, 0, P_QUERY)
    return to_bf16_bits(g.standard_normal((w.Hq, w.D), dtype=np.float32))


def batched_lengths(n_requests: int = 64, lo: int = 512, hi: int = 8192) -> np.ndarray:
    g = rng(4, 0, 0, 0, 0, P_LENGTHS)
    return g.integers(lo, hi + 1, size=n_requests).astype(np.int64)


def hidden_states(T: int, d: int, n_states: int, workload: int = 3, request: int = 0, layer: int = 0) -> List[np.ndarray]:
    """BF16 bit patterns [T, d] of H[1] .. H[n_states] (recipe in the module docstring)."""
    g = rng(workload, request, layer, 0, 0, P_HIDDEN)
    mag = np.exp(g.uniform(math.log(0.5), math.log(2.0), (T, 1))).astype(np.float32)
    y = g.standard_normal((T, d), dtype=np.float32) * mag
    out = [to_bf16_bits(y)]
    for r in range(1, n_states):
        gs = rng(workload, request, layer, 0, r, P_HSTEP)
        size = np.exp(gs.uniform(math.log(0.01), 0.0, (T, 1))).astype(np.float32)
        y = y + gs.standard_normal((T, d), dtype=np.float32) * size
        out.append(to_bf16_bits(y))
    return out


def device_trajectory(T: int, H: int, D: int, n_loops: int, seed: int, sigma: float = 0.1,
                      chunk: int = 1 << 16, device: str = "cuda") -> List[torch.Tensor]:
    """Dense BF16 inputs X[1..n_loops], each [T, H, D], drawn on the device: Y[1] ~ N(0,1),
    Y[r] = Y[r-1] + N(0, sigma^2) per element, X[r] = bf16(Y[r]) (round-to-nearest-even)."""
    xs = [torch.empty((T, H, D), dtype=torch.bfloat16, device=device) for _ in range(n_loops)]
    g = torch.Generator(device=device)
    for c, r0 in enumerate(range(0, T, chunk)):
        r1 = min(T, r0 + chunk)
        g.manual_seed(seed * (1 << 20) + c)
        y = torch.randn((r1 - r0, H, D), generator=g, device=device)
        xs[0][r0:r1] = y.to(torch.bfloat16)
        for r in range(1, n_loops):
            y += sigma * torch.randn((r1 - r0, H, D), generator=g, device=device)
            xs[r][r0:r1] = y.to(torch.bfloat16)
        del y
    return xs
