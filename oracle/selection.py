"""Oracle of token selection for sparse prefill: change scores, nested window top-k, compact maps
and the stable partition of a submission's rows.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and its binding)
never imports this module, and this module never imports the product.

What it follows: the FlashLoop integration RFC (vllm-rlt issue #156), section 3.1
("Token-sparse prefill": the score, the top-k over the previous active set, FP32 scores,
budgets against the window length, nested sets, ties by absolute position), section 3.1's
serving paragraph on fixed selection windows, and section 6.2 (gather indices built by a stable
partition, decode rows first, with a scatter map).

Readings taken where the RFC leaves a step open:
- H[r-1] and H[r-2] are BF16 [T, d] tensors indexed by token position;
- norm(.) is the Euclidean norm; every step is one binary32 operation rounded to nearest-even:
  each difference, each square, each addition, the square root and the quotient;
- a sum of squares is taken in pairwise order, the complete binary tree over the channel index,
  with the channel count padded by zeros to a power of two (a zero leaves every partial sum
  unchanged).  A fixed order makes the score, and so the selection, a function of the inputs
  alone, which the RFC's rule that packing and batch order must not change the result needs;
- epsilon is the caller's (a positive binary32);
- window w covers positions [w*W, min((w+1)*W, T)); its budget is ceil(pct * len / 100) in
  integers, never more than its tokens still eligible;
- top-k by score, equal scores to the lower position; the active set is listed ascending.
Scores are assumed finite (finite inputs whose squares do not overflow).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

ROW_INACTIVE, ROW_ACTIVE, ROW_DECODE = 0, 1, 2


def f32_of_bf16(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) to binary32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def pairwise_sum_f32(x: np.ndarray) -> np.ndarray:
    """Binary32 sum over the last axis in pairwise order: element pairs (0,1), (2,3), ... are
    added first, then pairs of those sums, and so on (zeros pad the length to a power of two)."""
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    p = 1
    while p < n:
        p *= 2
    if p != n:
        x = np.concatenate([x, np.zeros(x.shape[:-1] + (p - n,), np.float32)], axis=-1)
    while x.shape[-1] > 1:
        x = x[..., 0::2] + x[..., 1::2]            # binary32 + binary32 -> binary32, rounded once
    return x[..., 0]


def change_scores(h1: np.ndarray, h2: np.ndarray, eps: float) -> np.ndarray:
    """score = norm(h1 - h2) / max(norm(h1), eps) per row, binary32 (RFC section 3.1).
    h1 = H[r-1] rows, h2 = H[r-2] rows, both BF16 bit patterns [n, d]."""
    a = f32_of_bf16(h1)
    b = f32_of_bf16(h2)
    diff = a - b
    num = np.sqrt(pairwise_sum_f32(diff * diff))
    den = np.sqrt(pairwise_sum_f32(a * a))
    return num / np.maximum(den, np.float32(eps))


def window_budget(length: int, pct: int) -> int:
    """ceil(pct * length / 100): the budget refers to the window's own length (RFC section 3.1)."""
    return (pct * length + 99) // 100


def top_k_positions(scores: np.ndarray, positions: np.ndarray, k: int) -> np.ndarray:
    """The k positions of largest score, equal scores to the lower position; ascending."""
    order = sorted(range(len(scores)), key=lambda i: (-float(scores[i]), int(positions[i])))
    return np.sort(np.asarray([positions[i] for i in order[:k]], np.int32))


def select_rows(h_prev: np.ndarray, h_prev2: np.ndarray, rows_prev: Optional[np.ndarray], window: int,
                pct: int, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """Loop r's active positions from H[r-1] = h_prev and H[r-2] = h_prev2 (BF16 [T, d]) and the
    positions active at loop r-1 (None = all T).  Returns (scores of the eligible rows in their
    order, the selected positions ascending)."""
    T = h_prev.shape[0]
    elig = np.arange(T, dtype=np.int32) if rows_prev is None else np.asarray(rows_prev, np.int32)
    scores = change_scores(h_prev[elig], h_prev2[elig], eps)
    chosen: List[np.ndarray] = []
    for w0 in range(0, T, window):
        length = min(window, T - w0)
        inside = (elig >= w0) & (elig < w0 + length)
        k = min(window_budget(length, pct), int(inside.sum()))
        chosen.append(top_k_positions(scores[inside], elig[inside], k))
    rows = np.concatenate(chosen).astype(np.int32) if chosen else np.zeros(0, np.int32)
    return scores, rows


def slot_map(rows: np.ndarray, T: int) -> np.ndarray:
    """Position -> index in rows, or -1 for a position not in rows."""
    slot = np.full(T, -1, np.int32)
    for j, p in enumerate(rows):
        slot[p] = j
    return slot


def select_count(T: int, window: int, pcts: Sequence[int]) -> int:
    """Active tokens after the budgets pcts are applied in turn to a dense loop's windows."""
    total = 0
    for w0 in range(0, T, window):
        length = min(window, T - w0)
        n = length
        for p in pcts:
            n = min(window_budget(length, p), n)
        total += n
    return total


def partition_rows(cls: Sequence[int]) -> Tuple[np.ndarray, np.ndarray, Tuple[int, int]]:
    """Stable partition of execution rows (RFC section 6.2): decode rows in their order, then
    active prefill rows in their order.  Returns (gather, scatter, (split offset, total))."""
    decode = [i for i, c in enumerate(cls) if c == ROW_DECODE]
    active = [i for i, c in enumerate(cls) if c == ROW_ACTIVE]
    gather = np.asarray(decode + active, np.int32)
    scatter = np.full(len(cls), -1, np.int32)
    for j, i in enumerate(gather):
        scatter[i] = j
    return gather, scatter, (len(decode), len(gather))
