"""GPU parity for token selection and the row partition (FlashLoop integration RFC, vllm-rlt
#156, sections 3.1 and 6.2), through the C ABI.

Both sides evaluate every score in binary32 with the same single roundings and the same
(pairwise) order of each sum of squares, so scores are compared bit for bit, and so are the
selected positions, the slot map and the partition.
"""
import numpy as np
import pytest
import torch

from oracle import selection as osel
from quantized_kv_cache_amd import flk, synth

from chain_runner import to_dev_bf16

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _gpu_select(h1, h2, prev, window, pct, eps, n_out, with_slot=True, spare=0):
    """One flk_select_rows call; returns host (scores or None, rows, slot or None, status, spare tail)."""
    T, d = h1.shape
    n_prev = T if prev is None else len(prev)
    hd1, hd2 = to_dev_bf16(h1), to_dev_bf16(h2)
    pd = None if prev is None else _dev_i32(prev)
    scores = torch.full((max(n_prev, 1),), float("nan"), dtype=torch.float32, device="cuda")
    out_buf = torch.full((n_out + spare,), -7, dtype=torch.int32, device="cuda")
    slot = torch.full((T,), -7, dtype=torch.int32, device="cuda") if with_slot else None
    ws = torch.empty(flk.select_workspace_bytes(T, window) // 4, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    flk.select_rows(hd1, hd2, pd, window, pct, eps, scores, out_buf[:n_out], ws, slot, status)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()[:n_prev] if 0 < pct < 100 else None
    ob = out_buf.cpu().numpy()
    return (sc, ob[:n_out], None if slot is None else slot.cpu().numpy(), int(status.item()), ob[n_out:])


def _check_loop(h1, h2, prev, window, pct, eps, tag):
    T = h1.shape[0]
    want_scores, want_rows = osel.select_rows(h1, h2, prev, window, pct, eps)
    sc, rows, slot, status, _ = _gpu_select(h1, h2, prev, window, pct, eps, n_out=len(want_rows))
    assert status == 0, f"{tag}: status {status}"
    if sc is not None:
        bad = np.flatnonzero(sc.view(np.uint32) != want_scores.view(np.uint32))
        assert len(bad) == 0, (f"{tag}: {len(bad)} of {len(sc)} scores differ; first at {bad[0]}: "
                               f"{sc[bad[0]]!r} vs {want_scores[bad[0]]!r}")
    assert np.array_equal(rows, want_rows), f"{tag}: selected positions differ"
    assert np.array_equal(slot, osel.slot_map(want_rows, T)), f"{tag}: slot map differs"
    return want_rows


def _hidden(rng, T, d, n):
    y = (rng.standard_normal((T, d)) * np.exp(rng.uniform(-1, 1, (T, 1)))).astype(np.float32)
    hs = [synth.to_bf16_bits(y)]
    for _ in range(n - 1):
        y = y + (rng.standard_normal((T, d)) * np.exp(rng.uniform(-4, 0, (T, 1)))).astype(np.float32)
        hs.append(synth.to_bf16_bits(y))
    return hs


@pytest.mark.parametrize("T,d,window,pcts", [
    (1, 8, 1, [50, 25]),
    (100, 24, 7, [50, 25]),            # ragged last window, d below one 512-channel chunk
    (1000, 520, 64, [25, 10]),         # d just over one chunk (two chunks, the second nearly empty)
    (300, 4096, 300, [33, 0]),         # one window; an all-off loop
    (513, 8200, 128, [50, 100]),       # 17 chunks (tree over 32); 100 % keeps every active token
    (64, 16384, 16, [60, 30]),         # the widest rows
    (5000, 1024, 5000, [10, 5]),       # one long window
    (4099, 256, 1, [50, 50]),          # windows of one token
])
def test_select_matches_oracle(T, d, window, pcts):
    rng = np.random.default_rng(T * 7 + d)
    hs = _hidden(rng, T, d, len(pcts) + 1)
    prev = None
    say(f"select T={T} d={d} window={window} pcts={pcts}")
    for i, p in enumerate(pcts):
        prev = _check_loop(hs[i + 1], hs[i], prev, window, p, 1e-6, f"T={T} d={d} loop {i + 3}")
        assert len(prev) == flk.select_count(T, window, pcts[:i + 1])


def test_select_ties_zero_rows_and_eps():
    """Identical rows (equal scores: lower positions win), unchanged rows (score 0) and zero
    rows (the denominator is eps)."""
    T, d = 200, 64
    rng = np.random.default_rng(1)
    h1, h2 = _hidden(rng, T, d, 2)
    h1[10:60], h2[10:60] = h1[5], h2[5]              # 51 identical tokens (5 and 10..59)
    h2[100:120] = h1[100:120]                        # no change: score 0
    h1[150:160] = 0                                  # ||H[r-1]|| = 0: divided by eps
    for window, pct in ((200, 20), (64, 50), (200, 95), (32, 3)):
        _check_loop(h1, h2, None, window, pct, 0.25, f"ties window={window} pct={pct}")


def test_select_empty_previous_set():
    T, d = 300, 32
    rng = np.random.default_rng(2)
    h1, h2 = _hidden(rng, T, d, 2)
    empty = np.zeros(0, np.int32)
    sc, rows, slot, status, _ = _gpu_select(h1, h2, empty, 64, 50, 1e-6, n_out=0)
    assert status == 0 and len(rows) == 0 and np.all(slot == -1)


def test_select_count_mismatch_sets_status_and_writes_nothing_past_n_out():
    """A previous set that is not nested under the same budgets: the windows' budgets add up to
    more than n_out; FLK_DEV_COUNT is set and the buffer past n_out is untouched."""
    T, d, W = 256, 64, 64
    rng = np.random.default_rng(3)
    h1, h2 = _hidden(rng, T, d, 2)
    prev = np.arange(T, dtype=np.int32)                 # all tokens: 50 % gives 128, not 100
    _, rows, _, status, tail = _gpu_select(h1, h2, prev, W, 50, 1e-6, n_out=100, spare=16)
    assert status & 8
    assert np.all(tail == -7)
    _, want = osel.select_rows(h1, h2, prev, W, 50, 1e-6)
    assert np.array_equal(rows, want[:100])


def test_select_long_prompt_workload():
    """T = 32768, d = 4096, windows of 2048: loop 3 keeps 50 % of a dense loop 2, loop 4 25 %."""
    T, d, W = 32768, 4096, 2048
    hs = synth.hidden_states(T, d, 3)
    say("select long prompt: loop 3")
    rows3 = _check_loop(hs[1], hs[0], None, W, 50, 1e-6, "long prompt loop 3")
    say("select long prompt: loop 4")
    rows4 = _check_loop(hs[2], hs[1], rows3, W, 25, 1e-6, "long prompt loop 4")
    assert len(rows3) == 16384 and len(rows4) == 8192


def _gpu_partition(cls):
    n = len(cls)
    c = torch.from_numpy(np.asarray(cls, np.uint8)).cuda() if n else torch.zeros(0, dtype=torch.uint8, device="cuda")
    gather = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    scatter = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    flk.partition_rows(c, gather[:n] if n else gather, scatter[:n] if n else scatter, counts, status)
    torch.cuda.synchronize()
    return gather.cpu().numpy()[:n], scatter.cpu().numpy()[:n], tuple(counts.cpu().numpy()), int(status.item())


@pytest.mark.parametrize("n,seed", [(6, -1), (0, 0), (1, 1), (4095, 2), (4097, 3), (100000, 4)])
def test_partition_matches_oracle(n, seed):
    if seed < 0:   # the RFC's example [P0, D0, P1, P2, D1, P3] with P1, P3 active
        cls = [0, 2, 1, 0, 2, 1]
    else:
        cls = list(np.random.default_rng(seed).integers(0, 3, n))
    gather, scatter, counts, status = _gpu_partition(cls)
    wg, ws, wc = osel.partition_rows(cls)
    assert status == 0
    assert counts == wc
    assert np.array_equal(gather[:wc[1]], wg) and np.all(gather[wc[1]:] == -1)
    assert np.array_equal(scatter, ws)


def test_partition_flags_unknown_class():
    gather, scatter, counts, status = _gpu_partition([2, 7, 1, 0])
    assert status & 16
    assert counts == (1, 2) and list(gather) == [0, 2, -1, -1] and list(scatter) == [0, -1, 1, -1]
