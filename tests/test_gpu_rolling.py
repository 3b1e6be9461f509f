"""GPU parity for page-local K groups and the rolling BF16 tail.

Tile (page-local) K groups follow the PR #166 review, item 3 "Group ownership vs 16-token
pages"; the rolling tail follows the RFC (vllm-rlt #156), section 3.3, last paragraph (at
least 64 BF16 tail tokens; whole 64-token groups are flushed).  Codes, params, tile indexes
and reconstructions must be bit-identical to the oracle's tile-grouped encoding; appended
streams must equal one-shot streams byte for byte; attention over a packed prefix plus a BF16
tail must agree with exact attention within 2e-2 (normwise per query head).
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from quantized_kv_cache_amd import flk, synth

from chain_runner import GpuChain, OracleChain, assert_same, compare_chains, to_dev_bf16, to_dev_rows, to_host_u16

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _rel_err(got, ref):
    return np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)


# --------------------------------------------------------------------------- one-shot parity

@pytest.mark.parametrize("wid", [1, 2])
def test_tile_groups_small_workloads_full_parity(wid):
    w = synth.WORKLOADS[wid]
    sets = synth.active_sets(w, w.T)
    for kind, tensor in ((flk.K, synth.K_TENSOR), (flk.V, synth.V_TENSOR)):
        c = synth.make_chain(w, tensor, sets=sets)
        say(f"tile groups {w.name} kind {kind}")
        g = GpuChain(kind, c.xs, c.rows, k_tiles=True)
        o = OracleChain(kind, c.xs, c.rows, k_tiles=True)
        compare_chains(g, o, tag=f"tiles {w.name}/{kind}")
        for depth in range(1, w.n_loops + 1):
            assert_same(g.reconstruct(depth), o.recons[depth - 1], f"reconstruct depth {depth}")


def test_tile_groups_long_prompt_sampled_heads():
    w = synth.WORKLOADS[3]
    sets = synth.active_sets(w, w.T)
    c = synth.make_chain(w, synth.K_TENSOR, sets=sets)
    say("tile groups long_prompt K: GPU chain")
    g = GpuChain(flk.K, c.xs, c.rows, k_tiles=True)
    assert_same(g.reconstruct(), g.recons[-1], "reconstruct vs in-place")
    for h in (0, 5):
        say(f"  oracle head {h}")
        o = OracleChain(flk.K, [x[:, h:h + 1] for x in c.xs], c.rows, k_tiles=True)
        compare_chains(g, o, head_slice=slice(h, h + 1), tag=f"tiles long_prompt h{h}")
    del g
    torch.cuda.empty_cache()


def _random_chain(rng, T, H, D, sizes, sigma=0.1):
    y = rng.standard_normal((T, H, D)).astype(np.float32)
    xs, rows, prev = [], [], np.arange(T, dtype=np.int32)
    for r, n in enumerate(sizes):
        if r:
            y = y + (sigma * rng.standard_normal((T, H, D))).astype(np.float32)
        xb = synth.to_bf16_bits(y)
        if n is None:
            xs.append(xb)
            rows.append(None)
        else:
            prev = np.sort(rng.choice(prev, size=n, replace=False)).astype(np.int32)
            xs.append(np.ascontiguousarray(xb[prev]))
            rows.append(prev)
    return xs, rows


def _values_for_rows(rng, T, H, D, rows, sigma=0.1):
    """Fresh values for an existing loop structure (so K and V share their active rows)."""
    y = rng.standard_normal((T, H, D)).astype(np.float32)
    xs = []
    for r, sel in enumerate(rows):
        if r:
            y = y + (sigma * rng.standard_normal((T, H, D))).astype(np.float32)
        xb = synth.to_bf16_bits(y)
        xs.append(xb if sel is None else np.ascontiguousarray(xb[sel]))
    return xs


def _clustered_rows(rng, T, n):
    """n positions bunched into a few tiles, so many tiles are empty and some are full."""
    tiles = (T + 63) // 64
    pick = rng.choice(tiles, size=max(1, tiles // 3), replace=False)
    cand = np.concatenate([np.arange(64 * t, min(T, 64 * t + 64)) for t in pick])
    n = min(n, cand.size)
    return np.sort(rng.choice(cand, size=n, replace=False)).astype(np.int32)


@pytest.mark.parametrize("T,H,D,sizes", [
    (1, 1, 8, [None, 1]),
    (65, 3, 24, [None, None, 33, 1]),
    (127, 2, 200, [None, 64, 63]),
    (300, 5, 40, [None, 17, 0]),
    (1000, 8, 96, [None, None, 500, 250]),
    (4097, 8, 128, [None, None, 2048, 1]),
])
def test_tile_groups_edge_shapes(T, H, D, sizes):
    rng = np.random.default_rng(T * 7 + H * 3 + D)
    xs, rows = _random_chain(rng, T, H, D, sizes)
    say(f"tile groups edge T={T} H={H} D={D} sizes={sizes}")
    g = GpuChain(flk.K, xs, rows, k_tiles=True)
    o = OracleChain(flk.K, xs, rows, k_tiles=True)
    compare_chains(g, o, tag=f"tiles edge {T},{H},{D}")
    assert_same(g.reconstruct(), o.reconstruct(), "reconstruct")


def test_tile_groups_empty_and_full_tiles():
    """Rows clustered in a third of the tiles: empty tiles get zero params, full tiles hold
    64 rows, and a later loop draws from the clustered set."""
    rng = np.random.default_rng(3)
    T, H, D = 2000, 8, 128
    y = rng.standard_normal((T, H, D)).astype(np.float32)
    r3 = _clustered_rows(rng, T, 500)
    r4 = np.sort(rng.choice(r3, size=100, replace=False)).astype(np.int32)
    xs = [synth.to_bf16_bits(y), synth.to_bf16_bits(y + 0.1)]
    y3 = synth.to_bf16_bits(y + 0.2)
    y4 = synth.to_bf16_bits(y + 0.3)
    xs += [np.ascontiguousarray(y3[r3]), np.ascontiguousarray(y4[r4])]
    rows = [None, None, r3, r4]
    g = GpuChain(flk.K, xs, rows, k_tiles=True)
    o = OracleChain(flk.K, xs, rows, k_tiles=True)
    compare_chains(g, o, tag="clustered")
    assert_same(g.reconstruct(), o.reconstruct(), "reconstruct")


@pytest.mark.parametrize("T,H,Hq,sizes", [
    (1025, 4, 16, [None, None, 700, 3]),
    (4096, 8, 128, [None, 4096, 2048, 1]),
])
def test_tile_groups_attention(T, H, Hq, sizes):
    D = 128
    rng = np.random.default_rng(T + 11 * H)
    xk, rows = _random_chain(rng, T, H, D, sizes)
    xv = _values_for_rows(rng, T, H, D, rows)
    g = {flk.K: GpuChain(flk.K, xk, rows, k_tiles=True), flk.V: GpuChain(flk.V, xv, rows)}
    o = {flk.K: OracleChain(flk.K, xk, rows, k_tiles=True), flk.V: OracleChain(flk.V, xv, rows)}
    q = synth.to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32))
    ws = torch.empty(flk.attn_workspace_bytes(H, D, T, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    say(f"tile-grouped attention T={T} H={H} Hq={Hq}")
    flk.decode_attn_packed(to_dev_bf16(q), g[flk.K].packed, g[flk.V].packed, T, H, scale, out, ws)
    torch.cuda.synchronize()
    ref = orc.decode_attn(q, o[flk.K].recons[-1], o[flk.V].recons[-1], scale)
    rel = _rel_err(out.float().cpu().numpy(), ref)
    assert np.all(rel <= 2e-2), rel


def test_tile_groups_batched_calls():
    """Tile-grouped K units in the batched calls write exactly what the single calls write, for
    compact loops short enough to search their tiles in-kernel and long ones that take the
    tile index pass."""
    rng = np.random.default_rng(44)
    H, D = 8, 128
    units = []
    for i in range(6):
        T = int(rng.integers(64, 3000))
        n3 = int(rng.integers(0, T + 1))
        if i < 2:                                    # compact loops long enough for the tile index pass
            T, n3 = 9000 + 500 * i, 6000
        xs, rows = _random_chain(rng, T, H, D, [None, None, n3, n3 // 3])
        units.append((flk.K if i % 2 == 0 else flk.V, xs, rows))
    dev = []
    for kind, xs, rows in units:
        T = xs[0].shape[0]
        recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
        xd = [to_dev_bf16(x) for x in xs]
        rd = [to_dev_rows(r) for r in rows]
        packs = [flk.Packed.empty(kind, H, D, x.shape[0], r, T=T, k_tiles=True) for x, r in zip(xs, rd)]
        dev.append((kind, xd, rd, recon, packs))
    flk.encode_base_batch([(k, xd[0], recon, packs[0]) for k, xd, rd, recon, packs in dev], H, D)
    for loop in range(1, 4):
        flk.encode_residual_batch([(k, xd[loop], rd[loop], recon, packs[loop]) for k, xd, rd, recon, packs in dev],
                                  H, D)
    outs = [torch.empty_like(recon) for _, _, _, recon, _ in dev]
    flk.reconstruct_batch([(k, packs, out) for (k, _, _, _, packs), out in zip(dev, outs)], H, D)
    torch.cuda.synchronize()
    for ui, ((kind, xs, rows), (_, _, _, recon, packs), out) in enumerate(zip(units, dev, outs)):
        gs = GpuChain(kind, xs, rows, k_tiles=True)
        for loop, p in enumerate(packs):
            if p.n_rows == 0:
                continue                     # an empty loop writes nothing
            assert_same(p.codes.cpu().numpy(), gs.packed[loop].codes.cpu().numpy(), f"u{ui} codes {loop}")
            assert_same(p.params.cpu().numpy(), gs.packed[loop].params.cpu().numpy(), f"u{ui} params {loop}")
        assert_same(to_host_u16(recon), gs.recons[-1], f"u{ui} recon")
        assert_same(to_host_u16(out), gs.recons[-1], f"u{ui} reconstruct")


# --------------------------------------------------------------------------- appends

class RollingStreams:
    """Full-capacity device streams of one tensor (4 loops) filled window by window with the
    append calls, the way a rolling cache flushes its tail."""

    def __init__(self, kind, H, D, cap_T, cap_rows, dense_loops):
        self.kind, self.H, self.D = kind, H, D
        self.dense = dense_loops
        self.packs = []
        self.n = [0] * len(cap_rows)
        for l, cap in enumerate(cap_rows):
            compact = not dense_loops[l]
            rows = torch.zeros(max(cap, 1), dtype=torch.int32, device="cuda") if compact else None
            p = flk.Packed.empty(kind, H, D, max(cap, 1), rows, T=cap_T, k_tiles=True, compact=compact)
            self.packs.append(p)

    def append(self, xs_w, rows_w, p0, n_pos):
        """xs_w[l]: X at the window's active rows of loop l; rows_w[l]: their absolute
        positions (None for dense loops).  Returns the window's final reconstruction."""
        recon = torch.empty((n_pos, self.H, self.D), dtype=torch.bfloat16, device="cuda")
        for l, (x, r) in enumerate(zip(xs_w, rows_w)):
            p = self.packs[l]
            n_w = x.shape[0] if x is not None else 0
            if l == 0:
                flk.append_base(self.kind, to_dev_bf16(x), p0, p, recon)
            elif self.dense[l]:
                flk.append_residual(self.kind, to_dev_bf16(x), None, n_pos, p0, n_pos, p0, recon, p)
            else:
                rd = None
                if n_w:
                    p.rows[self.n[l]:self.n[l] + n_w].copy_(torch.from_numpy(r))
                    rd = p.rows[self.n[l]:self.n[l] + n_w]
                flk.append_residual(self.kind, to_dev_bf16(x) if n_w else None, rd, n_w, p0, n_pos, self.n[l],
                                    recon, p)
            self.n[l] += n_w if not self.dense[l] else n_pos
        return recon

    def chain(self, T):
        """Views of the streams as they stand after positions [0, T) were appended."""
        out = []
        tiles = (T + 63) // 64
        for l, p in enumerate(self.packs):
            n = self.n[l]
            params = p.params[:tiles] if self.kind == flk.K else p.params[:n]
            if self.dense[l]:
                out.append(flk.Packed(n, None, p.codes[:n], params, None, p.k_tiles))
            else:
                out.append(flk.Packed(n, p.rows[:n], p.codes[:n], params, p.tile_start[:tiles + 1], p.k_tiles))
        return out


def _window_inputs(X, rows, lo, hi):
    """Per loop: X at the active rows inside [lo, hi) and those rows (None for dense)."""
    xs_w, rows_w = [], []
    for l, r in enumerate(rows):
        if r is None:
            xs_w.append(np.ascontiguousarray(X[l][lo:hi]))
            rows_w.append(None)
        else:
            sel = r[(r >= lo) & (r < hi)]
            xs_w.append(np.ascontiguousarray(X[l][sel]) if sel.size else None)
            rows_w.append(sel.astype(np.int32))
    return xs_w, rows_w


def _prefix_inputs(X, rows, P):
    xs, rp = [], []
    for l, r in enumerate(rows):
        if r is None:
            xs.append(np.ascontiguousarray(X[l][:P]))
            rp.append(None)
        else:
            sel = r[r < P].astype(np.int32)
            xs.append(np.ascontiguousarray(X[l][sel]))
            rp.append(sel)
    return xs, rp


def _decode_depths(rng, n_tok):
    """Per-token exit depth: every token runs loops 1-2; half continue to loop 3, a quarter
    to loop 4.  Returns the depths and the nested active rows of each loop."""
    u = rng.random(n_tok)
    depth = np.where(u < 0.25, 4, np.where(u < 0.5, 3, 2))
    rows = [None, None, np.nonzero(depth >= 3)[0].astype(np.int32), np.nonzero(depth >= 4)[0].astype(np.int32)]
    return depth, rows


def _decode_values(rng, depth, H, D, scale):
    """Four loops of values at every position, and each token's last-exited version."""
    n_tok = depth.size
    y = (rng.standard_normal((n_tok, H, D)) * scale).astype(np.float32)
    X = [synth.to_bf16_bits(y)]
    for _ in range(3):
        y = y + (0.05 * scale * rng.standard_normal((n_tok, H, D))).astype(np.float32)
        X.append(synth.to_bf16_bits(y))
    final = np.stack([X[d - 1][t] for t, d in enumerate(depth)])
    return X, final


def _compare_prefix(rs: RollingStreams, X, rows, P, tag):
    """The appended streams against the oracle's one-shot tile-grouped encoding of [0, P)."""
    xs, rp = _prefix_inputs(X, rows, P)
    o = OracleChain(rs.kind, xs, rp, k_tiles=True)
    ch = rs.chain(P)
    for l, (p, st) in enumerate(zip(ch, o.streams)):
        assert p.n_rows == st.n_rows, f"{tag} loop {l} rows {p.n_rows} vs {st.n_rows}"
        assert_same(p.codes.cpu().numpy(), st.codes, f"{tag} codes loop {l + 1}")
        assert_same(p.params.cpu().numpy().view(np.uint32), st.params, f"{tag} params loop {l + 1}")
        if st.rows is not None:
            assert np.array_equal(p.rows.cpu().numpy(), st.rows), f"{tag} rows loop {l + 1}"
            assert np.array_equal(p.tile_start.cpu().numpy(), orc.tile_index(st.rows, P)), f"{tag} tile index {l + 1}"
    out = torch.empty((P, rs.H, rs.D), dtype=torch.bfloat16, device="cuda")
    flk.reconstruct(rs.kind, ch, out)
    torch.cuda.synchronize()
    assert_same(to_host_u16(out), o.recons[-1], f"{tag} reconstruct")
    return o


@pytest.mark.parametrize("H,D", [(8, 128), (3, 64)])
def test_append_windows_equal_one_shot(H, D):
    """Windows of 64, 192, 64 (one without loop-3/4 rows) and 320 positions appended one after
    another give the one-shot streams of the whole prefix, for K (tile groups) and V."""
    rng = np.random.default_rng(H * 100 + D)
    bounds = [0, 64, 256, 320, 640]
    n_tok = bounds[-1]
    for kind in (flk.K, flk.V):
        _, rows = _decode_depths(rng, n_tok)
        X = _decode_values(rng, np.full(n_tok, 4), H, D, 2.0 if kind == flk.K else 1.0)[0]
        # empty the window [256, 320) of loops 3 and 4
        rows[2] = rows[2][(rows[2] < 256) | (rows[2] >= 320)]
        rows[3] = np.intersect1d(rows[3], rows[2]).astype(np.int32)
        cap = [n_tok, n_tok, rows[2].size, rows[3].size]
        rs = RollingStreams(kind, H, D, n_tok, cap, [True, True, False, False])
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            say(f"append kind {kind} H={H} D={D} window [{lo}, {hi})")
            xs_w, rows_w = _window_inputs(X, rows, lo, hi)
            rs.append(xs_w, rows_w, lo, hi - lo)
            torch.cuda.synchronize()
            _compare_prefix(rs, X, rows, hi, f"kind {kind} after [{lo},{hi})")


@pytest.mark.parametrize("H,Hq,prompt,steps", [(8, 32, 300, 700), (2, 4, 20, 200), (1, 2, 10, 100)])
def test_rolling_decode_simulation(H, Hq, prompt, steps):
    """A prompt, then one token per step: the cache keeps rolling_prefix(n) positions packed
    and flushes whole tiles from the BF16 tail as the prefix grows.  At the end the packed
    streams equal the one-shot encoding of the prefix, and attention over prefix + tail
    agrees with exact attention."""
    D = 128
    rng = np.random.default_rng(H * 1000 + prompt)
    n_tok = prompt + steps
    depth, rows = _decode_depths(rng, n_tok)
    Xk, fk = _decode_values(rng, depth, H, D, 2.0)
    Xv, fv = _decode_values(rng, depth, H, D, 1.0)
    cap = [n_tok, n_tok, rows[2].size, rows[3].size]
    streams = {flk.K: RollingStreams(flk.K, H, D, n_tok, cap, [True, True, False, False]),
               flk.V: RollingStreams(flk.V, H, D, n_tok, cap, [True, True, False, False])}
    P = 0
    flushes = 0
    for n in [prompt] + list(range(prompt + 1, n_tok + 1)):
        newP = flk.rolling_prefix(n)
        assert newP == orc.rolling_prefix(n)
        if newP > P:
            for kind, X in ((flk.K, Xk), (flk.V, Xv)):
                xs_w, rows_w = _window_inputs(X, rows, P, newP)
                streams[kind].append(xs_w, rows_w, P, newP - P)
            P = newP
            flushes += 1
    torch.cuda.synchronize()
    say(f"rolling H={H}: {flushes} flushes, prefix {P}, tail {n_tok - P}")
    assert 64 <= n_tok - P <= 127 or n_tok < 128
    ok = _compare_prefix(streams[flk.K], Xk, rows, P, "rolling K") if P else None
    ov = _compare_prefix(streams[flk.V], Xv, rows, P, "rolling V") if P else None
    # attention over packed prefix + BF16 tail
    q = synth.to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32))
    k_tail, v_tail = np.ascontiguousarray(fk[P:]), np.ascontiguousarray(fv[P:])
    ws = torch.empty(flk.attn_workspace_bytes(H, D, n_tok, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    kc = streams[flk.K].chain(P) if P else []
    vc = streams[flk.V].chain(P) if P else []
    flk.decode_attn_rolling(to_dev_bf16(q), kc, vc, P, H, to_dev_bf16(k_tail), to_dev_bf16(v_tail), scale, out, ws)
    torch.cuda.synchronize()
    kp = ok.recons[-1] if P else np.zeros((0, H, D), np.uint16)
    vp = ov.recons[-1] if P else np.zeros((0, H, D), np.uint16)
    ref = orc.decode_attn_rolling(q, kp, vp, k_tail, v_tail, scale)
    rel = _rel_err(out.float().cpu().numpy(), ref)
    say(f"  rolling attention max rel err {rel.max():.2e}")
    assert np.all(rel <= 2e-2), rel


@pytest.mark.parametrize("tail_len", [1, 127, 300])
def test_rolling_attention_tail_only_and_long_tail(tail_len):
    """No packed prefix (T = 0): a single token, a rolling tail and a tail of several tiles
    ending in a partial one."""
    H, Hq, D = 8, 32, 128
    rng = np.random.default_rng(tail_len)
    kt = synth.to_bf16_bits((2 * rng.standard_normal((tail_len, H, D))).astype(np.float32))
    vt = synth.to_bf16_bits(rng.standard_normal((tail_len, H, D)).astype(np.float32))
    q = synth.to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32))
    ws = torch.empty(flk.attn_workspace_bytes(H, D, tail_len, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    flk.decode_attn_rolling(to_dev_bf16(q), [], [], 0, H, to_dev_bf16(kt), to_dev_bf16(vt), scale, out, ws)
    torch.cuda.synchronize()
    ref = orc.decode_attn(q, kt, vt, scale)
    rel = _rel_err(out.float().cpu().numpy(), ref)
    assert np.all(rel <= 2e-2), rel


@pytest.mark.parametrize("H,D", [(8, 128), (3, 64)])
def test_batched_appends_equal_single_appends(H, D):
    """A flush of many tensors through flk_append_*_batch writes exactly what the single
    append calls write: K and V mixed, windows of 192/64/256 positions, one compact window
    with no rows, streams at different lengths."""
    rng = np.random.default_rng(H * 7 + D)
    n_tok = 512
    bounds = [0, 192, 256, 512]
    tensors = []
    for i in range(6):
        kind = flk.K if i % 2 == 0 else flk.V
        _, rows = _decode_depths(rng, n_tok)
        if i == 2:                                   # no loop-3/4 rows in [192, 256)
            rows[2] = rows[2][(rows[2] < 192) | (rows[2] >= 256)]
            rows[3] = np.intersect1d(rows[3], rows[2]).astype(np.int32)
        X = _decode_values(rng, np.full(n_tok, 4), H, D, 1.0)[0]
        tensors.append((kind, X, rows))
    single, batched = [], []
    for kind, X, rows in tensors:
        cap = [n_tok, n_tok, rows[2].size, rows[3].size]
        single.append(RollingStreams(kind, H, D, n_tok, cap, [True, True, False, False]))
        batched.append(RollingStreams(kind, H, D, n_tok, cap, [True, True, False, False]))
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        say(f"batched appends H={H} D={D} window [{lo}, {hi})")
        wins = [_window_inputs(X, rows, lo, hi) for _, X, rows in tensors]
        rec_s = [rs.append(xw, rw, lo, hi - lo) for rs, (xw, rw) in zip(single, wins)]
        rec_b = [torch.empty((hi - lo, H, D), dtype=torch.bfloat16, device="cuda") for _ in tensors]
        keep = []
        for l in range(4):
            items = []
            for rs, (xw, rw), rec in zip(batched, wins, rec_b):
                p = rs.packs[l]
                xd = None if xw[l] is None else to_dev_bf16(xw[l])
                keep.append(xd)
                if l == 0:
                    items.append((rs.kind, xd, lo, rec, p))
                elif rs.dense[l]:
                    items.append((rs.kind, xd, None, hi - lo, lo, hi - lo, lo, rec, p))
                else:
                    n_w = 0 if xw[l] is None else xw[l].shape[0]
                    rd = None
                    if n_w:
                        p.rows[rs.n[l]:rs.n[l] + n_w].copy_(torch.from_numpy(rw[l]))
                        rd = p.rows[rs.n[l]:rs.n[l] + n_w]
                    items.append((rs.kind, xd, rd, n_w, lo, hi - lo, rs.n[l], rec, p))
            if l == 0:
                flk.append_base_batch(items, H, D)
            else:
                flk.append_residual_batch(items, H, D)
            for rs, (xw, rw) in zip(batched, wins):
                rs.n[l] += (hi - lo) if rs.dense[l] else (0 if xw[l] is None else xw[l].shape[0])
        torch.cuda.synchronize()
        for ti, (a, b, ra, rb) in enumerate(zip(single, batched, rec_s, rec_b)):
            assert_same(to_host_u16(rb), to_host_u16(ra), f"t{ti} window recon [{lo},{hi})")
            for l, (ca, cb) in enumerate(zip(a.chain(hi), b.chain(hi))):
                assert ca.n_rows == cb.n_rows
                assert_same(cb.codes.cpu().numpy(), ca.codes.cpu().numpy(), f"t{ti} codes loop {l}")
                assert_same(cb.params.cpu().numpy(), ca.params.cpu().numpy(), f"t{ti} params loop {l}")
                if ca.tile_start is not None:
                    assert torch.equal(ca.tile_start, cb.tile_start), f"t{ti} tile index loop {l}"


@pytest.mark.parametrize("before", [0, 5])
def test_empty_v_window_needs_no_stream_buffers(before):
    """An empty compact V window writes only its tile index entries, so it may come without codes
    and params (V has no per-tile params); the result must not depend on rows_before."""
    import ctypes
    H, D, p0, n_pos = 2, 64, 128, 128
    say(f"empty V window, rows_before {before}")
    tile = torch.full((p0 // 64 + n_pos // 64 + 1,), -7, dtype=torch.int32, device="cuda")
    recon = torch.zeros((n_pos, H, D), dtype=torch.bfloat16, device="cuda")
    st = flk.lib().flk_append_residual(ctypes.byref(flk.desc(flk.V, H, D)), None, None, 0, p0, n_pos, before,
                                       ctypes.c_void_p(recon.data_ptr()), None, None,
                                       ctypes.c_void_p(tile.data_ptr()), None, None)
    torch.cuda.synchronize()
    assert st == 0, flk.lib().flk_status_string(st).decode()
    got = tile.cpu().numpy()
    assert list(got[:p0 // 64]) == [-7] * (p0 // 64)            # entries before the window untouched
    assert np.all(got[p0 // 64:] == before)
