"""GPU parity for sparse decode attention over packed chains (RFC, vllm-rlt #156, section 3.2).

The selection S is decided by binary32 scores on the GPU and binary64 scores in the oracle, so
it is compared for what is unique: S must be k distinct ascending positions and a valid top-k
of the oracle's scores up to the binary32 rounding of a score (every selected score at least
every unselected one, within that bound).  The statistics and outputs are then compared with
the oracle evaluated on the GPU's S: mass within 1e-4 relative, O_ref, C_ref and the loop
outputs within 2e-2 normwise per query head (the attention tolerance).
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from quantized_kv_cache_amd import flk, synth

from chain_runner import GpuChain, OracleChain, to_dev_bf16

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _rel(got, ref):
    return np.abs(got - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)


def _check_selection(sel, scores, q, khat, scale, G, tag):
    """sel [Hq, k] from the GPU; scores [Hq, T] binary64 from the oracle."""
    Hq, k = sel.shape
    T = scores.shape[1]
    qf = orc.f32_from_bf16(q).astype(np.float64)
    kf = orc.f32_from_bf16(khat).astype(np.float64)
    for i in range(Hq):
        s = sel[i]
        assert s.min() >= 0 and s.max() < T, f"{tag} head {i}: position out of range"
        assert np.all(np.diff(s) > 0), f"{tag} head {i}: not ascending and distinct"
        if k == T:
            continue
        rest = np.setdiff1d(np.arange(T), s)
        # bound on a binary32 score's rounding: the terms' magnitudes times 2^-20
        eps = scale * (np.abs(kf[:, i // G]) @ np.abs(qf[i])).max() * 2.0 ** -20 + 1e-30
        lo, hi = scores[i, s].min(), scores[i, rest].max()
        assert lo >= hi - eps, f"{tag} head {i}: selected score {lo} below unselected {hi} (eps {eps})"


def _chains(rng, T, H, D, sizes):
    """K and V loop chains sharing their active rows (sizes[r] None = dense)."""
    yk = (2.0 * rng.standard_normal((T, H, D))).astype(np.float32)
    yv = rng.standard_normal((T, H, D)).astype(np.float32)
    xs = {flk.K: [], flk.V: []}
    rows, prev = [], np.arange(T, dtype=np.int32)
    for r, n in enumerate(sizes):
        if r:
            yk = yk + (0.1 * rng.standard_normal((T, H, D))).astype(np.float32)
            yv = yv + (0.1 * rng.standard_normal((T, H, D))).astype(np.float32)
        if n is not None:
            prev = np.sort(rng.choice(prev, size=n, replace=False)).astype(np.int32)
        sel = None if n is None else prev
        for kind, yy in ((flk.K, yk), (flk.V, yv)):
            xb = synth.to_bf16_bits(yy)
            xs[kind].append(xb if sel is None else np.ascontiguousarray(xb[sel]))
        rows.append(sel)
    return xs, rows


def _run_sparse(g, T, H, Hq, k, qs, scale, ref_depth=2):
    """GPU reference at ref_depth, then every later loop; returns host arrays."""
    D = 128
    n_loops = len(g[flk.K].packed)
    ws = torch.empty(flk.sparse_workspace_bytes(H, D, T, Hq, k, n_loops) // 4 + 64, dtype=torch.float32,
                     device="cuda")
    ws = ws[(-ws.data_ptr() // 4) % 64:]                      # 256-byte aligned
    st = flk.SparseState.empty(Hq, D, k)
    out_ref = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    flk.sparse_attn_reference(to_dev_bf16(qs[ref_depth]), g[flk.K].packed[:ref_depth], g[flk.V].packed[:ref_depth],
                              T, H, k, scale, out_ref, st, ws)
    outs = {}
    for depth in range(ref_depth + 1, n_loops + 1):
        o = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
        flk.sparse_attn_loop(to_dev_bf16(qs[depth]), g[flk.K].packed[:depth], g[flk.V].packed[:depth], T, H, k,
                             scale, st, o, ws)
        outs[depth] = o
    torch.cuda.synchronize()
    host = {d: o.float().cpu().numpy() for d, o in outs.items()}
    return (st.sel.cpu().numpy(), st.mass.cpu().numpy().astype(np.float64), st.o_ref.cpu().numpy().astype(np.float64),
            st.c_ref.cpu().numpy().astype(np.float64), out_ref.float().cpu().numpy(), host)


def _compare(gpu, o, qs, scale, H, Hq, k, head_slice=None, tag=""):
    """gpu: _run_sparse output; o: {K, V: OracleChain} (on the head slice if given)."""
    sel, mass, o_ref, c_ref, out_ref, outs = gpu
    G = Hq // H
    qsl = slice(None) if head_slice is None else slice(head_slice * G, (head_slice + 1) * G)
    sel, mass, o_ref, c_ref, out_ref = sel[qsl], mass[qsl], o_ref[qsl], c_ref[qsl], out_ref[qsl]
    k2, v2 = o[flk.K].recons[1], o[flk.V].recons[1]
    scores = orc.attn_scores(qs[2][qsl], k2, scale)
    _check_selection(sel, scores, qs[2][qsl], k2, scale, G, tag)
    ref = orc.sparse_reference_given(qs[2][qsl], k2, v2, scale, sel)
    assert np.all(np.abs(mass - ref.mass) <= 1e-4 * np.maximum(ref.mass, 1e-6)), f"{tag} mass"
    assert np.all(_rel(o_ref, ref.o_ref) <= 2e-2), f"{tag} O_ref {_rel(o_ref, ref.o_ref).max()}"
    assert np.all(_rel(out_ref, ref.o_ref) <= 2e-2), f"{tag} reference output"
    assert np.all(np.abs(c_ref - ref.c_ref).max(axis=1) <= 2e-2 * np.abs(ref.o_ref).max(axis=1) + 1e-6), f"{tag} C_ref"
    for depth, got in outs.items():
        want = orc.sparse_loop(qs[depth][qsl], o[flk.K].recons[depth - 1], o[flk.V].recons[depth - 1], scale, ref)
        rel = _rel(got[qsl], want)
        say(f"  {tag} loop {depth}: max rel err {rel.max():.2e}")
        assert np.all(rel <= 2e-2), f"{tag} loop {depth}: {rel}"
    # the oracle's own selection agrees except where two scores fall within rounding of each other
    own = orc.sparse_reference(qs[2][qsl], k2, v2, scale, k)
    same = np.mean([np.array_equal(a, b) for a, b in zip(own.sel, sel)])
    say(f"  {tag}: {same:.0%} of heads select exactly the oracle's S")


@pytest.mark.parametrize("T,H,Hq,sizes,k,k_tiles", [
    (1000, 2, 8, [None, None, 500, 250], 37, False),
    (1000, 2, 8, [None, None, 500, 250], 1, True),
    (1000, 2, 8, [None, None, 500, 250], 1000, False),   # every key kept: loops are dense attention
    (2049, 4, 64, [None, 2049, 1024, 1], 300, True),     # G = 16, a 1-row compact loop
    (700, 1, 2, [None, None, 0, None], 64, False),       # an empty loop, a dense loop 4
])
def test_sparse_attention_small(T, H, Hq, sizes, k, k_tiles):
    D = 128
    rng = np.random.default_rng(T + H + k)
    xs, rows = _chains(rng, T, H, D, sizes)
    g = {kind: GpuChain(kind, xs[kind], rows, k_tiles=k_tiles and kind == flk.K) for kind in (flk.K, flk.V)}
    o = {kind: OracleChain(kind, xs[kind], rows, k_tiles=k_tiles and kind == flk.K) for kind in (flk.K, flk.V)}
    qs = {d: synth.to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32)) for d in range(2, len(sizes) + 1)}
    scale = 1.0 / math.sqrt(D)
    say(f"sparse attention T={T} H={H} Hq={Hq} k={k} tiles={k_tiles}")
    gpu = _run_sparse(g, T, H, Hq, k, qs, scale)
    _compare(gpu, o, qs, scale, H, Hq, k, tag=f"T={T} k={k}")
    if k == T:
        assert np.allclose(gpu[1], 1.0, atol=1e-5)
        for depth, got in gpu[5].items():
            dense = orc.decode_attn(qs[depth], o[flk.K].recons[depth - 1], o[flk.V].recons[depth - 1], scale)
            assert np.all(_rel(got, dense) <= 2e-2)


def test_sparse_attention_long_context():
    """The decode workload (131072 tokens, 8 KV heads, 32 query heads, 4 loops at 100/100/50/25%)
    with 4096 keys per query head; the oracle runs on the query heads of two KV heads."""
    w = synth.WORKLOADS[5]
    T, H, D, Hq = w.T, w.H, w.D, w.Hq
    k = 4096
    sets = synth.active_sets(w, T)
    host, g = {}, {}
    for kind, tensor in ((flk.K, synth.K_TENSOR), (flk.V, synth.V_TENSOR)):
        c = synth.make_chain(w, tensor, sets=sets)
        host[kind] = c
        g[kind] = GpuChain(kind, c.xs, c.rows, k_tiles=kind == flk.K)
    rng = np.random.default_rng(5)
    qs = {d: synth.to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32)) for d in (2, 3, 4)}
    scale = 1.0 / math.sqrt(D)
    say(f"sparse attention T={T} k={k}: GPU")
    gpu = _run_sparse(g, T, H, Hq, k, qs, scale)
    for h in (0, 5):
        say(f"  oracle kv head {h}")
        o = {kind: OracleChain(kind, [x[:, h:h + 1] for x in host[kind].xs], host[kind].rows,
                               k_tiles=kind == flk.K) for kind in (flk.K, flk.V)}
        _compare(gpu, o, qs, scale, H, Hq, k, head_slice=h, tag=f"kv head {h}")
