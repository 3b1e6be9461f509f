"""GPU parity for sparse decode attention over packed chains (RFC, vllm-rlt #156, section 3.2).

The selection S is decided by binary32 scores on the GPU and binary64 scores in the oracle.  For a
query head whose oracle scores leave a gap wider than twice the binary32 rounding bound between
the k-th and the (k+1)-th key, S is unique and must equal the oracle's S exactly; the head's mass,
O_ref, C_ref and reference output are then compared with the oracle's (mass within 1e-4 relative,
the others within 2e-2 normwise per query head, the attention tolerance).  For any other head S is
only checked for validity: k distinct ascending positions, every selected score at least every
unselected one within the rounding bound.

The later loops are checked twice: the GPU loop call fed the oracle's own reference state against
the oracle's loop output (every head), and the GPU loop fed the GPU's reference state against the
same oracle output (heads with a unique S).  Nothing the GPU computes is passed to the oracle.
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp4 as ofp4
from oracle import oracle as orc
from quantized_kv_cache_amd import flk, synth

from chain_runner import GpuChain, OracleChain, to_dev_bf16

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _rel(got, ref):
    return np.abs(got - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30)


def _round_bound(q, khat, scale, G):
    """[Hq] bound on a binary32 score's rounding: the terms' magnitudes times 2^-20."""
    qf = orc.f32_from_bf16(q).astype(np.float64)
    kf = orc.f32_from_bf16(khat).astype(np.float64)
    return np.array([scale * (np.abs(kf[:, i // G]) @ np.abs(qf[i])).max() * 2.0 ** -20 + 1e-30
                     for i in range(q.shape[0])])


def _unique_heads(scores, k, eps):
    """Heads whose top-k under the oracle's scores cannot change by binary32 rounding: a gap of
    more than twice the rounding bound at the k-th key, or an exact tie there whose scores are
    the only ones within that bound (identical keys score identically on both sides, and the
    tie goes to the lower positions)."""
    T = scores.shape[1]
    if k == T:
        return np.ones(scores.shape[0], bool)
    part = -np.partition(-scores, (k - 1, k), axis=1)
    gap = part[:, k - 1] - part[:, k] > 2 * eps
    kth = part[:, k - 1:k]
    near = np.abs(scores - kth) <= 2 * eps[:, None]
    clean_tie = (part[:, k - 1] == part[:, k]) & np.all(~near | (scores == kth), axis=1)
    return gap | clean_tie


def _check_selection(sel, scores, eps, tag):
    Hq, k = sel.shape
    T = scores.shape[1]
    for i in range(Hq):
        s = sel[i]
        assert s.min() >= 0 and s.max() < T, f"{tag} head {i}: position out of range"
        assert np.all(np.diff(s) > 0), f"{tag} head {i}: not ascending and distinct"
        if k < T:
            lo, hi = scores[i, s].min(), np.delete(scores[i], s).max()
            assert lo >= hi - eps[i], f"{tag} head {i}: selected score {lo} below unselected {hi}"


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


def _workspace(T, H, Hq, k, n_loops):
    ws = torch.empty(flk.sparse_workspace_bytes(H, 128, T, Hq, k, n_loops) // 4 + 64, dtype=torch.float32,
                     device="cuda")
    return ws[(-ws.data_ptr() // 4) % 64:]                   # 256-byte aligned


def _gpu_reference(g, T, H, Hq, k, qs, scale, ws):
    """GPU reference at loop 2 and the later loops fed its state; returns host arrays."""
    D = 128
    n_loops = len(g[flk.K].packed)
    st = flk.SparseState.empty(Hq, D, k)
    out_ref = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    flk.sparse_attn_reference(to_dev_bf16(qs[2]), g[flk.K].packed[:2], g[flk.V].packed[:2],
                              T, H, k, scale, out_ref, st, ws)
    outs = _gpu_loops(g, T, H, Hq, k, qs, scale, st, ws)
    return dict(sel=st.sel.cpu().numpy(), mass=st.mass.cpu().numpy().astype(np.float64),
                o_ref=st.o_ref.cpu().numpy().astype(np.float64), c_ref=st.c_ref.cpu().numpy().astype(np.float64),
                out_ref=out_ref.float().cpu().numpy(), outs=outs)


def _gpu_loops(g, T, H, Hq, k, qs, scale, st, ws):
    outs = {}
    for depth in range(3, len(g[flk.K].packed) + 1):
        o = torch.empty((Hq, 128), dtype=torch.bfloat16, device="cuda")
        flk.sparse_attn_loop(to_dev_bf16(qs[depth]), g[flk.K].packed[:depth], g[flk.V].packed[:depth], T, H, k,
                             scale, st, o, ws)
        outs[depth] = o
    torch.cuda.synchronize()
    return {d: o.float().cpu().numpy() for d, o in outs.items()}


def _state_from(ref_parts, Hq, k):
    """Device SparseState holding the oracle's state on the heads it covers (others: the first k
    positions, zero statistics, whose outputs are not compared)."""
    sel = np.tile(np.arange(k, dtype=np.int32), (Hq, 1))
    mass = np.zeros(Hq, np.float32)
    o_ref = np.zeros((Hq, 128), np.float32)
    c_ref = np.zeros((Hq, 128), np.float32)
    for qsl, ref in ref_parts:
        sel[qsl], mass[qsl], o_ref[qsl], c_ref[qsl] = ref.sel, ref.mass, ref.o_ref, ref.c_ref
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return flk.SparseState(dev(sel), dev(mass), dev(o_ref), dev(c_ref))


def _compare(gpu, fed, o, qs, scale, H, Hq, k, qsl, tag):
    """gpu: _gpu_reference output; fed: GPU loop outputs from the oracle's state; o: {K, V: OracleChain}
    on the query heads qsl."""
    G = Hq // H
    k2, v2 = o[flk.K].recons[1], o[flk.V].recons[1]
    ref = orc.sparse_reference(qs[2][qsl], k2, v2, scale, k)
    scores = orc.attn_scores(qs[2][qsl], k2, scale)
    eps = _round_bound(qs[2][qsl], k2, scale, G)
    sel = gpu["sel"][qsl]
    _check_selection(sel, scores, eps, tag)
    uniq = _unique_heads(scores, k, eps)
    say(f"  {tag}: {uniq.mean():.0%} of heads have a unique S")
    assert uniq.mean() >= 0.5, f"{tag}: too few heads with a unique selection to compare"
    u = np.flatnonzero(uniq)
    assert np.array_equal(sel[u], ref.sel[u]), f"{tag}: S differs from the oracle's on a unique head"
    mass = gpu["mass"][qsl][u]
    assert np.all(np.abs(mass - ref.mass[u]) <= 1e-4 * np.maximum(ref.mass[u], 1e-6)), f"{tag} mass"
    assert np.all(_rel(gpu["o_ref"][qsl][u], ref.o_ref[u]) <= 2e-2), f"{tag} O_ref"
    assert np.all(_rel(gpu["out_ref"][qsl][u], ref.o_ref[u]) <= 2e-2), f"{tag} reference output"
    err_c = np.abs(gpu["c_ref"][qsl][u] - ref.c_ref[u]).max(axis=1)
    assert np.all(err_c <= 2e-2 * np.abs(ref.o_ref[u]).max(axis=1) + 1e-6), f"{tag} C_ref"
    for depth in fed:
        want = orc.sparse_loop(qs[depth][qsl], o[flk.K].recons[depth - 1], o[flk.V].recons[depth - 1], scale, ref)
        rel_fed = _rel(fed[depth][qsl], want)
        rel_own = _rel(gpu["outs"][depth][qsl][u], want[u])
        say(f"  {tag} loop {depth}: max rel err {rel_fed.max():.2e} (oracle state), {rel_own.max():.2e} (GPU state)")
        assert np.all(rel_fed <= 2e-2), f"{tag} loop {depth} from the oracle's state: {rel_fed}"
        assert np.all(rel_own <= 2e-2), f"{tag} loop {depth} from the GPU's state: {rel_own}"
    return ref


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
    ws = _workspace(T, H, Hq, k, len(sizes))
    gpu = _gpu_reference(g, T, H, Hq, k, qs, scale, ws)
    ref = orc.sparse_reference(qs[2], o[flk.K].recons[1], o[flk.V].recons[1], scale, k)
    fed = _gpu_loops(g, T, H, Hq, k, qs, scale, _state_from([(slice(None), ref)], Hq, k), ws)
    _compare(gpu, fed, o, qs, scale, H, Hq, k, slice(None), tag=f"T={T} k={k}")
    if k == T:
        assert np.allclose(gpu["mass"], 1.0, atol=1e-5)
        for depth, got in gpu["outs"].items():
            dense = orc.decode_attn(qs[depth], o[flk.K].recons[depth - 1], o[flk.V].recons[depth - 1], scale)
            assert np.all(_rel(got, dense) <= 2e-2)


@pytest.mark.parametrize("T,k,tied", [(20000, 777, False), (40000, 3000, True)])
def test_sparse_attention_split_selection(T, k, tied):
    """Rows longer than the split threshold take the segmented top-k; with every key identical
    all scores tie, the selection is the first k positions and need runs through all segments."""
    H, Hq, D = 1, 4, 128
    rng = np.random.default_rng(T + k)
    xs, rows = _chains(rng, T, H, D, [None, None, T // 2])
    if tied:
        row = xs[flk.K][0][:1]
        xs[flk.K] = [np.ascontiguousarray(np.broadcast_to(row, x.shape)) for x in xs[flk.K]]
    g = {kind: GpuChain(kind, xs[kind], rows, k_tiles=kind == flk.K) for kind in (flk.K, flk.V)}
    o = {kind: OracleChain(kind, xs[kind], rows, k_tiles=kind == flk.K) for kind in (flk.K, flk.V)}
    qs = {d: synth.to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32)) for d in (2, 3)}
    scale = 1.0 / math.sqrt(D)
    say(f"sparse attention split top-k T={T} k={k} tied={tied}")
    ws = _workspace(T, H, Hq, k, 3)
    gpu = _gpu_reference(g, T, H, Hq, k, qs, scale, ws)
    ref = orc.sparse_reference(qs[2], o[flk.K].recons[1], o[flk.V].recons[1], scale, k)
    fed = _gpu_loops(g, T, H, Hq, k, qs, scale, _state_from([(slice(None), ref)], Hq, k), ws)
    _compare(gpu, fed, o, qs, scale, H, Hq, k, slice(None), tag=f"split T={T}")
    if tied:
        assert np.array_equal(gpu["sel"], np.tile(np.arange(k, dtype=np.int32), (Hq, 1)))


def test_sparse_attention_long_context():
    """The decode workload (131072 tokens, 8 KV heads, 32 query heads, 4 loops at 100/100/50/25%)
    with 4096 keys per query head; the oracle runs on the query heads of two KV heads."""
    w = synth.WORKLOADS[5]
    T, H, D, Hq = w.T, w.H, w.D, w.Hq
    G = Hq // H
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
    ws = _workspace(T, H, Hq, k, 4)
    gpu = _gpu_reference(g, T, H, Hq, k, qs, scale, ws)
    orcs, parts = {}, []
    for h in (0, 5):
        say(f"  oracle kv head {h}")
        orcs[h] = {kind: OracleChain(kind, [x[:, h:h + 1] for x in host[kind].xs], host[kind].rows,
                                     k_tiles=kind == flk.K) for kind in (flk.K, flk.V)}
        qsl = slice(h * G, (h + 1) * G)
        parts.append((qsl, orc.sparse_reference(qs[2][qsl], orcs[h][flk.K].recons[1], orcs[h][flk.V].recons[1],
                                                scale, k)))
    fed = _gpu_loops(g, T, H, Hq, k, qs, scale, _state_from(parts, Hq, k), ws)
    for h in (0, 5):
        _compare(gpu, fed, orcs[h], qs, scale, H, Hq, k, slice(h * G, (h + 1) * G), tag=f"kv head {h}")


class _Fp4Oracle:
    """The oracle's reconstructions after every loop of an FP4 chain (NVFP4 or MXFP4 residual
    loops on an INT4 or same-format base)."""

    def __init__(self, kind, xs, rows, fmt, int4_base):
        mx = fmt == "mxfp4"
        _, recon = orc.encode_base(kind, xs[0]) if int4_base else ofp4.encode_base(xs[0], mx=mx)
        self.recons = [recon.copy()]
        for x, r in zip(xs[1:], rows[1:]):
            ofp4.encode_residual(x, r, recon, mx=mx)
            self.recons.append(recon.copy())


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("int4_base", [False, True])
@pytest.mark.parametrize("T,H,Hq,sizes,k", [
    (1000, 2, 8, [None, None, 500, 250], 37),
    (2049, 4, 64, [None, 2049, 1024, 1], 300),           # G = 16, a 1-row compact loop
])
def test_sparse_attention_fp4(T, H, Hq, sizes, k, int4_base, fmt):
    """The reference and later loops over FP4 chains (keys and values decoded from NVFP4 or MXFP4
    residual loops, on an INT4 or FP4 base), against the oracle's sparse attention over the FP4
    oracle's reconstructions."""
    D = 128
    rng = np.random.default_rng(T + H + k + 7)
    xs, rows = _chains(rng, T, H, D, sizes)
    base = "int4" if int4_base else fmt
    g = {kind: GpuChain(kind, xs[kind], rows, fmt=fmt, base_fmt=base) for kind in (flk.K, flk.V)}
    o = {kind: _Fp4Oracle(kind, xs[kind], rows, fmt, int4_base) for kind in (flk.K, flk.V)}
    for kind in (flk.K, flk.V):                          # the chains themselves agree bit for bit
        for loop in range(len(sizes)):
            assert np.array_equal(g[kind].recons[loop], o[kind].recons[loop]), f"{fmt} recon loop {loop + 1}"
    qs = {d: synth.to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32)) for d in range(2, len(sizes) + 1)}
    scale = 1.0 / math.sqrt(D)
    say(f"sparse attention {fmt} int4_base={int4_base} T={T} H={H} Hq={Hq} k={k}")
    ws = _workspace(T, H, Hq, k, len(sizes))
    gpu = _gpu_reference(g, T, H, Hq, k, qs, scale, ws)
    ref = orc.sparse_reference(qs[2], o[flk.K].recons[1], o[flk.V].recons[1], scale, k)
    fed = _gpu_loops(g, T, H, Hq, k, qs, scale, _state_from([(slice(None), ref)], Hq, k), ws)
    _compare(gpu, fed, o, qs, scale, H, Hq, k, slice(None), tag=f"{fmt} int4_base={int4_base} T={T} k={k}")
