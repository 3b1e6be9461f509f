"""GPU parity on the two workloads beyond the long prompt: the batched cache (many requests and
layers with seeded lengths, so K groups end in random tails) and single-token decode attention
over 131072 packed tokens.  Everything goes through the C ABI; the oracle runs on head slices
so it finishes in seconds."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from quantized_kv_cache_amd import flk, synth
from chain_runner import GpuChain, OracleChain, assert_same, compare_chains, to_dev_bf16

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


# (request, layer) units of the batched workload, with the seeded length of their request;
# the last two override the length to force a 1-row K tail group (L % 64 == 1) and a short
# request whose compact loops fall below one group.
LENGTHS = synth.batched_lengths()
UNITS = [(0, 0, None), (1, 7, None), (2, 23, None), (3, 11, None), (17, 3, None), (63, 22, None),
         (5, 5, 64 * 9 + 1), (6, 1, 100)]


@pytest.mark.parametrize("req,layer,length", UNITS)
def test_batched_cache_units(req, layer, length):
    w = synth.WORKLOADS[4]
    T = int(LENGTHS[req]) if length is None else length
    sets = synth.active_sets(w, T, request=req, layer=layer)
    assert [None if s is None else len(s) for s in sets] == [None, None] + \
        [synth.budget_rows(p, T) for p in w.budgets[2:]]
    heads = (0, 9)
    for kind, tensor in ((flk.K, synth.K_TENSOR), (flk.V, synth.V_TENSOR)):
        c = synth.make_chain(w, tensor, T=T, H=w.H, request=req, layer=layer, sets=sets)
        say(f"batched unit req={req} layer={layer} T={T} kind={kind}")
        g = GpuChain(kind, c.xs, c.rows)
        assert_same(g.reconstruct(), g.recons[-1], "reconstruct vs in-place")
        for h in heads:
            o = OracleChain(kind, [x[:, h:h + 1] for x in c.xs], c.rows)
            compare_chains(g, o, head_slice=slice(h, h + 1), tag=f"unit {req},{layer} kind {kind} h{h}")


def _attn_rel_err(got, ref):
    """Per query head: max |got - ref| / max |ref| (the benchmark's normwise tolerance)."""
    return np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)


def test_decode_attention_long_context():
    w = synth.WORKLOADS[5]
    T, H, D, Hq = w.T, w.H, w.D, w.Hq
    G = Hq // H
    sets = synth.active_sets(w, T)
    say(f"decode attention T={T} Hkv={H} Hq={Hq}: encoding K and V chains on the GPU")
    gpu = {}
    host = {}
    for kind, tensor in ((flk.K, synth.K_TENSOR), (flk.V, synth.V_TENSOR)):
        c = synth.make_chain(w, tensor, sets=sets)
        g = GpuChain(kind, c.xs, c.rows)
        gpu[kind] = g
        host[kind] = c
    q = synth.make_query(w)
    qd = to_dev_bf16(q)
    ws = torch.empty(flk.attn_workspace_bytes(H, D, T, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    flk.decode_attn_packed(qd, gpu[flk.K].packed, gpu[flk.V].packed, T, H, scale, out, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    for h in (0, 5):
        say(f"  oracle kv head {h}")
        kh = OracleChain(flk.K, [x[:, h:h + 1] for x in host[flk.K].xs], host[flk.K].rows)
        vh = OracleChain(flk.V, [x[:, h:h + 1] for x in host[flk.V].xs], host[flk.V].rows)
        # the packed streams the GPU wrote for this head equal the oracle's
        compare_chains(gpu[flk.K], kh, head_slice=slice(h, h + 1), tag=f"attn K h{h}")
        compare_chains(gpu[flk.V], vh, head_slice=slice(h, h + 1), tag=f"attn V h{h}")
        ref = orc.decode_attn(q[h * G:(h + 1) * G], kh.recons[-1], vh.recons[-1], scale)
        rel = _attn_rel_err(got[h * G:(h + 1) * G], ref)
        say(f"  kv head {h}: max rel err {rel.max():.2e}")
        assert np.all(rel <= 2e-2), rel


@pytest.mark.parametrize("T,H,Hq,sizes", [
    (1, 1, 1, [None]),                        # one token: softmax weight 1
    (63, 2, 8, [None, None]),                 # a single partial tile
    (1025, 4, 16, [None, None, 700, 3]),      # a split boundary plus one token; sparse tails
    (4096, 8, 128, [None, 4096, 2048, 1]),    # G = 16, a dense residual passed as compact rows
])
def test_decode_attention_shapes(T, H, Hq, sizes):
    D = 128
    rng = np.random.default_rng(T + H)
    y = rng.standard_normal((T, H, D)).astype(np.float32)
    xs = {flk.K: [], flk.V: []}
    rows = []
    prev = np.arange(T, dtype=np.int32)
    yk, yv = y * 2.0, rng.standard_normal((T, H, D)).astype(np.float32)
    for r, n in enumerate(sizes):
        if r:
            yk = yk + (0.05 * rng.standard_normal((T, H, D))).astype(np.float32)
            yv = yv + (0.05 * rng.standard_normal((T, H, D))).astype(np.float32)
        if n is not None:
            prev = np.sort(rng.choice(prev, size=n, replace=False)).astype(np.int32)
        sel = None if n is None else prev
        for kind, yy in ((flk.K, yk), (flk.V, yv)):
            xb = synth.to_bf16_bits(yy)
            xs[kind].append(xb if sel is None else np.ascontiguousarray(xb[sel]))
        rows.append(sel)
    g = {k: GpuChain(k, xs[k], rows) for k in (flk.K, flk.V)}
    o = {k: OracleChain(k, xs[k], rows) for k in (flk.K, flk.V)}
    q = synth.to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32))
    ws = torch.empty(flk.attn_workspace_bytes(H, D, T, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    say(f"attention shape T={T} H={H} Hq={Hq} sizes={sizes}")
    flk.decode_attn_packed(to_dev_bf16(q), g[flk.K].packed, g[flk.V].packed, T, H, scale, out, ws)
    torch.cuda.synchronize()
    ref = orc.decode_attn(q, o[flk.K].recons[-1], o[flk.V].recons[-1], scale)
    rel = _attn_rel_err(out.float().cpu().numpy(), ref)
    assert np.all(rel <= 2e-2), rel


@pytest.mark.parametrize("T,tail_len,H,Hq,sizes", [
    (1, 1, 1, 1, [None]),                     # one packed token, one tail token
    (63, 300, 2, 8, [None, None]),            # a partial tile, a tail of several slices
    (1025, 17, 4, 16, [None, None, 700, 3]),  # a split boundary; a tail slice plus one token
    (4096, 127, 8, 128, [None, 4096, 2048, 1]),  # G = 16, a rolling cache's longest tail
])
def test_decode_attention_packed_prefix_and_tail(T, tail_len, H, Hq, sizes):
    """Attention over packed INT4 chains plus a BF16 tail (flk_decode_attn_rolling with T > 0):
    the tail's scores follow the packed ones in both passes.  Against the oracle's exact
    attention over the reconstruction followed by the tail, within 2e-2 normwise per head."""
    D = 128
    rng = np.random.default_rng(7 * T + tail_len)
    xs = {flk.K: [], flk.V: []}
    rows = []
    prev = np.arange(T, dtype=np.int32)
    yk = (2.0 * rng.standard_normal((T, H, D))).astype(np.float32)
    yv = rng.standard_normal((T, H, D)).astype(np.float32)
    for r, n in enumerate(sizes):
        if r:
            yk = yk + (0.05 * rng.standard_normal((T, H, D))).astype(np.float32)
            yv = yv + (0.05 * rng.standard_normal((T, H, D))).astype(np.float32)
        if n is not None:
            prev = np.sort(rng.choice(prev, size=n, replace=False)).astype(np.int32)
        sel = None if n is None else prev
        for kind, yy in ((flk.K, yk), (flk.V, yv)):
            xb = synth.to_bf16_bits(yy)
            xs[kind].append(xb if sel is None else np.ascontiguousarray(xb[sel]))
        rows.append(sel)
    g = {k: GpuChain(k, xs[k], rows) for k in (flk.K, flk.V)}
    o = {k: OracleChain(k, xs[k], rows) for k in (flk.K, flk.V)}
    kt = synth.to_bf16_bits((2 * rng.standard_normal((tail_len, H, D))).astype(np.float32))
    vt = synth.to_bf16_bits(rng.standard_normal((tail_len, H, D)).astype(np.float32))
    q = synth.to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32))
    ws = torch.empty(flk.attn_workspace_bytes(H, D, T + tail_len, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    say(f"attention prefix T={T} tail={tail_len} H={H} Hq={Hq} sizes={sizes}")
    flk.decode_attn_rolling(to_dev_bf16(q), g[flk.K].packed, g[flk.V].packed, T, H, to_dev_bf16(kt),
                            to_dev_bf16(vt), scale, out, ws)
    torch.cuda.synchronize()
    ref = orc.decode_attn_rolling(q, o[flk.K].recons[-1], o[flk.V].recons[-1], kt, vt, scale)
    rel = _attn_rel_err(out.float().cpu().numpy(), ref)
    say(f"  max rel err {rel.max():.2e}")
    assert np.all(rel <= 2e-2), rel


def test_reconstruct_then_attend_matches_oracle():
    """The plain path the fused reader is measured against: rebuild K_hat and V_hat in BF16
    (flk_reconstruct), then attend over the BF16 cache (flk_decode_attn_rolling with no packed
    part).  Against the oracle's exact attention on the oracle's K_hat / V_hat, within 2e-2
    normwise per query head, on the decode workload's recipe at 16384 tokens and 4 KV heads."""
    w = synth.WORKLOADS[5]
    T, H, D, Hq = 16384, 4, 128, 16
    G = Hq // H
    sets = synth.active_sets(w, T)
    say(f"reconstruct-then-attend T={T} Hkv={H} Hq={Hq}")
    gpu, host = {}, {}
    for kind, tensor in ((flk.K, synth.K_TENSOR), (flk.V, synth.V_TENSOR)):
        c = synth.make_chain(w, tensor, T=T, H=H, sets=sets)
        gpu[kind] = GpuChain(kind, c.xs, c.rows)
        host[kind] = c
    q = synth.to_bf16_bits(np.random.default_rng(21).standard_normal((Hq, D)).astype(np.float32))
    kfull = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    vfull = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    flk.reconstruct(flk.K, gpu[flk.K].packed, kfull)
    flk.reconstruct(flk.V, gpu[flk.V].packed, vfull)
    ws = torch.empty(flk.attn_workspace_bytes(H, D, T, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    flk.decode_attn_rolling(to_dev_bf16(q), [], [], 0, H, kfull, vfull, scale, out, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    for h in range(H):
        kh = OracleChain(flk.K, [x[:, h:h + 1] for x in host[flk.K].xs], host[flk.K].rows)
        vh = OracleChain(flk.V, [x[:, h:h + 1] for x in host[flk.V].xs], host[flk.V].rows)
        ref = orc.decode_attn(q[h * G:(h + 1) * G], kh.recons[-1], vh.recons[-1], scale)
        rel = _attn_rel_err(got[h * G:(h + 1) * G], ref)
        say(f"  kv head {h}: max rel err {rel.max():.2e}")
        assert np.all(rel <= 2e-2), rel
