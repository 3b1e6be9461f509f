"""Batched calls against the single calls and the oracle: a batch must write exactly what the
single call writes for each of its units, whatever mix of K and V, lengths, compact and empty
loops and shapes it holds (shapes the batched kernels do not cover fall back to single
launches inside the same call)."""
import numpy as np
import pytest
import torch

from quantized_kv_cache_amd import flk, synth

from chain_runner import GpuChain, OracleChain, assert_same, compare_chains, to_dev_bf16, to_dev_rows, to_host_u16

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def run_batched(units, H, D):
    """units: list of (kind, xs, rows) chains of equal loop count.  Encodes every loop of every
    unit with one batched call per loop, then rebuilds all with one batched reconstruct.
    Returns per unit (packed list, per-loop recon copies, reconstruct output)."""
    n_loops = len(units[0][1])
    dev = []
    for kind, xs, rows in units:
        T = xs[0].shape[0]
        recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
        xd = [to_dev_bf16(x) for x in xs]
        rd = [to_dev_rows(r) for r in rows]
        packs = [flk.Packed.empty(kind, H, D, x.shape[0], r, T=T) for x, r in zip(xs, rd)]
        dev.append((kind, xd, rd, recon, packs, []))
    for loop in range(n_loops):
        if loop == 0:
            flk.encode_base_batch([(k, xd[0], recon, packs[0]) for k, xd, rd, recon, packs, _ in dev], H, D)
        else:
            flk.encode_residual_batch([(k, xd[loop], rd[loop], recon, packs[loop])
                                       for k, xd, rd, recon, packs, _ in dev], H, D)
        for k, xd, rd, recon, packs, copies in dev:
            copies.append(to_host_u16(recon))
    outs = [torch.empty_like(recon) for _, _, _, recon, _, _ in dev]
    flk.reconstruct_batch([(k, packs, out) for (k, _, _, _, packs, _), out in zip(dev, outs)], H, D)
    torch.cuda.synchronize()
    return [(packs, copies, to_host_u16(out)) for (_, _, _, _, packs, copies), out in zip(dev, outs)]


def assert_same_as_single(units, H, D, got, tag):
    for ui, ((kind, xs, rows), (packs, copies, out)) in enumerate(zip(units, got)):
        g = GpuChain(kind, xs, rows)
        for loop, p in enumerate(packs):
            assert_same(p.codes.cpu().numpy(), g.packed[loop].codes.cpu().numpy(), f"{tag} u{ui} codes {loop}")
            assert_same(p.params.cpu().numpy(), g.packed[loop].params.cpu().numpy(), f"{tag} u{ui} params {loop}")
            assert_same(copies[loop], g.recons[loop], f"{tag} u{ui} recon {loop}")
            if p.tile_start is not None and p.n_rows:
                assert torch.equal(p.tile_start, g.packed[loop].tile_start), f"{tag} u{ui} tile index {loop}"
        assert_same(out, g.recons[-1], f"{tag} u{ui} reconstruct")


def test_batched_cache_units_kv_together():
    """Four (request, layer) units of the batched workload, K and V of each in the same calls."""
    w = synth.WORKLOADS[4]
    L = synth.batched_lengths()
    picks = [(0, 0), (1, 7), (2, 23), (9, 13)]
    units = []
    for req, layer in picks:
        T = int(L[req])
        sets = synth.active_sets(w, T, request=req, layer=layer)
        for kind, tensor in ((flk.K, synth.K_TENSOR), (flk.V, synth.V_TENSOR)):
            c = synth.make_chain(w, tensor, T=T, request=req, layer=layer, sets=sets)
            units.append((kind, c.xs, c.rows))
    say(f"batched calls over {len(units)} tensors")
    got = run_batched(units, w.H, w.D)
    assert_same_as_single(units, w.H, w.D, got, "batched cache")
    # and one unit against the oracle on a head slice
    kind, xs, rows = units[3]
    o = OracleChain(kind, [x[:, 4:5] for x in xs], rows)
    packs, copies, out = got[3]
    for loop in range(len(xs)):
        assert_same(packs[loop].codes.cpu().numpy()[:, 4:5], o.streams[loop].codes, f"oracle codes {loop}")
        assert_same(packs[loop].params.cpu().numpy().view(np.uint32)[:, 4:5], o.streams[loop].params,
                    f"oracle params {loop}")
    assert_same(out[:, 4:5], o.recons[-1], "oracle reconstruct")


def _chain(rng, T, H, D, sizes):
    y = rng.standard_normal((T, H, D)).astype(np.float32)
    xs, rows, prev = [], [], np.arange(T, dtype=np.int32)
    for r, n in enumerate(sizes):
        if r:
            y = y + (0.1 * rng.standard_normal((T, H, D))).astype(np.float32)
        xb = synth.to_bf16_bits(y)
        if n is None:
            xs.append(xb)
            rows.append(None)
        else:
            prev = np.sort(rng.choice(prev, size=n, replace=False)).astype(np.int32)
            xs.append(np.ascontiguousarray(xb[prev]))
            rows.append(prev)
    return xs, rows


@pytest.mark.parametrize("H,D", [(8, 128), (8, 96), (3, 64), (1, 512)])
def test_mixed_batch_shapes_and_chunks(H, D):
    """20 tensors (more than one launch holds), K and V alternating, with varied lengths, a
    1-row compact loop and an empty loop; D = 96 and H*D < 1024 exercise the fallbacks."""
    rng = np.random.default_rng(H * 1000 + D)
    units = []
    for i in range(20):
        T = int(rng.integers(1, 700))
        s3 = int(rng.integers(0, T + 1))
        s4 = int(rng.integers(0, s3 + 1)) if i % 5 else (1 if s3 else 0)
        sizes = [None, None, s3, s4]
        xs, rows = _chain(rng, T, H, D, sizes)
        units.append((flk.K if i % 2 == 0 else flk.V, xs, rows))
    say(f"mixed batch H={H} D={D}")
    got = run_batched(units, H, D)
    assert_same_as_single(units, H, D, got, f"mixed {H}x{D}")
