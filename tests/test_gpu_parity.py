"""GPU parity: the HIP codec against the CPU oracle, element by element, on seeded inputs.

Codes, params and every loop's BF16 reconstruction must be bit-identical; reconstruction
from the packed chain alone must equal the encoder's in-place result.  Full-size workloads
compare a sample of KV heads: K groups are per (head, channel) and V groups per (row, head),
so the oracle run on one head's slice computes exactly that head's share of the output.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from quantized_kv_cache_amd import flk, synth

from chain_runner import GpuChain, OracleChain, assert_same, compare_chains, to_dev_bf16, to_host_u16

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def workload_chains(wid: int, head_slice=None):
    w = synth.WORKLOADS[wid]
    sets = synth.active_sets(w, w.T)
    kc = synth.make_chain(w, synth.K_TENSOR, sets=sets)
    vc = synth.make_chain(w, synth.V_TENSOR, sets=sets)
    return w, sets, kc, vc


@pytest.mark.parametrize("wid", [1, 2])
def test_small_workloads_full_parity(wid):
    w, sets, kc, vc = workload_chains(wid)
    for kind, c in ((flk.K, kc), (flk.V, vc)):
        say(f"workload {w.name} kind {kind} T={w.T} H={w.H} D={w.D}")
        g = GpuChain(kind, c.xs, c.rows)
        o = OracleChain(kind, c.xs, c.rows)
        compare_chains(g, o, tag=f"{w.name}/{kind}")
        for depth in range(1, w.n_loops + 1):
            assert_same(g.reconstruct(depth), o.recons[depth - 1], f"reconstruct depth {depth}")


def test_long_prompt_sampled_heads():
    w = synth.WORKLOADS[3]
    sets = synth.active_sets(w, w.T)
    for kind, tensor in ((flk.K, synth.K_TENSOR), (flk.V, synth.V_TENSOR)):
        c = synth.make_chain(w, tensor, sets=sets)
        say(f"long_prompt kind {kind}: GPU chain")
        g = GpuChain(kind, c.xs, c.rows)
        full = g.reconstruct()
        assert_same(full, g.recons[-1], "reconstruct vs in-place")
        for h in (0, 5):
            say(f"  oracle head {h}")
            o = OracleChain(kind, [x[:, h:h + 1] for x in c.xs], c.rows)
            compare_chains(g, o, head_slice=slice(h, h + 1), tag=f"long_prompt/{kind}/h{h}")
        del g, c
        torch.cuda.empty_cache()


def _random_chain(rng, T, H, D, sizes, sigma=0.1, scale=1.0):
    """sizes[r] = None for dense, else the row count of loop r (nested, ascending)."""
    y = (rng.standard_normal((T, H, D)) * scale).astype(np.float32)
    xs, rows = [], []
    prev = np.arange(T, dtype=np.int32)
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


EDGE_CASES = [
    # (T, H, D, sizes)
    (1, 1, 8, [None, None]),
    (65, 3, 24, [None, None, 33, 1]),        # K tail of 1, V single partial group, 1-row loop
    (127, 2, 200, [None, 64, 63]),           # V tail group of 8, K groups of 64 and 63 rows
    (130, 1, 512, [None, None, 129]),        # widest head: 64 lanes per head
    (300, 5, 40, [None, 0, None]),           # empty residual loop in the middle
    (513, 2, 64, [None, 512, 257, 1]),
    (64, 16, 128, [None, None, 64, 64]),
]


@pytest.mark.parametrize("T,H,D,sizes", EDGE_CASES)
def test_edge_shapes(T, H, D, sizes):
    rng = np.random.default_rng(T * 1000 + H * 10 + D)
    xs, rows = _random_chain(rng, T, H, D, sizes)
    for kind in (flk.K, flk.V):
        say(f"edge T={T} H={H} D={D} sizes={sizes} kind={kind}")
        g = GpuChain(kind, xs, rows)
        o = OracleChain(kind, xs, rows)
        compare_chains(g, o, tag=f"edge {T},{H},{D} kind {kind}")
        assert_same(g.reconstruct(), o.reconstruct(), "reconstruct")


def test_last_position_and_distributions():
    rng = np.random.default_rng(77)
    T, H, D = 700, 4, 128
    for scale in (1e-4, 1.0, 300.0):
        xs, rows = _random_chain(rng, T, H, D, [None, None, 350, 90], scale=scale, sigma=0.05 * scale)
        for kind in (flk.K, flk.V):
            say(f"scale {scale} kind {kind}")
            g = GpuChain(kind, xs, rows)
            o = OracleChain(kind, xs, rows)
            compare_chains(g, o, tag=f"scale {scale} kind {kind}")
            assert_same(g.reconstruct(), o.reconstruct(), "reconstruct")


def test_special_values():
    """Signed zeros, constant groups, lossless grids, tiny (FP16-subnormal) ranges and exact
    half-integer ties, all bit-exact against the oracle."""
    T, H, D = 128, 2, 64
    rng = np.random.default_rng(5)
    y = np.zeros((T, H, D), np.float32)
    y[:, 0, :] = -0.0
    y[::3, 0, ::5] = 0.0                              # mixed signed zeros
    k = rng.integers(0, 16, size=(T, D)).astype(np.float32)
    k[np.arange(T), np.arange(T) % D] = 0
    k[np.arange(T), (np.arange(T) + 1) % D] = 15
    y[:, 1, :] = 0.5 * k                              # exact grid with ties on quarter steps
    y[64:, 1, :32] = 1e-6 * rng.standard_normal((64, 32))   # FP16-subnormal minima and scales
    y[100:, 1, 40:] = 3.25                            # constant V groups
    xs = [synth.to_bf16_bits(y)]
    y2 = y.copy()
    y2[:, 1, :] += 0.25 * rng.integers(0, 16, size=(T, D)) - 1.0
    xs.append(synth.to_bf16_bits(y2))
    xs.append(synth.to_bf16_bits(y2))                # zero residual: constant groups
    for kind in (flk.K, flk.V):
        g = GpuChain(kind, xs, [None, None, None])
        o = OracleChain(kind, xs, [None, None, None])
        compare_chains(g, o, tag=f"special kind {kind}")


def test_device_status_word():
    T, H, D = 64, 1, 64
    base = np.ones((T, H, D), np.float32)
    for val, bit in ((np.inf, flk.DEV_NONFINITE), (np.nan, flk.DEV_NONFINITE), (1e6, flk.DEV_RANGE)):
        y = base.copy()
        y[5, 0, 7] = val
        for kind in (flk.K, flk.V):
            status = torch.zeros(1, dtype=torch.int32, device="cuda")
            GpuChain(kind, [synth.to_bf16_bits(y)], [None], status=status)
            assert int(status.item()) & bit, (val, kind)
    for kind in (flk.K, flk.V):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        GpuChain(kind, [synth.to_bf16_bits(base)], [None], status=status)
        assert int(status.item()) == 0


def test_determinism_and_no_stray_writes():
    """Two runs give identical bytes; bytes just past every output stay untouched."""
    rng = np.random.default_rng(9)
    T, H, D = 200, 3, 96
    xs, rows = _random_chain(rng, T, H, D, [None, None, 77])
    for kind in (flk.K, flk.V):
        outs = []
        for _ in range(2):
            pad = 4096
            recon_buf = torch.full((T * H * D + pad,), 0x5A5A, dtype=torch.int16, device="cuda")
            recon = recon_buf[: T * H * D].view(torch.bfloat16).view(T, H, D)
            packs = []
            for loop, (x, r) in enumerate(zip(xs, rows)):
                n = x.shape[0]
                cb = torch.full((flk.codes_bytes(kind, H, D, n) + pad,), 0xA5, dtype=torch.uint8, device="cuda")
                pb_n = flk.params_bytes(kind, H, D, n) // 4
                pb = torch.full((pb_n + pad,), 0x3C3C3C3C, dtype=torch.int32, device="cuda")
                rd = None if r is None else torch.from_numpy(r).cuda()
                ts = None if r is None else torch.empty(flk.tile_index_bytes(T) // 4, dtype=torch.int32,
                                                         device="cuda")
                p = flk.Packed(n, rd, cb[: n * H * D // 2].view(n, H, D // 2),
                               pb[:pb_n].view(flk.params_shape(kind, H, D, n)), ts)
                xd = to_dev_bf16(x)
                if loop == 0:
                    flk.encode_base(kind, xd, p, recon)
                else:
                    flk.encode_residual(kind, xd, rd, recon, p)
                packs.append((cb, pb, pb_n, n))
            torch.cuda.synchronize()
            assert torch.all(recon_buf[T * H * D:] == 0x5A5A)
            for cb, pb, pb_n, n in packs:
                assert torch.all(cb[n * H * D // 2:] == 0xA5)
                assert torch.all(pb[pb_n:] == 0x3C3C3C3C)
            outs.append([to_host_u16(recon)] + [cb.cpu().numpy() for cb, _, _, _ in packs]
                        + [pb.cpu().numpy() for _, pb, _, _ in packs])
        for a, b in zip(*outs):
            assert np.array_equal(a, b)
        # reconstruct leaves the bytes past its output alone too
        g = GpuChain(kind, xs, rows)
        out_buf = torch.full((T * H * D + 4096,), 0x5A5A, dtype=torch.int16, device="cuda")
        out = out_buf[: T * H * D].view(torch.bfloat16).view(T, H, D)
        flk.reconstruct(kind, g.packed, out)
        torch.cuda.synchronize()
        assert torch.all(out_buf[T * H * D:] == 0x5A5A)
        assert_same(to_host_u16(out), g.recons[-1], "reconstruct")
