"""GPU parity for the FP4 codec variants through the C ABI -- NVFP4 (vllm-rlt PR #166, review
item 2) and MXFP4 (OCP MX v1.0, section 6): codes, params (NVFP4: header and E4M3 block scales;
MXFP4: E8M0 block scales), the tile index of compact loops, every loop's reconstruction and the
reconstruction from the streams, bit for bit against the oracle, for FP4 chains and for an INT4
base with FP4 residuals; and decode attention fused over such chains against exact attention
over the oracle's reconstructions (within 2e-2 per head)."""
import math

import numpy as np
import pytest
import torch

from oracle import fp4 as ofp4
from oracle import oracle as orc
from quantized_kv_cache_amd import flk, synth

from chain_runner import assert_same, to_dev_bf16, to_dev_rows, to_host_u16

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


FMTS = ["nvfp4", "mxfp4"]


def _gpu_chain(kind, xs, rows, int4_base, fmt, status=None):
    T, H, D = xs[0].shape
    recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    packs, recons = [], []
    for loop, (x, r) in enumerate(zip(xs, rows)):
        xd, rd = to_dev_bf16(x), to_dev_rows(r)
        p = flk.Packed.empty(kind, H, D, x.shape[0], rd, T=T, fmt="int4" if loop == 0 and int4_base else fmt)
        if loop == 0:
            flk.encode_base(kind, xd, p, recon, status)
        else:
            flk.encode_residual(kind, xd, rd, recon, p, status)
        packs.append(p)
        recons.append(to_host_u16(recon))
    out = torch.empty_like(recon)
    flk.reconstruct(kind, packs, out)
    torch.cuda.synchronize()
    return packs, recons, to_host_u16(out)


def _oracle_chain(kind, xs, rows, int4_base, fmt):
    mx = fmt == "mxfp4"
    if int4_base:
        base, recon = orc.encode_base(kind, xs[0])
    else:
        base, recon = ofp4.encode_base(xs[0], mx=mx)
    recons, streams = [recon.copy()], [base]
    for x, r in zip(xs[1:], rows[1:]):
        streams.append(ofp4.encode_residual(x, r, recon, mx=mx))
        recons.append(recon.copy())
    return streams, recons


def _compare(kind, xs, rows, int4_base, tag, fmt):
    T, H, D = xs[0].shape
    tag = f"{fmt} {tag}"
    packs, g_recons, g_out = _gpu_chain(kind, xs, rows, int4_base, fmt)
    streams, o_recons = _oracle_chain(kind, xs, rows, int4_base, fmt)
    for loop, (p, s) in enumerate(zip(packs, streams)):
        assert_same(g_recons[loop], o_recons[loop], f"{tag} recon loop {loop + 1}")
        if p.n_rows == 0:
            continue
        assert_same(p.codes.cpu().numpy(), s.codes, f"{tag} codes loop {loop + 1}")
        if loop == 0 and int4_base:
            assert_same(p.params.cpu().numpy().view(np.uint32), s.params, f"{tag} INT4 params loop 1")
            continue
        want = s.params_bytes()
        got = p.params.cpu().numpy().view(np.uint8)[:len(want)]
        assert_same(got, want, f"{tag} params loop {loop + 1}")
        if s.rows is not None:
            assert np.array_equal(p.tile_start.cpu().numpy(), orc.tile_index(s.rows, T)), f"{tag} tile index"
    assert_same(g_out, o_recons[-1], f"{tag} reconstruct")


def _chain_inputs(rng, T, H, D, sizes, scale=1.0):
    y = (scale * rng.standard_normal((T, H, D))).astype(np.float32)
    xs, rows, prev = [], [], np.arange(T, dtype=np.int32)
    for r, n in enumerate(sizes):
        if r:
            y = y + (0.1 * scale * rng.standard_normal((T, H, D))).astype(np.float32)
        if n is not None:
            prev = np.sort(rng.choice(prev, size=n, replace=False)).astype(np.int32)
        xb = synth.to_bf16_bits(y)
        xs.append(xb if n is None else np.ascontiguousarray(xb[prev]))
        rows.append(None if n is None else prev.copy())
    return xs, rows


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("int4_base", [False, True])
@pytest.mark.parametrize("kind", [flk.K, flk.V])
@pytest.mark.parametrize("T,H,D,sizes", [
    (256, 2, 64, [None, None, None, None]),
    (1000, 8, 96, [None, None, 500, 250]),
    (1, 1, 16, [None, None, 1, 1]),
    (1, 1, 32, [None, None, 1, 1]),
    (65, 3, 48, [None, 65, 1, 0]),           # a dense loop given as rows, a 1-row loop, an empty loop
    (65, 3, 96, [None, 65, 1, 0]),
    (300, 5, 32, [None, None, 0, None]),     # an empty loop, then a dense one
    (513, 2, 128, [None, None, 200, 3]),
])
def test_fp4_chain_matches_oracle(T, H, D, sizes, kind, int4_base, fmt):
    if fmt == "mxfp4" and D % 32:
        pytest.skip("MXFP4 blocks are 32 channels")
    rng = np.random.default_rng(T * 31 + H * 7 + D + kind)
    xs, rows = _chain_inputs(rng, T, H, D, sizes)
    say(f"{fmt} T={T} H={H} D={D} kind={kind} int4_base={int4_base}")
    _compare(kind, xs, rows, int4_base, f"T={T} H={H} D={D} kind={kind} int4_base={int4_base}", fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("scale", [1e-36, 1e-20, 3e-3, 1.0, 300.0, 1e30])
def test_fp4_magnitudes(scale, fmt):
    """From scales in the binary32 subnormal range (NVFP4: the division decides every code;
    MXFP4: the smallest E8M0 scales) to large ones."""
    rng = np.random.default_rng(int(abs(np.log10(scale))) + 1)
    xs, rows = _chain_inputs(rng, 200, 2, 64, [None, None, 100], scale=scale)
    say(f"{fmt} magnitudes scale={scale}")
    for int4_base in (False, True):
        if int4_base and scale > 1e4:
            continue                                     # INT4's FP16 params overflow there
        if int4_base and scale < 1e-6:
            continue                                     # below FP16's range
        _compare(flk.V, xs, rows, int4_base, f"scale {scale} int4_base={int4_base}", fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp4_special_values(fmt):
    """Signed zeros, grid values times powers of two, constant and all-zero blocks, a residual
    loop equal to the reconstruction (NVFP4: amax 0, s_g = 1, every code +0; MXFP4: the
    smallest scale)."""
    T, H, D = 64, 2, 64
    rng = np.random.default_rng(11)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    x = (rng.choice(grid, (T, H, D)) * np.where(rng.random((T, H, D)) < 0.5, -1, 1)).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-8, 8, (T, H, 1)).astype(np.float32)
    x[:8] = -0.0
    x[8:16] = 0.0
    x[16:24, :, :16] = 2.5
    xb = synth.to_bf16_bits(x)
    _, r1 = ofp4.encode_base(xb, mx=fmt == "mxfp4")
    xs = [xb, r1.copy(), xb]                              # loop 2 equals X_hat_1 exactly
    rows = [None, None, None]
    _compare(flk.K, xs, rows, False, "special values", fmt)
    z = np.zeros((T, H, D), np.uint16)
    _compare(flk.V, [z, z], [None, None], False, "all zero", fmt)
    nz = np.full((T, H, D), 0x8000, np.uint16)           # every value -0
    _compare(flk.V, [nz, nz], [None, None], False, "all -0", fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp4_nonfinite_sets_status(fmt):
    T, H, D = 64, 1, 32
    x = np.zeros((T, H, D), np.float32)
    x[3, 0, 5] = np.nan
    xd = to_dev_bf16(synth.to_bf16_bits(x))
    recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    p = flk.Packed.empty(flk.K, H, D, T, fmt=fmt)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    flk.encode_base(flk.K, xd, p, recon, status)
    torch.cuda.synchronize()
    assert int(status.item()) & 1


@pytest.mark.parametrize("fmt", FMTS)
def test_fp4_long_prompt_k_chain(fmt):
    """The long-prompt K chain (32768 x 8 x 128, Student-t with per-channel multipliers,
    budgets 100/100/50/25 %) in full, FP4 and INT4 base + FP4 residuals."""
    w = synth.WORKLOADS[3]
    c = synth.make_chain(w, synth.K_TENSOR)
    for int4_base in (True, False):
        say(f"{fmt} long prompt K int4_base={int4_base}")
        _compare(flk.K, c.xs, c.rows, int4_base, f"long prompt K int4_base={int4_base}", fmt)


def _rel(got, ref):
    return np.abs(got - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("int4_base", [False, True])
@pytest.mark.parametrize("T,H,Hq,sizes", [
    (1000, 2, 8, [None, None, 500, 250]),
    (700, 1, 16, [None, None, 0, None]),        # an empty loop dropped from the chain, then a dense one
    (16384, 8, 32, [None, None, 8192, 4096]),   # 8 KV heads, 32 query heads
])
def test_fp4_decode_attention(T, H, Hq, sizes, int4_base, fmt):
    """Fused decode attention over FP4 (or INT4 base + FP4 residual) chains against exact
    attention over the oracle's reconstructions, within 2e-2 per query head."""
    D = 128
    rng = np.random.default_rng(T + H + int(int4_base))
    xk, rows = _chain_inputs(rng, T, H, D, sizes, scale=2.0)
    xv, _ = _chain_inputs(np.random.default_rng(T + 7), T, H, D, [None] * len(sizes))
    xv = [xv[0]] + [x if r is None else np.ascontiguousarray(x[r]) for x, r in zip(xv[1:], rows[1:])]
    say(f"{fmt} attention T={T} H={H} Hq={Hq} int4_base={int4_base}")
    kp, _, _ = _gpu_chain(flk.K, xk, rows, int4_base, fmt)
    vp, _, _ = _gpu_chain(flk.V, xv, rows, int4_base, fmt)
    q = synth.to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32))
    ws = torch.empty(flk.attn_workspace_bytes(H, D, T, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    flk.decode_attn_mixed(to_dev_bf16(q), kp, vp, T, H, scale, out, ws)
    torch.cuda.synchronize()
    _, ok = _oracle_chain(flk.K, xk, rows, int4_base, fmt)
    _, ov = _oracle_chain(flk.V, xv, rows, int4_base, fmt)
    ref = orc.decode_attn(q, ok[-1], ov[-1], scale)
    rel = _rel(out.float().cpu().numpy(), ref)
    say(f"  max rel err {rel.max():.2e}")
    assert np.all(rel <= 2e-2), rel
