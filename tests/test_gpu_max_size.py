"""The largest tensors the library accepts: H = 8, D = 128 and T = 2,097,151 positions, the
largest T with T*H*D < 2^31 elements (4 GiB of BF16 per tensor; the kernels address rows with
32-bit byte offsets), for K and V.  A 4-loop chain: two dense loops, then compact loops holding
the even positions and the multiples of 4, so that every 256-position window is a sub-problem
of its own: its K groups (64 consecutive compact rows) and its V groups (within a row) hold
only its own tokens.  Codes, params, the reconstruction after the last loop and flk_reconstruct
are compared bit for bit with the oracle run on sampled windows, the first, the last (255
positions: ragged dense and compact tails at the end of the address range) and windows between;
the tile indices are compared whole with their closed form."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from quantized_kv_cache_amd import flk, synth

from chain_runner import assert_same, to_host_u16

pytestmark = pytest.mark.gpu

H, D = 8, 128
W = H * D
T = (1 << 31) // W - 1                       # 2,097,151
WIN = 256


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("kind", [flk.K, flk.V])
def test_largest_tensor_chain(kind):
    assert T * W < (1 << 31) <= (T + 1) * W
    say(f"max size kind={kind}: drawing 4 x {T} x {H} x {D} BF16 on the device")
    xs = synth.device_trajectory(T, H, D, 4, seed=31 + kind)
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    rows = [None, None, pos[0::2].contiguous(), pos[0::4].contiguous()]
    x3 = xs[2].index_select(0, rows[2])
    x4 = xs[3].index_select(0, rows[3])
    host3 = {}
    host4 = {}
    last = (T - 1) // WIN
    windows = sorted({0, 1, 2047, 4096, 5000, last - 1, last})
    for w in windows:                        # keep the sampled inputs of the compact loops
        p0, p1 = w * WIN, min(T, (w + 1) * WIN)
        host3[w] = to_host_u16(x3[p0 // 2:(p1 + 1) // 2])
        host4[w] = to_host_u16(x4[p0 // 4:(p1 + 3) // 4])
    xs[2] = xs[3] = None
    torch.cuda.empty_cache()

    recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    packs = []
    for l, (x, r) in enumerate(zip([xs[0], xs[1], x3, x4], rows)):
        p = flk.Packed.empty(kind, H, D, x.shape[0], r, T=T)
        if l == 0:
            flk.encode_base(kind, x, p, recon)
        else:
            flk.encode_residual(kind, x, r, recon, p)
        packs.append(p)
    out = torch.empty_like(recon)
    flk.reconstruct(kind, packs, out)
    torch.cuda.synchronize()
    say("encoded and reconstructed; comparing windows with the oracle")

    # tile indices: the compact rows before position 64t are ceil(min(64t, T) / step)
    t64 = np.minimum(64 * np.arange((T + 63) // 64 + 1, dtype=np.int64), T)
    for l, step in ((2, 2), (3, 4)):
        assert np.array_equal(packs[l].tile_start.cpu().numpy(), (t64 + step - 1) // step), f"tile index loop {l + 1}"

    for w in windows:
        p0, p1 = w * WIN, min(T, (w + 1) * WIN)
        n = p1 - p0
        sub_rows = [None, None, np.arange(0, n, 2, dtype=np.int32), np.arange(0, n, 4, dtype=np.int32)]
        xh = [to_host_u16(xs[0][p0:p1]), to_host_u16(xs[1][p0:p1]), host3[w], host4[w]]
        base, rc = orc.encode_base(kind, xh[0])
        streams = [base]
        for x, r in zip(xh[1:], sub_rows[1:]):
            streams.append(orc.encode_residual(kind, x, r, rc))
        tag = f"kind={kind} window {w} [{p0}, {p1})"
        firsts = [p0, p0, p0 // 2, p0 // 4]
        for l, (s, j0) in enumerate(zip(streams, firsts)):
            m = s.codes.shape[0]
            assert_same(packs[l].codes[j0:j0 + m].cpu().numpy(), s.codes, f"{tag} codes loop {l + 1}")
            if kind == flk.K:
                g0 = j0 // 64
                got = packs[l].params[g0:g0 + s.params.shape[0]]
            else:
                got = packs[l].params[j0:j0 + m]
            assert_same(got.cpu().numpy().view(np.uint32), s.params, f"{tag} params loop {l + 1}")
        assert_same(to_host_u16(recon[p0:p1]), rc, f"{tag} recon after loop 4")
        assert_same(to_host_u16(out[p0:p1]), rc, f"{tag} reconstruct")
    say(f"windows {windows} equal the oracle")
