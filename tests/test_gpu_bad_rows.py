"""A compact loop whose rows list a position outside [0, T): the encoders flag FLK_DEV_ROWS,
skip that row (no X_hat write, and its values stay out of every group's extremes) and encode
the other rows exactly as the oracle encodes the loop without it.  The bad entry is the last
(largest) one, so the compact rows before it keep their indices and groups."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from quantized_kv_cache_amd import flk, synth

from chain_runner import assert_same, to_dev_bf16, to_host_u16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,D,n", [(300, 8, 128, 150), (640, 8, 128, 256), (1000, 3, 96, 333)])
def test_out_of_range_row_is_skipped(T, H, D, n):
    rng = np.random.default_rng(T + n)
    y0 = rng.standard_normal((T, H, D)).astype(np.float32)
    x0 = synth.to_bf16_bits(y0)
    good = np.sort(rng.choice(T, n - 1, replace=False)).astype(np.int32)
    rows = np.concatenate([good, np.array([T + 5], np.int32)])          # the last entry is out of range
    x1 = synth.to_bf16_bits(y0[np.minimum(rows, T - 1)] + 0.1 * rng.standard_normal((n, H, D)).astype(np.float32))
    for kind in (flk.K, flk.V):
        print(f"bad rows: T={T} H={H} D={D} n={n} kind={kind}", flush=True)
        # the oracle encodes the loop over the valid rows only
        base, recon_o = orc.encode_base(kind, x0)
        st_o = orc.encode_residual(kind, x1[: n - 1], good, recon_o)
        # the GPU gets every row, the bad one last
        recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
        p0 = flk.Packed.empty(kind, H, D, T, None, T=T)
        flk.encode_base(kind, to_dev_bf16(x0), p0, recon)
        rd = torch.from_numpy(rows).cuda()
        p1 = flk.Packed.empty(kind, H, D, n, rd, T=T)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        flk.encode_residual(kind, to_dev_bf16(x1), rd, recon, p1, status)
        torch.cuda.synchronize()
        assert int(status.item()) & flk.DEV_ROWS, "FLK_DEV_ROWS not set"
        assert_same(to_host_u16(recon), recon_o, f"recon kind {kind}")
        assert_same(p1.codes.cpu().numpy()[: n - 1], st_o.codes, f"codes kind {kind}")
        params = p1.params.cpu().numpy().view(np.uint32)
        if kind == flk.V:
            params = params[: n - 1]
        assert_same(params, st_o.params, f"params kind {kind}")
