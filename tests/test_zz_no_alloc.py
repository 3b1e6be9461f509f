"""The allocation-free decode attention (flk_decode_attn_packed_noalloc) against
flk_decode_attn_packed with a caller workspace, through the C ABI.

Both run the same kernels with the same split of the tokens, so their outputs must agree bit
for bit; both are also held to the oracle's exact attention within 2e-2 (normwise per query
head, RFC section 3.3 consumer).  Two calls in a row on one device, the second over a smaller
input, check that the scratch array's leftovers from the first call do not leak into the
second.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from quantized_kv_cache_amd import flk

from chain_runner import GpuChain, to_dev_bf16

pytestmark = pytest.mark.gpu


def _case(seed, T, H, D, Hq, fracs):
    """Seeded K and V chains (dense base and loop 2, compact later loops at `fracs` of T) and
    a query."""
    rng = np.random.default_rng(seed)
    rows = [None, None]
    prev = np.arange(T, dtype=np.int32)
    for f in fracs:
        prev = np.sort(rng.choice(prev, max(1, int(f * T)), replace=False)).astype(np.int32)
        rows.append(prev)
    chains = {}
    for kind in (flk.K, flk.V):
        y = rng.standard_normal((T, H, D)).astype(np.float32) * (3.0 if kind == flk.K else 1.0)
        xs = []
        for r in rows:
            if xs:
                y = y + 0.05 * rng.standard_normal((T, H, D)).astype(np.float32)
            u = y.view(np.uint32).astype(np.uint64)
            xb = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
            xs.append(xb if r is None else np.ascontiguousarray(xb[r]))
        chains[kind] = GpuChain(kind, xs, rows)
    u = rng.standard_normal((Hq, D)).astype(np.float32).view(np.uint32).astype(np.uint64)
    q = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return chains, q


@pytest.mark.parametrize("first,second", [((1, 2048, 8, 128, 32, [0.5, 0.25]), (2, 300, 2, 128, 8, [0.4])),
                                          ((3, 4160, 4, 128, 64, [0.5]), (4, 64, 1, 128, 16, []))])
def test_noalloc_matches_workspace_call(first, second):
    for seed, T, H, D, Hq, fracs in (first, second):
        print(f"noalloc attention seed={seed} T={T} H={H} Hq={Hq} loops={2 + len(fracs)}", flush=True)
        chains, q = _case(seed, T, H, D, Hq, fracs)
        kc, vc = chains[flk.K], chains[flk.V]
        qd = to_dev_bf16(q)
        scale = 1.0 / math.sqrt(D)
        ws = torch.empty(flk.attn_workspace_bytes(H, D, T, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
        want = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
        got = torch.full((Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        flk.decode_attn_packed(qd, kc.packed, vc.packed, T, H, scale, want, ws)
        flk.decode_attn_packed_noalloc(qd, kc.packed, vc.packed, T, H, scale, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "noalloc differs from the workspace call"
        ref = orc.decode_attn(q, kc.recons[-1], vc.recons[-1], scale)
        g = got.float().cpu().numpy()
        rel = np.abs(g - ref).max(axis=1) / np.abs(ref).max(axis=1)
        assert np.all(rel <= 2e-2), f"rel err {rel.max():.3e}"
