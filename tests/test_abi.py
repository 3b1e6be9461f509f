"""CPU-side checks of the C ABI: the library loads, exports what include/flk.h declares, the
size functions agree with the closed forms, and host validation rejects bad calls before
anything is enqueued (no kernel runs here: every call below fails validation)."""
import ctypes
import os
import re

import numpy as np
import pytest

from quantized_kv_cache_amd import flk
from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flk_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = flk.lib()
    names = declared_functions()
    assert "flk_encode_base" in names and "flk_decode_attn_packed" in names
    for n in names:
        assert hasattr(L, n), n
    assert L.flk_abi_version() == 2


@pytest.mark.parametrize("kind", [flk.K, flk.V])
@pytest.mark.parametrize("H,D,n", [(1, 8, 1), (2, 64, 256), (8, 96, 1000), (8, 128, 32768), (16, 128, 4353),
                                   (3, 24, 65), (1, 512, 130)])
def test_sizes_match_closed_forms(kind, H, D, n):
    assert flk.codes_bytes(kind, H, D, n) == n * H * D // 2 == orc.codes_bytes(H, D, n)
    assert flk.params_bytes(kind, H, D, n) == orc.params_bytes(kind, H, D, n)
    groups = -(-n // 64) * H * D if kind == flk.K else n * H * -(-D // 64)
    assert flk.params_bytes(kind, H, D, n) == 4 * groups
    assert flk.rows_bytes(n, True) == 4 * n and flk.rows_bytes(n, False) == 0
    assert flk.tile_index_bytes(n) == 4 * (-(-n // 64) + 1) == orc.tile_index(np.arange(0), n).nbytes


@pytest.mark.parametrize("H,D,n,T", [(1, 8, 1, 1), (2, 64, 100, 256), (8, 96, 500, 1000), (8, 128, 8192, 32768),
                                     (3, 24, 0, 65)])
def test_tile_grouped_sizes(H, D, n, T):
    """Tile-grouped K stores one parameter row per 64-position tile, whatever the stream's
    row count; V and dense K are unchanged; stream_bytes adds rows and the tile index."""
    assert flk.params_bytes(flk.K, H, D, n, T, k_tiles=True) == orc.k_tile_params_bytes(H, D, T)
    assert flk.params_bytes(flk.K, H, D, T, T, k_tiles=True) == flk.params_bytes(flk.K, H, D, T)
    assert flk.params_bytes(flk.V, H, D, n, T, k_tiles=True) == orc.params_bytes(flk.V, H, D, n)
    for kind in (flk.K, flk.V):
        for kt in (False, True):
            want = (orc.codes_bytes(H, D, n) + flk.params_bytes(kind, H, D, n, T, kt) + 4 * n +
                    4 * (-(-T // 64) + 1))
            assert flk.stream_bytes(kind, H, D, n, T, True, kt) == want
    assert flk.stream_bytes(flk.K, H, D, T, T, False) == orc.codes_bytes(H, D, T) + orc.params_bytes(flk.K, H, D, T)


def test_rolling_prefix_matches_oracle():
    for n in list(range(-3, 1200)) + [32767, 131072, 131072 + 127, 2**31 - 1]:
        assert flk.rolling_prefix(n) == (orc.rolling_prefix(n) if n >= 0 and n < 10**6 else
                                         (0 if n < 128 else ((n - 64) // 64) * 64)), n


def test_descriptor_checks():
    L = flk.lib()
    d = flk.desc(flk.K, 8, 128)
    assert L.flk_desc_check(ctypes.byref(d)) == 0
    assert L.flk_desc_check(None) == 1
    for field, bad in [("abi_version", 1), ("format", 0), ("kind", 2), ("group", 32), ("param_dtype", 0),
                       ("nibble_order", 2), ("k_grouping", 2)]:
        e = flk.desc(flk.K, 8, 128)
        setattr(e, field, bad)
        assert L.flk_desc_check(ctypes.byref(e)) == 4, field
    e = flk.desc(flk.K, 8, 128, k_tiles=True)
    assert L.flk_desc_check(ctypes.byref(e)) == 0
    e.reserved[1] = 1
    assert L.flk_desc_check(ctypes.byref(e)) == 4
    for H, D in [(0, 128), (8, 0), (8, 4), (8, 100), (8, 520), (-1, 64)]:
        assert L.flk_desc_check(ctypes.byref(flk.desc(flk.V, H, D))) == 2, (H, D)
    assert flk.codes_bytes(flk.K, 8, 100, 10) == 0


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced (validation fails first)
MIS = ctypes.c_void_p((1 << 20) + 2)     # misaligned


def _encode_base(d, x, T, codes, params, recon):
    return flk.lib().flk_encode_base(ctypes.byref(d), x, T, codes, params, recon, None, None)


def test_encode_base_validation():
    d = flk.desc(flk.K, 2, 64)
    assert _encode_base(d, None, 16, FAKE, FAKE, FAKE) == 1
    assert _encode_base(d, FAKE, 16, None, FAKE, FAKE) == 1
    assert _encode_base(d, FAKE, 16, FAKE, FAKE, None) == 1
    assert _encode_base(d, FAKE, 0, FAKE, FAKE, FAKE) == 2
    big = flk.desc(flk.K, 16, 512)                      # T*H*D = 2^31 elements: a 4 GiB tensor
    assert _encode_base(big, FAKE, 1 << 18, FAKE, FAKE, FAKE) == 2
    assert _encode_base(d, MIS, 16, FAKE, FAKE, FAKE) == 3
    assert _encode_base(d, FAKE, 16, FAKE, MIS, FAKE) == 3
    bad = flk.desc(flk.K, 2, 64)
    bad.group = 128
    assert _encode_base(bad, FAKE, 16, FAKE, FAKE, FAKE) == 4


def test_encode_residual_validation():
    L = flk.lib()
    d = flk.desc(flk.V, 2, 64)

    def call(x, rows, n, T, recon=FAKE, codes=FAKE, params=FAKE, tile=FAKE):
        return L.flk_encode_residual(ctypes.byref(d), x, rows, n, T, recon, codes, params, tile, None, None)
    assert call(FAKE, None, 10, 16) == 2            # dense needs n == T
    assert call(FAKE, FAKE, 17, 16) == 2            # n > T
    assert call(FAKE, FAKE, -1, 16) == 2
    assert call(None, FAKE, 4, 16) == 1
    assert call(FAKE, FAKE, 4, 16, recon=None) == 1
    assert call(FAKE, ctypes.c_void_p((1 << 20) + 1), 4, 16) == 3
    assert call(FAKE, FAKE, 4, 16, tile=None) == 1   # a compact loop writes its tile index
    assert call(FAKE, FAKE, 4, 16, tile=ctypes.c_void_p((1 << 20) + 2)) == 3
    # an empty residual loop is valid and enqueues nothing
    assert call(None, FAKE, 0, 16, codes=None, params=None, tile=None) == 0


def test_reconstruct_validation():
    L = flk.lib()
    d = flk.desc(flk.K, 2, 64)
    S = flk.StreamC

    def call(chain, n_loops, T=64, out=FAKE):
        arr = (S * max(1, len(chain)))(*chain) if chain else None
        return L.flk_reconstruct(ctypes.byref(d), T, arr, n_loops, out, None)
    base = S(64, 0, None, FAKE.value, FAKE.value, None)
    assert call([], 1) == 1
    assert call([base], 0) == 2
    assert call([base] * 9, 9) == 2
    assert call([S(32, 0, None, FAKE.value, FAKE.value, None)], 1) == 2      # base must be dense n == T
    assert call([S(64, 0, FAKE.value, FAKE.value, FAKE.value, FAKE.value)], 1) == 2
    assert call([base, S(65, 0, FAKE.value, FAKE.value, FAKE.value, FAKE.value)], 2) == 2
    assert call([base, S(10, 0, None, FAKE.value, FAKE.value, None)], 2) == 2
    assert call([base, S(10, 7, FAKE.value, FAKE.value, FAKE.value, FAKE.value)], 2) == 4
    assert call([base, S(10, 0, FAKE.value, None, FAKE.value, FAKE.value)], 2) == 1
    assert call([base, S(10, 0, FAKE.value, MIS.value, FAKE.value, FAKE.value)], 2) == 3
    assert call([base, S(10, 0, FAKE.value, FAKE.value, FAKE.value, None)], 2) == 1   # no tile index
    assert call([base], 1, out=None) == 1
    assert call([base], 1, out=MIS) == 3


def test_attention_validation():
    L = flk.lib()
    kd, vd = flk.desc(flk.K, 8, 128), flk.desc(flk.V, 8, 128)
    S = flk.StreamC
    T = 256
    chain = (S * 1)(S(T, 0, None, FAKE.value, FAKE.value, None))
    ws = flk.attn_workspace_bytes(8, 128, T, 32)
    assert ws > 0

    def call(kd=kd, vd=vd, q=FAKE, hq=32, out=FAKE, w=FAKE, wb=ws, n_loops=1):
        return L.flk_decode_attn_packed(ctypes.byref(kd), ctypes.byref(vd), T, q, hq, chain, chain, n_loops,
                                        0.088, out, w, wb, None)
    assert call(kd=vd, vd=kd) == 4
    assert call(q=None) == 1
    assert call(hq=30) == 2
    assert call(wb=64) == 6                   # below any launch's need
    assert call(w=None) == 6
    assert call(hq=8 * 17) == 5
    d64k, d64v = flk.desc(flk.K, 8, 64), flk.desc(flk.V, 8, 64)
    assert call(kd=d64k, vd=d64v) == 5
    assert call(n_loops=0) == 2


def test_noalloc_attention_validation():
    """The allocation-free decode attention validates like flk_decode_attn_packed and rejects a
    call whose partials would not fit the library's scratch array before touching the device."""
    L = flk.lib()
    S = flk.StreamC

    def call(H=8, hq=32, T=256, q=FAKE, n_loops=1, kind_swap=False):
        kd, vd = flk.desc(flk.K, H, 128), flk.desc(flk.V, H, 128)
        if kind_swap:
            kd, vd = vd, kd
        chain = (S * 1)(S(T, 0, None, FAKE.value, FAKE.value, None))
        return L.flk_decode_attn_packed_noalloc(ctypes.byref(kd), ctypes.byref(vd), T, q, hq, chain, chain, n_loops,
                                                0.088, FAKE, None)
    assert call(kind_swap=True) == 4
    assert call(q=None) == 1
    assert call(hq=30) == 2
    assert call(hq=8 * 17) == 5
    assert call(n_loops=0) == 2
    # one KV head with 16 query heads over 2^21 tokens needs more than the scratch array holds
    assert flk.attn_workspace_bytes(1, 128, 1 << 21, 16) > 64 << 20
    assert call(H=1, hq=16, T=1 << 21) == 6


def test_status_strings():
    L = flk.lib()
    for s in range(8):
        assert L.flk_status_string(s)


def test_batch_validation():
    L = flk.lib()
    kd, vd = flk.desc(flk.K, 2, 64), flk.desc(flk.V, 2, 64)
    U = flk.UnitC

    def unit(kind=flk.K, x=FAKE.value, rows=None, recon=FAKE.value, n=16, T=16, tile=None, reserved=0):
        return U(x, rows, recon, FAKE.value, FAKE.value, tile, n, T, kind, reserved)

    def base(units, k=kd, v=vd, n=None):
        arr = (U * max(1, len(units)))(*units) if units else None
        return L.flk_encode_base_batch(ctypes.byref(k) if k else None, ctypes.byref(v) if v else None, arr,
                                       len(units) if n is None else n, None, None)

    def resid(units, k=kd, v=vd):
        arr = (U * len(units))(*units)
        return L.flk_encode_residual_batch(ctypes.byref(k), ctypes.byref(v), arr, len(units), None, None)
    assert base([]) == 0                                     # nothing to do
    assert base([], n=-1) == 2
    assert base([], n=3) == 1                                # NULL table
    assert base([unit(kind=2)]) == 4
    assert base([unit(reserved=1)]) == 4
    assert base([unit(kind=flk.V)], v=None) == 1             # no descriptor for a V unit
    assert base([unit()], k=vd) == 4                         # k_desc must describe K
    assert base([unit(rows=FAKE.value, tile=FAKE.value)]) == 2   # a base is dense
    assert base([unit(n=8)]) == 2
    # a valid unit followed by a bad one: validation fails before anything is launched
    assert base([unit(), unit(kind=flk.V, x=MIS.value)]) == 3
    assert base([unit(), unit(kind=flk.V, recon=None)]) == 1
    assert resid([unit(rows=FAKE.value, n=4, tile=None)]) == 1   # compact needs its tile index
    assert resid([unit(rows=None, n=4)]) == 2                    # dense needs n == T
    assert resid([unit(n=17)]) == 2
    big = flk.desc(flk.K, 16, 512)
    assert base([unit(n=1 << 18, T=1 << 18)], k=big) == 2    # a 4 GiB tensor

    R = flk.ReconUnitC
    chain = (flk.StreamC * 1)(flk.StreamC(64, 0, None, FAKE.value, FAKE.value, None))

    def rec(units, k=kd, v=vd):
        arr = (R * len(units))(*units)
        return L.flk_reconstruct_batch(ctypes.byref(k), ctypes.byref(v), arr, len(units), None)
    good = ctypes.cast(chain, ctypes.POINTER(flk.StreamC))
    assert rec([R(None, FAKE.value, 64, 1, flk.K, 0)]) == 1
    assert rec([R(good, FAKE.value, 64, 0, flk.K, 0)]) == 2
    assert rec([R(good, MIS.value, 64, 1, flk.V, 0)]) == 3
    assert rec([R(good, FAKE.value, 64, 1, 5, 0)]) == 4
    assert rec([R(good, FAKE.value, 64, 1, flk.K, 3)]) == 4
    assert rec([R(good, None, 64, 1, flk.K, 0)]) == 1
    assert rec([R(good, FAKE.value, 65, 1, flk.K, 0)]) == 2      # base must have n == T


def test_append_validation():
    L = flk.lib()
    kt = flk.desc(flk.K, 2, 64, k_tiles=True)
    kr = flk.desc(flk.K, 2, 64)
    vd = flk.desc(flk.V, 2, 64)

    def base(d, p0=64, n_pos=128, x=FAKE, codes=FAKE, recon=FAKE):
        return L.flk_append_base(ctypes.byref(d), x, p0, n_pos, codes, FAKE, recon, None, None)
    assert base(kt, p0=32) == 2
    assert base(kt, n_pos=100) == 2
    assert base(kt, n_pos=0) == 2
    assert base(kt, p0=-64) == 2
    assert base(kt, x=None) == 1
    assert base(kt, codes=MIS) == 3
    big = flk.desc(flk.K, 16, 512)
    assert base(big, p0=1 << 18, n_pos=64) == 2

    def resid(d, rows=FAKE, n=10, p0=64, n_pos=128, before=20, x=FAKE, tile=FAKE, recon=FAKE):
        return L.flk_append_residual(ctypes.byref(d), x, rows, n, p0, n_pos, before, recon, FAKE, FAKE, tile,
                                     None, None)
    assert resid(kr) == 5                       # compact K needs tile groups
    assert resid(kt, n=129) == 2
    assert resid(kt, before=65) == 2            # more rows before p0 than positions
    assert resid(kt, before=-1) == 2
    assert resid(kt, p0=65) == 2
    assert resid(kt, rows=None, n=100) == 2     # dense needs n == n_pos
    assert resid(kt, rows=None, n=128, before=10) == 2   # and rows_before == p0
    assert resid(kt, tile=None) == 1
    assert resid(vd, tile=None) == 1
    assert resid(kt, x=None) == 1
    assert resid(kt, recon=None) == 1
    assert resid(kt, rows=MIS) == 3
    assert resid(vd, x=MIS) == 3


def test_rolling_attention_validation():
    L = flk.lib()
    kd, vd = flk.desc(flk.K, 8, 128), flk.desc(flk.V, 8, 128)
    S = flk.StreamC
    T = 256
    chain = (S * 1)(S(T, 0, None, FAKE.value, FAKE.value, None))
    ws = flk.attn_workspace_bytes(8, 128, T, 32)
    assert flk.attn_workspace_bytes(8, 128, 1, 32) >= 32 * 130 * 4     # at least one partial

    def call(T=T, tail=FAKE, tl=100, w=FAKE, wb=ws, n_loops=1, q=FAKE):
        return L.flk_decode_attn_rolling(ctypes.byref(kd), ctypes.byref(vd), T, q, 32, chain, chain, n_loops,
                                         tail, tail, tl, 0.088, FAKE, w, wb, None)
    assert call(T=0, tl=0) == 2                 # nothing to attend to
    assert call(T=-1) == 2
    assert call(tl=-1) == 2
    assert call(tail=None) == 1
    assert call(tail=MIS) == 3
    assert call(wb=64) == 6
    assert call(q=None) == 1
    assert call(n_loops=0) == 2


def test_batched_append_validation():
    L = flk.lib()
    kt, vd = flk.desc(flk.K, 2, 64, k_tiles=True), flk.desc(flk.V, 2, 64)
    kr = flk.desc(flk.K, 2, 64)
    A = flk.AppendUnitC

    def unit(kind=flk.K, x=FAKE.value, rows=FAKE.value, n=10, p0=64, n_pos=64, before=5, tile=FAKE.value,
             reserved=0):
        return A(x, rows, FAKE.value, FAKE.value, FAKE.value, tile, n, p0, n_pos, before, kind, reserved)

    def call(units, resid=True, k=kt, v=vd):
        arr = (A * max(1, len(units)))(*units)
        f = L.flk_append_residual_batch if resid else L.flk_append_base_batch
        return f(ctypes.byref(k) if k else None, ctypes.byref(v) if v else None, arr, len(units), None, None)
    assert call([]) == 0
    assert call([unit(kind=3)]) == 4
    assert call([unit(reserved=1)]) == 4
    assert call([unit(p0=32)]) == 2
    assert call([unit(tile=None)]) == 1
    assert call([unit()], k=kr) == 5                    # compact K needs tile groups
    assert call([unit(kind=flk.V)], v=None) == 1
    assert call([unit()], resid=False) == 2             # loop 1 is dense
    # every unit is checked before anything launches: a bad last unit fails the call
    assert call([unit(kind=flk.V), unit(n=65)]) == 2


def test_sparse_attention_validation():
    L = flk.lib()
    kd, vd = flk.desc(flk.K, 8, 128), flk.desc(flk.V, 8, 128)
    S = flk.StreamC
    T = 256
    chain = (S * 1)(S(T, 0, None, FAKE.value, FAKE.value, None))
    ws = flk.sparse_workspace_bytes(8, 128, T, 32, 16, 1)
    assert ws > 32 * T * 4                       # holds the reference scores
    assert flk.sparse_workspace_bytes(8, 128, T, 32, T + 1, 1) == 0
    assert flk.sparse_workspace_bytes(8, 128, T, 32, 16, 0) == 0

    def ref(k=16, q=FAKE, sel=FAKE, w=FAKE, wb=ws, n_loops=1, hq=32, kd=kd, vd=vd, c=FAKE):
        return L.flk_sparse_attn_reference(ctypes.byref(kd), ctypes.byref(vd), T, q, hq, chain, chain, n_loops, k,
                                           0.088, FAKE, sel, FAKE, FAKE, c, w, wb, None)

    def loop(k=16, sel=FAKE, wb=ws, c=FAKE):
        return L.flk_sparse_attn_loop(ctypes.byref(kd), ctypes.byref(vd), T, FAKE, 32, chain, chain, 1, k, 0.088,
                                      sel, FAKE, FAKE, c, FAKE, FAKE, wb, None)
    assert ref(kd=vd, vd=kd) == 4
    assert ref(q=None) == 1
    assert ref(sel=None) == 1
    assert ref(k=0) == 2
    assert ref(k=T + 1) == 2
    assert ref(hq=30) == 2
    assert ref(hq=8 * 17) == 5
    assert ref(n_loops=0) == 2
    assert ref(sel=MIS) == 3
    assert ref(c=MIS) == 3
    assert ref(wb=64) == 6
    assert ref(w=None) == 6
    assert ref(w=ctypes.c_void_p((1 << 20) + 16)) == 3   # the workspace is 256-byte aligned
    assert loop(k=0) == 2
    assert loop(sel=None) == 1
    assert loop(wb=64) == 6
    assert loop(c=MIS) == 3


def test_select_count_matches_oracle():
    from oracle import selection as osel
    for T, W, p in [(32768, 2048, [50]), (32768, 2048, [50, 25]), (1000, 7, [33, 10]), (20, 30, [50, 50]),
                    (33, 1, [100, 0]), (5, 8, []), (0, 4, [50])]:
        assert flk.select_count(T, W, p) == osel.select_count(T, W, p)
    L = flk.lib()
    arr = (ctypes.c_int32 * 1)(101)
    assert L.flk_select_count(10, 4, arr, 1) == -1
    assert L.flk_select_count(10, 0, arr, 0) == -1
    assert L.flk_select_count(10, 4, None, 1) == -1
    assert flk.select_workspace_bytes(32768, 2048) == 256
    assert flk.select_workspace_bytes(100000, 1) == (4 * 100001 + 255) // 256 * 256
    assert flk.select_workspace_bytes(0, 8) == 0


def test_select_rows_validation():
    L = flk.lib()
    T, d, W = 100, 64, 16
    ws = flk.select_workspace_bytes(T, W)
    H2 = ctypes.c_void_p((1 << 21))

    def call(h1=FAKE, h2=H2, T=T, d=d, rows=None, n_prev=T, W=W, pct=50, eps=1e-6, sc=FAKE, out=FAKE, n_out=56,
             w=FAKE, wb=ws):
        return L.flk_select_rows(h1, h2, T, d, rows, n_prev, W, pct, eps, sc, out, n_out, None, w, wb, None, None)
    assert call(h1=None) == 1
    assert call(out=None) == 1
    assert call(sc=None) == 1                            # 0 < pct < 100 writes scores
    assert call(T=0) == 2
    assert call(d=12) == 2
    assert call(d=16392) == 2
    assert call(n_prev=50) == 2                          # dense needs n_prev == T
    assert call(rows=FAKE, n_prev=T + 1) == 2
    assert call(W=0) == 2
    assert call(pct=101) == 2
    assert call(pct=-1) == 2
    assert call(n_out=T + 1) == 2
    assert call(eps=0.0) == 2
    assert call(eps=float("inf")) == 2
    assert call(h2=FAKE) == 2                            # the two hidden states alias
    assert call(h1=ctypes.c_void_p((1 << 20) + 8)) == 3
    assert call(rows=ctypes.c_void_p((1 << 20) + 2), n_prev=50, n_out=25) == 3
    assert call(wb=ws - 4) == 6
    assert call(w=None) == 6
    assert call(w=ctypes.c_void_p((1 << 20) + 2)) == 3


def test_partition_rows_validation():
    L = flk.lib()

    def call(cls=FAKE, n=10, g=FAKE, s=FAKE, c=FAKE):
        return L.flk_partition_rows(cls, n, g, s, c, None, None)
    assert call(c=None) == 1
    assert call(cls=None) == 1
    assert call(g=None) == 1
    assert call(n=-1) == 2
    assert call(g=ctypes.c_void_p((1 << 20) + 2)) == 3


def test_nvfp4_descriptor_sizes_and_unsupported_entry_points():
    L = flk.lib()
    d = flk.desc(flk.K, 8, 128, nvfp4=True)
    assert L.flk_desc_check(ctypes.byref(d)) == 0
    assert (d.format, d.group, d.param_dtype, d.k_grouping) == (2, 16, 2, 0)
    assert flk.codes_bytes(flk.K, 8, 128, 100) == 100 * 8 * 64
    assert flk.params_bytes(flk.K, 8, 128, 100, nvfp4=True) == 16 + 100 * 8 * 8
    assert flk.stream_bytes(flk.V, 8, 128, 100, 1000, True, nvfp4=True) == \
        100 * 8 * 64 + 16 + 100 * 64 + 400 + flk.tile_index_bytes(1000)
    bad = flk.desc(flk.K, 8, 120, nvfp4=True)           # D % 16 != 0
    assert L.flk_desc_check(ctypes.byref(bad)) == 2
    tiles = flk.desc(flk.K, 8, 128, nvfp4=True)
    tiles.k_grouping = 1                                  # NVFP4 has no tile groups
    assert L.flk_desc_check(ctypes.byref(tiles)) == 4
    mixed = flk.desc(flk.K, 8, 128)
    mixed.group = 16                                      # INT4 with an NVFP4 block size
    assert L.flk_desc_check(ctypes.byref(mixed)) == 4
    # INT4-only entry points answer "unsupported" for a well-formed NVFP4 descriptor
    vd = flk.desc(flk.V, 8, 128)
    S = flk.StreamC
    chain = (S * 1)(S(256, 0, None, FAKE.value, FAKE.value, None))
    assert L.flk_decode_attn_packed(ctypes.byref(d), ctypes.byref(vd), 256, FAKE, 32, chain, chain, 1, 0.088, FAKE,
                                    FAKE, 1 << 24, None) == 5
    assert L.flk_attn_workspace_bytes(ctypes.byref(d), 256, 32) == 0
    assert L.flk_sparse_workspace_bytes(ctypes.byref(d), 256, 32, 16, 1) == 0


def test_mxfp4_descriptor_and_sizes():
    L = flk.lib()
    d = flk.desc(flk.K, 8, 128, fmt="mxfp4")
    assert L.flk_desc_check(ctypes.byref(d)) == 0
    assert (d.format, d.group, d.param_dtype, d.k_grouping) == (3, 32, 3, 0)
    assert flk.params_bytes(flk.K, 8, 128, 100, fmt="mxfp4") == 100 * 8 * 4     # one byte per 32 elements
    assert flk.stream_bytes(flk.V, 8, 128, 100, 1000, True, fmt="mxfp4") == \
        100 * 8 * 64 + 100 * 8 * 4 + 400 + flk.tile_index_bytes(1000)
    assert L.flk_desc_check(ctypes.byref(flk.desc(flk.K, 8, 48, fmt="mxfp4"))) == 2    # D % 32 != 0
    assert L.flk_desc_check(ctypes.byref(flk.desc(flk.K, 8, 48, fmt="nvfp4"))) == 0    # NVFP4 needs D % 16
    tiles = flk.desc(flk.K, 8, 128, fmt="mxfp4")
    tiles.k_grouping = 1
    assert L.flk_desc_check(ctypes.byref(tiles)) == 4
    wrong = flk.desc(flk.K, 8, 128, fmt="mxfp4")
    wrong.param_dtype = 2                                 # MXFP4 blocks with NVFP4 scales
    assert L.flk_desc_check(ctypes.byref(wrong)) == 4
    with pytest.raises(ValueError):
        flk.desc(flk.K, 8, 128, nvfp4=True, fmt="mxfp4")
    assert L.flk_attn_workspace_bytes(ctypes.byref(d), 256, 32) == 0


def test_reconstruct_mixed_validation():
    L = flk.lib()
    S = flk.StreamC
    T = 256
    base = S(T, 0, None, FAKE.value, FAKE.value, None)
    chain = (S * 2)(base, S(T, 0, None, FAKE.value, FAKE.value, None))
    i4, f4 = flk.desc(flk.K, 8, 128), flk.desc(flk.K, 8, 128, nvfp4=True)
    f4v, f4h = flk.desc(flk.V, 8, 128, nvfp4=True), flk.desc(flk.K, 4, 128, nvfp4=True)

    def call(bd, rd, out=FAKE, n=2, T=T):
        return L.flk_reconstruct_mixed(ctypes.byref(bd), ctypes.byref(rd), T, chain, n, out, None)
    assert call(i4, f4v) == 4                             # kinds disagree
    assert call(i4, f4h) == 4                             # head counts disagree
    assert call(f4, i4) == 5                              # NVFP4 base, INT4 residuals
    mx = flk.desc(flk.K, 8, 128, fmt="mxfp4")
    assert call(f4, mx) == 5 and call(mx, f4) == 5        # NVFP4 mixed with MXFP4
    assert call(i4, f4, out=None) == 1
    assert call(i4, f4, T=0) == 2
    assert call(i4, f4, n=0) == 2
    assert call(i4, f4, out=MIS) == 3


def test_decode_attn_mixed_validation():
    L = flk.lib()
    S = flk.StreamC
    T = 256
    chain = (S * 2)(S(T, 0, None, FAKE.value, FAKE.value, None), S(T, 0, None, FAKE.value, FAKE.value, None))
    ki4, kf4 = flk.desc(flk.K, 8, 128), flk.desc(flk.K, 8, 128, nvfp4=True)
    vi4, vf4 = flk.desc(flk.V, 8, 128), flk.desc(flk.V, 8, 128, nvfp4=True)
    ws = flk.attn_workspace_bytes(8, 128, T, 32)

    def call(kb, kr, vb, vr, q=FAKE, hq=32, wb=ws):
        return L.flk_decode_attn_mixed(ctypes.byref(kb), ctypes.byref(kr), ctypes.byref(vb), ctypes.byref(vr), T, q,
                                       hq, chain, chain, 2, 0.088, FAKE, FAKE, wb, None)
    assert call(vi4, kf4, vi4, vf4) == 4                        # a V descriptor for K
    assert call(ki4, kf4, vi4, vi4) == 5                        # K and V formats differ
    assert call(kf4, ki4, vf4, vi4) == 5                        # NVFP4 base, INT4 residuals
    assert call(ki4, kf4, vi4, vf4, q=None) == 1
    assert call(ki4, kf4, vi4, vf4, hq=30) == 2
    assert call(ki4, kf4, vi4, vf4, wb=64) == 6
    kt = flk.desc(flk.K, 8, 128, k_tiles=True)
    assert call(kt, kf4, vi4, vf4) == 5                         # tile-grouped K with NVFP4 residuals
    kmx, vmx = flk.desc(flk.K, 8, 128, fmt="mxfp4"), flk.desc(flk.V, 8, 128, fmt="mxfp4")
    assert call(kf4, kmx, vf4, vmx) == 5                        # NVFP4 base, MXFP4 residuals
    assert call(ki4, kmx, vi4, vf4) == 5                        # K MXFP4, V NVFP4 residuals
    assert call(ki4, kmx, vi4, vmx, hq=30) == 2                 # a valid combination reaches the shape checks


def test_largest_tensor_bound():
    """T*H*D must stay below 2^31 elements (4 GiB of BF16, the kernels' 32-bit byte offsets):
    one position past the largest accepted T is rejected before anything is launched."""
    L = flk.lib()
    H, D = 8, 128
    T = (1 << 31) // (H * D)                 # 2,097,152: T*H*D == 2^31
    for kind in (flk.K, flk.V):
        d = flk.desc(kind, H, D)
        assert L.flk_encode_base(ctypes.byref(d), FAKE, T, FAKE, FAKE, FAKE, None, None) == 2
        assert L.flk_encode_residual(ctypes.byref(d), FAKE, None, T, T, FAKE, FAKE, FAKE, None, None, None) == 2
        chain = (flk.StreamC * 1)(flk.StreamC(T, 0, None, FAKE.value, FAKE.value, None))
        assert L.flk_reconstruct(ctypes.byref(d), T, chain, 1, FAKE, None) == 2


def test_sparse_mixed_validation():
    """The sparse *_mixed calls resolve formats as flk_decode_attn_mixed does, then apply the
    INT4 calls' checks; the INT4 calls still refuse FP4 descriptors."""
    L = flk.lib()
    S = flk.StreamC
    T, Hq, k = 256, 32, 16
    chain = (S * 2)(S(T, 0, None, FAKE.value, FAKE.value, None), S(T, 0, None, FAKE.value, FAKE.value, None))
    ki4, kf4, kmx = (flk.desc(flk.K, 8, 128, fmt=f) for f in ("int4", "nvfp4", "mxfp4"))
    vi4, vf4, vmx = (flk.desc(flk.V, 8, 128, fmt=f) for f in ("int4", "nvfp4", "mxfp4"))
    ws = flk.sparse_workspace_bytes(8, 128, T, Hq, k, 2)

    def ref(kb, kr, vb, vr, q=FAKE, kk=k, wb=ws):
        return L.flk_sparse_attn_reference_mixed(ctypes.byref(kb), ctypes.byref(kr), ctypes.byref(vb),
                                                 ctypes.byref(vr), T, q, Hq, chain, chain, 2, kk, 0.088, FAKE,
                                                 FAKE, FAKE, FAKE, FAKE, FAKE, wb, None)

    def loop(kb, kr, vb, vr, q=FAKE):
        return L.flk_sparse_attn_loop_mixed(ctypes.byref(kb), ctypes.byref(kr), ctypes.byref(vb), ctypes.byref(vr),
                                            T, q, Hq, chain, chain, 2, k, 0.088, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            ws, None)
    assert ref(vi4, kf4, vi4, vf4) == 4                   # a V descriptor for K
    assert ref(kf4, kmx, vf4, vmx) == 5                   # NVFP4 base, MXFP4 residuals
    assert ref(ki4, kf4, vi4, vmx) == 5                   # K and V formats differ
    assert ref(kf4, ki4, vf4, vi4) == 5                   # FP4 base, INT4 residuals
    assert ref(ki4, kf4, vi4, vf4, q=None) == 1
    assert ref(ki4, kmx, vi4, vmx, kk=0) == 2
    assert ref(ki4, kmx, vi4, vmx, wb=64) == 6
    assert loop(ki4, kf4, vi4, vf4, q=None) == 1
    assert loop(kf4, kmx, vf4, vmx) == 5
    kt = flk.desc(flk.K, 8, 128, k_tiles=True)
    assert ref(kt, kf4, vi4, vf4) == 5                    # tile-grouped K with FP4 residuals
    # the INT4-only calls refuse FP4 descriptors
    assert L.flk_sparse_attn_reference(ctypes.byref(kf4), ctypes.byref(vi4), T, FAKE, Hq, chain, chain, 2, k, 0.088,
                                       FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 5
