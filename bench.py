"""Benchmark: packed-KV encode + reconstruct throughput of a 4-loop residual chain on one GPU.

Workload (long prompt layer): one request/layer, K and V each [T=32768, H=8, D=128] BF16,
4 loops with retention budgets 100/100/50/25% (loops 3 and 4 compact-sparse over nested
active sets), K Student-t(3) with per-channel multipliers, V N(0,1), loop deltas N(0,0.05).

One step = for K and for V: encode the base, encode the residuals of loops 2..4, rebuild the
final depth.  By default the single calls run with the K chain and the V chain on two streams
(flk_encode_base, flk_encode_residual x 3, flk_reconstruct each; the chains are independent,
so one chain's next loop overlaps the other's ramp and drain); --mode batched issues one
batched call per loop covering both tensors (flk_encode_base_batch, flk_encode_residual_batch
x 3, flk_reconstruct_batch) on one stream, and --mode serial the single calls on one stream.
The timed region holds the steps alone: events around single launches cost about 9 us per step
(each event record drains its stream and writes back the L2), so the per-launch events of the
overlapped step run on min(10, steps) further steps after it.  Then every call is also timed
alone (one stream, nothing overlapping) and reported per call, with the dominant kernel's
roofline at that isolated duration.  `value` = algorithmic bytes of the step (each input read once, each output
written once) / wall time per step, inputs already resident in HBM.  Steps rotate over
several independent buffer sets (> 1 GB in total) so the 256 MB MALL holds no timed data.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import math
import os
import sys
import time
from types import SimpleNamespace

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from quantized_kv_cache_amd import flk, synth  # noqa: E402

METRIC = "packed-KV encode+reconstruct GB/s and % of HBM peak, 4-loop residual chain"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- bytes

def stream_bytes(kind, H, D, n, T, sparse, k_tiles=False):
    return flk.codes_bytes(kind, H, D, n) + flk.params_bytes(kind, H, D, n, T, k_tiles) + flk.rows_bytes(n, sparse)


def call_bytes(kind, H, D, T, rows_list, k_tiles=False):
    """Algorithmic bytes of each call of one tensor's chain, in launch order.  With tile
    (page-local) K groups a compact loop's params are one row per tile."""
    e = 2  # BF16
    W = H * D
    # base: read X, write codes + params, write recon
    out = [("base", e * T * W + flk.codes_bytes(kind, H, D, T) + flk.params_bytes(kind, H, D, T, T, k_tiles)
            + e * T * W)]
    for rows in rows_list[1:]:
        n = T if rows is None else len(rows)
        sparse = rows is not None
        # read X_r rows, read recon at rows, write codes + params, write recon at rows, read rows
        b = e * n * W + e * n * W + flk.codes_bytes(kind, H, D, n) + flk.params_bytes(kind, H, D, n, T, k_tiles) \
            + e * n * W + flk.rows_bytes(n, sparse)
        out.append(("dense_residual" if not sparse else "sparse_residual", b))
    rec = sum(stream_bytes(kind, H, D, T if r is None else len(r), T, r is not None, k_tiles) for r in rows_list) \
        + e * T * W
    out.append(("reconstruct", rec))
    return out


KV = -1    # a batched call covering the K and the V tensor


def batched_symbol(call, rows_list):
    """Kernel a batched call launches for the long-prompt shapes (K and V both take the batched
    kernels there); mirrors csrc/flk_encode.hip and csrc/flk_reconstruct.hip."""
    if call == "reconstruct":
        n_loops = len(rows_list)
        if n_loops <= 4:
            mask = sum(1 << l for l, r in enumerate(rows_list) if r is not None)
            return f"reconstruct_batch_kernel<{n_loops}, {mask}u, false>"
        return f"reconstruct_batch_kernel<{n_loops}, 0u, true>"
    return f"encode_batch_kernel<{str(call != 'base').lower()}, {str(call == 'sparse_residual').lower()}>"


def kernel_symbol(kind, call, H, D, rows_list):
    """Name of the kernel (as the profiler prints it, without namespace and arguments) that the
    library launches for one call; mirrors the routing in csrc/flk_encode.hip and
    csrc/flk_reconstruct.hip."""
    W = H * D
    if call == "reconstruct":
        n_loops = len(rows_list)
        if W // 8 >= 64:
            if n_loops <= 4:
                mask = sum(1 << l for l, r in enumerate(rows_list) if r is not None)
                return f"reconstruct_wide_kernel<{kind}, {n_loops}, {mask}u, false>"
            return f"reconstruct_wide_kernel<{kind}, {n_loops}, 0u, true>"
        return f"reconstruct_kernel<{kind}, {n_loops}>"
    resid = str(call != "base").lower()
    sparse = str(call == "sparse_residual").lower()
    if kind == flk.K:
        return f"encode_k_kernel<{resid}, {sparse}>"
    if D % 64 == 0 and W % 1024 == 0:
        return f"encode_v_wide_kernel<{resid}, {sparse}>"
    cph = D // 8
    lph = 8 if cph <= 8 else 16 if cph <= 16 else 32 if cph <= 32 else 64
    return f"encode_v_kernel<{resid}, {sparse}, {lph}>"


# ----------------------------------------------------------------------------- device state

class ChainSet:
    """One independent set of device buffers for the K and V chains."""

    def __init__(self, w, host, sets, batched=True, k_tiles=False):
        self.tensors = []
        self.batched = batched
        self.k_tiles = k_tiles
        H, D, T = w.H, w.D, w.T
        for kind in (flk.K, flk.V):
            xs = [torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) for x in host[kind].xs]
            rows = [None if r is None else torch.from_numpy(r).cuda() for r in sets]
            recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
            out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
            packed = [flk.Packed.empty(kind, H, D, x.shape[0], r, T=T, k_tiles=k_tiles) for x, r in zip(xs, rows)]
            self.tensors.append((kind, xs, rows, recon, out, packed))
        self._prepare(w)

    def _prepare(self, w):
        """Marshal every call's arguments once, so a step only issues the C calls.  Batched:
        one call per loop (and one reconstruct) covers K and V; else one call per tensor."""
        L = flk.lib()
        self.calls = []     # (name, kind or KV, fn, args)
        self._keep = []
        P = ctypes.c_void_p
        if self.batched:
            kd, vd = flk.desc(flk.K, w.H, w.D, self.k_tiles), flk.desc(flk.V, w.H, w.D)
            self._keep += [kd, vd]
            n_loops = len(self.tensors[0][1])
            for l in range(n_loops):
                units = []
                for kind, xs, rows, recon, out, packed in self.tensors:
                    r = rows[l]
                    units.append(flk.UnitC(xs[l].data_ptr(), None if r is None else r.data_ptr(), recon.data_ptr(),
                                           packed[l].codes.data_ptr(), packed[l].params.data_ptr(),
                                           None if r is None else packed[l].tile_start.data_ptr(),
                                           xs[l].shape[0], w.T, kind, 0))
                arr = (flk.UnitC * len(units))(*units)
                self._keep.append(arr)
                name = "base" if l == 0 else ("sparse_residual" if rows[l] is not None else "dense_residual")
                fn = L.flk_encode_base_batch if l == 0 else L.flk_encode_residual_batch
                self.calls.append((name, KV, fn, (ctypes.byref(kd), ctypes.byref(vd), arr, len(units), None)))
            runits = []
            for kind, xs, rows, recon, out, packed in self.tensors:
                chain = (flk.StreamC * len(packed))(*[p.c() for p in packed])
                self._keep.append(chain)
                runits.append(flk.ReconUnitC(ctypes.cast(chain, ctypes.POINTER(flk.StreamC)), out.data_ptr(), w.T,
                                             len(packed), kind, 0))
            rarr = (flk.ReconUnitC * len(runits))(*runits)
            self._keep.append(rarr)
            self.calls.append(("reconstruct", KV, L.flk_reconstruct_batch,
                               (ctypes.byref(kd), ctypes.byref(vd), rarr, len(runits))))
            return
        for kind, xs, rows, recon, out, packed in self.tensors:
            d = flk.desc(kind, w.H, w.D, self.k_tiles)
            self._keep.append(d)
            dp = ctypes.byref(d)
            self.calls.append(("base", kind, L.flk_encode_base,
                               (dp, P(xs[0].data_ptr()), w.T, P(packed[0].codes.data_ptr()),
                                P(packed[0].params.data_ptr()), P(recon.data_ptr()), None)))
            for l in range(1, len(xs)):
                r = rows[l]
                self.calls.append(("sparse_residual" if r is not None else "dense_residual", kind,
                                   L.flk_encode_residual,
                                   (dp, P(xs[l].data_ptr()), None if r is None else P(r.data_ptr()),
                                    xs[l].shape[0], w.T, P(recon.data_ptr()), P(packed[l].codes.data_ptr()),
                                    P(packed[l].params.data_ptr()),
                                    None if r is None else P(packed[l].tile_start.data_ptr()), None)))
            arr = (flk.StreamC * len(packed))(*[p.c() for p in packed])
            self._keep.append(arr)
            self.calls.append(("reconstruct", kind, L.flk_reconstruct,
                               (dp, w.T, arr, len(packed), P(out.data_ptr()))))

    def call(self, i, stream_ptr):
        """Issue call i alone on the stream stream_ptr."""
        name, _, fn, args = self.calls[i]
        st = fn(*args, stream_ptr)
        if st != 0:
            raise flk.FlkError(st, name)

    def run(self, streams, ev=None):
        """Issue one step: every call on the stream of its tensor (streams[kind]); ev[i], when
        given, is a pair of events recorded around call i on that same stream."""
        for i, (name, kind, fn, args) in enumerate(self.calls):
            ts, sp = streams[flk.K if kind == KV else kind]
            if ev is not None and ev[i] is not None:
                ev[i][0].record(ts)
            st = fn(*args, sp)
            if st != 0:
                raise flk.FlkError(st, name)
            if ev is not None and ev[i] is not None:
                ev[i][1].record(ts)


# ----------------------------------------------------------------------------- page-local K groups

def page_local_leg(w, host, sets, streams, steps, warmup, rotate):
    """The same step with tile (page-local) K groups: every K group owns the compact rows of one
    64-position tile, so a page's metadata never mixes with distant positions.  Same timing
    procedure as the headline (continuous warmup, then `steps` steps between synchronizations);
    its bytes count one K parameter row per tile for the compact loops.  Also each K call timed
    alone."""
    cs = [ChainSet(w, host, sets, batched=False, k_tiles=True) for _ in range(rotate)]
    per_call = []
    for kind in (flk.K, flk.V):
        per_call += [(kind, name, b) for name, b in call_bytes(kind, w.H, w.D, w.T, sets, k_tiles=kind == flk.K)]
    step_bytes = sum(b for _, _, b in per_call)
    torch.cuda.synchronize()
    for i in range(warmup):
        cs[i % rotate].run(streams)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        cs[k % rotate].run(streams)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    iso_us = isolated_calls(cs, 10)
    k_calls = [{"call": name, "bytes": int(b), "us": round(float(t), 2), "gbs": round(b / t / 1e3, 1)}
               for (kind, name, b), t in zip(per_call, iso_us) if kind == flk.K]
    rows_k = call_bytes(flk.K, w.H, w.D, w.T, sets)
    return {"k_grouping": "tile", "value": round(step_bytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 4), "hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "step_bytes": int(step_bytes), "steps": steps, "warmup": warmup,
            "extra_param_bytes_vs_rows": int(sum(b for _, b in call_bytes(flk.K, w.H, w.D, w.T, sets, True))
                                             - sum(b for _, b in rows_k)),
            "k_calls_isolated": k_calls}


def isolated_calls(chain_sets, reps):
    """Duration (us) of every call of a step run alone: per call, `reps` launches back to back on
    one stream (rotating over the buffer sets, so the MALL holds none of a launch's inputs), one
    pair of events around them, the mean per launch.  A spin kernel queued first keeps the GPU
    busy while the host issues the launches, so the events see no issue latency, and one event
    pair per `reps` launches keeps the events' own cost (a cache flush each) out of the figure."""
    iso_stream = torch.cuda.Stream()
    sp = ctypes.c_void_p(iso_stream.cuda_stream)
    n_calls = len(chain_sets[0].calls)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_calls)]
    for i in range(n_calls):
        with torch.cuda.stream(iso_stream):
            torch.cuda._sleep(ISO_SPIN_CYCLES)
        ev[i][0].record(iso_stream)
        for r in range(reps):
            chain_sets[r % len(chain_sets)].call(i, sp)
        ev[i][1].record(iso_stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev]) * 1e3 / reps


ISO_SPIN_CYCLES = 5_000_000       # about 2 ms at the shader clock: longer than the host's issue of the launches
OVERLAP_STEPS = 10                # steps after the timed region that carry per-launch events


# ----------------------------------------------------------------------------- cpu baseline

def host_threads():
    """Worker threads for the host baseline: the process's CPU share (OMP_NUM_THREADS where the
    environment sets it), never more than the CPUs the process may run on."""
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", avail))
    except ValueError:
        share = avail
    return max(1, min(avail, share))


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_unit(kind, h, host, sets, w):
    """The oracle's 4-loop chain + reconstruct of one KV head of one tensor (one independent unit:
    K groups run within a head's channels, V groups within a head's row); returns its bytes."""
    from oracle import oracle as orc
    xs = [np.ascontiguousarray(x[:, h:h + 1]) for x in host[kind].xs]
    chain, recon = orc.encode_chain(kind, xs, sets)
    out = orc.reconstruct(kind, chain, w.T, 1, w.D)
    assert np.array_equal(out, recon)
    return sum(b for _, b in call_bytes(kind, 1, w.D, w.T, sets))


def cpu_baseline(w, host, sets):
    """Time the oracle (as it stands) on the host: the whole long-prompt step (every KV head of K
    and V, full T) on a thread pool over the 2 x H independent (tensor, head) units -- the C
    oracle releases the interpreter lock -- and, single-threaded, the units of KV head 0."""
    from concurrent.futures import ThreadPoolExecutor
    units = [(kind, h) for kind in (flk.K, flk.V) for h in range(w.H)]
    n_threads = min(host_threads(), len(units))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n_threads) as ex:
        total = sum(ex.map(lambda u: _oracle_unit(u[0], u[1], host, sets, w), units))
    dt = time.perf_counter() - t0
    t1 = time.perf_counter()
    one = sum(_oracle_unit(kind, 0, host, sets, w) for kind in (flk.K, flk.V))
    dt1 = time.perf_counter() - t1
    return {"value": round(total / dt / 1e9, 4), "unit": "GB/s", "cores": n_threads, "kind": "oracle",
            "sample": f"the whole step (K and V, all {w.H} KV heads, T={w.T}, 4-loop chain + reconstruct) as "
                      f"{len(units)} (tensor, head) units on {n_threads} threads: {dt:.2f} s wall",
            "single_thread": {"value": round(one / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"KV head 0 of K and V (1/{w.H} of the step): {dt1:.2f} s"},
            "host": {"cpu_model": host_cpu_model(), "nproc": os.cpu_count(),
                     "threads_allowed": host_threads()},
            "rows": cpu_baseline_rows(w, host, sets)}


def cpu_baseline_rows(w, host, sets):
    """The oracle (as it stands, single thread) on bounded samples of the other legs' workloads,
    each in the unit its leg reports."""
    from oracle import fp4 as ofp4
    from oracle import oracle as orc
    from oracle import selection as osel
    rows = {}
    # token selection: loop 3 (50 %) over the first two windows (4096 tokens, d = 4096)
    T_s, d, W = 4096, 4096, 2048
    hs = synth.hidden_states(T_s, d, 2)
    t0 = time.perf_counter()
    osel.select_rows(hs[1], hs[0], None, W, 50, 1e-6)
    dt = time.perf_counter() - t0
    b = 2 * T_s * d * 2 + 4 * T_s
    rows["token_selection"] = {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "sample": f"loop 3 over windows 0-1 ({T_s} of 32768 tokens, d={d}): {dt:.2f} s"}
    # NVFP4: the long-prompt K chain of KV head 0 (1/8 of the tensor), encode + reconstruct
    xs = [np.ascontiguousarray(x[:, 0:1]) for x in host[flk.K].xs]
    t0 = time.perf_counter()
    _, recon = ofp4.encode_base(xs[0])
    base = recon.copy()
    streams = [ofp4.encode_residual(x, r, recon) for x, r in zip(xs[1:], sets[1:])]
    ofp4.apply_residuals(base, streams)
    dt = time.perf_counter() - t0
    b, _ = _format_bytes(flk.K, SimpleNamespace(H=1, D=w.D, T=w.T), sets, "nvfp4", "nvfp4")
    rows["nvfp4"] = {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                     "sample": f"K chain of KV head 0 (1/{w.H} of the tensor), 4 loops + reconstruct: {dt:.2f} s"}
    t0 = time.perf_counter()
    _, recon = ofp4.encode_base(xs[0], mx=True)
    base = recon.copy()
    streams = [ofp4.encode_residual(x, r, recon, mx=True) for x, r in zip(xs[1:], sets[1:])]
    ofp4.apply_residuals(base, streams)
    dt = time.perf_counter() - t0
    b, _ = _format_bytes(flk.K, SimpleNamespace(H=1, D=w.D, T=w.T), sets, "mxfp4", "mxfp4")
    rows["mxfp4"] = {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                     "sample": f"K chain of KV head 0 (1/{w.H} of the tensor), 4 loops + reconstruct: {dt:.2f} s"}
    # sparse decode attention: the reference and one later loop for the 4 query heads of one KV
    # head over 131072 tokens (BF16 K/V drawn like the decode workload's), k = 4096
    wd = synth.WORKLOADS[5]
    g = synth.rng(wd.wid, 0, 0, 0, 0, synth.P_VALUES)
    kh = synth.to_bf16_bits(g.standard_normal((wd.T, 1, wd.D), dtype=np.float32))
    vh = synth.to_bf16_bits(g.standard_normal((wd.T, 1, wd.D), dtype=np.float32))
    q = synth.to_bf16_bits(g.standard_normal((wd.Hq // wd.H, wd.D), dtype=np.float32))
    t0 = time.perf_counter()
    ref = orc.sparse_reference(q, kh, vh, 1.0 / math.sqrt(wd.D), 4096)
    t1 = time.perf_counter()
    orc.sparse_loop(q, kh, vh, 1.0 / math.sqrt(wd.D), ref)
    t2 = time.perf_counter()
    rows["sparse_attention"] = {"value": round((t1 - t0) * 1e6 * wd.H, 1), "unit": "us per reference call",
                                "loop_us": round((t2 - t1) * 1e6 * wd.H, 1), "cores": 1,
                                "sample": f"1 of {wd.H} KV heads ({wd.Hq // wd.H} query heads), T={wd.T}, k=4096, "
                                          f"scaled by {wd.H}: reference {t1 - t0:.2f} s, loop {t2 - t1:.2f} s"}
    return rows


# ----------------------------------------------------------------------------- decode attention

def attention_leg(reps=20):
    """Time flk_decode_attn_packed, the chains' consumer, on the decode workload (T=131072,
    8 KV heads, 32 query heads, D=128, chains at 100/100/50/25%), with the chains encoded by
    the library from the seeded inputs.  Each timed call is preceded by a 512 MiB read so the
    MALL holds none of the packed chains; the figure is the median of `reps` calls."""
    w = synth.WORKLOADS[5]
    T, H, D, Hq = w.T, w.H, w.D, w.Hq
    sets = synth.active_sets(w, T)
    chains, packed_bytes = {}, 0
    for kind, tensor in ((flk.K, synth.K_TENSOR), (flk.V, synth.V_TENSOR)):
        c = synth.make_chain(w, tensor, sets=sets)
        recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
        packs = []
        for l, (x, r) in enumerate(zip(c.xs, c.rows)):
            xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
            rd = None if r is None else torch.from_numpy(r).cuda()
            p = flk.Packed.empty(kind, H, D, x.shape[0], rd, T=T)
            if l == 0:
                flk.encode_base(kind, xd, p, recon)
            else:
                flk.encode_residual(kind, xd, rd, recon, p)
            packs.append(p)
            packed_bytes += flk.codes_bytes(kind, H, D, p.n_rows) + flk.params_bytes(kind, H, D, p.n_rows)
        chains[kind] = packs
        del recon
    packed_bytes += sum(4 * len(r) for r in sets if r is not None)      # one rows array per loop
    q = torch.from_numpy(synth.make_query(w).view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(flk.attn_workspace_bytes(H, D, T, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(D)
    algo = packed_bytes + 2 * Hq * D * 2                                # + q read + out write
    for _ in range(3):
        flk.decode_attn_packed(q, chains[flk.K], chains[flk.V], T, H, scale, out, ws)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        flush.view(torch.int64).sum()                                  # clean MALL (see _timed_us)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flk.decode_attn_packed(q, chains[flk.K], chains[flk.V], T, H, scale, out, ws)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    us = float(np.median(times))
    fused = out.float().clone()
    # the same call back to back: a second copy of the chains at other addresses, calls
    # alternating between the two (each reads 0.4 GB, so the 256 MB MALL holds none of the next
    # call's chains), queued behind a spin kernel, one event pair around BACK_TO_BACK calls -- the
    # per-call event pairs and the flush above add their own cost to every call
    twin = {kind: [dataclasses.replace(p, rows=None if p.rows is None else p.rows.clone(), codes=p.codes.clone(),
                                       params=p.params.clone(),
                                       tile_start=None if p.tile_start is None else p.tile_start.clone())
                   for p in packs] for kind, packs in chains.items()}
    copies = [chains, twin]
    b2b_us = _back_to_back_us(
        lambda i: flk.decode_attn_packed(q, copies[i % 2][flk.K], copies[i % 2][flk.V], T, H, scale, out, ws))
    # the same attention the plain way: rebuild K_hat and V_hat in BF16 (flk_reconstruct), then
    # attend over the BF16 cache (the BF16-tail reader of flk_decode_attn_rolling, no packed part)
    kfull = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    vfull = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")

    def rta_call():
        flk.reconstruct(flk.K, chains[flk.K], kfull)
        flk.reconstruct(flk.V, chains[flk.V], vfull)
        flk.decode_attn_rolling(q, [], [], 0, H, kfull, vfull, scale, out2, ws)
    for _ in range(3):
        rta_call()
    torch.cuda.synchronize()
    rta_us = _timed_us(rta_call, reps, flush)

    def rta_call_i(i):
        flk.reconstruct(flk.K, copies[i % 2][flk.K], kfull)
        flk.reconstruct(flk.V, copies[i % 2][flk.V], vfull)
        flk.decode_attn_rolling(q, [], [], 0, H, kfull, vfull, scale, out2, ws)
    rta_b2b_us = _back_to_back_us(rta_call_i)
    del twin, copies
    o2 = out2.float()
    rta_diff = float(((fused - o2).abs().amax(dim=1) / o2.abs().amax(dim=1)).max())
    # bytes of that path: the packed chains read once, K_hat and V_hat written, then read back
    rta = packed_bytes + 4 * 2 * T * H * D + 2 * Hq * D * 2
    return {"workload": "decode_attn", "T": T, "Hkv": H, "Hq": Hq, "D": D, "loops": w.n_loops,
            "budgets_pct": list(w.budgets), "median_us": round(us, 2),
            "p10_us": round(float(np.percentile(times, 10)), 2), "p90_us": round(float(np.percentile(times, 90)), 2),
            "algorithmic_bytes": int(algo), "gbs": round(algo / us / 1e3, 1),
            "hbm_frac": round(algo / us / 1e3 / HBM_PEAK_GBS, 4),
            "reconstruct_then_attend_us": round(rta_us, 2), "reconstruct_then_attend_bytes": int(rta),
            "reconstruct_then_attend_gbs": round(rta / rta_us / 1e3, 1),
            "fused_speedup": round(rta_us / us, 3),
            "back_to_back_us": round(b2b_us, 2), "back_to_back_gbs": round(algo / b2b_us / 1e3, 1),
            "back_to_back_hbm_frac": round(algo / b2b_us / 1e3 / HBM_PEAK_GBS, 4),
            "reconstruct_then_attend_back_to_back_us": round(rta_b2b_us, 2),
            "back_to_back_timing": f"{BACK_TO_BACK} calls alternating two copies of the chains, queued behind a "
                                   "spin kernel, one event pair, mean per call",
            "fused_vs_reconstruct_max_rel_diff": round(rta_diff, 6)}


# ----------------------------------------------------------------------------- batched cache

def _student_t3(shape, g):
    """Student-t(3) draws on the device: N(0,1) / sqrt(chi2(3) / 3)."""
    z = torch.randn(shape, device="cuda", generator=g)
    c = (torch.randn(shape, device="cuda", generator=g) ** 2 + torch.randn(shape, device="cuda", generator=g) ** 2
         + torch.randn(shape, device="cuda", generator=g) ** 2) / 3.0
    return z / torch.sqrt(c)


def batched_cache_leg(layers=24, requests=64):
    """The batched cache: 64 requests with seeded lengths L ~ U{512..8192}, 16 KV heads, D = 128,
    4 loops at 100/100/50/25 % of each request's L (compact loops over nested seeded active sets,
    per request and layer), K and V of every (request, layer).  The library encodes one layer at
    a time -- the base of all 128 of the layer's tensors in one flk_encode_base_batch call, then
    one flk_encode_residual_batch call per loop -- and afterwards rebuilds every tensor of every
    layer with flk_reconstruct_batch, one call per layer.  `layers` of the 24 layers are run (the
    request lengths, and so every layer's shapes and bytes, are the same for all 24).  Inputs are
    drawn on the device per layer (K: Student-t(3) times a per-(head, channel) multiplier
    exp(U(ln 0.1, ln 10)); V: N(0,1); loop deltas N(0, 0.05)) outside the timed calls; each
    layer's calls are timed with events, after a 512 MiB read that evicts the MALL.  GB/s from
    the exact algorithmic bytes of the seeded lengths (each input read once, each output written
    once)."""
    w = synth.WORKLOADS[4]
    H, D = w.H, w.D
    lengths = [int(x) for x in synth.batched_lengths(requests)]
    L_tot = sum(lengths)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    g = torch.Generator(device="cuda")
    g.manual_seed(20261204)
    L = flk.lib()
    kd, vd = flk.desc(flk.K, H, D), flk.desc(flk.V, H, D)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    recon = {k: torch.empty((L_tot, H, D), dtype=torch.bfloat16, device="cuda") for k in (flk.K, flk.V)}
    outs = {k: torch.empty((L_tot, H, D), dtype=torch.bfloat16, device="cuda") for k in (flk.K, flk.V)}
    enc_bytes = rec_bytes = 0
    enc_us, rec_us = [], []
    streams = []                     # per layer: (kind, chain) per tensor, kept for the reconstruct
    keep = []
    for layer in range(layers):
        sets = [synth.active_sets(w, Lr, request=r, layer=layer) for r, Lr in enumerate(lengths)]
        # inputs of the layer: one trajectory per tensor over all requests' rows
        xs = {}
        for kind in (flk.K, flk.V):
            if kind == flk.K:
                mult = torch.exp(torch.empty((H, D), device="cuda").uniform_(math.log(0.1), math.log(10.0), generator=g))
                y = _student_t3((L_tot, H, D), g) * mult
            else:
                y = torch.randn((L_tot, H, D), device="cuda", generator=g)
            per_loop = []
            for loop in range(w.n_loops):
                if loop:
                    y.add_(torch.randn((L_tot, H, D), device="cuda", generator=g), alpha=w.sigma)
                xb = y.to(torch.bfloat16)
                if sets[0][loop] is None:
                    per_loop.append([xb[off[r]:off[r + 1]] for r in range(requests)])
                else:
                    per_loop.append([xb[off[r]:off[r + 1]][torch.from_numpy(sets[r][loop]).cuda().long()].contiguous()
                                     for r in range(requests)])
            xs[kind] = per_loop
            del y
        rows = [[None if sets[r][loop] is None else torch.from_numpy(sets[r][loop]).cuda()
                 for loop in range(w.n_loops)] for r in range(requests)]
        tables, layer_streams = [], []
        chains = {}
        for loop in range(w.n_loops):
            units = []
            for r, Lr in enumerate(lengths):
                for kind in (flk.K, flk.V):
                    rr = rows[r][loop]
                    n = Lr if rr is None else len(rr)
                    pk = flk.Packed.empty(kind, H, D, n, rr, T=Lr)
                    chains.setdefault((r, kind), []).append(pk)
                    rec = recon[kind][off[r]:off[r + 1]]
                    x = xs[kind][loop][r]
                    units.append(flk.UnitC(x.data_ptr(), None if rr is None else rr.data_ptr(), rec.data_ptr(),
                                           pk.codes.data_ptr(), pk.params.data_ptr(),
                                           None if rr is None else pk.tile_start.data_ptr(), n, Lr, kind, 0))
                    if loop == 0:
                        enc_bytes += 2 * Lr * H * D * 2 + flk.codes_bytes(kind, H, D, Lr) + \
                            flk.params_bytes(kind, H, D, Lr, Lr)
                    else:
                        enc_bytes += 3 * n * H * D * 2 + flk.codes_bytes(kind, H, D, n) + \
                            flk.params_bytes(kind, H, D, n, Lr) + flk.rows_bytes(n, rr is not None)
            tables.append((flk.UnitC * len(units))(*units))
        runits = []
        for r, Lr in enumerate(lengths):
            for kind in (flk.K, flk.V):
                ch = chains[(r, kind)]
                arr = (flk.StreamC * len(ch))(*[p.c() for p in ch])
                keep.append(arr)
                runits.append(flk.ReconUnitC(ctypes.cast(arr, ctypes.POINTER(flk.StreamC)),
                                             outs[kind][off[r]:off[r + 1]].data_ptr(), Lr, len(ch), kind, 0))
                rec_bytes += sum(flk.codes_bytes(kind, H, D, p.n_rows) + flk.params_bytes(kind, H, D, p.n_rows, Lr)
                                 + flk.rows_bytes(p.n_rows, p.rows is not None) for p in ch) + Lr * H * D * 2
        rtab = (flk.ReconUnitC * len(runits))(*runits)
        keep += [tables, rtab, rows, chains]
        streams.append(rtab)
        torch.cuda.synchronize()
        flush.view(torch.int64).sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        st = L.flk_encode_base_batch(ctypes.byref(kd), ctypes.byref(vd), tables[0], len(tables[0]), None, sp)
        for t in tables[1:]:
            st = st or L.flk_encode_residual_batch(ctypes.byref(kd), ctypes.byref(vd), t, len(t), None, sp)
        e1.record()
        torch.cuda.synchronize()
        if st != 0:
            raise flk.FlkError(st, "batched encode")
        enc_us.append(e0.elapsed_time(e1) * 1e3)
        del xs
    for layer, rtab in enumerate(streams):
        flush.view(torch.int64).sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        st = L.flk_reconstruct_batch(ctypes.byref(kd), ctypes.byref(vd), rtab, len(rtab), sp)
        e1.record()
        torch.cuda.synchronize()
        if st != 0:
            raise flk.FlkError(st, "batched reconstruct")
        rec_us.append(e0.elapsed_time(e1) * 1e3)
    enc_t, rec_t = sum(enc_us), sum(rec_us)
    res = {"workload": "batched_cache", "requests": requests, "layers_run": layers, "layers_config": 24,
           "H": H, "D": D, "tokens_per_layer": L_tot, "budgets_pct": list(w.budgets),
           "tensors_per_layer": 2 * requests,
           "encode": {"bytes": int(enc_bytes), "us": round(enc_t, 1), "gbs": round(enc_bytes / enc_t / 1e3, 1),
                      "hbm_frac": round(enc_bytes / enc_t / 1e3 / HBM_PEAK_GBS, 4),
                      "per_layer_us": [round(x, 1) for x in enc_us]},
           "reconstruct": {"bytes": int(rec_bytes), "us": round(rec_t, 1), "gbs": round(rec_bytes / rec_t / 1e3, 1),
                           "hbm_frac": round(rec_bytes / rec_t / 1e3 / HBM_PEAK_GBS, 4),
                           "per_layer_us": [round(x, 1) for x in rec_us]},
           "all_24_layers_estimate_s": round(24 * (enc_t + rec_t) / layers / 1e6, 3)}
    del keep, streams, recon, outs
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- rolling tail

BACK_TO_BACK = 20


def _back_to_back_us(fn_i, n=BACK_TO_BACK):
    """Mean duration (us) of fn_i(0) .. fn_i(n-1) issued back to back on the current stream
    behind a spin kernel (so the host's issue never shows), one event pair around them."""
    for i in range(2):
        fn_i(i)
    torch.cuda.synchronize()
    torch.cuda._sleep(ISO_SPIN_CYCLES)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn_i(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def _timed_us(fn, reps, flush=None):
    """Median of `reps` calls of fn (HIP events on the current stream); `flush`, when given, is
    read before each call so the MALL holds none of fn's data.  Reading leaves clean lines: a
    flush by writing would leave dirty lines whose write-back then falls inside fn's time."""
    times = []
    for _ in range(reps):
        if flush is not None:
            flush.view(torch.int64).sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(times))


def decode_chains(w, k_tiles):
    """The decode workload's K and V chains, encoded by the library from the seeded inputs."""
    T, H, D = w.T, w.H, w.D
    sets = synth.active_sets(w, T)
    chains = {}
    for kind, tensor in ((flk.K, synth.K_TENSOR), (flk.V, synth.V_TENSOR)):
        c = synth.make_chain(w, tensor, sets=sets)
        recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
        packs = []
        for l, (x, r) in enumerate(zip(c.xs, c.rows)):
            xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
            rd = None if r is None else torch.from_numpy(r).cuda()
            p = flk.Packed.empty(kind, H, D, x.shape[0], rd, T=T, k_tiles=k_tiles)
            if l == 0:
                flk.encode_base(kind, xd, p, recon)
            else:
                flk.encode_residual(kind, xd, rd, recon, p)
            packs.append(p)
        chains[kind] = packs
        del recon
    return chains


def sparse_leg(k=4096, reps=20):
    """Sparse decode attention (RFC section 3.2) on the decode workload (131072 packed tokens,
    8 KV heads, 32 query heads, D=128, chains at 100/100/50/25% with tile-grouped K), k keys
    per query head: the reference call at loop 2 (full attention writing the scores, the top-k
    selection, the selected keys' mass and C_ref), the loop calls at loops 3 and 4 (only the
    selected keys, read through the chains at depth 3 and 4), next to dense packed attention
    at the same depths.  Each call is timed with a cold MALL (a 512 MiB read before it)."""
    w = synth.WORKLOADS[5]
    T, H, D, Hq = w.T, w.H, w.D, w.Hq
    chains = decode_chains(w, k_tiles=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    qs = {d: torch.randn((Hq, D), device="cuda", generator=g).to(torch.bfloat16) for d in (2, 3, 4)}
    scale = 1.0 / math.sqrt(D)
    ws = torch.empty(max(flk.sparse_workspace_bytes(H, D, T, Hq, k, 4), flk.attn_workspace_bytes(H, D, T, Hq)) // 4
                     + 64, dtype=torch.float32, device="cuda")
    ws = ws[(-ws.data_ptr() // 4) % 64:]
    st = flk.SparseState.empty(Hq, D, k)
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    K, V = chains[flk.K], chains[flk.V]
    ref = lambda: flk.sparse_attn_reference(qs[2], K[:2], V[:2], T, H, k, scale, out, st, ws)
    loop = {d: (lambda d=d: flk.sparse_attn_loop(qs[d], K[:d], V[:d], T, H, k, scale, st, out, ws)) for d in (3, 4)}
    dense = {d: (lambda d=d: flk.decode_attn_packed(qs[d], K[:d], V[:d], T, H, scale, out, ws)) for d in (2, 3, 4)}
    for _ in range(3):
        ref()
        for d in (3, 4):
            loop[d]()
        for d in (2, 3, 4):
            dense[d]()
    torch.cuda.synchronize()
    res = {"workload": "decode_attn", "T": T, "Hkv": H, "Hq": Hq, "D": D, "k": k, "k_grouping": "tile",
           "reference_us": round(_timed_us(ref, reps, flush), 2)}
    for d in (3, 4):
        res[f"loop{d}_us"] = round(_timed_us(loop[d], reps, flush), 2)
    for d in (2, 3, 4):
        res[f"dense_depth{d}_us"] = round(_timed_us(dense[d], reps, flush), 2)
    res["sparse_loops_3_4_us"] = round(res["loop3_us"] + res["loop4_us"], 2)
    res["dense_loops_3_4_us"] = round(res["dense_depth3_us"] + res["dense_depth4_us"], 2)
    # bytes of a loop call: the packed rows of the selected keys only
    sel = st.sel.cpu().numpy()
    sets = synth.active_sets(w, T)
    for d in (3, 4):
        b = sparse_loop_bytes(sel, sets[:d], T, H, D, Hq)
        res[f"loop{d}_algorithmic_bytes"] = int(b)
        res[f"loop{d}_gbs"] = round(b / res[f"loop{d}_us"] / 1e3, 1)
        res[f"loop{d}_hbm_frac"] = round(b / res[f"loop{d}_us"] / 1e3 / HBM_PEAK_GBS, 4)
    return res


def sparse_loop_bytes(sel, sets, T, H, D, Hq):
    """Algorithmic bytes of a sparse loop call at depth len(sets) over tile-grouped K: per KV head,
    the union of its query heads' selected positions; per such position and loop that lists it,
    the K and V code rows (D/2 bytes each) and the V parameter row (4 bytes per 64 channels); per
    (loop, 64-position tile) holding such a position, the tile's K parameter row (4 bytes per
    channel); plus q, the reference state (mass, O_ref, C_ref), the selection and the output."""
    G = Hq // H
    total = 0
    for h in range(H):
        u = np.unique(sel[h * G:(h + 1) * G].ravel())
        u = u[(u >= 0) & (u < T)]
        for rows in sets:
            listed = u if rows is None else u[np.isin(u, rows)]
            total += len(listed) * (D // 2 + D // 2 + 4 * ((D + 63) // 64))
            total += len(np.unique(listed // 64)) * 4 * D
    total += Hq * D * 2 + Hq * (1 + 2 * D) * 4 + sel.size * 4 + Hq * D * 2
    return total


def selection_leg(reps=20):
    """Token selection for sparse prefill (RFC section 3.1) on the long prompt: T=32768 tokens,
    hidden width d=4096, selection windows of 2048 tokens; loop 3 keeps 50 % of a dense loop 2,
    loop 4 keeps 25 % of each window's length from loop 3's tokens.  The hidden states follow
    the recipe of synth.hidden_states, drawn on the GPU from a seeded generator.  A call reads
    the eligible rows of H[r-1] and H[r-2] once (512 MiB at loop 3, 256 MiB at loop 4) and
    writes the scores, the selected positions and the slot map."""
    T, d, W = 32768, 4096, 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(20261203)
    mag = torch.exp(torch.empty((T, 1), device="cuda").uniform_(math.log(0.5), math.log(2.0), generator=g))
    y = torch.randn((T, d), device="cuda", generator=g) * mag
    hs = [y.to(torch.bfloat16)]
    for _ in range(2):
        size = torch.exp(torch.empty((T, 1), device="cuda").uniform_(math.log(0.01), 0.0, generator=g))
        y = y + torch.randn((T, d), device="cuda", generator=g) * size
        hs.append(y.to(torch.bfloat16))
    del y, mag, size
    n3, n4 = flk.select_count(T, W, [50]), flk.select_count(T, W, [50, 25])
    i32 = dict(dtype=torch.int32, device="cuda")
    scores = torch.empty(T, dtype=torch.float32, device="cuda")
    rows3, rows4, slot = torch.empty(n3, **i32), torch.empty(n4, **i32), torch.empty(T, **i32)
    ws = torch.empty(flk.select_workspace_bytes(T, W) // 4, **i32)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    l3 = lambda: flk.select_rows(hs[1], hs[0], None, W, 50, 1e-6, scores, rows3, ws, slot)
    l4 = lambda: flk.select_rows(hs[2], hs[1], rows3, W, 25, 1e-6, scores, rows4, ws, slot)
    for _ in range(3):
        l3()
        l4()
    torch.cuda.synchronize()
    res = {"workload": "token_selection", "T": T, "d": d, "window": W, "budgets_pct": [50, 25]}
    # scoring reads both hidden rows (and the eligible list) and writes a score; the top-k
    # reads the scores (and the list), writes the positions and the slot map
    for name, fn, n_prev, n_out, compact in (("loop3", l3, T, n3, False), ("loop4", l4, n3, n4, True)):
        us = _timed_us(fn, reps, flush)
        b = 2 * n_prev * d * 2 + 4 * n_prev + 4 * n_prev + 4 * n_out + 4 * T + (8 * n_prev if compact else 0)
        res[f"{name}_us"] = round(us, 2)
        res[f"{name}_gbs"] = round(b / us / 1e3, 1)
        res[f"{name}_hbm_frac"] = round(b / us / 1e3 / HBM_PEAK_GBS, 4)
    return res


# The chain formats the FP4 leg compares: (name, base loop's format, residual loops' format).
CHAIN_FORMATS = (("int4", "int4", "int4"), ("nvfp4", "nvfp4", "nvfp4"), ("int4_base_nvfp4_residuals", "int4", "nvfp4"),
                 ("mxfp4", "mxfp4", "mxfp4"), ("int4_base_mxfp4_residuals", "int4", "mxfp4"))


def _format_calls(kind, w, xs, rows, recon, out, packed, base_fmt, resid_fmt):
    """Prepared C calls of one tensor's chain in a format: base, residual loops, reconstruct."""
    L = flk.lib()
    P = ctypes.c_void_p
    bd = flk.desc(kind, w.H, w.D, fmt=base_fmt)
    rd = flk.desc(kind, w.H, w.D, fmt=resid_fmt)
    keep = [bd, rd]
    calls = [(L.flk_encode_base, (ctypes.byref(bd), P(xs[0].data_ptr()), w.T, P(packed[0].codes.data_ptr()),
                                  P(packed[0].params.data_ptr()), P(recon.data_ptr()), None))]
    for l in range(1, len(xs)):
        r = rows[l]
        calls.append((L.flk_encode_residual,
                      (ctypes.byref(rd), P(xs[l].data_ptr()), None if r is None else P(r.data_ptr()), xs[l].shape[0],
                       w.T, P(recon.data_ptr()), P(packed[l].codes.data_ptr()), P(packed[l].params.data_ptr()),
                       None if r is None else P(packed[l].tile_start.data_ptr()), None)))
    arr = (flk.StreamC * len(packed))(*[p.c() for p in packed])
    keep.append(arr)
    calls.append((L.flk_reconstruct_mixed, (ctypes.byref(bd), ctypes.byref(rd), w.T, arr, len(packed),
                                            P(out.data_ptr()))))
    return calls, keep


def fp4_attention_times(flush, reps=20, k=4096):
    """The chains' consumers on the decode workload (131072 tokens, 8 KV heads, 32 query heads,
    chains of 4 loops at 100/100/50/25 %) in each format: fused decode attention at depth 4, and
    sparse decode attention with k keys per query head (the reference call at loop 2, the loop
    calls at depths 3 and 4).  Median microseconds per call, each after a 512 MiB read that
    evicts the MALL."""
    w = synth.WORKLOADS[5]
    T, H, D, Hq = w.T, w.H, w.D, w.Hq
    sets = synth.active_sets(w, T)
    host = {kind: synth.make_chain(w, tensor, sets=sets) for kind, tensor in ((flk.K, synth.K_TENSOR),
                                                                                (flk.V, synth.V_TENSOR))}
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    q = torch.randn((Hq, D), device="cuda", generator=g).to(torch.bfloat16)
    ws = torch.empty(max(flk.sparse_workspace_bytes(H, D, T, Hq, k, 4), flk.attn_workspace_bytes(H, D, T, Hq)) // 4
                     + 64, dtype=torch.float32, device="cuda")
    ws = ws[(-ws.data_ptr() // 4) % 64:]                         # 256-byte aligned
    st = flk.SparseState.empty(Hq, D, k)
    out = torch.empty((Hq, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    times = {}
    for name, base_fmt, resid_fmt in CHAIN_FORMATS:
        chains = {}
        for kind in (flk.K, flk.V):
            recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
            packs = []
            for l, (x, r) in enumerate(zip(host[kind].xs, host[kind].rows)):
                xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
                rd = None if r is None else torch.from_numpy(r).cuda()
                p = flk.Packed.empty(kind, H, D, x.shape[0], rd, T=T, fmt=base_fmt if l == 0 else resid_fmt)
                if l == 0:
                    flk.encode_base(kind, xd, p, recon)
                else:
                    flk.encode_residual(kind, xd, rd, recon, p)
                packs.append(p)
            chains[kind] = packs
            del recon
        Kc, Vc = chains[flk.K], chains[flk.V]
        fn = lambda: flk.decode_attn_mixed(q, Kc, Vc, T, H, scale, out, ws)
        ref = lambda: flk.sparse_attn_reference(q, Kc[:2], Vc[:2], T, H, k, scale, out, st, ws)
        loop = {d: (lambda d=d: flk.sparse_attn_loop(q, Kc[:d], Vc[:d], T, H, k, scale, st, out, ws)) for d in (3, 4)}
        for _ in range(3):
            fn()
            ref()
            loop[3]()
            loop[4]()
        torch.cuda.synchronize()
        times[name] = {"decode_attention_us": round(_timed_us(fn, reps, flush), 2),
                       "sparse_reference_us": round(_timed_us(ref, reps, flush), 2),
                       "sparse_loop3_us": round(_timed_us(loop[3], reps, flush), 2),
                       "sparse_loop4_us": round(_timed_us(loop[4], reps, flush), 2)}
        del chains, Kc, Vc
    return times


def _format_bytes(kind, w, sets, base_fmt, resid_fmt):
    """Algorithmic bytes of one tensor's chain (each input read once, each output written once);
    the stream-amax pass of an NVFP4 loop re-reads its input and is not counted."""
    H, D, T = w.H, w.D, w.T
    W = H * D

    def stream(n, fmt, sparse):
        return flk.stream_bytes(kind, H, D, n, T, sparse, fmt=fmt) - (flk.tile_index_bytes(T) if sparse else 0)
    b = 2 * T * W + stream(T, base_fmt, False) + 2 * T * W
    total_streams = stream(T, base_fmt, False)
    for r in sets[1:]:
        n = T if r is None else len(r)
        st = stream(n, resid_fmt, r is not None)
        b += 6 * n * W + st
        total_streams += st
    return b + total_streams + 2 * T * W, total_streams


def fp4_leg(w, host, sets, reps=30, rotate=2):
    """The FP4 variants (NVFP4, PR #166 review item 2; MXFP4, OCP MX v1.0) on the long prompt, K
    and V chains of 4 loops (100/100/50/25 %), against INT4 at about the same bits per element
    (4.5; MXFP4 4.25): INT4 throughout, NVFP4 or MXFP4 throughout, INT4 base + NVFP4 or MXFP4
    residuals.  Per format: the chain step (encode base, three
    residual encodes, reconstruct, for K and V; events around the step, `rotate` buffer sets),
    the stored bytes, and the accuracy of the depth-4 reconstruction X_hat against the BF16
    inputs: relative Frobenius error per tensor, and decode attention (32 query heads over the
    8 KV heads, binary32 on the GPU) from X_hat against attention from the inputs.  Also the
    fused decode attention's and the sparse decode attention's times per call on the decode
    workload in each format."""
    H, D, T = w.H, w.D, w.T
    dev = {}
    for kind in (flk.K, flk.V):
        xs = [torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) for x in host[kind].xs]
        rows = [None if r is None else torch.from_numpy(r).cuda() for r in sets]
        truth = xs[0].clone()                                  # the logical BF16 tensor after loop 4
        for x, r in zip(xs[1:], rows[1:]):
            if r is None:
                truth.copy_(x)
            else:
                truth[r.long()] = x
        dev[kind] = (xs, rows, truth)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    Hq = 32
    q = torch.randn((Hq, D), device="cuda", generator=g).to(torch.bfloat16).float()

    def attend(kt, vt):
        kf = kt.float().permute(1, 2, 0).contiguous()          # [H, D, T]
        vf = vt.float().permute(1, 0, 2).contiguous()          # [H, T, D]
        qh = q.view(H, Hq // H, D)
        p = torch.softmax(torch.bmm(qh, kf) / math.sqrt(D), dim=-1)
        return torch.bmm(p, vf).reshape(Hq, D)

    ref_out = attend(dev[flk.K][2], dev[flk.V][2])
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    attn_us = fp4_attention_times(flush)
    res = {"workload": "long_prompt", "T": T, "H": H, "D": D, "budgets_pct": list(w.budgets), "formats": {}}
    for name, base_fmt, resid_fmt in CHAIN_FORMATS:
        sets_dev, keep, outs = [], [], {}
        for _ in range(rotate):
            calls = []
            for kind in (flk.K, flk.V):
                xs, rows, _ = dev[kind]
                recon = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
                out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
                packed = [flk.Packed.empty(kind, H, D, x.shape[0], r, T=T, fmt=base_fmt if l == 0 else resid_fmt)
                          for l, (x, r) in enumerate(zip(xs, rows))]
                c, k = _format_calls(kind, w, xs, rows, recon, out, packed, base_fmt, resid_fmt)
                calls += c
                keep += [k, packed, recon, out]
                outs.setdefault(kind, out)
            sets_dev.append(calls)
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        def step(i):
            for fn, args in sets_dev[i % rotate]:
                st = fn(*args, sp)
                if st != 0:
                    raise flk.FlkError(st, name)
        for i in range(5):
            step(i)
        torch.cuda.synchronize()
        times = []
        for i in range(reps):
            flush.view(torch.int64).sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step(i)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        step(0)                                                # outs[] hold set 0's reconstruction
        torch.cuda.synchronize()
        us = float(np.median(times))
        b_k, s_k = _format_bytes(flk.K, w, sets, base_fmt, resid_fmt)
        b_v, s_v = _format_bytes(flk.V, w, sets, base_fmt, resid_fmt)
        acc = {}
        for kind, tag in ((flk.K, "k"), (flk.V, "v")):
            t = dev[kind][2].float()
            acc[f"{tag}_rel_fro_err"] = float((outs[kind].float() - t).norm() / t.norm())
        o = attend(outs[flk.K], outs[flk.V])
        rel = ((o - ref_out).abs().amax(dim=1) / ref_out.abs().amax(dim=1)).cpu().numpy()
        res["formats"][name] = {
            **attn_us[name],
            "step_us": round(us, 2), "step_bytes": int(b_k + b_v), "gbs": round((b_k + b_v) / us / 1e3, 1),
            "hbm_frac": round((b_k + b_v) / us / 1e3 / HBM_PEAK_GBS, 4),
            "stored_bytes": int(s_k + s_v),
            "bits_per_element": round(8 * (s_k + s_v) / (2 * sum((T if r is None else len(r)) for r in sets) * H * D), 4),
            **{k: round(v, 6) for k, v in acc.items()},
            "attn_rel_err_max": round(float(rel.max()), 6), "attn_rel_err_mean": round(float(rel.mean()), 6)}
        del sets_dev, keep, outs
    return res


def rolling_leg(reps=50):
    """The rolling BF16 tail (RFC section 3.3): decode tokens wait in BF16 until a whole
    64-token group can be flushed into the packed streams, whose K groups are tile-local.

    flush: one decode step's flush for a request of the batched-cache shape (24 layers, K and V,
    16 KV heads, D=128, 4 loops): the 64-position window [4096, 4160) appended to every
    layer's streams -- loops 1-2 dense, loops 3/4 over the window's tokens that ran that deep
    (seeded exit depths: a half reach loop 3, a quarter loop 4).  Timed as 4 batched calls
    (flk_append_base_batch + 3 x flk_append_residual_batch, 48 tensors each) and as 192
    one-tensor calls, back to back with the unit tables prepared once.  attention: flk_decode_attn_rolling over the decode workload's 131072 packed
    tokens (tile-grouped K) plus a 127-token BF16 tail, next to flk_decode_attn_packed over
    the same packed tokens alone."""
    out = {}
    H, D, layers, p0, win = 16, 128, 24, 4096, 64
    rng = np.random.default_rng(20261202)
    u = rng.random(win)
    depth = np.where(u < 0.25, 4, np.where(u < 0.5, 3, 2))
    rows_w = [None, None, (p0 + np.nonzero(depth >= 3)[0]).astype(np.int32),
              (p0 + np.nonzero(depth >= 4)[0]).astype(np.int32)]
    before = [p0, p0, p0 // 2, p0 // 4]                # compact rows already in the streams
    T_cap = p0 + win
    units = []
    for layer in range(layers):
        for kind in (flk.K, flk.V):
            xs = [torch.randn((win if r is None else len(r), H, D), device="cuda").to(torch.bfloat16)
                  for r in rows_w]
            recon = torch.empty((win, H, D), dtype=torch.bfloat16, device="cuda")
            packs = []
            for l, r in enumerate(rows_w):
                n_cap = before[l] + (win if r is None else len(r))
                rows = None
                if r is not None:
                    rows = torch.empty(n_cap, dtype=torch.int32, device="cuda")
                    rows[before[l]:].copy_(torch.from_numpy(r))
                packs.append(flk.Packed.empty(kind, H, D, n_cap, rows, T=T_cap, k_tiles=True,
                                              compact=r is not None))
            units.append((kind, xs, recon, packs))

    def items(l):
        if l == 0:
            return [(k, xs[0], p0, rec, pk[0]) for k, xs, rec, pk in units]
        r = rows_w[l]
        return [(k, xs[l], None if r is None else pk[l].rows[before[l]:], win if r is None else len(r), p0, win,
                 before[l], rec, pk[l]) for k, xs, rec, pk in units]
    # unit tables marshalled once, as a serving loop would keep them: a flush is 4 C calls
    L = flk.lib()
    kd, vd = flk.desc(flk.K, H, D, True), flk.desc(flk.V, H, D)
    tables = []
    for l in range(4):
        its = items(l)
        us_ = [flk._append_unit(k, x, None, x.shape[0], q0, x.shape[0], q0, rec, pk) for k, x, q0, rec, pk in its] \
            if l == 0 else [flk._append_unit(*it) for it in its]
        tables.append((flk.AppendUnitC * len(us_))(*us_))
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def flush_batched():
        assert L.flk_append_base_batch(ctypes.byref(kd), ctypes.byref(vd), tables[0], len(tables[0]), None, sp) == 0
        for l in range(1, 4):
            assert L.flk_append_residual_batch(ctypes.byref(kd), ctypes.byref(vd), tables[l], len(tables[l]), None,
                                               sp) == 0

    def flush_single():
        for l in range(4):
            for u in tables[l]:
                one = (flk.AppendUnitC * 1)(u)
                f = L.flk_append_base_batch if l == 0 else L.flk_append_residual_batch
                assert f(ctypes.byref(kd), ctypes.byref(vd), one, 1, None, sp) == 0

    def back_to_back(fn, n=50):
        return lambda: [fn() for _ in range(n)]

    for _ in range(5):
        flush_batched()
        flush_single()
    torch.cuda.synchronize()
    nb = 0
    for kind in (flk.K, flk.V):
        calls = call_bytes(kind, H, D, win, [None if r is None else r - p0 for r in rows_w], k_tiles=kind == flk.K)
        nb += layers * sum(b for name, b in calls if name != "reconstruct")
    us_b = _timed_us(back_to_back(flush_batched), 5) / 50
    us_s = _timed_us(back_to_back(flush_single, 10), 3) / 10
    out["flush"] = {"workload": "decode_flush", "tensors": 2 * layers, "H": H, "D": D, "window": win,
                    "window_rows": [win, win, len(rows_w[2]), len(rows_w[3])], "algorithmic_bytes": int(nb),
                    "batched_us": round(us_b, 2), "batched_gbs": round(nb / us_b / 1e3, 1),
                    "single_calls_us": round(us_s, 2), "calls_batched": 4, "calls_single": 8 * layers,
                    "timing": "wall per flush over back-to-back flushes, unit tables prepared once"}
    del units, tables
    torch.cuda.empty_cache()

    # attention over 131072 packed tokens (tile-grouped K) + a 127-token BF16 tail
    w = synth.WORKLOADS[5]
    T, Hk, Dk, Hq = w.T, w.H, w.D, w.Hq
    chains = decode_chains(w, k_tiles=True)
    tail = 127
    assert flk.rolling_prefix(T + tail) == T
    kt = torch.randn((tail, Hk, Dk), device="cuda").to(torch.bfloat16)
    vt = torch.randn((tail, Hk, Dk), device="cuda").to(torch.bfloat16)
    q = torch.from_numpy(synth.make_query(w).view(np.int16)).cuda().view(torch.bfloat16)
    o = torch.empty((Hq, Dk), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(flk.attn_workspace_bytes(Hk, Dk, T + tail, Hq) // 4 + 1, dtype=torch.float32, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(Dk)
    roll = lambda: flk.decode_attn_rolling(q, chains[flk.K], chains[flk.V], T, Hk, kt, vt, scale, o, ws)
    packed = lambda: flk.decode_attn_packed(q, chains[flk.K], chains[flk.V], T, Hk, scale, o, ws)
    for _ in range(3):
        roll()
        packed()
    torch.cuda.synchronize()
    out["attention"] = {"workload": "decode_attn", "T_packed": T, "tail": tail, "Hkv": Hk, "Hq": Hq, "D": Dk,
                        "k_grouping": "tile", "rolling_us": round(_timed_us(roll, 20, flush), 2),
                        "packed_only_us": round(_timed_us(packed, 20, flush), 2)}
    return out


# ----------------------------------------------------------------------------- HBM traffic

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_long_prompt.txt")
COPY_PROBE_BYTES = 1 << 29     # plain copy used to calibrate FETCH_SIZE / WRITE_SIZE (2x the MALL)


# The sources the codec kernels (encode, residual encode, reconstruct) are compiled from.
CODEC_SOURCES = ("flk_device.h", "flk_encode.hip", "flk_internal.h", "flk_reconstruct.hip")


def source_digest():
    """sha256 over CODEC_SOURCES: a traffic figure taken from other kernel sources than the ones
    built now is not reported."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_kv_cache_amd", "csrc")
    for name in CODEC_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def copy_probe(warm_s=0.3, reps=100):
    """The practical ceiling: plain copies of COPY_PROBE_BYTES (read once, written once) by an
    elementwise kernel whose name contains 'bitwise_not', timed at steady clocks -- about warm_s
    seconds of copies first (the GPU reaches its sustained clocks only after some hundred
    milliseconds of load), then `reps` copies between two events.  The counter runs also divide
    its FETCH_SIZE / WRITE_SIZE into the known size to get the scale applied to the codec
    kernels.  Returns the copy's GB/s (bytes read + written)."""
    src = torch.zeros(COPY_PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t_end = time.perf_counter() + warm_s
    while time.perf_counter() < t_end:
        for _ in range(50):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)
    ev[1].record()
    torch.cuda.synchronize()
    gbs = 2 * COPY_PROBE_BYTES * reps / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
    del src, dst
    return gbs


def _short_name(kernel_name):
    if "at::native::" in kernel_name:                # torch's kernels: the op's functor name
        import re
        m = re.search(r"at::native::(?:[A-Za-z_]\w*::)*?(\w*(?:_kernel_cuda|Functor_\w+|_kernel_impl\w*|reduce_kernel))",
                      kernel_name)
        return "torch " + (m.group(1) if m else kernel_name.split("<")[0].split()[-1])
    n = kernel_name.replace("(anonymous namespace)::", "").split("(")[0].strip()
    for pre in ("void ", "flk::"):
        if n.startswith(pre):
            n = n[len(pre):]
    return n


def summarize_pmc(dirs):
    """Turn rocprofv3 --pmc counter CSVs (one run with FETCH_SIZE, one with WRITE_SIZE, each of
    `bench.py --copy-probe`) into the per-launch HBM traffic table that bench.py reports."""
    import csv
    import glob
    vals = {}                                   # (counter, kernel) -> [per-dispatch values]
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                key = (r["Counter_Name"], _short_name(r["Kernel_Name"]))
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
    w = synth.WORKLOADS[3]
    sets = synth.active_sets(w, w.T)
    algo = {}
    for kind in (flk.K, flk.V):
        for name, b in call_bytes(kind, w.H, w.D, w.T, sets):
            algo.setdefault(kernel_symbol(kind, name, w.H, w.D, sets), []).append(b)
    # the page-local leg's tile-grouped compact K loops (its other kernels are the headline's)
    for name, b in call_bytes(flk.K, w.H, w.D, w.T, sets, k_tiles=True):
        if name == "sparse_residual":
            algo.setdefault("encode_k_tile_kernel<true>", []).append(b)

    def mean(counter, pred):
        xs = [v for (c, k), vs in vals.items() if c == counter and pred(k) for v in vs]
        return (sum(xs) / len(xs), len(xs)) if xs else (float("nan"), 0)
    probe_kib = COPY_PROBE_BYTES / 1024
    fetch_copy, nf = mean("FETCH_SIZE", lambda k: "bitwise_not" in k)
    write_copy, nw = mean("WRITE_SIZE", lambda k: "bitwise_not" in k)
    fs, ws_ = probe_kib / fetch_copy, probe_kib / write_copy
    lines = [f"source_sha256 {source_digest()}",
             f"copy_probe bytes {COPY_PROBE_BYTES} fetch_kib {fetch_copy:.1f} write_kib {write_copy:.1f} "
             f"fetch_scale {fs:.4f} write_scale {ws_:.4f} dispatches {nf}/{nw}"]
    # the two-pass decode attention, when the run had the attention leg: pass 1 reads the K
    # chain (and the loops' rows) and writes the scores rows, pass 2 reads the V chain, the rows
    # and the scores; the algorithmic bytes count the chains alone, so the scores' round trip
    # (Hq * T * 4 bytes written, then read) shows in the ratio
    if any(c == "FETCH_SIZE" and k.startswith("attn_scores_kernel<4") for (c, k) in vals):
        wa = synth.WORKLOADS[5]
        sa = synth.active_sets(wa, wa.T)
        rows_b = sum(4 * len(r) for r in sa if r is not None)
        chain_b = {kind: sum(flk.codes_bytes(kind, wa.H, wa.D, n) + flk.params_bytes(kind, wa.H, wa.D, n)
                             for n in (wa.T if r is None else len(r) for r in sa)) + rows_b
                   for kind in (flk.K, flk.V)}
        for sym, a in (("attn_scores_kernel<4, false>", chain_b[flk.K]), ("attn_pv_kernel<4>", chain_b[flk.V])):
            algo[sym] = [a]
    for sym, bs in algo.items():
        f, n1 = mean("FETCH_SIZE", lambda k, s=sym: k == s)
        wr, n2 = mean("WRITE_SIZE", lambda k, s=sym: k == s)
        if n1 == 0 and n2 == 0:
            continue
        traffic = (f * fs + wr * ws_) * 1024
        a = sum(bs) / len(bs)
        lines.append(f"kernel {sym} | dispatches {n1}/{n2} | fetch_kib {f:.1f} | write_kib {wr:.1f} | "
                     f"traffic_bytes {traffic:.0f} | algorithmic_bytes {a:.0f} | ratio {traffic / a:.4f}")
    return "\n".join(lines)


def headline_launches():
    """Kernel symbol -> launches per step of the headline (long-prompt, single calls)."""
    w = synth.WORKLOADS[3]
    sets = synth.active_sets(w, w.T)
    per = {}
    for kind in (flk.K, flk.V):
        for name, _ in call_bytes(kind, w.H, w.D, w.T, sets):
            sym = kernel_symbol(kind, name, w.H, w.D, sets)
            per[sym] = per.get(sym, 0) + 1
    return per


def summarize_trace(trace_dir, warmup, steps, isolated=10):
    """Per-kernel durations from a rocprofv3 kernel trace of `bench.py` (default mode): over all
    calls, and for the headline's kernels over its timed region and over its isolated launches.
    A headline kernel runs c times per step and the headline's launches come first in dispatch
    order (warmup steps, timed steps, min(10, steps) steps with per-launch events, then
    `isolated` launches of each call alone), so its timed calls are launches
    [c*warmup, c*(warmup+steps)) and its isolated ones the c*isolated after the evented steps."""
    import csv
    import glob
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    per = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            per.setdefault(_short_name(r["Kernel_Name"]), []).append(
                (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    head = headline_launches()
    lines = [f"{'kernel':52s} {'calls':>6s} {'all_avg_us':>11s} {'timed_avg_us':>13s} {'isolated_avg_us':>16s}"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        v.sort()
        d = np.array([x for _, x in v])
        timed = iso = ""
        c = head.get(name, 0)
        ov = min(OVERLAP_STEPS, steps)
        if c and len(d) >= c * (warmup + steps + ov + isolated):
            timed = f"{d[warmup * c:(warmup + steps) * c].mean():13.2f}"
            iso = f"{d[(warmup + steps + ov) * c:(warmup + steps + ov + isolated) * c].mean():16.2f}"
        lines.append(f"{name[:52]:52s} {len(d):6d} {d.mean():11.2f} {timed:>13s} {iso:>16s}")
    return "\n".join(lines)


def summarize_stats(stats_csv, top=40, match=None):
    """rocprofv3 --stats kernel statistics (kernel_stats.csv) as a short table: per kernel the
    calls, mean / min / max duration (us) and share of the summed kernel time; the `top`
    kernels by summed time, or every kernel whose short name matches the regex `match`."""
    import csv
    import re
    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    if match:
        rows = [r for r in rows if re.search(match, _short_name(r["Name"]))]
        top = len(rows)
    lines = [f"{'kernel':52s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share_%':>8s}"]
    for r in rows[:top]:
        lines.append(f"{_short_name(r['Name'])[:52]:52s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):8.2f}")
    return "\n".join(lines)


TRACE_FILE = os.path.join(ROOT, "profiles", "kernel_trace_long_prompt.txt")


def read_trace(symbol):
    """(timed-region, isolated-step) average durations (us) of `symbol` in the committed
    kernel-trace summary of the benchmark command, or (None, None)."""
    if not os.path.exists(TRACE_FILE):
        return None, None
    for line in open(TRACE_FILE):
        if line[:52].strip() == symbol[:52]:
            parts = line[52:].split()
            if len(parts) == 4:
                return float(parts[2]), float(parts[3])
    return None, None


def summarize_counters(dirs, n_cu=256, clock_mhz=2400.0):
    """Per-kernel instruction and occupancy counters from rocprofv3 --pmc runs (CSV output, one
    counter set per run; every run over the same command), as a table of per-dispatch medians.
    Derived columns use the dispatch's duration at the nominal 2.4 GHz clock: VALU issue share
    (SQ_INSTS_VALU against one VALU wave-instruction per CU per cycle) and mean resident waves
    per CU (SQ_WAVE_CYCLES counts wave quad-cycles); also VALU instructions per wave."""
    import csv
    import glob
    import statistics
    vals, dur = {}, {}
    for d in dirs:
        seen = set()
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                k = _short_name(r["Kernel_Name"])
                if not (k.startswith(("encode", "reconstruct", "attn", "sparse", "fp4", "select"))):
                    continue
                vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                key = (path, r["Dispatch_Id"])
                if key not in seen:
                    seen.add(key)
                    dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = []
    for k in sorted(vals, key=lambda k: -statistics.median(dur[k]) * len(dur[k])):
        med = {c: statistics.median(v) for c, v in vals[k].items()}
        us = statistics.median(dur[k])
        lines.append(f"kernel {k} | dispatches {len(dur[k])} | median_us {us:.2f}")
        lines.append("  " + " | ".join(f"{c} {v:.0f}" for c, v in sorted(med.items())))
        derived = []
        cyc = us * clock_mhz
        if "SQ_INSTS_VALU" in med:
            derived.append(f"valu_issue_share {med['SQ_INSTS_VALU'] / (n_cu * cyc):.3f}")
        if "SQ_WAVE_CYCLES" in med:
            derived.append(f"mean_waves_per_cu {4 * med['SQ_WAVE_CYCLES'] / (n_cu * cyc):.1f}")
        if "SQ_INSTS_VALU" in med and med.get("SQ_WAVES"):
            derived.append(f"valu_per_wave {med['SQ_INSTS_VALU'] / med['SQ_WAVES']:.0f}")
        if derived:
            lines.append("  derived: " + " | ".join(derived))
    return "\n".join(lines)


def read_traffic(symbol):
    """Per-launch HBM bytes of `symbol` from the committed counter summary, or None when there is
    none or it was taken from other sources than the ones built now."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest, found = None, None
    for line in open(TRAFFIC_FILE):
        if line.startswith("source_sha256 "):
            digest = line.split()[1]
        elif line.startswith("kernel ") and line.split("|")[0][len("kernel "):].strip() == symbol:
            for field in line.split("|"):
                kv = field.split()
                if kv and kv[0] == "traffic_bytes":
                    found = float(kv[1])
    return found if digest == source_digest() else None


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU reaches steady clocks only after some hundred milliseconds of load: 1000 warmup
    # steps (about 0.25 s) before 2000 timed ones (about 0.5 s) measure the steady state.
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--rotate", type=int, default=4, help="independent buffer sets cycled across steps")
    ap.add_argument("--mode", default="streams", choices=("batched", "streams", "serial"),
                    help="batched: one batched call per loop covers K and V (one stream); streams: "
                         "single calls, the K chain and the V chain on two streams; serial: single calls "
                         "on one stream")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attention", action="store_true", help="skip the decode-attention leg")
    ap.add_argument("--no-page-local", action="store_true", help="skip the page-local K grouping leg")
    ap.add_argument("--no-rolling", action="store_true", help="skip the rolling-tail flush and attention leg")
    ap.add_argument("--no-sparse", action="store_true", help="skip the sparse decode attention leg")
    ap.add_argument("--no-selection", action="store_true", help="skip the token selection leg")
    ap.add_argument("--no-fp4", action="store_true", help="skip the FP4 (NVFP4, MXFP4) variant leg")
    ap.add_argument("--no-batched", action="store_true", help="skip the batched-cache leg")
    ap.add_argument("--batched-layers", type=int, default=24,
                    help="layers of the batched cache (64 requests each) the batched-cache leg runs (24 = all)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="accepted for older command lines: the copy of known size (which calibrates the HBM "
                         "byte counters) now always runs")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="print the traffic table from rocprofv3 counter output and exit (no GPU)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="print per-kernel instruction/occupancy counters from rocprofv3 --pmc CSV runs, and exit "
                         "(no GPU)")
    ap.add_argument("--summarize-stats", metavar="CSV",
                    help="print a rocprofv3 kernel_stats.csv as a short table and exit")
    ap.add_argument("--stats-match", metavar="REGEX",
                    help="with --summarize-stats: every kernel whose name matches, instead of the top 40")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print per-kernel durations (all calls, timed region) from a rocprofv3 kernel trace "
                         "of a run with the same --warmup/--steps, and exit (no GPU)")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats, match=args.stats_match))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.warmup, args.steps))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the codec runs per request/layer on a single device); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    flk.lib()

    w = synth.WORKLOADS[3]
    log(f"generating workload {w.name}: T={w.T} H={w.H} D={w.D}")
    sets = synth.active_sets(w, w.T)
    host = {flk.K: synth.make_chain(w, synth.K_TENSOR, sets=sets),
            flk.V: synth.make_chain(w, synth.V_TENSOR, sets=sets)}
    batched = args.mode == "batched"
    chain_sets = [ChainSet(w, host, sets, batched=batched) for _ in range(args.rotate)]
    torch.cuda.synchronize()

    per_call = []
    if batched:
        kb = call_bytes(flk.K, w.H, w.D, w.T, sets)
        vb = call_bytes(flk.V, w.H, w.D, w.T, sets)
        per_call = [(KV, name, b + b2) for (name, b), (_, b2) in zip(kb, vb)]
    else:
        for kind in (flk.K, flk.V):
            per_call += [(kind, name, b) for name, b in call_bytes(kind, w.H, w.D, w.T, sets)]
    step_bytes = sum(b for _, _, b in per_call)
    # the practical ceiling, measured at steady clocks right before the headline (the GPU then
    # enters the headline's warmup at the clocks sustained load gives it)
    log("copy ceiling ...")
    copy_gbs = copy_probe()
    # default-priority streams only; in "streams" mode the K chain and the V chain overlap
    ts = [torch.cuda.Stream(), torch.cuda.Stream()] if args.mode == "streams" else [torch.cuda.Stream()] * 2
    streams = {k: (ts[i], ctypes.c_void_p(ts[i].cuda_stream)) for i, k in enumerate((flk.K, flk.V))}

    # warmup: every step back to back (no idle gaps while the clocks settle), events around each
    # call of the last min(10, W) steps on the call's stream; they pick the kernel with the largest
    # share of the overlapped step
    n_calls = len(chain_sets[0].calls)
    n_warm = max(args.warmup, 1)
    n_ev = min(10, n_warm)
    wev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_calls)]
           for _ in range(n_ev)]
    for i in range(n_warm):
        k = i - (n_warm - n_ev)
        chain_sets[i % args.rotate].run(streams, wev[k] if k >= 0 else None)
    torch.cuda.synchronize()
    times = np.sum([[a.elapsed_time(b) for a, b in e] for e in wev], axis=0)
    counted = n_ev
    symbols = [batched_symbol(name, sets) if kind == KV else kernel_symbol(kind, name, w.H, w.D, sets)
               for kind, name, _ in per_call]
    sym_time = {}
    for sy, t in zip(symbols, times):
        sym_time[sy] = sym_time.get(sy, 0.0) + t
    dominant = max(sym_time, key=sym_time.get)
    dom_idx = [i for i, sy in enumerate(symbols) if sy == dominant]
    log("warmup per-call us: " + ", ".join(f"{sy}={t / counted * 1e3:.1f}" for sy, t in zip(symbols, times)))

    # timed region: exactly `steps` steps, nothing else on the streams
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        chain_sets[k % args.rotate].run(streams)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # the dominant kernel inside the overlapped step: min(10, steps) further steps, back to back
    # as in the timed region, with events around that kernel's launches on the stream that
    # launches it (kept out of the timed region: each event pair drains its stream)
    n_ov = min(OVERLAP_STEPS, args.steps)
    dom_ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               if i in dom_idx else None for i in range(n_calls)] for _ in range(n_ov)]
    for k in range(n_ov):
        chain_sets[(args.steps + k) % args.rotate].run(streams, dom_ev[k])
    torch.cuda.synchronize()

    # each call alone: one stream, events around every call, nothing overlapping
    iso_us = isolated_calls(chain_sets, 10)
    per_call_iso = [{"tensor": {flk.K: "K", flk.V: "V", KV: "K+V"}[kind], "call": name, "kernel": sy,
                     "bytes": int(b), "us": round(float(t), 2), "gbs": round(b / t / 1e3, 1)}
                    for (kind, name, b), sy, t in zip(per_call, symbols, iso_us)]

    # the overlapped steps' event durations of the warmup's dominant kernel: with two streams they
    # include waiting for compute units the other chain holds, so they are reported apart
    dom_ms = [dom_ev[k][i][0].elapsed_time(dom_ev[k][i][1]) for k in range(n_ov) for i in dom_idx]
    dom_bytes = float(np.mean([per_call[i][2] for i in dom_idx]))
    dom_avg_ms = float(np.mean(dom_ms))
    prof_timed, _ = read_trace(dominant)
    roofline_overlapped = {"kernel": dominant, "launch_avg_us": round(dom_avg_ms * 1e3, 2),
                           "achieved": round(dom_bytes / (dom_avg_ms * 1e-3) / 1e9, 1),
                           "frac": round(dom_bytes / (dom_avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "note": f"HIP events on the kernel's stream around its launches in {n_ov} steps run "
                                   "right after the timed region as it runs (two streams, overlapping the other "
                                   "chain)",
                           "profile_launch_avg_us": prof_timed}

    # the roofline's kernel: the largest summed time per step with every call timed alone (one
    # stream, nothing overlapping), its duration the mean of its isolated launches; the committed
    # kernel trace of this command gives the same launches' duration for comparison
    iso_sym = {}
    for sy, t in zip(symbols, iso_us):
        iso_sym[sy] = iso_sym.get(sy, 0.0) + float(t)
    rdom = max(iso_sym, key=iso_sym.get)
    r_idx = [i for i, sy in enumerate(symbols) if sy == rdom]
    r_bytes = float(np.mean([per_call[i][2] for i in r_idx]))
    r_us = float(np.mean([iso_us[i] for i in r_idx]))
    traffic = read_traffic(rdom)
    _, prof_us = read_trace(rdom)
    roofline = {"bound": "hbm", "kernel": rdom, "achieved": round(r_bytes / r_us / 1e3, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(r_bytes / r_us / 1e3 / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else int(traffic), "traffic_unit": "bytes per launch",
                "launches_per_step": len(r_idx), "launch_avg_us": round(r_us, 2),
                "algorithmic_bytes_per_launch": int(r_bytes),
                "timing": "HIP events on the kernel's stream around 10 back-to-back launches of its call "
                          "alone (rotating buffer sets, queued behind a spin kernel), mean per launch",
                "profile_launch_avg_us": None if prof_us is None else prof_us,
                "profile_frac": None if prof_us is None else round(r_bytes / prof_us / 1e3 / HBM_PEAK_GBS, 4),
                "profile": os.path.relpath(TRACE_FILE, ROOT)}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "copy_ceiling_gbs": round(copy_gbs, 1), "copy_frac": round(value / copy_gbs, 4),
        "config": {"workload": "long_prompt", "T": w.T, "H": w.H, "D": w.D, "loops": w.n_loops,
                   "budgets_pct": list(w.budgets), "tensors": "K+V", "step_bytes": int(step_bytes),
                   "rotate_sets": args.rotate, "mode": args.mode},
        "roofline": roofline,
        "roofline_overlapped": roofline_overlapped,
    }
    result["per_call_isolated"] = per_call_iso
    result["isolated_step_us"] = round(float(iso_us.sum()), 2)
    if not args.no_page_local and args.mode != "batched":
        log("the same step with page-local K groups ...")
        result["page_local"] = page_local_leg(w, host, sets, streams, args.steps, args.warmup, args.rotate)
    if not args.no_attention:
        log("decode attention over the packed chains ...")
        result["decode_attention"] = attention_leg()
    if not args.no_batched:
        log(f"batched cache: {args.batched_layers} layers x 64 requests ...")
        result["batched_cache"] = batched_cache_leg(layers=args.batched_layers)
    if not args.no_rolling:
        log("rolling tail: flush and attention ...")
        result["rolling"] = rolling_leg()
    if not args.no_sparse:
        log("sparse decode attention ...")
        result["sparse_attention"] = sparse_leg()
    if not args.no_fp4:
        log("FP4 variants against INT4 ...")
        result["fp4"] = fp4_leg(w, host, sets)
    if not args.no_selection:
        log("token selection ...")
        result["token_selection"] = selection_leg()
    if not args.no_cpu_baseline:
        log("timing the oracle on a head sample ...")
        result["cpu_baseline"] = cpu_baseline(w, host, sets)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
