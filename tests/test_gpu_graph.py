"""Graph capture of the codec path (RFC vllm-rlt #156, section 6.7, CUDA Graphs: stable-address
storage, bounded selection buffers, and no batch's selection captured as a constant).  One
graph holds the base encode, a dense residual loop, the device token selection of loop 3 (50 %
per window), the gather of the selected rows, the compact residual encode and the
reconstruction.  It is replayed over new inputs written in place; each replay must equal the
same calls made eagerly, bit for bit, and the selected rows must follow the inputs."""
import numpy as np
import pytest
import torch

from quantized_kv_cache_amd import flk

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


T, H, D, d, W, PCT = 4096, 2, 128, 512, 1024, 50


class Bufs:
    """Every tensor of one run of the path, allocated once (stable addresses)."""

    def __init__(self, kind):
        dev = "cuda"
        self.kind = kind
        self.n3 = flk.select_count(T, W, [PCT])
        self.x = [torch.empty((T, H, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
        self.hp = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
        self.hp2 = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
        self.rows3 = torch.empty(self.n3, dtype=torch.int32, device=dev)
        self.slot = torch.empty(T, dtype=torch.int32, device=dev)
        self.scores = torch.empty(T, dtype=torch.float32, device=dev)
        self.ws = torch.empty(flk.select_workspace_bytes(T, W) // 4 + 1, dtype=torch.int32, device=dev)
        self.x3rows = torch.empty((self.n3, H, D), dtype=torch.bfloat16, device=dev)
        self.recon = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
        self.p = [flk.Packed.empty(kind, H, D, T), flk.Packed.empty(kind, H, D, T),
                  flk.Packed.empty(kind, H, D, self.n3, self.rows3, T=T)]

    def load(self, xs, hp, hp2):
        for dst, src in zip(self.x, xs):
            dst.copy_(src)
        self.hp.copy_(hp)
        self.hp2.copy_(hp2)

    def run(self):
        k = self.kind
        flk.encode_base(k, self.x[0], self.p[0], self.recon)
        flk.encode_residual(k, self.x[1], None, self.recon, self.p[1])
        flk.select_rows(self.hp, self.hp2, None, W, PCT, 1e-6, self.scores, self.rows3, self.ws, slot=self.slot)
        torch.index_select(self.x[2], 0, self.rows3, out=self.x3rows)
        flk.encode_residual(k, self.x3rows, self.rows3, self.recon, self.p[2])
        flk.reconstruct(k, self.p, self.out)

    def outputs(self):
        o = [self.rows3, self.slot, self.recon, self.out]
        for p in self.p:
            o += [p.codes, p.params] + ([p.tile_start] if p.tile_start is not None else [])
        return [t.clone() for t in o]


@pytest.mark.parametrize("kind", [flk.K, flk.V])
def test_selection_encode_reconstruct_graph_replays(kind):
    g_bufs, e_bufs = Bufs(kind), Bufs(kind)
    gen = torch.Generator(device="cuda")

    def inputs(seed):
        gen.manual_seed(seed)
        y = torch.randn((T, H, D), device="cuda", generator=gen)
        xs = [y]
        for _ in range(2):
            y = y + 0.1 * torch.randn((T, H, D), device="cuda", generator=gen)
            xs.append(y)
        hp2 = torch.randn((T, d), device="cuda", generator=gen)
        hp = hp2 + torch.rand((T, 1), device="cuda", generator=gen) * torch.randn((T, d), device="cuda", generator=gen)
        return [x.to(torch.bfloat16) for x in xs], hp.to(torch.bfloat16), hp2.to(torch.bfloat16)

    g_bufs.load(*inputs(100))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # warm up outside the capture
        g_bufs.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_bufs.run()
    torch.cuda.synchronize()

    selections = []
    for rep in range(4):
        say(f"graph replay {rep} kind={kind}")
        xs, hp, hp2 = inputs(rep)
        g_bufs.load(xs, hp, hp2)
        graph.replay()
        torch.cuda.synchronize()
        got = g_bufs.outputs()
        e_bufs.load(xs, hp, hp2)                     # the same calls, eagerly, between replays
        e_bufs.run()
        torch.cuda.synchronize()
        want = e_bufs.outputs()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), f"replay {rep}, output {i}"
        assert torch.equal(g_bufs.out.view(torch.int16), g_bufs.recon.view(torch.int16))
        selections.append(g_bufs.rows3.cpu().numpy())
        r = selections[-1]
        assert np.all(np.diff(r) > 0) and r[0] >= 0 and r[-1] < T
    # the selection follows each replay's hidden states: it was not captured as a constant
    assert any(not np.array_equal(selections[0], r) for r in selections[1:])
