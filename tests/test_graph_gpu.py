"""The library's entry points can be captured into a HIP graph: they enqueue
only kernels on the caller's stream (no allocation, no memset, no
synchronisation).  Each captured graph is replayed several times with new
input data written eagerly in between, and every replay is compared bit for
bit with an eager call on the same data (all kernels are deterministic)."""
import pytest
import torch

from io_aware_exact_amd import fa, inputs

pytestmark = pytest.mark.gpu


def test_graph_fwd_bwd_replays():
    B, S, H, d = 1, 1000, 4, 128
    print(f"graph fwd+bwd B={B} S={S} H={H} d={d}", flush=True)
    q, k, v, do = (torch.empty((B, S, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(q) for _ in range(3))
    a = fa.bwd_args(q, k, v, o, do, lse, *grads, True, None)
    ws = torch.empty(int(fa.lib().fa_bwd_workspace_size(fa.ctypes.byref(a))), dtype=torch.uint8,
                     device="cuda")

    def step():
        fa.fwd(q, k, v, True, out=o, lse=lse)
        fa.bwd(q, k, v, o, do, lse, True, out=grads, workspace=ws)

    def load(seed):
        src = inputs.qkv(B, S, S, H, H, d, seed, device="cuda", with_dout=True)
        for dst, x in zip((q, k, v, do), src):
            dst.copy_(x)

    load(1)
    step()                                   # warm up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for seed in (2, 3, 4):
        load(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, *grads)]
        step()
        torch.cuda.synchronize()
        for x, y in zip(got, (o, lse, *grads)):
            assert torch.equal(x, y), f"replay with seed {seed} differs from eager"


def test_graph_kvcache_decode_replays():
    B, L, Hq, Hkv, d, ps = 8, 3000, 16, 4, 128, 64
    print(f"graph kvcache decode B={B} L={L}", flush=True)
    per = (L + 1 + ps - 1) // ps
    kc = torch.randn((B * per, ps, Hkv, d), device="cuda").to(torch.bfloat16)
    vc = torch.randn((B * per, ps, Hkv, d), device="cuda").to(torch.bfloat16)
    bt = torch.randperm(B * per, device="cuda").to(torch.int32).view(B, per)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q = torch.empty((B, 1, Hq, d), dtype=torch.bfloat16, device="cuda")
    kn = torch.empty((B, 1, Hkv, d), dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(kn)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    a = fa.kvcache_args(q, kc, vc, lens, bt, kn, vn, o, lse, True, None)
    ws = torch.empty(int(fa.lib().fa_fwd_kvcache_workspace_size(fa.ctypes.byref(a))),
                     dtype=torch.uint8, device="cuda")

    def step():
        fa.fwd_kvcache(q, kc, vc, lens, bt, kn, vn, True, out=o, lse=lse, workspace=ws)

    def load(seed):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        for t in (q, kn, vn):
            t.copy_(torch.randn(t.shape, generator=gen, device="cuda"))

    load(10)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for seed in (11, 12, 13):
        load(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (o.clone(), lse.clone())
        step()
        torch.cuda.synchronize()
        assert torch.equal(got[0], o) and torch.equal(got[1], lse), f"replay {seed}"
