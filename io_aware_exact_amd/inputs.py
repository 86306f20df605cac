"""Seeded synthetic inputs for attention workloads.

This module draws random numbers and packs sequence lengths; it holds none of
the attention arithmetic, so both the HIP path's callers and the oracle's
callers can share it.  Every generator takes an explicit seed and fills its
tensors in a fixed order, so a (shape, seed) pair always names the same data.
"""
import torch


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed, dtype=torch.bfloat16, device="cpu"):
    """iid N(0, 1) drawn in fp32, then cast (round-to-nearest-even)."""
    x = torch.randn(shape, generator=_gen(device, seed), dtype=torch.float32,
                    device=device)
    return x.to(dtype)


def qkv(B, Sq, Sk, Hq, Hkv, d, seed, dtype=torch.bfloat16, device="cpu",
        with_dout=False):
    """Q [B,Sq,Hq,d], K and V [B,Sk,Hkv,d] (and dO [B,Sq,Hq,d]) iid N(0,1),
    drawn from one generator in the order Q, K, V, dO."""
    g = _gen(device, seed)
    shapes = [(B, Sq, Hq, d), (B, Sk, Hkv, d), (B, Sk, Hkv, d)]
    if with_dout:
        shapes.append((B, Sq, Hq, d))
    out = []
    for s in shapes:
        x = torch.randn(s, generator=g, dtype=torch.float32, device=device)
        out.append(x.to(dtype))
    return tuple(out)


def varlen_lengths(nseq, lo, hi, seed):
    """nseq integers uniform on [lo, hi] inclusive (CPU generator)."""
    g = _gen("cpu", seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (nseq,), generator=g)]


def cu_seqlens(lengths, device="cpu"):
    """Cumulative offsets [0, L0, L0+L1, ...] as int32."""
    out = [0]
    for L in lengths:
        out.append(out[-1] + int(L))
    return torch.tensor(out, dtype=torch.int32, device=device)


def packed_qkv(lengths_q, lengths_k, Hq, Hkv, d, seed, dtype=torch.bfloat16,
               device="cpu"):
    """Packed Q [sum Lq, Hq, d], K and V [sum Lk, Hkv, d], iid N(0,1)."""
    g = _gen(device, seed)
    Tq, Tk = sum(lengths_q), sum(lengths_k)
    out = []
    for s in [(Tq, Hq, d), (Tk, Hkv, d), (Tk, Hkv, d)]:
        x = torch.randn(s, generator=g, dtype=torch.float32, device=device)
        out.append(x.to(dtype))
    return tuple(out)


def outlier_normal(shape, seed, p=0.001, outlier_std=10.0, device="cpu"):
    """fp32 N(0,1) plus, where Bernoulli(p) fires, an extra N(0, outlier_std^2)
    term (variance 100 for outlier_std = 10)."""
    g = _gen(device, seed)
    base = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    mask = torch.rand(shape, generator=g, dtype=torch.float32, device=device) < p
    extra = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    return base + mask.to(torch.float32) * extra * outlier_std


def sample_indices(n, count, seed, always=()):
    """`count` distinct seeded indices in [0, n), plus the listed ones."""
    g = _gen("cpu", seed)
    picks = set(int(i) % n for i in always if n > 0)
    if n > 0:
        perm = torch.randperm(n, generator=g)[: max(0, count)]
        picks.update(int(i) for i in perm)
    return sorted(picks)
