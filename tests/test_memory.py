"""The memory claim of the method: no buffer the size of the attention matrix.

"Dao and colleagues: IO-aware exact attention with FlashAttention" (research
record, summary) computes exact attention without materialising the full
attention matrix, and "Flash Attention and Efficient Transformer Mechanisms"
states the memory requirement as linear instead of quadratic in the sequence
length.  The library allocates nothing itself, so the only memory it can ask
for is the caller's workspace; these checks assert that every workspace query
grows at most linearly in Sq + Sk (never with Sq * Sk), and, on the GPU, that
a forward and backward at S = 16384 take no device memory beyond the caller's
tensors.
"""
import ctypes

import pytest
import torch

from io_aware_exact_amd import fa

FAKE = 0x7F0000000000  # size queries never dereference pointers


def _t(H, d, S):
    return fa.FaTensor(FAKE, S * H * d, H * d, d)


def fwd_ws(B, Sq, Sk, Hq, Hkv, d):
    a = fa.FwdArgs(fa.FA_BF16, B, Sq, Sk, Hq, Hkv, d, 1, d ** -0.5, _t(Hq, d, Sq), _t(Hkv, d, Sk),
                   _t(Hkv, d, Sk), _t(Hq, d, Sq), FAKE, None, None, None, None, 0)
    return int(fa.lib().fa_fwd_workspace_size(ctypes.byref(a)))


def bwd_ws(B, Sq, Sk, Hq, Hkv, d):
    tq, tk = _t(Hq, d, Sq), _t(Hkv, d, Sk)
    a = fa.BwdArgs(fa.FA_BF16, B, Sq, Sk, Hq, Hkv, d, 1, d ** -0.5, tq, tk, tk, tq, tq, tq, tk, tk,
                   FAKE, None, 0, 0)
    return int(fa.lib().fa_bwd_workspace_size(ctypes.byref(a)))


def bwd_varlen_ws(nseq, L, Hq, Hkv, d):
    st = Hq * d
    a = fa.BwdVarlenArgs(fa.FA_BF16, nseq, Hq, Hkv, d, L, L, nseq * L, nseq * L, 1, d ** -0.5,
                         *([FAKE] * 8), *([st, d] * 8), FAKE, FAKE, FAKE, None, 0)
    return int(fa.lib().fa_bwd_varlen_workspace_size(ctypes.byref(a)))


def kvcache_ws(B, Sq, L, Hq, Hkv, d):
    ps = 256
    pages = (L + ps - 1) // ps
    a = fa.FwdKvcacheArgs(fa.FA_BF16, B, Sq, Hq, Hkv, d, 0, 1, d ** -0.5, _t(Hq, d, Sq),
                          _t(Hq, d, Sq), FAKE, FAKE, FAKE, ps * Hkv * d, Hkv * d, d,
                          ps * Hkv * d, Hkv * d, d, B * pages, ps, pages, L, FAKE, pages, FAKE,
                          fa.FaTensor(None, 0, 0, 0), fa.FaTensor(None, 0, 0, 0), None, 0)
    return int(fa.lib().fa_fwd_kvcache_workspace_size(ctypes.byref(a)))


LENGTHS = [1, 7, 64, 128, 1000, 4096, 8192, 32768, 131072]


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_workspace_linear_in_sq_and_free_of_sk(d):
    B, Hq, Hkv = 2, 16, 4
    for Sk in LENGTHS:
        sizes = [bwd_ws(B, Sq, Sk, Hq, Hkv, d) for Sq in LENGTHS]
        for Sq, n in zip(LENGTHS, sizes):
            # D = rowsum(dO o O): one fp32 per query row and head, 256-byte aligned
            assert n <= B * Hq * Sq * 4 + 255, (Sq, Sk, n)
            assert n == bwd_ws(B, Sq, 1, Hq, Hkv, d), "workspace depends on Sk"
    # doubling both lengths at most doubles it
    for S in LENGTHS[:-1]:
        assert bwd_ws(B, 2 * S, 2 * S, Hq, Hkv, d) <= 2 * bwd_ws(B, S, S, Hq, Hkv, d) + 256


def test_bwd_varlen_workspace_linear_in_tokens():
    for L in LENGTHS:
        n = bwd_varlen_ws(3, L, 8, 2, 128)
        assert n <= 8 * 3 * L * 4 + 255, (L, n)


@pytest.mark.parametrize("Sq,Hq,Hkv", [(1, 32, 8), (4, 8, 8), (1, 8, 1), (8, 16, 4)])
def test_decode_workspace_bounded_in_sk(Sq, Hq, Hkv):
    """The split-KV partials are (rows x splits x d) with at most 64 splits:
    bounded however long the key sequence, and proportional to the rows."""
    B, d = 4, 128
    rows = B * Hq * Sq
    cap = rows * 64 * (d + 1) * 4 + 512
    for Sk in LENGTHS + [1 << 20, (1 << 31) - 1024]:
        n = fwd_ws(B, Sq, Sk, Hq, Hkv, d)
        assert 0 < n <= cap, (Sk, n)
        nk = kvcache_ws(B, Sq, min(Sk, 1 << 24), Hq, Hkv, d)
        assert 0 < nk <= cap, (Sk, nk)


@pytest.mark.parametrize("Sq,Hq,Hkv,split", [
    (1, 32, 8, True),      # 4 rows: one block
    (8, 16, 4, True),      # 32 rows: one block
    (1, 64, 1, True),      # 64 rows in 2 blocks, 64 query heads per kv head
    (16, 32, 8, True),     # 64 rows in 2 blocks, group 4
    (24, 32, 8, True),     # 96 rows in 3 blocks, group 4
    (32, 32, 8, False),    # 128 rows in 4 blocks: as many as the group's heads
    (64, 32, 32, False),   # 64 rows, group 1
    (33, 1, 1, False),     # 33 rows, group 1
    (1, 160, 1, False),    # 160 rows: over four blocks
])
def test_decode_row_block_rule(Sq, Hq, Hkv, split):
    """The split-KV path takes up to four 32-row blocks of a kv head's query
    rows, when the blocks are fewer than the group's query heads (each block
    reads the kv head's keys; the tiled kernels read them once per query
    head): its workspace is non-zero exactly then, for the dense and the
    KV-cache entry points alike."""
    assert (fwd_ws(2, Sq, 4096, Hq, Hkv, 128) > 0) == split
    assert (kvcache_ws(2, Sq, 4096, Hq, Hkv, 128) > 0) == split


def test_tiled_shapes_need_no_workspace():
    for S in LENGTHS:
        assert fwd_ws(2, max(S, 64), S, 16, 16, 128) == 0
        assert kvcache_ws(2, 128, S + 128, 16, 16, 128) == 0


@pytest.mark.gpu
def test_no_device_allocation_at_16k():
    """fa_fwd and fa_bwd at B=1, H=16, S=16384, d=128 with caller-owned
    outputs and workspace: free device memory is the same before and after
    (the library allocates nothing; a materialised score matrix alone would
    be 16 x 16384^2 x 4 B = 17 GB)."""
    from io_aware_exact_amd import inputs
    B, S, H, d = 1, 16384, 16, 128
    q, k, v, do = inputs.qkv(B, S, S, H, H, d, 5, device="cuda", with_dout=True)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(q) for _ in range(3))
    a = fa.bwd_args(q, k, v, o, do, lse, *grads, True, None)
    ws = torch.empty(int(fa.lib().fa_bwd_workspace_size(ctypes.byref(a))), dtype=torch.uint8,
                     device="cuda")
    assert ws.numel() == B * H * S * 4
    # first calls load the kernels
    fa.fwd(q, k, v, True, out=o, lse=lse)
    fa.bwd(q, k, v, o, do, lse, True, out=grads, workspace=ws)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(2):
        fa.fwd(q, k, v, True, out=o, lse=lse)
        fa.bwd(q, k, v, o, do, lse, True, out=grads, workspace=ws)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    print(f"free device memory before {free0}, after {free1}", flush=True)
    assert free1 >= free0 - (2 << 20)
    assert bool(torch.isfinite(grads[0]).all())
