"""fa_bwd_noalloc: the dense backward with no workspace and no allocation.

Its scratch is a fixed per-device array inside the library, looked up once
per device; the kernels are fa_bwd's, so the gradients must be bitwise those
of fa_bwd with a caller workspace.  Two calls in a row (the second smaller)
also show that the array keeps nothing that a later call depends on.
"""
import ctypes

import pytest
import torch

from io_aware_exact_amd import fa, inputs

FAKE = 0x7F0000000000


def test_rejects_beyond_scratch_without_gpu():
    """B * Hq * Sq * 4 bytes of D above the 32 MiB array: FA_ERR_WORKSPACE,
    decided on the host before anything touches a device."""
    B, S, H, d = 1, 131073, 64, 64      # 8,388,672 rows x heads > 8,388,608
    t = fa.FaTensor(FAKE, S * H * d, H * d, d)
    a = fa.BwdArgs(fa.FA_BF16, B, S, 16, H, H, d, 0, 0.125, t, t, t, t, t, t, t, t,
                   FAKE, None, 0, 0)
    assert fa.lib().fa_bwd_noalloc(ctypes.byref(a), None) == 7
    assert fa.lib().fa_bwd_noalloc(None, None) == 1


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [False, True])
def test_matches_fa_bwd_twice(causal):
    shapes = [(2, 700, 700, 8, 2, 128, 31), (1, 300, 257, 4, 4, 64, 32)]
    for B, Sq, Sk, Hq, Hkv, d, seed in shapes:
        print(f"noalloc bwd B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}",
              flush=True)
        q, k, v, do = inputs.qkv(B, Sq, Sk, Hq, Hkv, d, seed, device="cuda", with_dout=True)
        o, lse = fa.fwd(q, k, v, causal)
        ref = fa.bwd(q, k, v, o, do, lse, causal)
        out = tuple(torch.full_like(x, float("nan")) for x in ref)
        got = fa.bwd_noalloc(q, k, v, o, do, lse, causal, out=out)
        torch.cuda.synchronize()
        for x, y in zip(got, ref):
            assert torch.equal(x, y)


@pytest.mark.gpu
def test_full_size_step():
    """The benchmark's backward shape (B=2, H=16, S=8192, d=128) through the
    no-allocation entry point equals fa_bwd bitwise."""
    B, S, H, d = 2, 8192, 16, 128
    q, k, v, do = inputs.qkv(B, S, S, H, H, d, 2000, device="cuda", with_dout=True)
    o, lse = fa.fwd(q, k, v, False)
    ref = fa.bwd(q, k, v, o, do, lse, False)
    got = fa.bwd_noalloc(q, k, v, o, do, lse, False)
    torch.cuda.synchronize()
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
