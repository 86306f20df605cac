"""GPU parity of the split-KV decode path of fa_fwd (few query rows against a
long KV cache) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_amd import fa, inputs
from parity import Guarded, check_lse, check_o

pytestmark = pytest.mark.gpu


def run_decode(B, Sq, Sk, Hq, Hkv, d, causal, seed, scale=None):
    print(f"decode B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} seed={seed}",
          flush=True)
    q, k, v = inputs.qkv(B, Sq, Sk, Hq, Hkv, d, seed, device="cuda")
    n = fa.fwd_workspace_bytes(q, k, v, causal, scale)
    assert n > 0, "decode path should apply"
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    go = Guarded((B, Sq, Hq, d), torch.bfloat16)
    gl = Guarded((B, Hq, Sq), torch.float32)
    fa.fwd(q, k, v, causal, scale, out=go.t, lse=gl.t, workspace=ws)
    torch.cuda.synchronize()
    go.check_guards()
    gl.check_guards()
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, causal, scale)
    check_o("O", go.t.float().cpu().numpy(), o_ref)
    check_lse("LSE", gl.t.cpu().numpy(), lse_ref)
    return q, k, v, go.t, gl.t


@pytest.mark.parametrize("shape", [
    (1, 1, 1, 1, 1, 64), (2, 1, 1, 4, 1, 128), (3, 1, 300, 8, 2, 128),
    (2, 1, 1000, 32, 8, 128), (1, 4, 777, 8, 1, 64), (2, 2, 5000, 4, 4, 128),
    (1, 1, 31, 32, 1, 128), (1, 1, 70000, 4, 1, 128), (2, 3, 2, 4, 2, 64),
])
@pytest.mark.parametrize("causal", [False, True])
def test_shapes(shape, causal):
    B, Sq, Sk, Hq, Hkv, d = shape
    run_decode(B, Sq, Sk, Hq, Hkv, d, causal, seed=300 + sum(shape))


@pytest.mark.parametrize("shape", [
    (2, 1, 3000, 64, 1, 128), (1, 16, 1000, 32, 8, 128), (2, 24, 777, 32, 8, 64),
    (1, 5, 4000, 20, 1, 128), (1, 3, 2, 40, 1, 64), (1, 3, 300, 16, 1, 128),
])
@pytest.mark.parametrize("causal", [False, True])
def test_shapes_several_row_blocks(shape, causal):
    # 33 to 128 query rows per kv head, fewer 32-row blocks than query heads
    # in the group: each block is its own workgroup over the same keys; block
    # boundaries inside a head's rows (Sq = 3, 5), causal rows that see no
    # key (Sq > Sk)
    B, Sq, Sk, Hq, Hkv, d = shape
    run_decode(B, Sq, Sk, Hq, Hkv, d, causal, seed=350 + sum(shape))


def test_scale():
    run_decode(2, 1, 900, 8, 2, 128, False, seed=31, scale=0.3)


def test_split_equals_unsplit():
    """The split-KV result and the tiled kernel's agree (different rounding
    order only); LSE to fp32 accuracy."""
    B, Sq, Sk, Hq, Hkv, d = 4, 1, 9000, 16, 4, 128
    q, k, v = inputs.qkv(B, Sq, Sk, Hq, Hkv, d, 32, device="cuda")
    o1, l1 = fa.fwd_decode(q, k, v, True)
    o2, l2 = fa.fwd(q, k, v, True)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-2
    assert float((l1 - l2).abs().max()) <= 1e-4


def test_deterministic():
    q, k, v = inputs.qkv(2, 1, 4000, 8, 2, 128, 33, device="cuda")
    outs = [fa.fwd_decode(q, k, v, False) for _ in range(3)]
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_full_size_decode():
    """Decode at batch 64, one new token, 32 query heads over 8 kv heads,
    d=128, against a 32768-key cache (8.6 GB of K/V), in the launch
    configuration the bench times; every one of the 2048 output rows is
    checked against the oracle."""
    B, Sq, Sk, Hq, Hkv, d = 64, 1, 32768, 32, 8, 128
    print("decode full size", flush=True)
    q, k, v = inputs.qkv(B, Sq, Sk, Hq, Hkv, d, 3100, device="cuda")
    o, lse = fa.fwd_decode(q, k, v, True)
    torch.cuda.synchronize()
    grp = Hq // Hkv
    o_got = o.float().cpu().numpy()
    l_got = lse.cpu().numpy()
    o_ref = np.zeros((B, Hq, d))
    l_ref = np.zeros((B, Hq))
    for b in range(B):
        for g in range(Hkv):
            hs = slice(g * grp, (g + 1) * grp)
            orf, lrf = oracle.head_fwd(q[b, 0, hs, :], np.zeros(grp, np.int64),
                                       k[b, :, g, :], v[b, :, g, :], Sk - Sq, True,
                                       1.0 / np.sqrt(d))
            o_ref[b, hs], l_ref[b, hs] = orf, lrf
    check_o("O", o_got[:, 0], o_ref)
    check_lse("LSE", l_got[:, :, 0], l_ref)
