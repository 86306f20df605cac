"""GPU checks of fa_merge, the exact merge of partial results over disjoint
key shards (the per-shard step of sequence-parallel attention): random
partials against the oracle's merge, a one-part merge that returns its input
bit for bit, and attention split over key shards on one GPU (each shard a
fa_fwd call, then the merge) against the fp64 oracle on the whole sequence,
causal and not, with GQA."""
import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_amd import fa, inputs
from parity import check_lse, check_o

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_merge_random_parts(dtype, d):
    P, B, S, H = 3, 2, 70, 3
    print(f"merge P={P} B={B} S={S} H={H} d={d} {dtype}", flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(5 + d)
    o_parts = torch.randn((P, B, S, H, d), generator=g).to(dtype)
    lse_parts = torch.randn((P, B, H, S), generator=g) * 3
    lse_parts[1, 0, 1, :10] = float("-inf")                  # one part sees no key
    lse_parts[:, 1, 2, 5] = float("-inf")                    # no part sees a key
    o, lse = fa.merge(o_parts.cuda(), lse_parts.cuda())
    torch.cuda.synchronize()
    o_r, lse_r = oracle.merge_partials(o_parts, lse_parts)
    check_o("O", o.float().cpu().numpy(), o_r)
    check_lse("LSE", lse.cpu().numpy(), lse_r)
    assert torch.all(o[1, 5, 2] == 0) and lse[1, 2, 5].item() == float("-inf")


def test_merge_single_part_is_identity():
    q, k, v = inputs.qkv(1, 200, 300, 4, 2, 128, 9, device="cuda")
    o, lse = fa.fwd(q, k, v, True)
    om, lm = fa.merge(o[None].contiguous(), lse[None].contiguous())
    assert torch.equal(om, o) and torch.equal(lm, lse)


@pytest.mark.parametrize("causal", [False, True])
def test_sequence_parallel_shards(causal):
    # query shard i sees key shards j <= i (causal) or all (not): key shards
    # before i in full, shard i with the causal mask, each one fa_fwd call
    B, S, Hq, Hkv, d, n = 1, 2048, 8, 2, 128, 4
    L = S // n
    print(f"sequence-parallel emulation S={S} shards={n} causal={causal}", flush=True)
    q, k, v = inputs.qkv(B, S, S, Hq, Hkv, d, 17, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    for i in range(n):
        qi = q[:, i * L:(i + 1) * L]
        js = range(i + 1) if causal else range(n)
        parts = [fa.fwd(qi, k[:, j * L:(j + 1) * L], v[:, j * L:(j + 1) * L], causal and j == i)
                 for j in js]
        om, lm = fa.merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]))
        o[:, i * L:(i + 1) * L] = om
        lse[:, :, i * L:(i + 1) * L] = lm
    torch.cuda.synchronize()
    o_r, lse_r = oracle.attention_fwd(q.cpu(), k.cpu(), v.cpu(), causal)
    check_o("O", o.float().cpu().numpy(), o_r)
    check_lse("LSE", lse.cpu().numpy(), lse_r)
