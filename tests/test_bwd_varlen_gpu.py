"""GPU parity of the packed variable-length backward (fa_bwd_varlen) against
the fp64 oracle (the dense backward run on every packed sequence alone), its
bitwise agreement with fa_bwd run on each sequence separately, run-to-run
reproducibility, the autograd wrapper, and a full-size packed batch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_amd import fa, inputs
from parity import Guarded, check_grad, check_lse, check_o

pytestmark = pytest.mark.gpu


def packed(lens_q, lens_k, Hq, Hkv, d, seed):
    q, k, v = inputs.packed_qkv(lens_q, lens_k, Hq, Hkv, d, seed, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    cq = inputs.cu_seqlens(lens_q, device="cuda")
    ck = inputs.cu_seqlens(lens_k, device="cuda")
    return q, k, v, do, cq, ck


def run_varlen_bwd(lens_q, lens_k, Hq, Hkv, d, causal, seed, scale=None):
    print(f"varlen bwd lens_q={lens_q} lens_k={lens_k} Hq={Hq} Hkv={Hkv} d={d} "
          f"causal={causal} seed={seed}", flush=True)
    q, k, v, do, cq, ck = packed(lens_q, lens_k, Hq, Hkv, d, seed)
    mq, mk = max(lens_q), max(lens_k)
    o, lse = fa.fwd_varlen(q, k, v, cq, ck, mq, mk, causal, scale)
    Tq, Tk = sum(lens_q), sum(lens_k)
    gq = Guarded((Tq, Hq, d), torch.bfloat16)
    gk = Guarded((Tk, Hkv, d), torch.bfloat16)
    gv = Guarded((Tk, Hkv, d), torch.bfloat16)
    fa.bwd_varlen(q, k, v, o, do, lse, cq, ck, mq, mk, causal, scale, out=(gq.t, gk.t, gv.t))
    torch.cuda.synchronize()
    for gbuf in (gq, gk, gv):
        gbuf.check_guards()
    o_r, lse_r, dq_r, dk_r, dv_r = oracle.attention_bwd_varlen(q, k, v, do, cq.cpu(), ck.cpu(),
                                                               causal, scale)
    check_o("O", o.float().cpu().numpy(), o_r)
    seen = np.isfinite(lse_r)
    check_lse("LSE", lse.cpu().numpy()[seen], lse_r[seen])
    check_grad("dQ", gq.t.float().cpu().numpy(), dq_r)
    check_grad("dK", gk.t.float().cpu().numpy(), dk_r)
    check_grad("dV", gv.t.float().cpu().numpy(), dv_r)
    return q, k, v, do, cq, ck, o, lse, (gq.t, gk.t, gv.t)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_bwd(d, causal):
    # tiles past a sequence end, an empty sequence, a one-token one, tails
    lens = [1, 0, 17, 128, 129, 300, 64, 255]
    run_varlen_bwd(lens, lens, 4, 2, d, causal, seed=31 + d)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_bwd_cross_lengths(causal):
    # Lq != Lk per sequence (bottom-right causal alignment), a sequence with
    # queries but no keys (dQ = 0) and one with keys but no queries (dK = dV = 0)
    lens_q = [100, 37, 5, 0, 256]
    lens_k = [150, 37, 0, 40, 300]
    run_varlen_bwd(lens_q, lens_k, 8, 2, 128, causal, seed=41)


def test_varlen_bwd_equals_dense_per_sequence():
    lens_q = [100, 37, 256, 1]
    lens_k = [150, 37, 300, 64]
    q, k, v, do, cq, ck = packed(lens_q, lens_k, 4, 1, 128, 51)
    o, lse = fa.fwd_varlen(q, k, v, cq, ck, max(lens_q), max(lens_k), True)
    dq, dk, dv = fa.bwd_varlen(q, k, v, o, do, lse, cq, ck, max(lens_q), max(lens_k), True)
    for z in range(len(lens_q)):
        qs, qe = int(cq[z]), int(cq[z + 1])
        ks, ke = int(ck[z]), int(ck[z + 1])
        od, ld = fa.fwd(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke], True)
        ddq, ddk, ddv = fa.bwd(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke], od,
                               do[None, qs:qe].contiguous(), ld, True)
        assert torch.equal(ddq[0], dq[qs:qe])
        assert torch.equal(ddk[0], dk[ks:ke]) and torch.equal(ddv[0], dv[ks:ke])


def test_varlen_bwd_deterministic():
    lens = [700, 33, 1000]
    q, k, v, do, cq, ck = packed(lens, lens, 8, 2, 128, 61)
    o, lse = fa.fwd_varlen(q, k, v, cq, ck, max(lens), max(lens), True)
    runs = [fa.bwd_varlen(q, k, v, o, do, lse, cq, ck, max(lens), max(lens), True)
            for _ in range(3)]
    for r in runs[1:]:
        for x, y in zip(r, runs[0]):
            assert torch.equal(x, y)


def test_varlen_bwd_no_rows():
    # every sequence empty on the query side: dK = dV = 0 and nothing else
    lens_q, lens_k = [0, 0], [5, 9]
    q, k, v, do, cq, ck = packed(lens_q, lens_k, 2, 2, 64, 71)
    o = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, 0), dtype=torch.float32, device="cuda")
    dk = torch.full(k.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    dv = torch.full(v.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    dq = torch.empty_like(q)
    fa.bwd_varlen(q, k, v, o, do, lse, cq, ck, 0, 9, False, out=(dq, dk, dv))
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk) == 0 and torch.count_nonzero(dv) == 0


def test_attention_varlen_autograd():
    lens = [50, 129, 7]
    q, k, v, do, cq, ck = packed(lens, lens, 4, 2, 64, 81)
    for t in (q, k, v):
        t.requires_grad_(True)
    o = fa.attention_varlen(q, k, v, cq, ck, max(lens), max(lens), causal=True)
    o.backward(do)
    _, _, dq_r, dk_r, dv_r = oracle.attention_bwd_varlen(q.detach(), k.detach(), v.detach(), do,
                                                         cq.cpu(), ck.cpu(), True)
    check_grad("dQ", q.grad.float().cpu().numpy(), dq_r)
    check_grad("dK", k.grad.float().cpu().numpy(), dk_r)
    check_grad("dV", v.grad.float().cpu().numpy(), dv_r)


def test_varlen_bwd_full_size_sampled():
    """The packed GQA workload of the forward benchmark (16 sequences, lengths
    uniform on [128, 32768], Hq=32, Hkv=8, d=128, causal): the shortest
    sequence against the oracle on kv heads 0 and 7 (all their query heads);
    on every sequence and head, the identities
    sum_j dK_j = 0 (the rows of dS sum to zero) and sum_j dV_j =
    sum over the group's heads of sum_i dO_i (the rows of P sum to one)."""
    lens = inputs.varlen_lengths(16, 128, 32768, 3000)
    print(f"varlen bwd full size lens={lens}", flush=True)
    q, k, v = inputs.packed_qkv(lens, lens, 32, 8, 128, 3001, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(3002)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    cu = inputs.cu_seqlens(lens, device="cuda")
    mx = max(lens)
    o, lse = fa.fwd_varlen(q, k, v, cu, cu, mx, mx, True)
    dq, dk, dv = fa.bwd_varlen(q, k, v, o, do, lse, cu, cu, mx, mx, True)
    torch.cuda.synchronize()
    z = min(range(16), key=lambda i: lens[i])
    cuc = cu.cpu().numpy()
    s, e = int(cuc[z]), int(cuc[z + 1])
    _, _, dq_r, dk_r, dv_r = oracle.attention_bwd(q[None, s:e].cpu(), k[None, s:e].cpu(),
                                                  v[None, s:e].cpu(), do[None, s:e].cpu(), True,
                                                  bh=[(0, 0), (0, 7)])
    for gk in (0, 7):
        hs = slice(4 * gk, 4 * gk + 4)
        check_grad(f"dQ seq {z} kv head {gk}", dq[s:e, hs].float().cpu().numpy(), dq_r[0, :, hs])
        check_grad(f"dK seq {z} kv head {gk}", dk[s:e, gk].float().cpu().numpy(), dk_r[0, :, gk])
        check_grad(f"dV seq {z} kv head {gk}", dv[s:e, gk].float().cpu().numpy(), dv_r[0, :, gk])
    for z in range(16):
        s, e = int(cuc[z]), int(cuc[z + 1])
        dkz, dvz = dk[s:e].double(), dv[s:e].double()
        doz = do[s:e].double().view(e - s, 8, 4, 128).sum(2)
        # sums of L bf16-rounded terms: allow the rounding of each term
        bound = 2.0 ** -8 * dkz.abs().sum(0) + 1e-3
        assert (dkz.sum(0).abs() <= bound).all(), f"sum dK seq {z}"
        bound = 2.0 ** -8 * (dvz.abs().sum(0) + doz.abs().sum(0)) + 1e-3
        assert ((dvz.sum(0) - doz.sum(0)).abs() <= bound).all(), f"sum dV seq {z}"
