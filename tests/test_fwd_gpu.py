"""GPU parity of the dense and packed forward against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_amd import fa, inputs
from parity import Guarded, check_lse, check_o

pytestmark = pytest.mark.gpu


def run_dense(B, Sq, Sk, Hq, Hkv, d, causal, seed, scale=None):
    print(f"dense B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} seed={seed}", flush=True)
    q, k, v = inputs.qkv(B, Sq, Sk, Hq, Hkv, d, seed, device="cuda")
    go = Guarded((B, Sq, Hq, d), torch.bfloat16)
    gl = Guarded((B, Hq, Sq), torch.float32)
    fa.fwd(q, k, v, causal, scale, out=go.t, lse=gl.t)
    torch.cuda.synchronize()
    go.check_guards()
    gl.check_guards()
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, causal, scale)
    check_o("O", go.t.float().cpu().numpy(), o_ref)
    check_lse("LSE", gl.t.cpu().numpy(), lse_ref)
    return go.t, gl.t


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_config(causal):
    # B=1, H=2, Sq=Sk=256, d=64, iid N(0,1), scale 1/sqrt(d)
    run_dense(1, 256, 256, 2, 2, 64, causal, seed=0)


@pytest.mark.parametrize("shape", [
    (1, 1, 1, 1, 1, 64), (1, 2, 2, 2, 2, 128), (2, 127, 127, 3, 3, 64),
    (1, 129, 129, 2, 2, 128), (1, 1000, 1000, 2, 1, 128), (2, 200, 333, 4, 2, 64),
    (1, 333, 200, 2, 2, 128), (1, 64, 1, 2, 1, 128), (1, 300, 257, 8, 1, 128),
    (1, 512, 512, 8, 2, 64),
])
@pytest.mark.parametrize("causal", [False, True])
def test_shapes(shape, causal):
    B, Sq, Sk, Hq, Hkv, d = shape
    run_dense(B, Sq, Sk, Hq, Hkv, d, causal, seed=sum(shape))


@pytest.mark.parametrize("shape", [
    (1, 300, 2100, 4, 2, 64), (2, 513, 2048, 2, 1, 64), (1, 700, 8250, 2, 1, 64),
    (1, 1100, 8192, 1, 1, 64),
])
@pytest.mark.parametrize("causal", [False, True])
def test_shapes_d64_long_keys(shape, causal):
    # d = 64 with 2048 keys or more (8192 when causal) runs the two-group
    # kernel: ragged query and key tails, GQA, Sq < Sk
    B, Sq, Sk, Hq, Hkv, d = shape
    run_dense(B, Sq, Sk, Hq, Hkv, d, causal, seed=7 + sum(shape))


@pytest.mark.parametrize("shape", [
    (1, 33, 40, 2, 1, 128), (2, 64, 3000, 4, 2, 128), (1, 128, 8192, 2, 2, 128),
    (1, 100, 517, 8, 1, 128), (3, 127, 127, 2, 2, 128), (1, 128, 64, 2, 2, 128),
])
@pytest.mark.parametrize("causal", [False, True])
def test_shapes_d128_few_rows(shape, causal):
    # d = 128 with at most 128 query rows (and more than 32 rows per kv head,
    # so not the split-KV path) runs the one-group kernel: GQA, Sq > Sk with
    # fully masked causal rows, long and ragged key sweeps
    B, Sq, Sk, Hq, Hkv, d = shape
    run_dense(B, Sq, Sk, Hq, Hkv, d, causal, seed=11 + sum(shape))


def test_scale_and_strided_views():
    # q/k/v as views into a packed [B,S,3,H,d] buffer (non-trivial strides)
    B, S, H, d = 2, 190, 4, 128
    qkv = inputs.normal((B, S, 3, H, d), 11, device="cuda")
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    o, lse = fa.fwd(q, k, v, False, 0.05)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, False, 0.05)
    check_o("O", o.float().cpu().numpy(), o_ref)
    check_lse("LSE", lse.cpu().numpy(), lse_ref)


def test_deterministic():
    q, k, v = inputs.qkv(2, 700, 700, 4, 2, 128, 5, device="cuda")
    outs = [fa.fwd(q, k, v, True) for _ in range(3)]
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_gqa_equals_repeated_heads():
    q, k, v = inputs.qkv(1, 300, 300, 8, 2, 128, 6, device="cuda")
    o1, l1 = fa.fwd(q, k, v, True)
    o2, l2 = fa.fwd(q, k.repeat_interleave(4, dim=2).contiguous(),
                    v.repeat_interleave(4, dim=2).contiguous(), True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", [[1, 0, 17, 128, 129, 300, 64, 255], [1, 0, 17, 128, 64, 100, 33]])
def test_varlen(d, causal, lens):
    # the second list has no sequence over 128 rows: at d = 128 it runs the
    # one-group kernel, the first the two-group kernel
    Hq, Hkv = 4, 2
    print(f"varlen lens={lens} d={d} causal={causal}", flush=True)
    q, k, v = inputs.packed_qkv(lens, lens, Hq, Hkv, d, 21, device="cuda")
    cu = inputs.cu_seqlens(lens, device="cuda")
    T = sum(lens)
    go = Guarded((T, Hq, d), torch.bfloat16)
    gl = Guarded((Hq, T), torch.float32)
    fa.fwd_varlen(q, k, v, cu, cu, max(lens), max(lens), causal, None, out=go.t, lse=gl.t)
    torch.cuda.synchronize()
    go.check_guards()
    gl.check_guards()
    o_ref, lse_ref = oracle.attention_fwd_varlen(q, k, v, cu.cpu(), cu.cpu(), causal)
    check_o("O", go.t.float().cpu().numpy(), o_ref)
    check_lse("LSE", gl.t.cpu().numpy(), lse_ref)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_short_queries_long_keys(causal):
    # packed d = 128 queries of at most 128 rows (the one-group kernel) over
    # key sequences of other lengths, up to 1000 keys and down to none
    lq, lk = [1, 64, 128, 33, 90], [500, 64, 1000, 10, 0]
    Hq, Hkv, d = 8, 2, 128
    print(f"varlen short queries lq={lq} lk={lk} causal={causal}", flush=True)
    q, k, v = inputs.packed_qkv(lq, lk, Hq, Hkv, d, 23, device="cuda")
    cq, ck = inputs.cu_seqlens(lq, device="cuda"), inputs.cu_seqlens(lk, device="cuda")
    o, lse = fa.fwd_varlen(q, k, v, cq, ck, max(lq), max(lk), causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd_varlen(q, k, v, cq.cpu(), ck.cpu(), causal)
    check_o("O", o.float().cpu().numpy(), o_ref)
    check_lse("LSE", lse.cpu().numpy(), lse_ref)


def test_varlen_d64_long_sequences():
    # packed d = 64, non-causal, longest sequence over 2048 keys: the
    # two-group kernel over every sequence of the pack, short ones included
    lens = [2100, 300, 2500, 17, 256, 1]
    Hq, Hkv, d = 4, 2, 64
    print(f"varlen d64 long lens={lens}", flush=True)
    q, k, v = inputs.packed_qkv(lens, lens, Hq, Hkv, d, 25, device="cuda")
    cu = inputs.cu_seqlens(lens, device="cuda")
    o, lse = fa.fwd_varlen(q, k, v, cu, cu, max(lens), max(lens), False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd_varlen(q, k, v, cu.cpu(), cu.cpu(), False)
    check_o("O", o.float().cpu().numpy(), o_ref)
    check_lse("LSE", lse.cpu().numpy(), lse_ref)


def test_varlen_equals_dense_per_sequence():
    lens_q = [100, 37, 256]
    lens_k = [150, 37, 300]
    q, k, v = inputs.packed_qkv(lens_q, lens_k, 4, 1, 128, 22, device="cuda")
    cq = inputs.cu_seqlens(lens_q, device="cuda")
    ck = inputs.cu_seqlens(lens_k, device="cuda")
    o, lse = fa.fwd_varlen(q, k, v, cq, ck, max(lens_q), max(lens_k), True)
    for z in range(3):
        qs, qe = int(cq[z]), int(cq[z + 1])
        ks, ke = int(ck[z]), int(ck[z + 1])
        od, ld = fa.fwd(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke], True)
        assert torch.equal(od[0], o[qs:qe]) and torch.equal(ld[0], lse[:, qs:qe])


def test_varlen_debug_check(monkeypatch):
    """FA_DEBUG: the packed calls check the cu_seqlens contents on the host
    and reject inconsistent ones before enqueuing anything (outputs keep
    their sentinel); valid ones run as without the check."""
    lens = [100, 37, 256]
    q, k, v = inputs.packed_qkv(lens, lens, 4, 1, 128, 23, device="cuda")
    good = inputs.cu_seqlens(lens, device="cuda")
    o_ref, lse_ref = fa.fwd_varlen(q, k, v, good, good, max(lens), max(lens), True)
    monkeypatch.setenv("FA_DEBUG", "1")
    o, lse = fa.fwd_varlen(q, k, v, good, good, max(lens), max(lens), True)
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    bad = [torch.tensor(c, dtype=torch.int32, device="cuda") for c in
           ([0, 150, 137, 393], [1, 101, 138, 393], [0, 100, 137, 392])]
    # a step above max_seqlen_q is also rejected
    tight = (good, max(lens) - 1)
    for cu, mx in [(c, max(lens)) for c in bad] + [tight]:
        out = torch.full_like(o, 7.0)
        with pytest.raises(fa.FaError) as e:
            fa.fwd_varlen(q, k, v, cu, good, mx, max(lens), True, out=out)
        assert e.value.status == 11
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
        dq, dk, dv = (torch.full_like(x, 7.0) for x in (q, k, v))
        with pytest.raises(fa.FaError) as e:
            fa.bwd_varlen(q, k, v, o, o, lse, good, cu, max(lens), mx, True, out=(dq, dk, dv))
        assert e.value.status == 11
        torch.cuda.synchronize()
        assert all(bool((x == 7.0).all()) for x in (dq, dk, dv))


def check_against_oracle(q, k, v, causal):
    o, lse = fa.fwd(q, k, v, causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, causal)
    check_o("O", o.float().cpu().numpy(), o_ref)
    seen = np.isfinite(lse_ref)
    check_lse("LSE", lse.cpu().numpy()[seen], lse_ref[seen])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores(d, causal):
    """Keys whose norm grows along the sequence (x1 to x4), so later key
    tiles hold much larger scores than the first ones: the running max has
    to move while the tiles stream, which the first tiles alone never ask."""
    print(f"growing scores d={d} causal={causal}", flush=True)
    q, k, v = inputs.qkv(1, 1000, 1000, 4, 2, d, 71 + d, device="cuda")
    ramp = torch.linspace(1.0, 4.0, 1000, device="cuda").view(1, 1000, 1, 1)
    k = (k.float() * ramp).to(torch.bfloat16)
    check_against_oracle(q, k, v, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_score_steps(d, causal):
    """Every query row is the all-ones vector and key j is beta_j times it,
    so every score of key j is exactly scale * d * beta_j.  The key blocks
    step through: 0 (the first 100 keys), +6 in exp2 units (probabilities of
    64 against the first max: partial row sums far above 2^8 while no single
    probability passes 2^8), -40 (probabilities that underflow), +12 (a max
    that grows past 2^8) and +6 again."""
    print(f"score steps d={d} causal={causal}", flush=True)
    S = 1000
    log2e = 1.0 / math.log(2.0)
    unit = (1.0 / math.sqrt(d)) * d * log2e          # exp2 units per unit of beta
    beta = torch.zeros(S)
    for lo, hi, e2 in [(100, 300, 6.0), (300, 450, -40.0), (450, 700, 12.0), (700, S, 6.0)]:
        beta[lo:hi] = e2 / unit
    q = torch.ones((1, S, 2, d), dtype=torch.bfloat16, device="cuda")
    k = (beta.view(1, S, 1, 1) * torch.ones((1, S, 1, d))).to(torch.bfloat16).cuda()
    _, _, v = inputs.qkv(1, S, S, 2, 1, d, 81 + d, device="cuda")
    check_against_oracle(q, k, v, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_growing_scores(d, causal):
    """Packed sequences whose keys grow along each sequence (x1 to x4), so the
    running max moves mid-sequence in every sequence of the pack."""
    lens = [700, 65, 300, 1000]
    print(f"varlen growing scores lens={lens} d={d} causal={causal}", flush=True)
    q, k, v = inputs.packed_qkv(lens, lens, 4, 2, d, 91 + d, device="cuda")
    ramp = torch.cat([torch.linspace(1.0, 4.0, n) for n in lens]).view(-1, 1, 1).cuda()
    k = (k.float() * ramp).to(torch.bfloat16)
    cu = inputs.cu_seqlens(lens, device="cuda")
    o, lse = fa.fwd_varlen(q, k, v, cu, cu, max(lens), max(lens), causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd_varlen(q, k, v, cu.cpu(), cu.cpu(), causal)
    check_o("O", o.float().cpu().numpy(), o_ref)
    check_lse("LSE", lse.cpu().numpy(), lse_ref)


@pytest.mark.parametrize("decode", [False, True])
def test_no_keys(decode):
    """Sk = 0: every row sees no key, so O = 0 and LSE = -inf (no NaN); the
    empty K/V are zero-length views, on the tiled and the split-KV paths."""
    q, k, v = inputs.qkv(2, 1 if decode else 100, 10, 8, 2, 128, 14, device="cuda")
    k, v = k[:, :0], v[:, :0]
    o, lse = (fa.fwd_decode if decode else fa.fwd)(q, k, v, True)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


# fp32 path: inputs and probabilities are not rounded below fp32, so the bars
# are those of fp32 arithmetic (a few fp32 ulps of O ~ 1 and LSE ~ 10 after a
# sum over up to a thousand products): O <= 1e-4 max-abs, LSE <= 1e-5 max-abs.
F32_O_MAX_ABS = 1e-4
F32_LSE_MAX_ABS = 1e-5


def run_dense_f32(B, Sq, Sk, Hq, Hkv, d, causal, seed, scale=None):
    print(f"fp32 B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} seed={seed}", flush=True)
    q, k, v = inputs.qkv(B, Sq, Sk, Hq, Hkv, d, seed, dtype=torch.float32, device="cuda")
    go = Guarded((B, Sq, Hq, d), torch.float32)
    gl = Guarded((B, Hq, Sq), torch.float32)
    fa.fwd(q, k, v, causal, scale, out=go.t, lse=gl.t)
    torch.cuda.synchronize()
    go.check_guards()
    gl.check_guards()
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, causal, scale)
    check_o("O", go.t.cpu().numpy(), o_ref, max_abs=F32_O_MAX_ABS, mean_abs=F32_O_MAX_ABS, rel=1e-5)
    check_lse("LSE", gl.t.cpu().numpy(), lse_ref, max_abs=F32_LSE_MAX_ABS)


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_config_fp32(causal):
    # B=1, H=2, Sq=Sk=256, d=64, iid N(0,1) in fp32, scale 1/sqrt(d)
    run_dense_f32(1, 256, 256, 2, 2, 64, causal, seed=0)


@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1, 64), (2, 127, 129, 4, 2, 128),
                                   (1, 300, 200, 2, 2, 64), (1, 200, 1000, 8, 1, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_shapes_fp32(shape, causal):
    B, Sq, Sk, Hq, Hkv, d = shape
    run_dense_f32(B, Sq, Sk, Hq, Hkv, d, causal, seed=50 + sum(shape))
