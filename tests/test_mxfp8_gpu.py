"""GPU checks of the MX FP8 path (E4M3 elements with one E8M0 scale per 32
elements along each product's reduction dimension): the quantiser bit for
bit against the oracle's MX encoder, and the forward against the fp64
oracle on the dequantised inputs, with the element-wise bound and relative L2
bars of the FP8 path (the probabilities are rounded to E4M3 at the running
maximum of the kernel's key order, which no plain definition fixes; the
bound on what that rounding can do is derived in tests/test_fp8_gpu.py and
holds unchanged here: the E8M0 block scales are powers of two applied
inside the matrix instruction, so the dequantised Q, K and V are exactly
what the products see)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
from io_aware_exact_amd import fa, inputs
from parity import Guarded
from test_fp8_gpu import (abs_dot_max, check_fp8_all_rows, check_lse_fp8, check_o_fp8, growing_keys,
                          o_bound_rows)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(1, 300, 3, 64), (2, 128, 2, 128), (1, 33, 1, 32),
                                   (2, 257, 4, 128), (1, 70, 1, 256)])
@pytest.mark.parametrize("axis", [0, 1])
def test_mx_quantiser_bit_exact(shape, axis):
    B, S, H, d = shape
    print(f"mx quantise shape={shape} axis={axis}", flush=True)
    x = inputs.outlier_normal((B, S, H, d), 60 + sum(shape), p=0.01)
    x[0, 0, 0, :32] = 0.0                         # an all-zero block along d
    x[0, :, 0, 1] = 0.0 if axis == 1 else x[0, :, 0, 1]   # and along the tokens
    codes, scales = fa.quantize_mxfp8(x.cuda(), axis)
    torch.cuda.synchronize()
    c_ref, s_ref = ofp8.quantize_mx(x.numpy(), "d" if axis == 0 else "s")
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)


def test_mx_quantiser_strided_and_special_values():
    base = inputs.normal((1, 70, 4, 64), 61, dtype=torch.float32)
    base[0, 3, 0, :8] = torch.tensor([0.0, -0.0, 1e-30, -1e-6, 3e38, -3e38, 5.0, -7.0])
    base[0, 5, 2, 32:] = 1e-40                    # subnormal fp32 block
    x = base[:, :, ::2]                           # head stride 2*d
    for axis in (0, 1):
        codes, scales = fa.quantize_mxfp8(x.cuda(), axis)
        torch.cuda.synchronize()
        c_ref, s_ref = ofp8.quantize_mx(x.contiguous().numpy(), "d" if axis == 0 else "s")
        assert np.array_equal(scales.cpu().numpy(), s_ref)
        assert np.array_equal(codes.cpu().numpy(), c_ref)


def run_mx(B, Sq, Sk, Hq, Hkv, d, causal, seed, scale=None, xs=None):
    """xs: the fp32 q, k, v to quantise (default: the outlier distribution)."""
    print(f"mxfp8 B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} seed={seed}",
          flush=True)
    if xs is None:
        xs = [inputs.outlier_normal(s, seed + i) for i, s in
              enumerate([(B, Sq, Hq, d), (B, Sk, Hkv, d), (B, Sk, Hkv, d)])]
    qc, qs = fa.quantize_mxfp8(xs[0].cuda(), 0)
    kc, ks = fa.quantize_mxfp8(xs[1].cuda(), 0)
    vc, vs = fa.quantize_mxfp8(xs[2].cuda(), 1)
    go = Guarded((B, Sq, Hq, d), torch.bfloat16)
    gl = Guarded((B, Hq, Sq), torch.float32)
    fa.fwd_mxfp8(qc, kc, vc, qs, ks, vs, causal, scale, out=go.t, lse=gl.t)
    torch.cuda.synchronize()
    go.check_guards()
    gl.check_guards()
    Q = ofp8.dequantize_mx(qc.cpu().numpy(), qs.cpu().numpy(), "d")
    K = ofp8.dequantize_mx(kc.cpu().numpy(), ks.cpu().numpy(), "d")
    V = ofp8.dequantize_mx(vc.cpu().numpy(), vs.cpu().numpy(), "s")
    o_ref, lse_ref = oracle.attention_fwd(Q, K, V, causal, scale)
    o = go.t.float().cpu().numpy()
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    check_lse_fp8(gl.t.cpu().numpy(), lse_ref, abs_dot_max(Q, K, Hq // Hkv, sc))
    check_fp8_all_rows(o, o_ref, lse_ref, Q, K, V, Hq // Hkv, sc, causal)


@pytest.mark.parametrize("shape", [(1, 256, 256, 2, 2, 64), (2, 300, 300, 4, 2, 128),
                                   (1, 129, 500, 2, 1, 128), (1, 700, 200, 2, 2, 64),
                                   (1, 1, 130, 4, 4, 128), (1, 100, 37, 2, 2, 128),
                                   (1, 600, 650, 2, 1, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_mx_forward(shape, causal):
    B, Sq, Sk, Hq, Hkv, d = shape
    run_mx(B, Sq, Sk, Hq, Hkv, d, causal, seed=700 + sum(shape))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_mx_growing_scores(d, causal):
    run_mx(1, 700, 900, 4, 2, d, causal, seed=93 + d, xs=growing_keys(700, 900, 4, 2, d, 93 + d))


def test_mx_forward_scale():
    run_mx(1, 200, 200, 2, 2, 128, False, seed=79, scale=0.2)


def test_mx_deterministic():
    x = inputs.outlier_normal((1, 600, 4, 128), 80, device="cuda")
    c, s = fa.quantize_mxfp8(x, 0)
    cv, sv = fa.quantize_mxfp8(x, 1)
    outs = [fa.fwd_mxfp8(c, c, cv, s, s, sv, True) for _ in range(3)]
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_mx_full_size():
    """B=1, H=16, S=16384, d=128, non-causal, the FP8 workload's inputs, in the
    launch configuration the bench times: 64 seeded rows of every head
    against the oracle on the dequantised inputs, and the RMS error against
    the oracle on the original fp32 inputs next to the 128-token per-block
    FP8 path's."""
    B, S, H, d = 1, 16384, 16, 128
    print("mxfp8 full size", flush=True)
    X = [inputs.outlier_normal((B, S, H, d), 4000 + i, device="cuda") for i in range(3)]
    mx = [fa.quantize_mxfp8(X[0], 0), fa.quantize_mxfp8(X[1], 0), fa.quantize_mxfp8(X[2], 1)]
    blk = [fa.quantize_fp8(x) for x in X]
    o_mx, l_mx = fa.fwd_mxfp8(*[c for c, _ in mx], *[s for _, s in mx], False)
    o_blk, _ = fa.fwd_fp8(*[c for c, _ in blk], *[s for _, s in blk], False)
    torch.cuda.synchronize()
    rows = inputs.sample_indices(S, 61, 4001, always=(0, 1, S - 1))
    bi = [0] * (len(rows) * H)
    hi = [h for h in range(H) for _ in rows]
    ii = [i for _ in range(H) for i in rows]
    deq = [ofp8.dequantize_mx(c.cpu().numpy(), s.cpu().numpy(), a)
           for (c, s), a in zip(mx, ("d", "d", "s"))]
    o_ref_m, l_ref_m = oracle.attention_fwd_rows(*deq, bi, hi, ii, False)
    got = o_mx[bi, ii, hi].float().cpu().numpy()
    print("  MX vs oracle on dequantised inputs:", flush=True)
    Qr = deq[0][0][np.asarray(ii), np.asarray(hi)]
    absdot = np.array([(np.abs(Qr[r]) @ np.abs(deq[1][0, :, hi[r]]).T).max() / np.sqrt(d)
                       for r in range(len(ii))])
    check_lse_fp8(l_mx[bi, hi, ii].cpu().numpy(), l_ref_m, absdot)
    bound = o_bound_rows(*deq, 1, 1.0 / np.sqrt(d), False, bi, hi, ii, l_ref_m, o_ref_m)
    check_o_fp8(got, o_ref_m, bound, bi, hi)
    o_ref, _ = oracle.attention_fwd_rows(*[x.cpu() for x in X], bi, hi, ii, False)
    deq_b = [ofp8.dequantize_blocks(c.cpu().numpy(), s.cpu().numpy()) for c, s in blk]
    o_deq_b, _ = oracle.attention_fwd_rows(*deq_b, bi, hi, ii, False)
    rms = {"exact_on_mx_inputs": float(np.sqrt(np.mean((o_ref_m - o_ref) ** 2))),
           "exact_on_block128_inputs": float(np.sqrt(np.mean((o_deq_b - o_ref) ** 2)))}
    for name, o in (("mxfp8", o_mx), ("fp8_block128", o_blk)):
        v = o[bi, ii, hi].float().cpu().numpy()
        rms[name] = float(np.sqrt(np.mean((v - o_ref) ** 2)))
    print(f"  RMS vs fp64 on original inputs: {rms}", flush=True)
    assert all(np.isfinite(v) for v in rms.values())
