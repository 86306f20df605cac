"""The Python binding rejects mismatched tensors before it calls the library.

The C ABI takes one dtype and raw element strides per call, so a k of another
dtype, an output of the wrong shape or a host tensor would become an
out-of-bounds access or a fault on the GPU.  These CPU-only checks make the
library unreachable (any call fails the test) and assert that each mismatch
raises ValueError first; a call whose tensors are right in every respect but
live in host memory is rejected for its device.
"""
import pytest
import torch

from io_aware_exact_amd import fa

bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def unreachable():
        raise AssertionError("the library was called before the arguments were checked")
    monkeypatch.setattr(fa, "lib", unreachable)


def dense(B=2, Sq=16, Sk=24, Hq=4, Hkv=2, d=64, dtype=bf):
    q = torch.zeros(B, Sq, Hq, d, dtype=dtype)
    k = torch.zeros(B, Sk, Hkv, d, dtype=dtype)
    v = torch.zeros(B, Sk, Hkv, d, dtype=dtype)
    return q, k, v


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_fwd_mismatches():
    q, k, v = dense()
    raises("share one dtype", fa.fwd, q, k.float(), v)
    raises("share one dtype", fa.fwd, q.float(), k, v)
    raises("same shape", fa.fwd, q, k, v[:, :20])
    raises("head dimension", fa.fwd, q, k[..., :32], v[..., :32])
    raises("batch size", fa.fwd, q, k[:1], v[:1])
    raises("not supported", fa.fwd, q.half(), k.half(), v.half())
    raises("out must have shape", fa.fwd, q, k, v, out=torch.zeros(2, 16, 4, 32, dtype=bf))
    raises("out must be", fa.fwd, q, k, v, out=torch.zeros(2, 16, 4, 64, dtype=f32))
    raises("out must be", fa.fwd, q.float(), k.float(), v.float(), out=torch.zeros(2, 16, 4, 64, dtype=bf))
    raises("lse must have shape", fa.fwd, q, k, v, lse=torch.zeros(2, 16, 4))
    raises("lse must be", fa.fwd, q, k, v, lse=torch.zeros(2, 4, 16, dtype=bf))
    raises("workspace", fa.fwd, q, k, v, workspace=torch.zeros(16, dtype=f32))
    raises("GPU tensor", fa.fwd, q, k, v)


def test_bwd_mismatches():
    q, k, v = dense()
    o, do = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros(2, 4, 16)
    grads = (torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v))
    raises("dout must have shape", fa.bwd, q, k, v, o, do[:, :8], lse, out=grads)
    raises("o must be", fa.bwd, q, k, v, o.float(), do, lse, out=grads)
    raises("dk must have shape", fa.bwd, q, k, v, o, do, lse, out=(grads[0], grads[0], grads[2]))
    raises("dv must be", fa.bwd, q, k, v, o, do, lse, out=(grads[0], grads[1], grads[2].float()))
    raises("lse must have shape", fa.bwd, q, k, v, o, do, torch.zeros(2, 16, 4), out=grads)
    raises("not supported", fa.bwd, q.float(), k.float(), v.float(), o, do, lse, out=grads)
    raises("GPU tensor", fa.bwd, q, k, v, o, do, lse, out=grads)


def test_varlen_mismatches():
    q = torch.zeros(40, 4, 64, dtype=bf)
    k = torch.zeros(50, 2, 64, dtype=bf)
    v = torch.zeros(50, 2, 64, dtype=bf)
    cu = torch.tensor([0, 20, 40], dtype=torch.int32)
    cuk = torch.tensor([0, 25, 50], dtype=torch.int32)
    raises("share one dtype", fa.fwd_varlen, q, k, v.float(), cu, cuk, 20, 25)
    raises("int32", fa.fwd_varlen, q, k, v, cu.long(), cuk, 20, 25)
    raises("nseq", fa.fwd_varlen, q, k, v, cu, cuk[:2], 20, 25)
    raises("lse must have shape", fa.fwd_varlen, q, k, v, cu, cuk, 20, 25, lse=torch.zeros(40, 4))
    raises("GPU tensor", fa.fwd_varlen, q, k, v, cu, cuk, 20, 25)
    o, do, lse = torch.zeros_like(q), torch.zeros_like(q), torch.zeros(4, 40)
    grads = (torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v))
    raises("dq must have shape", fa.bwd_varlen, q, k, v, o, do, lse, cu, cuk, 20, 25,
           out=(grads[1], grads[1], grads[2]))
    raises("GPU tensor", fa.bwd_varlen, q, k, v, o, do, lse, cu, cuk, 20, 25, out=grads)


def test_kvcache_mismatches():
    B, Hq, Hkv, d, ps = 2, 4, 2, 64, 16
    q = torch.zeros(B, 1, Hq, d, dtype=bf)
    kc = torch.zeros(8, ps, Hkv, d, dtype=bf)
    vc = torch.zeros(8, ps, Hkv, d, dtype=bf)
    lens = torch.zeros(B, dtype=torch.int32)
    bt = torch.zeros(B, 4, dtype=torch.int32)
    kn = torch.zeros(B, 1, Hkv, d, dtype=bf)
    raises("same shape", fa.fwd_kvcache, q, kc, vc[:4], lens, bt, workspace=torch.zeros(1, dtype=u8))
    raises("bf16", fa.fwd_kvcache, q, kc.float(), vc, lens, bt, workspace=torch.zeros(1, dtype=u8))
    raises("cache_seqlens", fa.fwd_kvcache, q, kc, vc, lens[:1], bt, workspace=torch.zeros(1, dtype=u8))
    raises("go together", fa.fwd_kvcache, q, kc, vc, lens, bt, kn, None, workspace=torch.zeros(1, dtype=u8))
    raises("v_new must have shape", fa.fwd_kvcache, q, kc, vc, lens, bt, kn, kn[:, :, :1],
           workspace=torch.zeros(1, dtype=u8))
    raises("block_table", fa.fwd_kvcache, q, kc, vc, lens, bt[:1], workspace=torch.zeros(1, dtype=u8))
    raises("GPU tensor", fa.fwd_kvcache, q, kc, vc, lens, bt, kn, kn.clone(),
           workspace=torch.zeros(1, dtype=u8))


def test_fp8_and_merge_mismatches():
    q8 = torch.zeros(1, 200, 2, 64, dtype=u8)
    k8 = torch.zeros(1, 300, 2, 64, dtype=u8)
    sq, sk = torch.zeros(1, 2, 2), torch.zeros(1, 2, 3)
    raises("same shape", fa.fwd_fp8, q8, k8, k8[:, :10], sq, sk, sk)
    raises("E4M3 codes", fa.fwd_fp8, q8.to(bf), k8, k8, sq, sk, sk)
    raises("k_descale must have shape", fa.fwd_fp8, q8, k8, k8, sq, sq, sk)
    raises("GPU tensor", fa.fwd_fp8, q8, k8, k8, sq, sk, sk)
    qs = torch.zeros(1, 200, 2, 2, dtype=u8)
    ks = torch.zeros(1, 300, 2, 2, dtype=u8)
    vs = torch.zeros(1, 2, 10, 64, dtype=u8)
    raises("v_scale must have shape", fa.fwd_mxfp8, q8, k8, k8, qs, ks, vs[:, :, :9])
    raises("GPU tensor", fa.fwd_mxfp8, q8, k8, k8, qs, ks, vs)
    parts = torch.zeros(3, 1, 8, 2, 64)
    raises("lse_parts must have shape", fa.merge, parts, torch.zeros(3, 1, 8, 2))
    raises("GPU tensor", fa.merge, parts, torch.zeros(3, 1, 2, 8))
    raises("fp32", fa.quantize_fp8, torch.zeros(1, 8, 2, 64, dtype=bf))
    raises("GPU tensor", fa.quantize_mxfp8, torch.zeros(1, 8, 2, 64), 0)
