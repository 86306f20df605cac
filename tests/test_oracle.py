"""Pins for the fp64 oracle: each test ties it to something other than itself
(a library routine computed a different way, a closed form, an invariant of
exact attention, brute force on tiny inputs, finite differences)."""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_amd import inputs

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def rnd(shape, seed):
    return inputs.normal(shape, seed, dtype=torch.float64).numpy()


def sdpa_ref(q, k, v, causal, scale):
    """torch's fp64 CPU attention with an explicit bottom-right causal mask and
    kv heads repeated for GQA.  Returns o [B,Sq,Hq,d], lse [B,Hq,Sq]."""
    q, k, v = (torch.from_numpy(np.asarray(x, np.float64)) for x in (q, k, v))
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    k = k.repeat_interleave(grp, dim=2)
    v = v.repeat_interleave(grp, dim=2)
    qt, kt, vt = (x.transpose(1, 2) for x in (q, k, v))
    mask = None
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        mask = j <= i + (Sk - Sq)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale)
    s = torch.matmul(qt, kt.transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.transpose(1, 2).numpy(), lse.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 7, 7, 2, 2, 4), (2, 33, 33, 4, 2, 16),
                                   (1, 5, 12, 3, 1, 8), (2, 64, 40, 2, 2, 64)])
def test_fwd_matches_sdpa_fp64(shape, causal):
    B, Sq, Sk, Hq, Hkv, d = shape
    q = rnd((B, Sq, Hq, d), 1)
    k = rnd((B, Sk, Hkv, d), 2)
    v = rnd((B, Sk, Hkv, d), 3)
    scale = 1.0 / math.sqrt(d)
    if causal and Sq > Sk:
        pytest.skip("fully masked rows are covered by test_fully_masked_rows")
    o, lse = oracle.attention_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = sdpa_ref(q, k, v, causal, scale)
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)


def test_single_key_closed_form():
    # Sk = 1: O = V, LSE = scale * <q, k>
    q = rnd((1, 4, 2, 8), 4)
    k = rnd((1, 1, 2, 8), 5)
    v = rnd((1, 1, 2, 8), 6)
    o, lse = oracle.attention_fwd(q, k, v, False, 0.7)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=1e-15)
    expect = 0.7 * np.einsum("bshd,bhd->bhs", q, k[:, 0])
    np.testing.assert_allclose(lse, expect, atol=1e-13)


def test_two_keys_closed_form():
    # Sk = 2: O = sigma(s1 - s2) v1 + sigma(s2 - s1) v2, LSE = logaddexp(s1, s2)
    q = rnd((1, 3, 1, 4), 7)
    k = rnd((1, 2, 1, 4), 8)
    v = rnd((1, 2, 1, 4), 9)
    scale = 0.5
    o, lse = oracle.attention_fwd(q, k, v, False, scale)
    for i in range(3):
        s1 = scale * float(q[0, i, 0] @ k[0, 0, 0])
        s2 = scale * float(q[0, i, 0] @ k[0, 1, 0])
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        w2 = 1.0 / (1.0 + math.exp(s1 - s2))
        np.testing.assert_allclose(o[0, i, 0], w1 * v[0, 0, 0] + w2 * v[0, 1, 0], atol=1e-14)
        assert abs(lse[0, 0, i] - np.logaddexp(s1, s2)) < 1e-14


def test_brute_force_hand_example():
    # B=H=1, Sq=2, Sk=3, d=2, scale=1: scores of row 0 are (1, 0, 0), row 1
    # (0, 2, 1).  Written out with math.e, no shared routine.
    q = np.array([[[[1.0, 0.0]], [[0.0, 1.0]]]])
    k = np.array([[[[1.0, 0.0]], [[0.0, 2.0]], [[0.0, 1.0]]]])
    v = np.array([[[[1.0, 10.0]], [[2.0, 20.0]], [[4.0, 40.0]]]])
    o, lse = oracle.attention_fwd(q, k, v, False, 1.0)
    e = math.e
    z0 = e + 2.0
    np.testing.assert_allclose(o[0, 0, 0], [(e * 1 + 2 + 4) / z0, (e * 10 + 20 + 40) / z0], atol=1e-14)
    assert abs(lse[0, 0, 0] - math.log(z0)) < 1e-14
    z1 = 1.0 + e * e + e
    np.testing.assert_allclose(o[0, 1, 0], [(1 + 2 * e * e + 4 * e) / z1, (10 + 20 * e * e + 40 * e) / z1], atol=1e-13)
    assert abs(lse[0, 0, 1] - math.log(z1)) < 1e-14
    # causal (bottom-right, diag = Sk - Sq = 1): row 0 sees keys 0..1, row 1 all
    o, lse = oracle.attention_fwd(q, k, v, True, 1.0)
    np.testing.assert_allclose(o[0, 0, 0], [(e * 1 + 2) / (e + 1), (e * 10 + 20) / (e + 1)], atol=1e-14)
    assert abs(lse[0, 0, 0] - math.log(e + 1)) < 1e-14
    np.testing.assert_allclose(o[0, 1, 0], [(1 + 2 * e * e + 4 * e) / z1, (10 + 20 * e * e + 40 * e) / z1], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows(causal):
    q = rnd((1, 19, 2, 8), 10)
    k = rnd((1, 23, 2, 8), 11)
    v = rnd((1, 23, 2, 8), 12)
    o, lse, p = oracle.attention_fwd(q, k, v, causal, 0.4, want_probs=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    assert (p >= 0).all()
    if causal:
        i = np.arange(19)[:, None]
        j = np.arange(23)[None, :]
        assert (p[..., ~(j <= i + 4)] == 0).all()
    # O is P V and lies in the per-column hull of the visible V rows
    o2 = np.einsum("bhij,bjhc->bihc", p, v)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    for h in range(2):
        for i in range(19):
            vis = p[0, h, i] > 0
            lo = v[0, vis, h].min(0)
            hi = v[0, vis, h].max(0)
            assert (o[0, i, h] >= lo - 1e-12).all() and (o[0, i, h] <= hi + 1e-12).all()


def test_identical_keys_mean():
    S, d = 17, 8
    q = rnd((1, S, 2, d), 13)
    k = np.broadcast_to(rnd((1, 1, 2, d), 14), (1, S, 2, d)).copy()
    v = rnd((1, S, 2, d), 15)
    scale = 0.3
    o, lse = oracle.attention_fwd(q, k, v, False, scale)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(1, keepdims=True), o.shape), atol=1e-13)
    expect = scale * np.einsum("bshd,bhd->bhs", q, k[:, 0]) + math.log(S)
    np.testing.assert_allclose(lse, expect, atol=1e-13)
    o, lse = oracle.attention_fwd(q, k, v, True, scale)
    prefix = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    np.testing.assert_allclose(o, prefix, atol=1e-13)


def test_causal_row0_is_v0():
    q = rnd((2, 9, 2, 16), 16)
    k = rnd((2, 9, 2, 16), 17)
    v = rnd((2, 9, 2, 16), 18)
    o, lse = oracle.attention_fwd(q, k, v, True, 0.25)
    np.testing.assert_allclose(o[:, 0], v[:, 0], atol=1e-15)
    np.testing.assert_allclose(lse[:, :, 0], 0.25 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]), atol=1e-13)


def test_fully_masked_rows():
    # Sq > Sk, causal, bottom-right: rows i < Sq - Sk see no key.
    q = rnd((1, 6, 1, 4), 19)
    k = rnd((1, 3, 1, 4), 20)
    v = rnd((1, 3, 1, 4), 21)
    o, lse = oracle.attention_fwd(q, k, v, True, 0.5)
    assert (o[0, :3] == 0).all() and np.isneginf(lse[0, 0, :3]).all()
    # row 3 sees key 0 only
    np.testing.assert_allclose(o[0, 3, 0], v[0, 0, 0], atol=1e-15)
    _, _, dq, dk, dv = oracle.attention_bwd(q, k, v, rnd((1, 6, 1, 4), 22), True, 0.5)
    assert (dq[0, :3] == 0).all()


def test_shift_permutation_linearity_scale0():
    q = rnd((1, 11, 2, 8), 23)
    k = rnd((1, 13, 2, 8), 24)
    v = rnd((1, 13, 2, 8), 25)
    scale = 0.35
    o, lse = oracle.attention_fwd(q, k, v, False, scale)
    u = rnd((1, 1, 2, 8), 26)
    o2, lse2 = oracle.attention_fwd(q, k + u, v, False, scale)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2 - lse, scale * np.einsum("bshd,bhd->bhs", q, u[:, 0]), atol=1e-12)
    perm = np.random.RandomState(0).permutation(13)
    o3, lse3 = oracle.attention_fwd(q, k[:, perm], v[:, perm], False, scale)
    np.testing.assert_allclose(o3, o, atol=1e-12)
    np.testing.assert_allclose(lse3, lse, atol=1e-12)
    w = rnd((1, 13, 2, 8), 27)
    oa, _ = oracle.attention_fwd(q, k, 2.0 * v - 3.0 * w, False, scale)
    ow, _ = oracle.attention_fwd(q, k, w, False, scale)
    np.testing.assert_allclose(oa, 2.0 * o - 3.0 * ow, atol=1e-12)
    o0, lse0 = oracle.attention_fwd(q, k, v, False, 0.0)
    np.testing.assert_allclose(o0, np.broadcast_to(v.mean(1, keepdims=True), o0.shape), atol=1e-13)
    np.testing.assert_allclose(lse0, math.log(13), atol=1e-13)


def test_gqa_equals_repeated_mha():
    q = rnd((2, 10, 8, 8), 28)
    k = rnd((2, 12, 2, 8), 29)
    v = rnd((2, 12, 2, 8), 30)
    do = rnd((2, 10, 8, 8), 31)
    kr, vr = k.repeat(4, axis=2), v.repeat(4, axis=2)
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, causal, 0.3)
        o2, lse2 = oracle.attention_fwd(q, kr, vr, causal, 0.3)
        np.testing.assert_allclose(o, o2, atol=1e-14)
        np.testing.assert_allclose(lse, lse2, atol=1e-14)
        _, _, dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, 0.3)
        _, _, dq2, dk2, dv2 = oracle.attention_bwd(q, kr, vr, do, causal, 0.3)
        np.testing.assert_allclose(dq, dq2, atol=1e-13)
        np.testing.assert_allclose(dk, dk2.reshape(2, 12, 2, 4, 8).sum(3), atol=1e-13)
        np.testing.assert_allclose(dv, dv2.reshape(2, 12, 2, 4, 8).sum(3), atol=1e-13)


def test_rows_entry_matches_dense():
    q = rnd((2, 40, 4, 16), 32)
    k = rnd((2, 40, 2, 16), 33)
    v = rnd((2, 40, 2, 16), 34)
    o, lse = oracle.attention_fwd(q, k, v, True, 0.25)
    b = [0, 1, 1, 0, 1]
    h = [0, 3, 2, 1, 0]
    i = [0, 39, 17, 5, 22]
    orow, lrow = oracle.attention_fwd_rows(q, k, v, b, h, i, True, 0.25)
    for r in range(5):
        np.testing.assert_allclose(orow[r], o[b[r], i[r], h[r]], atol=1e-15)
        assert abs(lrow[r] - lse[b[r], h[r], i[r]]) < 1e-15


def test_varlen_matches_block_diagonal_sdpa():
    lens = [5, 1, 17, 9]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    T = cu[-1]
    q = rnd((T, 4, 8), 35)
    k = rnd((T, 2, 8), 36)
    v = rnd((T, 2, 8), 37)
    for causal in (False, True):
        o, lse = oracle.attention_fwd_varlen(q, k, v, cu, cu, causal, 0.3)
        seq = np.repeat(np.arange(len(lens)), lens)
        pos = np.concatenate([np.arange(L) for L in lens])
        allowed = seq[:, None] == seq[None, :]
        if causal:
            allowed &= pos[None, :] <= pos[:, None]
        qt = torch.from_numpy(q).transpose(0, 1)
        kt = torch.from_numpy(k).repeat_interleave(2, dim=1).transpose(0, 1)
        vt = torch.from_numpy(v).repeat_interleave(2, dim=1).transpose(0, 1)
        m = torch.from_numpy(allowed)
        o_ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=0.3)
        s = (qt @ kt.transpose(-1, -2) * 0.3).masked_fill(~m, float("-inf"))
        np.testing.assert_allclose(o, o_ref.transpose(0, 1).numpy(), atol=1e-12)
        np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-12)


def torch_fwd_bwd(q, k, v, do, causal, scale):
    """fp64 autograd through an independent torch implementation."""
    q, k, v, do = (torch.from_numpy(np.asarray(x, np.float64)) for x in (q, k, v, do))
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    Hq, Hkv = q.shape[2], k.shape[2]
    kr = k.repeat_interleave(Hq // Hkv, dim=2)
    vr = v.repeat_interleave(Hq // Hkv, dim=2)
    Sq, Sk = q.shape[1], k.shape[1]
    s = torch.einsum("bihd,bjhd->bhij", q, kr) * scale
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        s = s.masked_fill(~(j <= i + Sk - Sq), float("-inf"))
    p = torch.softmax(s, -1)
    o = torch.einsum("bhij,bjhd->bihd", p, vr)
    o.backward(do)
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 8, 8, 2, 2, 4), (2, 21, 21, 4, 2, 16), (1, 7, 19, 2, 1, 8)])
def test_bwd_matches_torch_autograd(shape, causal):
    B, Sq, Sk, Hq, Hkv, d = shape
    q = rnd((B, Sq, Hq, d), 40)
    k = rnd((B, Sk, Hkv, d), 41)
    v = rnd((B, Sk, Hkv, d), 42)
    do = rnd((B, Sq, Hq, d), 43)
    scale = 1.0 / math.sqrt(d)
    o, lse, dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale)
    o_t, dq_t, dk_t, dv_t = torch_fwd_bwd(q, k, v, do, causal, scale)
    np.testing.assert_allclose(o, o_t, atol=1e-12)
    np.testing.assert_allclose(dq, dq_t, atol=1e-12)
    np.testing.assert_allclose(dk, dk_t, atol=1e-12)
    np.testing.assert_allclose(dv, dv_t, atol=1e-12)
    o2, lse2 = oracle.attention_fwd(q, k, v, causal, scale)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_finite_differences(causal):
    # dL/dx for L = sum(dO * O) by central differences of the oracle forward
    B, S, Hq, Hkv, d = 1, 6, 2, 1, 4
    q = rnd((B, S, Hq, d), 44)
    k = rnd((B, S, Hkv, d), 45)
    v = rnd((B, S, Hkv, d), 46)
    do = rnd((B, S, Hq, d), 47)
    scale = 0.6
    _, _, dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale)
    eps = 1e-6

    def loss(q_, k_, v_):
        o, _ = oracle.attention_fwd(q_, k_, v_, causal, scale)
        return float((o * do).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7, (name, idx, fd, g[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(causal):
    q = rnd((2, 15, 4, 8), 48)
    k = rnd((2, 15, 2, 8), 49)
    v = rnd((2, 15, 2, 8), 50)
    do = rnd((2, 15, 4, 8), 51)
    o, lse, dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, 0.4)
    # sum_j dS_ij = 0  =>  sum_j dK_j = 0 per kv head
    np.testing.assert_allclose(dk.sum(1), 0.0, atol=1e-12)
    # sum_j dV_j = sum over the group's query heads and rows of dO
    np.testing.assert_allclose(dv.sum(1), do.reshape(2, 15, 2, 2, 8).sum((1, 3)), atol=1e-12)
    if causal:
        np.testing.assert_allclose(dq[:, 0], 0.0, atol=1e-15)


def test_bwd_selected_slices():
    q = rnd((2, 9, 4, 8), 52)
    k = rnd((2, 9, 2, 8), 53)
    v = rnd((2, 9, 2, 8), 54)
    do = rnd((2, 9, 4, 8), 55)
    full = oracle.attention_bwd(q, k, v, do, True, 0.3)
    part = oracle.attention_bwd(q, k, v, do, True, 0.3, bh=[(1, 0)])
    np.testing.assert_allclose(part[2][1, :, 0:2], full[2][1, :, 0:2], atol=0)
    np.testing.assert_allclose(part[3][1, :, 0], full[3][1, :, 0], atol=0)
    assert (part[3][0] == 0).all()


def test_num_threads_positive():
    assert oracle.num_threads() >= 1


def test_varlen_bwd_matches_block_diagonal_autograd():
    """The packed backward oracle (the dense backward run per sequence) against
    fp64 autograd through the whole packed batch with a block-diagonal mask,
    including an empty sequence, one with no keys and one with no queries."""
    lens_q = [5, 0, 17, 9, 3, 0]
    lens_k = [7, 4, 17, 9, 0, 0]
    cq, ck = [0], [0]
    for a, b in zip(lens_q, lens_k):
        cq.append(cq[-1] + a)
        ck.append(ck[-1] + b)
    Tq, Tk = cq[-1], ck[-1]
    q = rnd((Tq, 4, 8), 41)
    k = rnd((Tk, 2, 8), 42)
    v = rnd((Tk, 2, 8), 43)
    do = rnd((Tq, 4, 8), 44)
    for causal in (False, True):
        o, lse, dq, dk, dv = oracle.attention_bwd_varlen(q, k, v, do, cq, ck, causal, 0.3)
        seq_q = np.repeat(np.arange(len(lens_q)), lens_q)
        seq_k = np.repeat(np.arange(len(lens_k)), lens_k)
        pos_q = np.concatenate([np.arange(L) for L in lens_q])
        pos_k = np.concatenate([np.arange(L) for L in lens_k])
        allowed = seq_q[:, None] == seq_k[None, :]
        if causal:
            diag = np.array(lens_k)[seq_q] - np.array(lens_q)[seq_q]
            allowed &= pos_k[None, :] <= pos_q[:, None] + diag[:, None]
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        kr = tk.repeat_interleave(2, dim=1)
        vr = tv.repeat_interleave(2, dim=1)
        s = torch.einsum("ihd,jhd->hij", tq, kr) * 0.3
        s = s.masked_fill(~torch.from_numpy(allowed)[None], float("-inf"))
        m = torch.amax(s, -1, keepdim=True)
        m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
        e = torch.exp(s - m)
        den = e.sum(-1, keepdim=True)
        p = e / torch.where(den > 0, den, torch.ones_like(den))
        o_ref = torch.einsum("hij,jhd->ihd", p, vr)
        o_ref.backward(torch.from_numpy(do))
        rows = seq_q >= 0
        np.testing.assert_allclose(o[rows], o_ref.detach().numpy()[rows], atol=1e-12)
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
        # rows with no visible key: LSE = -inf
        no_key = ~allowed.any(1)
        assert np.all(np.isneginf(lse[:, no_key]))


# ---- KV-cache oracle (append + paged cache) ----------------------------------

def paged_case(seed, lens, snew, sq, Hq=4, Hkv=2, d=16, page_size=4, npages=24):
    """A paged cache whose pages are handed out to the sequences in a
    shuffled order, plus new rows to append and queries."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    per = max(-(-(L + snew) // page_size) for L in lens)
    assert B * per <= npages
    phys = rng.permutation(npages)[:B * per].reshape(B, per)
    kc = rng.standard_normal((npages, page_size, Hkv, d))
    vc = rng.standard_normal((npages, page_size, Hkv, d))
    kn = rng.standard_normal((B, snew, Hkv, d))
    vn = rng.standard_normal((B, snew, Hkv, d))
    q = rng.standard_normal((B, sq, Hq, d))
    return q, kc, vc, np.asarray(lens), phys, kn, vn


def walk_pages(cache, table_row, n, page_size):
    """Tokens 0..n-1 of one sequence by concatenating its pages in order."""
    parts, left, p = [], n, 0
    while left > 0:
        take = min(page_size, left)
        parts.append(cache[table_row[p], :take])
        left -= take
        p += 1
    return np.concatenate(parts) if parts else cache[:0, 0]


@pytest.mark.parametrize("causal", [False, True])
def test_kvcache_matches_sdpa_on_page_walk(causal):
    # the append written by hand into a copy of the cache, the sequence read
    # back page by page, then torch's attention per sequence
    lens, snew, sq = [5, 0, 13, 8], 3, 3
    q, kc, vc, lens, bt, kn, vn = paged_case(1, lens, snew, sq)
    o, lse = oracle.attention_kvcache(q, kc, vc, lens, bt, kn, vn, causal, 0.3)
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(len(lens)):
        for i in range(snew):
            j = lens[b] + i
            kc2[bt[b, j // 4], j % 4] = kn[b, i]
            vc2[bt[b, j // 4], j % 4] = vn[b, i]
    for b in range(len(lens)):
        L = lens[b] + snew
        kk = walk_pages(kc2, bt[b], L, 4)[None]
        vv = walk_pages(vc2, bt[b], L, 4)[None]
        o_r, lse_r = sdpa_ref(q[b:b + 1], kk, vv, causal, 0.3)
        np.testing.assert_allclose(o[b], o_r[0], atol=1e-12)
        np.testing.assert_allclose(lse[b], lse_r[0], atol=1e-12)


def test_kvcache_append_writes_only_the_new_rows():
    lens, snew = [5, 0, 13], 3
    q, kc, vc, lens, bt, kn, vn = paged_case(2, lens, snew, 1)
    kc2, vc2 = oracle.kvcache_append(kc, vc, lens, kn, vn, bt)
    written = np.zeros(kc.shape[:2], dtype=bool)
    for b in range(len(lens)):
        for i in range(snew):
            j = lens[b] + i
            p, s = bt[b, j // 4], j % 4
            assert np.array_equal(kc2[p, s], kn[b, i]) and np.array_equal(vc2[p, s], vn[b, i])
            written[p, s] = True
    assert np.array_equal(kc2[~written], kc[~written]) and np.array_equal(vc2[~written], vc[~written])


def test_kvcache_invariant_under_page_permutation():
    # moving the physical pages and rewriting the block table changes nothing
    q, kc, vc, lens, bt, kn, vn = paged_case(3, [6, 11, 1], 2, 2)
    perm = np.random.default_rng(9).permutation(kc.shape[0])
    inv = np.argsort(perm)
    kcp, vcp = kc[perm], vc[perm]          # new page x holds old page perm[x]
    btp = inv[bt]
    o1, l1 = oracle.attention_kvcache(q, kc, vc, lens, bt, kn, vn, True)
    o2, l2 = oracle.attention_kvcache(q, kcp, vcp, lens, btp, kn, vn, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_kvcache_append_equals_prefilled_cache():
    # appending Snew rows = a cache that already holds them, with no append
    q, kc, vc, lens, bt, kn, vn = paged_case(4, [6, 0, 9], 3, 3)
    o1, l1 = oracle.attention_kvcache(q, kc, vc, lens, bt, kn, vn, True)
    kc2, vc2 = oracle.kvcache_append(kc, vc, lens, kn, vn, bt)
    o2, l2 = oracle.attention_kvcache(q, kc2, vc2, lens + 3, bt, None, None, True)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_kvcache_dense_cache_equals_dense_attention():
    # without a block table sequence b owns cache row b; a full cache with no
    # append is the dense forward, and shorter lengths are its prefix
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 4, 16))
    kc = rng.standard_normal((2, 10, 2, 16))
    vc = rng.standard_normal((2, 10, 2, 16))
    o1, l1 = oracle.attention_kvcache(q, kc, vc, [10, 10], None, None, None, True)
    o2, l2 = oracle.attention_fwd(q, kc, vc, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = oracle.attention_kvcache(q, kc, vc, [7, 10], None, None, None, False)
    o4, l4 = oracle.attention_fwd(q[:1], kc[:1, :7], vc[:1, :7], False)
    assert np.array_equal(o3[:1], o4) and np.array_equal(l3[:1], l4)


def test_kvcache_empty_sequence():
    # no cached tokens and nothing appended: O = 0, LSE = -inf
    q, kc, vc, lens, bt, kn, vn = paged_case(6, [0, 3], 0, 2)
    o, lse = oracle.attention_kvcache(q, kc, vc, lens, bt, None, None, False)
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(lse[1]))


def test_merge_of_key_shards_is_full_attention():
    # attention over all keys equals the merge of attention over key shards
    # (computed directly, no merge involved on the reference side)
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 9, 4, 16))
    k = rng.standard_normal((2, 23, 2, 16))
    v = rng.standard_normal((2, 23, 2, 16))
    o, lse = oracle.attention_fwd(q, k, v, False, 0.4)
    cuts = [0, 5, 6, 17, 23]
    parts = [oracle.attention_fwd(q, k[:, a:b], v[:, a:b], False, 0.4) for a, b in zip(cuts, cuts[1:])]
    om, lm = oracle.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(om, o, atol=1e-13)
    np.testing.assert_allclose(lm, lse, atol=1e-13)


def test_merge_with_empty_parts():
    # a part that sees no key (LSE = -inf) has no weight; a row no part sees
    # is O = 0, LSE = -inf
    rng = np.random.default_rng(13)
    o_parts = rng.standard_normal((3, 1, 2, 1, 8))
    lse = np.array([[[[0.5, -np.inf]]], [[[-np.inf, -np.inf]]], [[[1.5, -np.inf]]]])   # [3,1,1,2]
    o, l = oracle.merge_partials(o_parts, lse)
    w = np.exp(np.array([0.5, 1.5]) - 1.5)
    np.testing.assert_allclose(o[0, 0, 0], (w[0] * o_parts[0, 0, 0, 0] + w[1] * o_parts[2, 0, 0, 0]) / w.sum())
    assert l[0, 0, 0] == 1.5 + np.log(w.sum())
    assert np.all(o[0, 1, 0] == 0) and l[0, 0, 1] == -np.inf
