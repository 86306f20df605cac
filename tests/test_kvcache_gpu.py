"""GPU parity of KV-cache attention (fa_fwd_kvcache): the append into a
paged or dense cache, then attention over each sequence's cached plus
appended tokens, against the fp64 oracle.  Covers the split-KV path (few
query rows per kv head) and the tiled path (chunked prefill against a
cache), page sizes from 16 to 256, sequences with no cached tokens, and
bitwise equality of the tiled path with the dense forward on the same keys.
Cache slots that hold no token of any sequence are filled with NaN, so a
read past a sequence's end shows up in the output."""
import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_amd import fa, inputs
from parity import Guarded, check_lse, check_o

pytestmark = pytest.mark.gpu


def same_cache(got, ref):
    """Bitwise equal where ref holds a number, NaN where ref holds NaN (the
    NaN payload does not survive the oracle's float64 round trip)."""
    got = got.cpu()
    nan = torch.isnan(ref)
    return bool(torch.equal(torch.isnan(got), nan) and
                torch.equal(got[~nan].view(torch.int16), ref[~nan].view(torch.int16)))


def build_case(lens, snew, sq, Hq, Hkv, d, page_size, paged, seed, spare=3, ramp=False):
    """Cache, block table and inputs.  Paged: each sequence gets
    ceil((len + snew) / page_size) pages, handed out in a shuffled order
    from a pool with `spare` unused pages.  Dense: a [B, capacity] cache.
    ramp: the key at position j of a sequence of total length n is scaled
    by 1 + 3 j / n, so later keys give larger scores."""
    B = len(lens)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    need = [-(-(L + snew) // page_size) for L in lens]
    if paged:
        npages = sum(need) + spare
        perm = torch.randperm(npages, generator=g)
        maxp = max(max(need), 1)
        bt = torch.zeros((B, maxp + 1), dtype=torch.int32)   # one spare column
        at = 0
        for b in range(B):
            bt[b, :need[b]] = perm[at:at + need[b]].to(torch.int32)
            at += need[b]
        cap = page_size
    else:
        npages, bt, cap = B, None, max(L + snew for L in lens) + 5
    kc = torch.full((npages, cap, Hkv, d), float("nan"))
    vc = torch.full((npages, cap, Hkv, d), float("nan"))
    grow = lambda j, b: (1.0 + 3.0 * j / (lens[b] + snew)) if ramp else 1.0
    for b, L in enumerate(lens):
        for j in range(L):
            p, s = (int(bt[b, j // page_size]), j % page_size) if paged else (b, j)
            kc[p, s] = torch.randn((Hkv, d), generator=g) * grow(j, b)
            vc[p, s] = torch.randn((Hkv, d), generator=g)
    kn = torch.randn((B, snew, Hkv, d), generator=g)
    for b, L in enumerate(lens):
        for i in range(snew):
            kn[b, i] *= grow(L + i, b)
    vn = torch.randn((B, snew, Hkv, d), generator=g)
    q = torch.randn((B, sq, Hq, d), generator=g)
    bf = lambda x: x.to(torch.bfloat16)
    return (bf(q), bf(kc), bf(vc), torch.tensor(lens, dtype=torch.int32), bt, bf(kn), bf(vn))


def run_kvcache(lens, snew, sq, Hq, Hkv, d, page_size, paged, causal, seed,
                use_workspace=True, scale=None, ramp=False):
    print(f"kvcache lens={lens} snew={snew} sq={sq} Hq={Hq} Hkv={Hkv} d={d} page={page_size} "
          f"paged={paged} causal={causal} ws={use_workspace} seed={seed} ramp={ramp}", flush=True)
    q, kc, vc, lens_t, bt, kn, vn = build_case(lens, snew, sq, Hq, Hkv, d, page_size, paged, seed,
                                               ramp=ramp)
    dq, dkc, dvc = q.cuda(), kc.cuda(), vc.cuda()
    dlens = lens_t.cuda()
    dbt = bt.cuda() if bt is not None else None
    dkn, dvn = (kn.cuda(), vn.cuda()) if snew else (None, None)
    B = len(lens)
    go = Guarded((B, sq, Hq, d), torch.bfloat16)
    gl = Guarded((B, Hq, sq), torch.float32)
    # without a workspace argument the binding allocates one when the split
    # path applies; an empty one forces the tiled path
    ws = None if use_workspace else torch.empty(0, dtype=torch.uint8, device="cuda")
    fa.fwd_kvcache(dq, dkc, dvc, dlens, dbt, dkn, dvn, causal, scale, out=go.t, lse=gl.t,
                   workspace=ws)
    torch.cuda.synchronize()
    go.check_guards()
    gl.check_guards()
    # the cache after the append: exactly the oracle's, bit for bit (NaN slots included)
    kc_r, vc_r = (kc, vc) if not snew else tuple(
        torch.from_numpy(x).to(torch.bfloat16) for x in
        oracle.kvcache_append(kc, vc, lens_t.numpy(), kn, vn, None if bt is None else bt.numpy()))
    assert same_cache(dkc, kc_r) and same_cache(dvc, vc_r)
    o_r, lse_r = oracle.attention_kvcache(q, kc, vc, lens_t.numpy(),
                                          None if bt is None else bt.numpy(),
                                          kn if snew else None, vn if snew else None, causal, scale)
    check_o("O", go.t.float().cpu().numpy(), o_r)
    check_lse("LSE", gl.t.cpu().numpy(), lse_r)
    return go.t, gl.t, (dq, dkc, dvc, dlens, dbt)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("page_size,paged", [(16, True), (64, True), (256, True), (0, False)])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_append(d, page_size, paged, causal):
    # one new token per sequence: an empty cache, a short one, tails
    run_kvcache([0, 37, 300, 129], 1, 1, 8, 2, d, page_size or 1, paged, causal, seed=11 + d)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_several_new_tokens(causal):
    # Sq = Snew = 4 rows per sequence, group 8: 32 query rows per kv head
    run_kvcache([5, 0, 250], 4, 4, 16, 2, 128, 32, True, causal, seed=21)


def test_decode_without_append():
    # attention over what is cached, nothing appended; a query longer than the
    # cache of one sequence (causal rows that see no key)
    run_kvcache([40, 3, 77], 0, 4, 4, 4, 64, 16, True, True, seed=31)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("page_size", [16, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_chunked_prefill(d, page_size, causal):
    # Sq = Snew = 200 new tokens appended after 0, 100 and 513 cached ones
    run_kvcache([0, 100, 513], 200, 200, 4, 1, d, page_size, True, causal, seed=41)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_chunked_prefill_growing_scores(d, causal):
    # keys grow along each sequence, so the running max moves while the
    # cached and the appended keys stream
    run_kvcache([0, 100, 513], 200, 200, 4, 1, d, 64, True, causal, seed=43, ramp=True)


@pytest.mark.parametrize("page_size", [16, 32, 64, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_short_chunk_d128(page_size, causal):
    # at most 128 new rows at d = 128 (the one-group kernel's cache paths):
    # small pages read row by row, larger ones tile by tile
    run_kvcache([0, 100, 513], 96, 96, 8, 2, 128, page_size, True, causal, seed=47 + page_size)


def test_decode_shape_without_workspace_takes_tiled_path():
    run_kvcache([300, 17], 1, 1, 8, 2, 128, 64, True, True, seed=51, use_workspace=False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_cache_prefill(d, causal):
    run_kvcache([64, 255], 70, 70, 8, 4, d, 1, False, causal, seed=61)


def test_tiled_path_equals_dense_forward():
    # the tiled kernels walk keys in the same order over the cache pages as
    # over a contiguous K/V, so results are bitwise those of fa_fwd
    lens, snew = [100, 513, 7], 150
    o, lse, (dq, dkc, dvc, dlens, dbt) = run_kvcache(lens, snew, snew, 4, 2, 128, 16, True, True,
                                                     seed=71)
    for b, L in enumerate(lens):
        n = L + snew
        j = torch.arange(n, device="cuda")
        pages = dbt[b].long()[j // 16]
        kk = dkc[pages, j % 16][None].contiguous()
        vv = dvc[pages, j % 16][None].contiguous()
        od, ld = fa.fwd(dq[b:b + 1], kk, vv, True)
        assert torch.equal(od[0], o[b]) and torch.equal(ld[0], lse[b])


def test_append_only():
    # Sq = 0: the call only writes the new rows into the cache
    q, kc, vc, lens_t, bt, kn, vn = build_case([3, 20], 5, 0, 2, 2, 64, 16, True, seed=81)
    dkc, dvc = kc.cuda(), vc.cuda()
    fa.fwd_kvcache(q.cuda(), dkc, dvc, lens_t.cuda(), bt.cuda(), kn.cuda(), vn.cuda())
    torch.cuda.synchronize()
    kc_r, vc_r = oracle.kvcache_append(kc, vc, lens_t.numpy(), kn, vn, bt.numpy())
    assert same_cache(dkc, torch.from_numpy(kc_r).to(torch.bfloat16))
    assert same_cache(dvc, torch.from_numpy(vc_r).to(torch.bfloat16))


def test_deterministic():
    q, kc, vc, lens_t, bt, kn, vn = build_case([500, 1000], 1, 1, 8, 2, 128, 64, True, seed=91)
    args = (q.cuda(), kc.cuda(), vc.cuda(), lens_t.cuda(), bt.cuda(), kn.cuda(), vn.cuda(), True)
    runs = [fa.fwd_kvcache(*args) for _ in range(3)]
    for o, l in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(l, runs[0][1])


def test_full_size_paged_decode():
    """Decode against a paged cache at the dense decode benchmark's size: B=64,
    Hq=32, Hkv=8, d=128, 32767 cached tokens plus one appended per sequence,
    256-token pages in a shuffled order.  Sampled sequences against the
    oracle (all heads), the cache's new rows checked bitwise."""
    B, Hq, Hkv, d, ps, L = 64, 32, 8, 128, 256, 32767
    print(f"kvcache full size B={B} L={L} page={ps}", flush=True)
    per = (L + 1 + ps - 1) // ps
    g = torch.Generator(device="cuda")
    g.manual_seed(3200)
    kc = torch.randn((B * per, ps, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((B * per, ps, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, 1, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn((B, 1, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((B, 1, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    gc = torch.Generator(device="cpu")
    gc.manual_seed(3201)
    bt = torch.randperm(B * per, generator=gc).to(torch.int32).view(B, per).cuda()
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o, lse = fa.fwd_kvcache(q, kc, vc, lens, bt, kn, vn, True)
    torch.cuda.synchronize()
    j = torch.arange(L + 1, device="cuda")
    for b in (0, 37, 63):
        pages = bt[b].long()[j // ps]
        kk = kc[pages, j % ps]
        vv = vc[pages, j % ps]
        assert torch.equal(kk[L], kn[b, 0]) and torch.equal(vv[L], vn[b, 0])
        o_r, lse_r = oracle.attention_fwd(q[b:b + 1].cpu(), kk[None].cpu(), vv[None].cpu(), True)
        check_o(f"O seq {b}", o[b:b + 1].float().cpu().numpy(), o_r)
        check_lse(f"LSE seq {b}", lse[b:b + 1].cpu().numpy(), lse_r)


def test_full_size_paged_prefill():
    """A prefill chunk against a paged cache at the benchmark's size: B=4,
    Hq=32, Hkv=8, d=128, 15360 cached tokens and 1024 appended per sequence,
    causal, 256-token pages in a shuffled order (the tiled path, pages read
    by DMA).  Sampled query rows of every sequence and head against the
    oracle, the cache's new rows checked bitwise."""
    B, Hq, Hkv, d, ps, L0, sn = 4, 32, 8, 128, 256, 15360, 1024
    L = L0 + sn
    grp = Hq // Hkv
    print(f"kvcache full size prefill B={B} cached={L0} new={sn} page={ps}", flush=True)
    per = (L + ps - 1) // ps
    g = torch.Generator(device="cuda")
    g.manual_seed(3300)
    kc = torch.randn((B * per, ps, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((B * per, ps, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, sn, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn((B, sn, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((B, sn, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    gc = torch.Generator(device="cpu")
    gc.manual_seed(3301)
    bt = torch.randperm(B * per, generator=gc).to(torch.int32).view(B, per).cuda()
    lens = torch.full((B,), L0, dtype=torch.int32, device="cuda")
    o, lse = fa.fwd_kvcache(q, kc, vc, lens, bt, kn, vn, True)
    torch.cuda.synchronize()
    j = torch.arange(L, device="cuda")
    for b in range(B):
        pages = bt[b].long()[j // ps]
        kk = kc[pages, j % ps]
        vv = vc[pages, j % ps]
        assert torch.equal(kk[L0:], kn[b]) and torch.equal(vv[L0:], vn[b])
        pos = np.asarray(inputs.sample_indices(sn, 12, 3302 + b, always=(0, 1, sn - 1)), np.int64)
        for kvh in range(Hkv):
            hs = list(range(kvh * grp, (kvh + 1) * grp))
            qr = q[b, pos][:, hs, :].transpose(0, 1).reshape(-1, d).cpu()
            o_r, l_r = oracle.head_fwd(qr, np.tile(pos, grp), kk[:, kvh].cpu(), vv[:, kvh].cpu(),
                                       L - sn, True, 1.0 / np.sqrt(d))
            got_o = o[b, pos][:, hs, :].transpose(0, 1).reshape(-1, d).float().cpu().numpy()
            got_l = lse[b, hs][:, pos].reshape(-1).cpu().numpy()
            check_o(f"O seq {b} kv head {kvh}", got_o, o_r)
            check_lse(f"LSE seq {b} kv head {kvh}", got_l, l_r)

