"""Parity at the full workload sizes, in the launch configurations the bench
times, on rows the oracle computes one by one:
  * the bf16 forward sweep: B*S = 16384 tokens, H = 16, d in {64, 128},
    S in {512, ..., 16384}, causal and not;
  * the packed varlen + GQA forward: 16 sequences with lengths uniform on
    [128, 32768], Hq = 32, Hkv = 8, d = 128, causal."""
import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_amd import fa, inputs
from parity import check_lse, check_o

pytestmark = pytest.mark.gpu

SWEEP_S = [512, 1024, 2048, 4096, 8192, 16384]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("S", SWEEP_S)
def test_forward_sweep_sampled(S, d, causal):
    B, H = 16384 // S, 16
    seed = 1000 + SWEEP_S.index(S) + 10 * (d == 128) + 100 * causal
    print(f"sweep B={B} S={S} H={H} d={d} causal={causal} seed={seed}", flush=True)
    q, k, v = inputs.qkv(B, S, S, H, H, d, seed, device="cuda")
    o, lse = fa.fwd(q, k, v, causal)
    torch.cuda.synchronize()
    rows = inputs.sample_indices(S, 13, seed, always=(0, 1, S - 1))
    bi, hi, ii = [], [], []
    for b in sorted({0, B - 1}):
        for h in range(H):
            for i in rows:
                bi.append(b), hi.append(h), ii.append(i)
    o_ref, lse_ref = oracle.attention_fwd_rows(q, k, v, bi, hi, ii, causal)
    check_o("O", o[bi, ii, hi].float().cpu().numpy(), o_ref)
    check_lse("LSE", lse[bi, hi, ii].cpu().numpy(), lse_ref)


def test_varlen_gqa_full_size_sampled():
    lens = inputs.varlen_lengths(16, 128, 32768, 3000)
    Hq, Hkv, d = 32, 8, 128
    grp = Hq // Hkv
    print(f"varlen full size lens={lens}", flush=True)
    q, k, v = inputs.packed_qkv(lens, lens, Hq, Hkv, d, 3001, device="cuda")
    cu = inputs.cu_seqlens(lens, device="cuda")
    o, lse = fa.fwd_varlen(q, k, v, cu, cu, max(lens), max(lens), True)
    torch.cuda.synchronize()
    cu_h = cu.cpu().numpy()
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for z, L in enumerate(lens):
        t0 = int(cu_h[z])
        pos = np.asarray(inputs.sample_indices(L, 14, 3002 + z, always=(0, L - 1)), np.int64)
        for g in range(Hkv):
            hs = list(range(g * grp, (g + 1) * grp))
            kz = k[t0:t0 + L, g, :].cpu()
            vz = v[t0:t0 + L, g, :].cpu()
            qr = q[t0 + pos][:, hs, :].transpose(0, 1).reshape(-1, d).cpu()   # [grp*n, d]
            orf, lrf = oracle.head_fwd(qr, np.tile(pos, grp), kz, vz, 0, True, 1.0 / np.sqrt(d))
            ref_o.append(orf)
            ref_l.append(lrf)
            got_o.append(o[t0 + pos][:, hs, :].transpose(0, 1).reshape(-1, d).float().cpu().numpy())
            got_l.append(lse[hs][:, t0 + pos].reshape(-1).cpu().numpy())
    check_o("O", np.concatenate(got_o), np.concatenate(ref_o))
    check_lse("LSE", np.concatenate(got_l), np.concatenate(ref_l))
