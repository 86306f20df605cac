"""Seeded random shapes through the dense and packed forward and backward,
against the fp64 oracle with the usual bars: head dimension, causal flag,
GQA grouping, unequal and ragged lengths (including a single row or key) and
the softmax scale drawn per case, so that tile, wave and stage boundaries
fall at varied places in every kernel (bf16 and FP8, forward and backward,
and the KV-cache paths).

The scale is drawn within [0.5, 1.5] / sqrt(d).  The absolute gradient bar
holds for scores of about unit spread; the backward forms D = rowsum(dO o O)
from the forward's bf16 output O, and with a much sharper softmax that
rounding alone moves dQ by more than the bar (at 2.8 / sqrt(d), d = 128, a
causal row with 14 keys: 6.1e-2 from D alone, measured against dQ computed
exactly but for D)."""
import numpy as np
import pytest

from test_bwd_fp8_gpu import run_fp8_bwd
from test_bwd_gpu import run_bwd
from test_bwd_varlen_gpu import run_varlen_bwd
from test_fp8_gpu import run_fp8
from test_fwd_gpu import run_dense
from test_kvcache_gpu import run_kvcache
from test_mxfp8_gpu import run_mx

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 2, 4]))
    lens = rng.integers(1, 700, size=2)
    if rng.random() < 0.2:
        lens[rng.integers(0, 2)] = 1
    causal = bool(rng.random() < 0.5)
    scale = None if rng.random() < 0.5 else float(rng.uniform(0.5, 1.5) / np.sqrt(d))
    return d, hkv, group, int(lens[0]), int(lens[1]), causal, scale


@pytest.mark.parametrize("seed", range(40))
def test_random_dense(seed):
    d, hkv, group, sq, sk, _, scale = draw(1000 + seed)
    causal = seed % 2 == 1
    B = 1 + seed % 3
    run_dense(B, sq, sk, hkv * group, hkv, d, causal, seed=2000 + seed, scale=scale)
    run_bwd(B, sq, sk, hkv * group, hkv, d, causal, seed=3000 + seed, scale=scale)


@pytest.mark.parametrize("seed", range(8))
def test_random_long_keys(seed):
    """Dense forward with 2048 to 9000 keys, where d = 64 takes the two-group
    kernel (causal from 8192 keys) and short query blocks end anywhere."""
    rng = np.random.default_rng(1500 + seed)
    d, hkv, group, _, _, _, scale = draw(1600 + seed)
    d = 64 if seed % 4 else d
    causal = seed % 2 == 1
    sk = int(rng.integers(8192, 9001) if causal else rng.integers(2048, 9001))
    sq = int(rng.integers(1, 900))
    run_dense(1, sq, sk, hkv * group, hkv, d, causal, seed=1700 + seed, scale=scale)


@pytest.mark.parametrize("seed", range(16))
def test_random_packed(seed):
    rng = np.random.default_rng(4000 + seed)
    d, hkv, group, _, _, _, scale = draw(4100 + seed)
    causal = seed % 2 == 0
    nseq = int(rng.integers(1, 5))
    lens_q = [int(x) for x in rng.integers(1, 400, size=nseq)]
    lens_k = [int(x) for x in rng.integers(1, 400, size=nseq)] if seed % 2 else list(lens_q)
    run_varlen_bwd(lens_q, lens_k, hkv * group, hkv, d, causal, seed=5000 + seed, scale=scale)


@pytest.mark.parametrize("seed", range(10))
def test_random_fp8(seed):
    """FP8 forward, per-block and MX scales, with the element-wise O bound."""
    d, hkv, group, sq, sk, _, scale = draw(6000 + seed)
    causal = seed % 2 == 1
    run_fp8(1, sq, sk, hkv * group, hkv, d, causal, seed=6100 + seed, scale=scale)
    run_mx(1, sq, sk, hkv * group, hkv, d, causal, seed=6200 + seed, scale=scale)


@pytest.mark.parametrize("seed", range(10))
def test_random_fp8_bwd(seed):
    """FP8 backward with the element-wise gradient bounds (the scale drawn
    as above, or 1/sqrt(d))."""
    d, hkv, group, sq, sk, _, scale = draw(6500 + seed)
    causal = seed % 2 == 0
    run_fp8_bwd(1 + seed % 2, sq, sk, hkv * group, hkv, d, causal, seed=6600 + seed, scale=scale)


@pytest.mark.parametrize("seed", range(12))
def test_random_kvcache(seed):
    """KV-cache attention: cached lengths, appended rows (decode or a chunk),
    page size (or an unpaged cache) drawn per case."""
    rng = np.random.default_rng(7000 + seed)
    d, hkv, group, _, _, _, scale = draw(7100 + seed)
    nseq = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(0, 900, size=nseq)]
    snew = int(rng.choice([1, 1, int(rng.integers(2, 300))]))
    page = int(rng.choice([16, 32, 64, 128, 256, 0]))
    run_kvcache(lens, snew, snew, hkv * group, hkv, d, page if page else 1, page > 0,
                seed % 2 == 0, seed=7200 + seed, scale=scale)
