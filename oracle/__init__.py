"""Reference oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow fp64 CPU implementation of the attention hot path, used by the
test suite, the smoke check and the benchmark's CPU-baseline leg to check the
HIP library.  The product path never imports it.  It shares no code with the
HIP library: the arithmetic lives in ``oracle.c`` (fp64, materialised score and
probability rows) and the fp8 encoder in ``fp8.py``; this module only slices
tensors into heads and sequences and calls them.

Sources (pages on IO-aware exact attention):
  * "Dao and colleagues: IO-aware exact attention with FlashAttention",
    research record, fields "summary" and "boundary": the method is exact
    attention computed with tiling and recomputation, without the full
    attention matrix; the result is the plain definition.
  * "Flash Attention and Efficient Transformer Mechanisms": the blockwise
    result is standard attention, nothing approximated.
  * "Dao-AILab" repository overview: the public surface has dense, packed
    variable-length (varlen) and KV-cache entry points -- the varlen oracle
    below is the dense oracle run on every packed sequence separately, and
    the KV-cache oracle is the dense oracle run on each sequence's keys as
    read from its cache pages, after the new keys are appended.

Layouts (readings; the pages give none): dense tensors are [B, S, H, d];
packed varlen tensors are [T, H, d] with cumulative sequence offsets; LSE is
[B, Hq, Sq] (dense) or [Hq, T] (varlen).  Query head h uses kv head
h // (Hq // Hkv) (grouped-query attention with contiguous groups).

All array arguments are numpy arrays (any float dtype; converted exactly to
float64) or torch CPU tensors.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i64, dbl, ip = ctypes.c_int64, ctypes.c_double, ctypes.c_int
        pd = ctypes.POINTER(ctypes.c_double)
        pi64 = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_head_fwd.argtypes = [i64, i64, i64, pd, pi64, i64, ip, dbl,
                                        pd, pd, pd, pd, pd]
        lib.oracle_head_fwd.restype = None
        lib.oracle_group_bwd.argtypes = [i64, i64, i64, i64, pd, pd, pd, pd,
                                         ip, dbl, pd, pd, pd, pd, pd]
        lib.oracle_group_bwd.restype = None
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads():
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all cores)."""
    return int(_load().oracle_num_threads())


def _f64(x):
    if hasattr(x, "detach"):  # torch tensor: bf16/fp16/fp8 -> fp32 is exact
        import torch
        x = x.detach().cpu()
        if x.dtype != torch.float64:
            x = x.to(torch.float32)
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _default_scale(d, scale):
    return 1.0 / np.sqrt(d) if scale is None else float(scale)


def head_fwd(q_rows, pos, k, v, diag, causal, scale, want_probs=False):
    """Exact attention for some query rows of one head.

    q_rows [n, d]; pos [n] integer position of each row in its sequence;
    k, v [sk, d]; diag = Sk - Sq of the sequence (bottom-right causal mask).
    Returns (o [n, d], lse [n]) and, if want_probs, P [n, sk].
    """
    lib = _load()
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    n, d = q_rows.shape
    sk = k.shape[0]
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    assert pos.shape == (n,) and k.shape == (sk, d) and v.shape == (sk, d)
    o = np.zeros((n, d))
    lse = np.zeros(n)
    p = np.zeros((n, sk)) if want_probs else None
    lib.oracle_head_fwd(n, sk, d, _ptr(q_rows),
                        pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                        int(diag), int(bool(causal)), float(scale), _ptr(k),
                        _ptr(v), _ptr(o), _ptr(lse),
                        _ptr(p) if want_probs else None)
    return (o, lse, p) if want_probs else (o, lse)


def attention_fwd(q, k, v, causal=False, scale=None, want_probs=False):
    """Dense forward.  q [B,Sq,Hq,d], k/v [B,Sk,Hkv,d] -> o [B,Sq,Hq,d],
    lse [B,Hq,Sq] (and P [B,Hq,Sq,Sk] if want_probs)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0
    scale = _default_scale(d, scale)
    grp = Hq // Hkv
    o = np.zeros((B, Sq, Hq, d))
    lse = np.zeros((B, Hq, Sq))
    probs = np.zeros((B, Hq, Sq, Sk)) if want_probs else None
    pos = np.arange(Sq)
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            res = head_fwd(q[b, :, h, :], pos, k[b, :, g, :], v[b, :, g, :],
                           Sk - Sq, causal, scale, want_probs)
            o[b, :, h, :], lse[b, h, :] = res[0], res[1]
            if want_probs:
                probs[b, h] = res[2]
    return (o, lse, probs) if want_probs else (o, lse)


def attention_fwd_rows(q, k, v, b_idx, h_idx, i_idx, causal=False, scale=None):
    """Dense forward evaluated only at the query rows (b_idx[n], h_idx[n],
    i_idx[n]).  Returns o [n, d], lse [n].  q/k/v may be torch tensors on any
    device; only the needed heads are copied to the host."""
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    scale = _default_scale(d, scale)
    grp = Hq // Hkv
    b_idx, h_idx, i_idx = (np.asarray(x, dtype=np.int64) for x in (b_idx, h_idx, i_idx))
    n = len(b_idx)
    o = np.zeros((n, d))
    lse = np.zeros(n)
    keys = {}
    for r in range(n):
        keys.setdefault((int(b_idx[r]), int(h_idx[r])), []).append(r)
    for (b, h), rows in keys.items():
        g = h // grp
        rows = np.asarray(rows)
        qr = _f64(q[b, :, h, :][i_idx[rows]] if not hasattr(q, "detach")
                  else q[b, i_idx[rows], h, :])
        o[rows], lse[rows] = head_fwd(qr, i_idx[rows], k[b, :, g, :],
                                      v[b, :, g, :], Sk - Sq, causal, scale)
    return o, lse


def attention_bwd(q, k, v, dout, causal=False, scale=None, bh=None):
    """Dense forward + backward.  Returns (o, lse, dq, dk, dv) in the dense
    layouts; dk/dv [B,Sk,Hkv,d] are summed over each kv head's query heads.
    With bh = [(b, g), ...] only those (batch, kv-head) slices are computed
    and the other entries are left at zero."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0
    scale = _default_scale(d, scale)
    grp = Hq // Hkv
    lib = _load()
    o = np.zeros((B, Sq, Hq, d))
    lse = np.zeros((B, Hq, Sq))
    dq = np.zeros((B, Sq, Hq, d))
    dk = np.zeros((B, Sk, Hkv, d))
    dv = np.zeros((B, Sk, Hkv, d))
    if bh is None:
        bh = [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in bh:
        hs = slice(g * grp, (g + 1) * grp)
        qg = np.ascontiguousarray(q[b, :, hs, :].transpose(1, 0, 2))
        dog = np.ascontiguousarray(dout[b, :, hs, :].transpose(1, 0, 2))
        kg = np.ascontiguousarray(k[b, :, g, :])
        vg = np.ascontiguousarray(v[b, :, g, :])
        og = np.zeros((grp, Sq, d))
        lg = np.zeros((grp, Sq))
        dqg = np.zeros((grp, Sq, d))
        dkg = np.zeros((Sk, d))
        dvg = np.zeros((Sk, d))
        lib.oracle_group_bwd(grp, Sq, Sk, d, _ptr(qg), _ptr(kg), _ptr(vg),
                             _ptr(dog), int(bool(causal)), scale, _ptr(og),
                             _ptr(lg), _ptr(dqg), _ptr(dkg), _ptr(dvg))
        o[b, :, hs, :] = og.transpose(1, 0, 2)
        lse[b, hs, :] = lg
        dq[b, :, hs, :] = dqg.transpose(1, 0, 2)
        dk[b, :, g, :] = dkg
        dv[b, :, g, :] = dvg
    return o, lse, dq, dk, dv


def attention_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, causal=False,
                         scale=None, seqs=None, rows_per_seq=None):
    """Packed variable-length forward: each sequence z attends only to its own
    keys.  q [Tq,Hq,d], k/v [Tk,Hkv,d], cu_seqlens_* [nseq+1] -> o [Tq,Hq,d],
    lse [Hq,Tq].  `seqs` restricts the work to some sequences and
    `rows_per_seq` (dict z -> positions) to some rows; rows not computed are
    left at zero (o) and nan (lse)."""
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = _default_scale(d, scale)
    grp = Hq // Hkv
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    o = np.zeros((Tq, Hq, d))
    lse = np.full((Hq, Tq), np.nan)
    nseq = len(cq) - 1
    for z in (range(nseq) if seqs is None else seqs):
        q0, q1, k0, k1 = cq[z], cq[z + 1], ck[z], ck[z + 1]
        lq, lk = q1 - q0, k1 - k0
        pos = np.arange(lq) if rows_per_seq is None else np.asarray(rows_per_seq[z], dtype=np.int64)
        for h in range(Hq):
            g = h // grp
            qr = q[q0 + pos, h, :] if len(pos) else q[q0:q0, h, :]
            res = head_fwd(qr, pos, k[k0:k1, g, :], v[k0:k1, g, :], lk - lq,
                           causal, scale)
            o[q0 + pos, h, :] = res[0]
            lse[h, q0 + pos] = res[1]
    return o, lse


def attention_bwd_varlen(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, causal=False,
                         scale=None, seqs=None):
    """Packed variable-length forward + backward: the dense backward run on
    each packed sequence alone (sequence z sees only its own keys, causal
    alignment per sequence).  q, dout [Tq,Hq,d], k/v [Tk,Hkv,d] ->
    (o [Tq,Hq,d], lse [Hq,Tq], dq [Tq,Hq,d], dk [Tk,Hkv,d], dv [Tk,Hkv,d]);
    dk/dv are summed over each kv head's query heads.  `seqs` restricts the
    work to some sequences; the other rows are left at zero (lse: nan)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    o = np.zeros((Tq, Hq, d))
    lse = np.full((Hq, Tq), np.nan)
    dq = np.zeros((Tq, Hq, d))
    dk = np.zeros((Tk, Hkv, d))
    dv = np.zeros((Tk, Hkv, d))
    nseq = len(cq) - 1
    for z in (range(nseq) if seqs is None else seqs):
        q0, q1, k0, k1 = cq[z], cq[z + 1], ck[z], ck[z + 1]
        if q1 == q0:
            continue        # no query rows: every gradient of this sequence is zero
        if k1 == k0:
            # no keys: the rows attend to nothing, O = 0, LSE = -inf, dQ = 0
            lse[:, q0:q1] = -np.inf
            continue
        oz, lz, dqz, dkz, dvz = attention_bwd(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1],
                                              dout[None, q0:q1], causal, scale)
        o[q0:q1] = oz[0]
        lse[:, q0:q1] = lz[0]
        dq[q0:q1] = dqz[0]
        dk[k0:k1] = dkz[0]
        dv[k0:k1] = dvz[0]
    return o, lse, dq, dk, dv



def _cache_rows(cache, pages, slots, g):
    """Rows cache[pages[i], slots[i], g, :] as float64 [n, d]."""
    if hasattr(cache, "detach"):
        import torch
        pages = torch.as_tensor(np.asarray(pages, dtype=np.int64))
        slots = torch.as_tensor(np.asarray(slots, dtype=np.int64))
    return _f64(cache[pages, slots, g, :])


def _seq_pages(b, n, page_size, block_table):
    """Page and slot of tokens 0..n-1 of sequence b: token j lives in page
    block_table[b][j // page_size] at slot j % page_size; without a block
    table, sequence b owns page b of capacity page_size."""
    j = np.arange(n, dtype=np.int64)
    if block_table is None:
        return np.full(n, b, dtype=np.int64), j
    row = np.asarray(block_table[b], dtype=np.int64)
    return row[j // page_size], j % page_size


def kvcache_append(k_cache, v_cache, cache_seqlens, k_new, v_new, block_table=None):
    """The cache after the append step of KV-cache attention, as float64
    copies: row i of k_new[b] / v_new[b] ([B, Snew, Hkv, d]) is written at
    token position cache_seqlens[b] + i of sequence b (page and slot as in
    _seq_pages); nothing else changes.  Caches are [pages, page_size, Hkv, d]
    (without a block table: [B, capacity, Hkv, d])."""
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    kn, vn = _f64(k_new), _f64(v_new)
    page_size = kc.shape[1]
    lens = np.asarray(cache_seqlens, dtype=np.int64)
    for b in range(kn.shape[0]):
        pages, slots = _seq_pages(b, lens[b] + kn.shape[1], page_size, block_table)
        for i in range(kn.shape[1]):
            j = lens[b] + i
            kc[pages[j], slots[j]] = kn[b, i]
            vc[pages[j], slots[j]] = vn[b, i]
    return kc, vc


def attention_kvcache(q, k_cache, v_cache, cache_seqlens, block_table=None, k_new=None,
                      v_new=None, causal=False, scale=None, seqs=None, rows=None):
    """KV-cache attention (the repository overview's KV-cache entry point).

    Sequence b holds L_b = cache_seqlens[b] + Snew keys: tokens
    0..cache_seqlens[b]-1 read from its cache pages (see _seq_pages), then
    the Snew rows of k_new[b] / v_new[b] (the append).  q [B,Sq,Hq,d]
    attends to them with the causal alignment of the dense path (query row i
    sees key j iff j <= i + L_b - Sq).  Returns o [B,Sq,Hq,d], lse [B,Hq,Sq].
    `seqs` restricts the work to some sequences and `rows` (list of query
    positions) to some rows; rows not computed are left at zero (o) and nan
    (lse)."""
    B, Sq, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    page_size = k_cache.shape[1]
    grp = Hq // Hkv
    scale = _default_scale(d, scale)
    lens = np.asarray(cache_seqlens, dtype=np.int64)
    snew = 0 if k_new is None else k_new.shape[1]
    o = np.zeros((B, Sq, Hq, d))
    lse = np.full((B, Hq, Sq), np.nan)
    pos = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    for b in (range(B) if seqs is None else seqs):
        pages, slots = _seq_pages(b, lens[b], page_size, block_table)
        L = int(lens[b]) + snew
        for g in range(Hkv):
            kk = _cache_rows(k_cache, pages, slots, g)
            vv = _cache_rows(v_cache, pages, slots, g)
            if snew:
                kk = np.concatenate([kk, _f64(k_new[b, :, g, :])])
                vv = np.concatenate([vv, _f64(v_new[b, :, g, :])])
            for h in range(g * grp, (g + 1) * grp):
                qr = _f64(q[b, :, h, :])[pos]
                ob, lb = head_fwd(qr, pos, kk.reshape(L, d), vv.reshape(L, d), L - Sq,
                                  causal, scale)
                o[b, pos, h, :] = ob
                lse[b, h, pos] = lb
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Exact merge of partial attention results over disjoint key sets
    (sequence-parallel attention; the same identity merges the split-KV
    decode chunks): o_parts [P,B,S,H,d], lse_parts [P,B,H,S] ->
    o [B,S,H,d], lse [B,H,S], with M = max_p LSE_p, w_p = exp(LSE_p - M),
    LSE = M + ln sum_p w_p and O = sum_p w_p O_p / sum_p w_p.  Rows where
    every part has LSE_p = -inf get O = 0, LSE = -inf."""
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    M = lse_parts.max(axis=0)                                   # [B,H,S]
    fin = np.isfinite(M)
    Ms = np.where(fin, M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Ms[None]), 0.0)   # [P,B,H,S]
    wsum = w.sum(axis=0)
    wt = w.transpose(0, 1, 3, 2)[..., None]                     # [P,B,S,H,1]
    o = (wt * o_parts).sum(axis=0)
    ws = wsum.transpose(0, 2, 1)[..., None]
    o = np.where(ws > 0, o / np.where(ws > 0, ws, 1.0), 0.0)
    lse = np.where(wsum > 0, Ms + np.log(np.where(wsum > 0, wsum, 1.0)), -np.inf)
    return o, lse
