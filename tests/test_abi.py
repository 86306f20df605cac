"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from io_aware_exact_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == set(fa.EXPORTS)
    L = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_strings():
    L = fa.lib()
    assert L.fa_abi_version() == 2
    assert L.fa_status_string(0) == b"ok"
    assert b"head dimension" in L.fa_status_string(3)


FAKE = 0x7F0000000000  # never dereferenced: validation fails first


def fwd_args(**kw):
    B, Sq, Sk, Hq, Hkv, d = 1, 16, 16, 2, 2, 64
    base = dict(dtype=0, B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, d=d, causal=0, softmax_scale=0.125)
    base.update({k: v for k, v in kw.items() if k in base})

    def t(ptr, H):
        return fa.FaTensor(ptr, base["Sq"] * H * base["d"], H * base["d"], base["d"])

    a = fa.FwdArgs(base["dtype"], base["B"], base["Sq"], base["Sk"], base["Hq"], base["Hkv"],
                   base["d"], base["causal"], base["softmax_scale"],
                   kw.get("q", t(FAKE, 2)), kw.get("k", t(FAKE + (1 << 24), 2)),
                   kw.get("v", t(FAKE + (2 << 24), 2)), kw.get("o", t(FAKE + (3 << 24), 2)),
                   kw.get("lse", FAKE + (4 << 24)), None, None, None, None, 0)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), 3), (dict(d=256), 3), (dict(Hq=3, Hkv=2), 5), (dict(Sq=-1), 2),
    (dict(dtype=7), 4), (dict(softmax_scale=float("nan")), 10),
    (dict(softmax_scale=0.0), 10), (dict(softmax_scale=-0.5), 10),
    (dict(dtype=2), 1),   # FP8 without descale arrays
    (dict(q=fa.FaTensor(0, 2048, 128, 64)), 1), (dict(lse=0), 1),
    (dict(q=fa.FaTensor(FAKE + 2, 2048, 128, 64)), 6),
    (dict(q=fa.FaTensor(FAKE, 2048, 130, 64)), 6),
    (dict(o=fa.FaTensor(FAKE + 64, 2048, 128, 64)), 8),
])
def test_fwd_rejects(kw, status):
    a = fwd_args(**kw)
    assert fa.lib().fa_fwd(ctypes.byref(a), None) == status


def test_fwd_null_args():
    assert fa.lib().fa_fwd(None, None) == 1
    assert fa.lib().fa_fwd_varlen(None, None) == 1
    assert fa.lib().fa_bwd(None, None) == 1


def test_fwd_empty_is_noop():
    a = fwd_args(Sq=0)
    assert fa.lib().fa_fwd(ctypes.byref(a), None) == 0


def test_quantize_rejects():
    L = fa.lib()
    ok = dict(x=FAKE, sb=2048, ss=128, sh=64, B=1, S=16, H=2, d=64, pt=0, c=FAKE + (1 << 24),
              s=FAKE + (2 << 24))

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.fa_quantize_fp8(a["x"], a["sb"], a["ss"], a["sh"], a["B"], a["S"], a["H"],
                                 a["d"], a["pt"], a["c"], a["s"], None)
    assert call(x=0) == 1
    assert call(d=24) == 3 and call(d=512) == 3
    assert call(H=0) == 2
    assert call(c=FAKE + 8) == 6
    assert call(c=FAKE + 64) == 8          # codes overlap the input
    assert call(S=0) == 0                  # empty: nothing to do


def test_workspace_size_queries():
    L = fa.lib()
    # decode-shaped: 1 query row x 4 heads per kv head -> split-KV workspace
    a = fwd_args(Sq=1, Sk=4096, Hq=8, Hkv=2)
    assert L.fa_fwd_workspace_size(ctypes.byref(a)) > 0
    # prefill-shaped: no workspace
    a = fwd_args(Sq=512, Sk=512)
    assert L.fa_fwd_workspace_size(ctypes.byref(a)) == 0
    assert L.fa_fwd_workspace_size(None) == 0


def test_bwd_rejects_bad_stages():
    t = fa.FaTensor(FAKE, 2048, 128, 64)
    a = fa.BwdArgs(0, 1, 16, 16, 2, 2, 64, 0, 0.125, t, t, t, t, t, t, t, t, FAKE, FAKE, 1 << 20, 9)
    assert fa.lib().fa_bwd(ctypes.byref(a), None) == 2


def test_fwd_varlen_rejects_fp32():
    a = fa.FwdVarlenArgs(1, 1, 2, 2, 64, 16, 16, 16, 16, 0, 0.125, FAKE, FAKE + (1 << 24),
                         FAKE + (2 << 24), FAKE + (3 << 24), 128, 64, 128, 64, 128, 64, 128, 64,
                         FAKE + (4 << 24), FAKE + (5 << 24), FAKE + (6 << 24))
    assert fa.lib().fa_fwd_varlen(ctypes.byref(a), None) == 4


def bwd_varlen_args(**kw):
    base = dict(dtype=0, nseq=2, Hq=2, Hkv=2, d=64, mq=16, mk=16, Tq=32, Tk=32, causal=0,
                scale=0.125, ws=FAKE + (12 << 24), ws_bytes=1 << 20)
    base.update(kw)
    ptr = {n: FAKE + (i << 24) for i, n in enumerate(
        ["q", "k", "v", "o", "do", "dq", "dk", "dv", "cuq", "cuk", "lse"])}
    ptr.update({n: kw[n] for n in ptr if n in kw})
    st = base["Hq"] * base["d"]
    return fa.BwdVarlenArgs(base["dtype"], base["nseq"], base["Hq"], base["Hkv"], base["d"],
                            base["mq"], base["mk"], base["Tq"], base["Tk"], base["causal"],
                            base["scale"], ptr["q"], ptr["k"], ptr["v"], ptr["o"], ptr["do"],
                            ptr["dq"], ptr["dk"], ptr["dv"], *([st, base["d"]] * 8),
                            ptr["cuq"], ptr["cuk"], ptr["lse"], base["ws"], base["ws_bytes"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=1), 4), (dict(d=96), 3), (dict(Hq=3, Hkv=2), 5), (dict(nseq=-1), 2),
    (dict(scale=0.0), 10), (dict(scale=float("inf")), 10),
    (dict(cuq=0), 1), (dict(dq=0), 1), (dict(lse=0), 1),
    (dict(dk=FAKE + (6 << 24) + 2), 6), (dict(ws=FAKE + (12 << 24) + 64), 6),
    (dict(ws=0), 7), (dict(ws_bytes=16), 7),
    (dict(dq=FAKE + 64), 8),               # dq overlaps q
])
def test_bwd_varlen_rejects(kw, status):
    a = bwd_varlen_args(**kw)
    assert fa.lib().fa_bwd_varlen(ctypes.byref(a), None) == status


def test_bwd_varlen_null_and_workspace_query():
    L = fa.lib()
    assert L.fa_bwd_varlen(None, None) == 1
    assert L.fa_bwd_varlen_workspace_size(None) == 0
    a = bwd_varlen_args(Hq=4, Hkv=2, Tq=1000)
    assert L.fa_bwd_varlen_workspace_size(ctypes.byref(a)) == 4 * 1000 * 4 // 256 * 256 + 256 * (4 * 1000 * 4 % 256 != 0)


def kvcache_args(**kw):
    """fa_fwd_kvcache_args over FAKE pointers: B=2, Sq=1, Hq=4, Hkv=2, d=64,
    4 pages of 16 tokens, block table [2, 2], Snew=1."""
    base = dict(dtype=0, B=2, Sq=1, Hq=4, Hkv=2, d=64, Snew=1, causal=1, softmax_scale=0.125,
                num_pages=4, page_size=16, max_pages_per_seq=2, max_seqlen_k=0,
                block_table=FAKE + (8 << 24), block_table_stride=2, cache_seqlens=FAKE + (9 << 24),
                k_stride_page=2048, k_stride_s=128, k_stride_h=64,
                v_stride_page=2048, v_stride_s=128, v_stride_h=64,
                k_cache=FAKE + (5 << 24), v_cache=FAKE + (6 << 24), lse=FAKE + (4 << 24),
                workspace=None, workspace_bytes=0)
    base.update({k: v for k, v in kw.items() if k in base})
    q = kw.get("q", fa.FaTensor(FAKE, 256, 256, 64))
    o = kw.get("o", fa.FaTensor(FAKE + (3 << 24), 256, 256, 64))
    kn = kw.get("k_new", fa.FaTensor(FAKE + (7 << 24), 128, 128, 64))
    vn = kw.get("v_new", fa.FaTensor(FAKE + (10 << 24), 128, 128, 64))
    b = base
    return fa.FwdKvcacheArgs(b["dtype"], b["B"], b["Sq"], b["Hq"], b["Hkv"], b["d"], b["Snew"],
                             b["causal"], b["softmax_scale"], q, o, b["lse"], b["k_cache"],
                             b["v_cache"], b["k_stride_page"], b["k_stride_s"], b["k_stride_h"],
                             b["v_stride_page"], b["v_stride_s"], b["v_stride_h"], b["num_pages"],
                             b["page_size"], b["max_pages_per_seq"], b["max_seqlen_k"],
                             b["block_table"], b["block_table_stride"], b["cache_seqlens"], kn, vn,
                             b["workspace"], b["workspace_bytes"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 4), (dict(d=96), 3), (dict(Hq=3), 5), (dict(softmax_scale=0.0), 10),
    (dict(page_size=48), 2),                         # paged: not a power of two
    (dict(page_size=8, max_pages_per_seq=4, block_table_stride=4), 2),   # paged: below 16
    (dict(max_pages_per_seq=0), 2), (dict(block_table_stride=1), 2),
    (dict(block_table=None, num_pages=1), 2),        # dense cache: one page per sequence
    (dict(max_seqlen_k=33), 2),                      # beyond the capacity 2 x 16
    (dict(Snew=40), 2), (dict(Sq=-1), 2),
    (dict(cache_seqlens=None), 1), (dict(k_new=fa.FaTensor(None, 0, 0, 0)), 1),
    (dict(k_cache=None), 1), (dict(lse=None), 1),
    (dict(q=fa.FaTensor(FAKE + 8, 256, 256, 64)), 6),
    (dict(k_stride_s=130), 6), (dict(cache_seqlens=FAKE + (9 << 24) + 2), 6),
    (dict(workspace=FAKE + (11 << 24) + 16, workspace_bytes=4096), 6),
    (dict(o=fa.FaTensor(FAKE + 64, 256, 256, 64)), 8),             # o overlaps q
    (dict(k_new=fa.FaTensor(FAKE + (5 << 24) + 256, 128, 128, 64)), 8),   # k_new in the cache
    (dict(lse=FAKE + (6 << 24) + 64), 8),                          # lse in the V cache
])
def test_kvcache_rejects(kw, status):
    a = kvcache_args(**kw)
    assert fa.lib().fa_fwd_kvcache(ctypes.byref(a), None) == status


def test_kvcache_noop_and_workspace_query():
    assert fa.lib().fa_fwd_kvcache(None, None) == 1
    a = kvcache_args(B=0)
    assert fa.lib().fa_fwd_kvcache(ctypes.byref(a), None) == 0
    # decode-shaped (Sq * group = 2 <= 32): a split-KV workspace; prefill-shaped: none
    assert fa.lib().fa_fwd_kvcache_workspace_size(ctypes.byref(kvcache_args())) > 0
    big = kvcache_args(Sq=64, q=fa.FaTensor(FAKE, 16384, 256, 64), o=fa.FaTensor(FAKE + (3 << 24), 16384, 256, 64))
    assert fa.lib().fa_fwd_kvcache_workspace_size(ctypes.byref(big)) == 0


def test_struct_layouts_match_header(tmp_path):
    """Every ctypes argument structure has the header's size and field offsets
    (checked with the host C compiler)."""
    structs = {"fa_fwd_args": fa.FwdArgs, "fa_fwd_varlen_args": fa.FwdVarlenArgs,
               "fa_bwd_args": fa.BwdArgs, "fa_bwd_varlen_args": fa.BwdVarlenArgs,
               "fa_fwd_kvcache_args": fa.FwdKvcacheArgs, "fa_fwd_mxfp8_args": fa.FwdMxfp8Args,
               "fa_merge_args": fa.MergeArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "fa.h"', 'int main(void) {']
    expect = []
    for cname, cls in structs.items():
        lines.append(f'  printf("%zu\\n", sizeof({cname}));')
        expect.append(ctypes.sizeof(cls))
        for fname, _ in cls._fields_:
            lines.append(f'  printf("%zu\\n", offsetof({cname}, {fname}));')
            expect.append(getattr(cls, fname).offset)
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got == expect


def mx_args(**kw):
    base = dict(B=1, Sq=16, Sk=16, Hq=2, Hkv=2, d=64, causal=0, softmax_scale=0.125)
    base.update({k: v for k, v in kw.items() if k in base})
    t = fa.FaTensor(FAKE, 2048, 128, 64)
    return fa.FwdMxfp8Args(base["B"], base["Sq"], base["Sk"], base["Hq"], base["Hkv"], base["d"],
                           base["causal"], base["softmax_scale"], kw.get("q", t),
                           fa.FaTensor(FAKE + (1 << 24), 2048, 128, 64),
                           fa.FaTensor(FAKE + (2 << 24), 2048, 128, 64),
                           kw.get("o", fa.FaTensor(FAKE + (3 << 24), 2048, 128, 64)),
                           FAKE + (4 << 24), kw.get("q_scale", FAKE + (5 << 24)),
                           FAKE + (6 << 24), kw.get("v_scale", FAKE + (7 << 24)))


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), 3), (dict(Hq=3), 5), (dict(softmax_scale=0.0), 10), (dict(Sq=-1), 2),
    (dict(q_scale=None), 1), (dict(q_scale=FAKE + (5 << 24) + 2), 6),
    (dict(q=fa.FaTensor(FAKE + 8, 2048, 128, 64)), 6),
    (dict(o=fa.FaTensor(FAKE + (7 << 24), 2048, 128, 64)), 8),   # o over the V scales
])
def test_mxfp8_rejects(kw, status):
    a = mx_args(**kw)
    assert fa.lib().fa_fwd_mxfp8(ctypes.byref(a), None) == status


def test_quantize_mxfp8_rejects():
    L = fa.lib()
    assert L.fa_quantize_mxfp8(None, 0, 0, 0, 1, 1, 1, 64, 0, FAKE, FAKE, None) == 1
    assert L.fa_quantize_mxfp8(FAKE, 0, 0, 0, 1, 1, 1, 48, 0, FAKE + (1 << 24), FAKE + (2 << 24), None) == 3
    assert L.fa_quantize_mxfp8(FAKE, 0, 0, 0, 1, 1, 1, 64, 2, FAKE + (1 << 24), FAKE + (2 << 24), None) == 2
    assert L.fa_quantize_mxfp8(FAKE, 0, 0, 0, 1, 1, 1, 64, 0, FAKE + (1 << 24) + 4, FAKE + (2 << 24), None) == 6
    assert L.fa_quantize_mxfp8(FAKE, 64, 64, 64, 1, 4, 1, 64, 1, FAKE + 16, FAKE + (2 << 24), None) == 8
    assert L.fa_quantize_mxfp8(FAKE, 0, 0, 0, 0, 1, 1, 64, 0, FAKE + (1 << 24), FAKE + (2 << 24), None) == 0


def test_merge_rejects():
    L = fa.lib()
    def m(**kw):
        base = dict(dtype=0, nparts=2, B=1, S=4, H=2, d=64)
        base.update({k: v for k, v in kw.items() if k in base})
        return fa.MergeArgs(base["dtype"], base["nparts"], base["B"], base["S"], base["H"], base["d"],
                            kw.get("o_parts", FAKE), kw.get("lse_parts", FAKE + (1 << 24)),
                            kw.get("o", fa.FaTensor(FAKE + (2 << 24), 512, 128, 64)),
                            kw.get("lse", FAKE + (3 << 24)))
    assert L.fa_merge(None, None) == 1
    for kw, st in ((dict(dtype=2), 4), (dict(nparts=0), 2), (dict(d=96), 3), (dict(lse=None), 1),
                   (dict(lse_parts=FAKE + (1 << 24) + 2), 6),
                   (dict(o=fa.FaTensor(FAKE + 256, 512, 128, 64)), 8)):
        assert L.fa_merge(ctypes.byref(m(**kw)), None) == st, kw
    assert L.fa_merge(ctypes.byref(m(S=0)), None) == 0


def test_fwd_rejects_slices_beyond_32bit_offsets():
    """A (batch, head) slice is addressed with 32-bit byte offsets up to the
    end of its last 256-row tile: with 64 KB rows (Hq = 512, d = 64) the
    largest accepted Sq is 65279; Sq = 65300 is refused even though it would
    fit with only 128 rows of padding.  (Sq = 65270 passes this check and
    fails the later overlap check instead, so nothing launches.)"""
    Hq, d = 512, 64
    row = Hq * d

    def args(Sq, o_ptr):
        t = fa.FaTensor(FAKE, Sq * row, row, d)
        o = fa.FaTensor(o_ptr, Sq * row, row, d)
        return fa.FwdArgs(0, 1, Sq, 16, Hq, Hq, d, 0, 0.125, t,
                          fa.FaTensor(FAKE + (1 << 40), 16 * row, row, d),
                          fa.FaTensor(FAKE + (2 << 40), 16 * row, row, d), o,
                          FAKE + (3 << 40), None, None, None, None, 0)
    assert fa.lib().fa_fwd(ctypes.byref(args(65300, FAKE + 64)), None) == 2
    assert fa.lib().fa_fwd(ctypes.byref(args(65270, FAKE + 64)), None) == 8


def test_fp8_bwd_rejects_and_workspace():
    """FP8 backward: descale arrays are required, q/k/v strides are in bytes
    (16-byte rows), and the workspace adds the dO codes and their scales."""
    d, S, H = 64, 16, 2
    def args(dtype=2, **kw):
        t8 = fa.FaTensor(FAKE, S * H * d, H * d, d)
        t16 = lambda i: fa.FaTensor(FAKE + (i << 24), S * H * d, H * d, d)
        a = fa.BwdArgs(dtype, 1, S, S, H, H, d, 0, 0.125, t8, fa.FaTensor(FAKE + (1 << 24), S * H * d, H * d, d),
                       fa.FaTensor(FAKE + (2 << 24), S * H * d, H * d, d), t16(3), t16(4), t16(5), t16(6), t16(7),
                       FAKE + (8 << 24), FAKE + (9 << 24), 1 << 20, 0)
        a.q_descale = kw.get("qd", FAKE + (10 << 24))
        a.k_descale = kw.get("kd", FAKE + (11 << 24))
        a.v_descale = kw.get("vd", FAKE + (12 << 24))
        return a
    L = fa.lib()
    assert L.fa_bwd(ctypes.byref(args(qd=None)), None) == 1
    assert L.fa_bwd(ctypes.byref(args(vd=None)), None) == 1
    assert L.fa_bwd(ctypes.byref(args(kd=FAKE + (11 << 24) + 2)), None) == 6
    assert L.fa_bwd(ctypes.byref(args(dtype=1)), None) == 4
    # D [1,2,16] fp32 (256 B) + codes [1,2,16,64] (2 KiB) + scales [1,2,1] int32 (256 B)
    assert L.fa_bwd_workspace_size(ctypes.byref(args())) == 256 + 2048 + 256
    assert L.fa_bwd_workspace_size(ctypes.byref(args(dtype=0))) == 256
