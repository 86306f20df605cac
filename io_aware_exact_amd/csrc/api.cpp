// Host entry points of libfa.so: argument checks, then kernel launches on the
// caller's stream.  Nothing here allocates device memory or synchronises.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

constexpr int kBM = 128;   // query rows per forward workgroup

// Workgroups of a packed-sequence grid (varlen_order): rows padded to a
// multiple of 8, tiles (per query head of a kv group) to whole runs of at
// most 8.  Holds for every kernel's run length.
static int64_t varlen_grid_bound(int64_t rows, int64_t tiles, int64_t group) {
  int64_t r;
  if (rows < 0 || tiles < 0 || group < 0 ||
      __builtin_mul_overflow((rows + 7) / 8 * 8, (tiles + 8), &r) || __builtin_mul_overflow(r, group, &r))
    return INT64_MAX;
  return r;
}

// Products of sizes saturate instead of overflowing: a caller may pass any
// int32 size or int64 stride, and a saturated product fails every range check.
int64_t mul_sat(int64_t a, int64_t b) {
  int64_t r;
  if (a <= 0 || b <= 0) return a == 0 || b == 0 ? 0 : -1;
  return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}
int64_t mul_sat(int64_t a, int64_t b, int64_t c) { return mul_sat(mul_sat(a, b), c); }
int64_t mul_sat(int64_t a, int64_t b, int64_t c, int64_t d) { return mul_sat(mul_sat(a, b, c), d); }

// No device allocation is this large; extents beyond it are rejected as
// FA_ERR_SHAPE before any overlap test.
constexpr int64_t kMaxExtentBytes = int64_t(1) << 56;

struct Span {
  uintptr_t lo, hi;  // [lo, hi) in bytes; empty when lo == hi
  bool bad;          // the extent overflows or exceeds kMaxExtentBytes
};

Span empty_span(const void* p) { return {(uintptr_t)p, (uintptr_t)p, false}; }

// n elements of esize bytes from p.
Span lin(const void* p, int64_t n, int64_t esize) {
  if (n <= 0) return empty_span(p);
  const int64_t bytes = mul_sat(n, esize);
  if (bytes > kMaxExtentBytes) return {(uintptr_t)p, (uintptr_t)p, true};
  return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes, false};
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Byte span of a [B,S,H,d] tensor with non-negative element strides.
Span span4(const void* ptr, int64_t B, int64_t S, int64_t H, int64_t d, int64_t sb, int64_t ss,
           int64_t sh, int64_t esize) {
  if (B <= 0 || S <= 0 || H <= 0 || d <= 0) return empty_span(ptr);
  if (sb < 0 || ss < 0 || sh < 0) return {(uintptr_t)ptr, (uintptr_t)ptr, true};
  int64_t last = d - 1, t;
  bool of = false;
  of |= __builtin_mul_overflow(B - 1, sb, &t) || __builtin_add_overflow(last, t, &last);
  of |= __builtin_mul_overflow(S - 1, ss, &t) || __builtin_add_overflow(last, t, &last);
  of |= __builtin_mul_overflow(H - 1, sh, &t) || __builtin_add_overflow(last, t, &last);
  if (of) return {(uintptr_t)ptr, (uintptr_t)ptr, true};
  return lin(ptr, last + 1, esize);
}

bool overlap(Span a, Span b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

template <size_t N>
bool any_bad(const Span (&s)[N]) {
  for (const Span& x : s)
    if (x.bad) return true;
  return false;
}

// Kernels address one (batch, head) slice with 32-bit byte offsets.  Rows
// past the end of the last tile are addressed too (and read as zero through
// the buffer bounds check), so the offsets must stay below 2^32 up to the end
// of the largest tile any kernel uses: 256 query rows (the two-group forward).
constexpr int64_t kMaxTileRows = 256;
bool fits32(int64_t rows, int64_t row_stride_elems, int64_t esize) {
  return mul_sat(rows + kMaxTileRows, row_stride_elems, esize) < (int64_t)0xffffffffLL;
}

bool strides_ok(const fa_tensor& t, int64_t mult) {
  return t.stride_b >= 0 && t.stride_s >= 0 && t.stride_h >= 0 && t.stride_b % mult == 0 &&
         t.stride_s % mult == 0 && t.stride_h % mult == 0;
}

fa_status hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// The kernels evaluate exp2(scale * log2(e) * s - m); masked scores are -inf,
// which needs a strictly positive scale.
bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// ---- split-KV decode plan: taken when the query rows of one kv head fit in
// a few 32-column MFMA tiles (row blocks), each a workgroup that reads the
// kv head's keys of its split.  With more than one row block it is taken
// only when the blocks are fewer than the group's query heads, i.e. when it
// streams each kv head's keys fewer times than the tiled kernels (one pass
// per query head).  Same box, d = 128, against the tiled path: B=8, 64 query
// heads on one kv head, one row each, 32768 keys: 855 -> 61 us; B=8, group
// 4, 16 rows per head, 8192 keys: 160 -> 110 us; the same with 32 rows per
// head (four blocks): 160 -> 153 us; B=4, group 1, 64 rows (two blocks):
// 166 -> 196 us.
constexpr int kDecodeTileRows = 32;
constexpr int kDecodeMaxRowBlocks = 4;
constexpr int kDecodeMaxRows = kDecodeTileRows * kDecodeMaxRowBlocks;
constexpr int64_t kDecodeTargetWaves = 4096;  // one wave per (batch, kv head, split)
constexpr int64_t kDecodeMinKeysPerSplit = 256;
constexpr int64_t kDecodeMaxSplits = 64;

struct DecodePlan {
  bool eligible;
  int nsplit, chunk, nrblk;
  size_t o_part_bytes, lse_part_bytes;
};

DecodePlan split_plan(fa_dtype dtype, int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv,
                      int64_t d) {
  DecodePlan pl = {false, 1, 32, 1, 0, 0};
  if (dtype != FA_BF16 || B <= 0 || Sq <= 0 || Sk < 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 ||
      (d != 64 && d != 128))
    return pl;
  const int64_t group = Hq / Hkv;
  if (Sq * group > kDecodeMaxRows) return pl;
  const int64_t nrblk = (Sq * group + kDecodeTileRows - 1) / kDecodeTileRows;
  if (nrblk > 1 && nrblk >= group) return pl;
  pl.eligible = true;
  pl.nrblk = (int)nrblk;
  if (Sk > 0) {
    const int64_t pairs = B * Hkv * pl.nrblk;
    int64_t ns = (kDecodeTargetWaves + pairs - 1) / pairs;
    const int64_t by_len = (Sk + kDecodeMinKeysPerSplit - 1) / kDecodeMinKeysPerSplit;
    if (ns > by_len) ns = by_len;
    if (ns > kDecodeMaxSplits) ns = kDecodeMaxSplits;
    if (ns < 1) ns = 1;
    const int64_t chunk = ((Sk + ns - 1) / ns + 31) / 32 * 32;
    pl.chunk = (int)chunk;
    pl.nsplit = (int)((Sk + chunk - 1) / chunk);
  }
  const size_t rows = (size_t)B * Hq * Sq * pl.nsplit;
  pl.o_part_bytes = align256(rows * d * 4);
  pl.lse_part_bytes = align256(rows * 4);
  return pl;
}

DecodePlan decode_plan(const fa_fwd_args* a) {
  return split_plan(a->dtype, a->B, a->Sq, a->Sk, a->Hq, a->Hkv, a->d);
}

fa_status check_fwd(const fa_fwd_args* a) {
  if (!a) return FA_ERR_NULL;
  if (a->dtype != FA_BF16 && a->dtype != FA_FP8_E4M3 && a->dtype != FA_FP32) return FA_ERR_DTYPE;
  const bool fp8 = a->dtype == FA_FP8_E4M3;
  const int64_t es = fp8 ? 1 : (a->dtype == FA_FP32 ? 4 : 2);   // bytes per q/k/v element
  const int64_t oes = a->dtype == FA_FP32 ? 4 : 2;                // bytes per o element
  if (a->B < 0 || a->Sq < 0 || a->Sk < 0 || a->Hq < 1 || a->Hkv < 1) return FA_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return FA_ERR_HEADDIM;
  if (a->Hq % a->Hkv != 0) return FA_ERR_GQA;
  if (!scale_ok(a->softmax_scale)) return FA_ERR_SCALE;
  // a pointer may be NULL exactly when its tensor has no elements
  const bool q_side = (int64_t)a->B * a->Sq > 0, k_side = (int64_t)a->B * a->Sk > 0;
  if (q_side && (!a->q.ptr || !a->o.ptr || !a->lse)) return FA_ERR_NULL;
  if (k_side && (!a->k.ptr || !a->v.ptr)) return FA_ERR_NULL;
  if (fp8 && q_side && !a->q_descale) return FA_ERR_NULL;
  if (fp8 && k_side && (!a->k_descale || !a->v_descale)) return FA_ERR_NULL;
  if (!aligned16(a->q.ptr) || !aligned16(a->k.ptr) || !aligned16(a->v.ptr) || !aligned16(a->o.ptr) ||
      ((uintptr_t)a->lse & 3u))
    return FA_ERR_ALIGN;
  if (fp8 && (((uintptr_t)a->q_descale & 3u) || ((uintptr_t)a->k_descale & 3u) ||
              ((uintptr_t)a->v_descale & 3u)))
    return FA_ERR_ALIGN;
  const int64_t smult = 16 / es;             // 16-byte rows
  if (!strides_ok(a->q, smult) || !strides_ok(a->k, smult) || !strides_ok(a->v, smult) ||
      !strides_ok(a->o, 16 / oes))
    return FA_ERR_ALIGN;
  const int64_t tiles = ((int64_t)a->Sq + kBM - 1) / kBM;
  if (mul_sat(tiles, a->Hq, a->B) > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (!fits32(a->Sq, a->q.stride_s, es) || !fits32(a->Sq, a->o.stride_s, oes) ||
      !fits32(a->Sk, a->k.stride_s, es) || !fits32(a->Sk, a->v.stride_s, es))
    return FA_ERR_SHAPE;
  const Span so = span4(a->o.ptr, a->B, a->Sq, a->Hq, a->d, a->o.stride_b, a->o.stride_s, a->o.stride_h, oes);
  const Span sl = lin(a->lse, mul_sat(a->B, a->Hq, a->Sq), 4);
  const Span sq = span4(a->q.ptr, a->B, a->Sq, a->Hq, a->d, a->q.stride_b, a->q.stride_s, a->q.stride_h, es);
  const Span sk = span4(a->k.ptr, a->B, a->Sk, a->Hkv, a->d, a->k.stride_b, a->k.stride_s, a->k.stride_h, es);
  const Span sv = span4(a->v.ptr, a->B, a->Sk, a->Hkv, a->d, a->v.stride_b, a->v.stride_s, a->v.stride_h, es);
  const Span all[5] = {so, sl, sq, sk, sv};
  if (any_bad(all)) return FA_ERR_SHAPE;
  if (overlap(so, sq) || overlap(so, sk) || overlap(so, sv) || overlap(so, sl) || overlap(sl, sq) ||
      overlap(sl, sk) || overlap(sl, sv))
    return FA_ERR_ALIAS;
  if (a->workspace && a->workspace_bytes > 0) {
    if ((uintptr_t)a->workspace & 255u) return FA_ERR_ALIGN;
    const Span sw = lin(a->workspace, a->workspace_bytes > (size_t)kMaxExtentBytes
                                          ? INT64_MAX : (int64_t)a->workspace_bytes, 1);
    if (sw.bad) return FA_ERR_WORKSPACE;
    if (overlap(sw, sq) || overlap(sw, sk) || overlap(sw, sv) || overlap(sw, so) || overlap(sw, sl))
      return FA_ERR_ALIAS;
  }
  return FA_OK;
}

// FA_DEBUG (read at every call): any value other than "0" turns on the
// host-side check of cu_seqlens contents.
bool debug_checks() {
  const char* e = getenv("FA_DEBUG");
  return e && *e && strcmp(e, "0") != 0;
}

// One cu_seqlens array of nseq + 1 entries: starts at 0, never decreases,
// ends at `total`, no step above `max_len`.
bool seqlens_ok(const std::vector<int32_t>& cu, int32_t total, int32_t max_len) {
  if (cu.empty() || cu[0] != 0 || cu.back() != total) return false;
  for (size_t i = 1; i < cu.size(); ++i) {
    const int64_t len = (int64_t)cu[i] - cu[i - 1];
    if (len < 0 || len > max_len) return false;
  }
  return true;
}

// The FA_DEBUG check of both arrays (after the argument check passed):
// synchronises the stream, copies them to the host and checks them.
fa_status check_seqlens_debug(const int32_t* cu_q, const int32_t* cu_k, int32_t nseq, int32_t total_q,
                              int32_t total_k, int32_t max_q, int32_t max_k, hipStream_t stream) {
  if (!debug_checks()) return FA_OK;
  std::vector<int32_t> hq((size_t)nseq + 1), hk((size_t)nseq + 1);
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(hq.data(), cu_q, hq.size() * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(hk.data(), cu_k, hk.size() * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return FA_ERR_HIP;
  if (!seqlens_ok(hq, total_q, max_q) || !seqlens_ok(hk, total_k, max_k)) return FA_ERR_SEQLENS;
  return FA_OK;
}

fa_status check_varlen(const fa_fwd_varlen_args* a) {
  if (!a) return FA_ERR_NULL;
  if (a->dtype != FA_BF16) return FA_ERR_DTYPE;
  if (a->nseq < 0 || a->Hq < 1 || a->Hkv < 1 || a->max_seqlen_q < 0 || a->max_seqlen_k < 0 ||
      a->total_q < 0 || a->total_k < 0)
    return FA_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return FA_ERR_HEADDIM;
  if (a->Hq % a->Hkv != 0) return FA_ERR_GQA;
  if (!scale_ok(a->softmax_scale)) return FA_ERR_SCALE;
  if (!a->cu_seqlens_q || !a->cu_seqlens_k) return FA_ERR_NULL;
  // a pointer may be NULL exactly when its tensor has no elements
  if (a->total_q > 0 && (!a->q || !a->o || !a->lse)) return FA_ERR_NULL;
  if (a->total_k > 0 && (!a->k || !a->v)) return FA_ERR_NULL;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o) ||
      ((uintptr_t)a->lse & 3u) || ((uintptr_t)a->cu_seqlens_q & 3u) || ((uintptr_t)a->cu_seqlens_k & 3u))
    return FA_ERR_ALIGN;
  const int64_t st[8] = {a->q_stride_t, a->q_stride_h, a->k_stride_t, a->k_stride_h,
                         a->v_stride_t, a->v_stride_h, a->o_stride_t, a->o_stride_h};
  for (int i = 0; i < 8; ++i)
    if (st[i] < 0 || st[i] % 8 != 0) return FA_ERR_ALIGN;
  const int64_t tiles = ((int64_t)a->max_seqlen_q + kBM - 1) / kBM;
  if (varlen_grid_bound(mul_sat(a->Hkv, a->nseq), tiles, a->Hq / a->Hkv) > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (!fits32(a->max_seqlen_q, a->q_stride_t, 2) || !fits32(a->max_seqlen_q, a->o_stride_t, 2) ||
      !fits32(a->max_seqlen_k, a->k_stride_t, 2) || !fits32(a->max_seqlen_k, a->v_stride_t, 2))
    return FA_ERR_SHAPE;
  const Span so = span4(a->o, 1, a->total_q, a->Hq, a->d, 0, a->o_stride_t, a->o_stride_h, 2);
  const Span sl = lin(a->lse, mul_sat(a->Hq, a->total_q), 4);
  const Span sq = span4(a->q, 1, a->total_q, a->Hq, a->d, 0, a->q_stride_t, a->q_stride_h, 2);
  const Span sk = span4(a->k, 1, a->total_k, a->Hkv, a->d, 0, a->k_stride_t, a->k_stride_h, 2);
  const Span sv = span4(a->v, 1, a->total_k, a->Hkv, a->d, 0, a->v_stride_t, a->v_stride_h, 2);
  const Span all[5] = {so, sl, sq, sk, sv};
  if (any_bad(all)) return FA_ERR_SHAPE;
  if (overlap(so, sq) || overlap(so, sk) || overlap(so, sv) || overlap(so, sl) || overlap(sl, sq) ||
      overlap(sl, sk) || overlap(sl, sv))
    return FA_ERR_ALIAS;
  return FA_OK;
}

// Backward workspace: D = rowsum(dO o O) [B,Hq,Sq] fp32; for FP8 also the
// E4M3 codes of dO [B,Hq,Sq,d] and their E8M0 scale bytes [B,Hq,nqb] (int32),
// each region 256-byte aligned.  Sizes saturate for impossible shapes, which
// the argument check rejects.
struct BwdWorkspace {
  size_t delta, do8, do_scale, total;
};

size_t region(int64_t n) { return n > kMaxExtentBytes ? (size_t)kMaxExtentBytes : align256((size_t)n); }

BwdWorkspace bwd_workspace(const fa_bwd_args* a) {
  const int64_t B = a->B > 0 ? a->B : 0, Hq = a->Hq > 0 ? a->Hq : 0, Sq = a->Sq > 0 ? a->Sq : 0;
  BwdWorkspace w = {region(mul_sat(B, Hq, Sq, 4)), 0, 0, 0};
  if (a->dtype == FA_FP8_E4M3) {
    w.do8 = region(mul_sat(B, Hq, Sq, a->d > 0 ? a->d : 0));
    w.do_scale = region(mul_sat(B, Hq, (Sq + 127) / 128, 4));
  }
  w.total = w.delta + w.do8 + w.do_scale;
  return w;
}

size_t bwd_delta_bytes(const fa_bwd_args* a) { return bwd_workspace(a).total; }

fa_status check_bwd(const fa_bwd_args* a) {
  if (!a) return FA_ERR_NULL;
  if (a->dtype != FA_BF16 && a->dtype != FA_FP8_E4M3) return FA_ERR_DTYPE;
  const bool fp8 = a->dtype == FA_FP8_E4M3;
  const int64_t es = fp8 ? 1 : 2;   // bytes per q, k, v element
  if (a->B < 0 || a->Sq < 0 || a->Sk < 0 || a->Hq < 1 || a->Hkv < 1) return FA_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return FA_ERR_HEADDIM;
  if (a->Hq % a->Hkv != 0) return FA_ERR_GQA;
  if (!scale_ok(a->softmax_scale)) return FA_ERR_SCALE;
  if (a->stages < 0 || a->stages > (FA_BWD_PREPROCESS | FA_BWD_DKDV | FA_BWD_DQ)) return FA_ERR_SHAPE;
  const fa_tensor* ts[8] = {&a->q, &a->k, &a->v, &a->o, &a->dout, &a->dq, &a->dk, &a->dv};
  // a pointer may be NULL exactly when its tensor has no elements
  const bool q_side = (int64_t)a->B * a->Sq > 0, k_side = (int64_t)a->B * a->Sk > 0;
  const bool is_q_side[8] = {true, false, false, true, true, true, false, false};
  for (int i = 0; i < 8; ++i)
    if (!ts[i]->ptr && (is_q_side[i] ? q_side : k_side)) return FA_ERR_NULL;
  if (!a->lse && q_side) return FA_ERR_NULL;
  if (fp8 && ((q_side && !a->q_descale) || (k_side && (!a->k_descale || !a->v_descale)))) return FA_ERR_NULL;
  for (int i = 0; i < 8; ++i)
    if (!aligned16(ts[i]->ptr) || !strides_ok(*ts[i], i < 3 ? 16 / es : 8)) return FA_ERR_ALIGN;
  if ((uintptr_t)a->lse & 3u) return FA_ERR_ALIGN;
  if (fp8 && (((uintptr_t)a->q_descale & 3u) || ((uintptr_t)a->k_descale & 3u) ||
              ((uintptr_t)a->v_descale & 3u)))
    return FA_ERR_ALIGN;
  const int64_t B = a->B, Sq = a->Sq, Sk = a->Sk, Hq = a->Hq, Hkv = a->Hkv, d = a->d;
  if (mul_sat((Sq + 127) / 128, Hq, B) > 0x7fffffffLL || mul_sat((Sk + 127) / 128, Hkv, B) > 0x7fffffffLL)
    return FA_ERR_SHAPE;
  if (mul_sat(B, Sq, Hq) > 0x7fffffffLL * 16) return FA_ERR_SHAPE;
  if (!fits32(Sq, a->q.stride_s, es) || !fits32(Sq, a->dout.stride_s, 2) ||
      !fits32(Sk, a->k.stride_s, es) || !fits32(Sk, a->v.stride_s, es))
    return FA_ERR_SHAPE;
  if (fp8 && !fits32(Sq, d, 1)) return FA_ERR_SHAPE;   // one head's dO codes in the workspace
  const size_t need = bwd_delta_bytes(a);
  if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if ((uintptr_t)a->workspace & 255u) return FA_ERR_ALIGN;
  // outputs must not overlap each other, the inputs or the workspace
  const int64_t nqb = (Sq + 127) / 128, nkb = (Sk + 127) / 128;
  const Span in[9] = {
      span4(a->q.ptr, B, Sq, Hq, d, a->q.stride_b, a->q.stride_s, a->q.stride_h, es),
      span4(a->k.ptr, B, Sk, Hkv, d, a->k.stride_b, a->k.stride_s, a->k.stride_h, es),
      span4(a->v.ptr, B, Sk, Hkv, d, a->v.stride_b, a->v.stride_s, a->v.stride_h, es),
      span4(a->o.ptr, B, Sq, Hq, d, a->o.stride_b, a->o.stride_s, a->o.stride_h, 2),
      span4(a->dout.ptr, B, Sq, Hq, d, a->dout.stride_b, a->dout.stride_s, a->dout.stride_h, 2),
      lin(a->lse, mul_sat(B, Hq, Sq), 4),
      fp8 ? lin(a->q_descale, mul_sat(B, Hq, nqb), 4) : empty_span(nullptr),
      fp8 ? lin(a->k_descale, mul_sat(B, Hkv, nkb), 4) : empty_span(nullptr),
      fp8 ? lin(a->v_descale, mul_sat(B, Hkv, nkb), 4) : empty_span(nullptr)};
  const Span out[4] = {
      span4(a->dq.ptr, B, Sq, Hq, d, a->dq.stride_b, a->dq.stride_s, a->dq.stride_h, 2),
      span4(a->dk.ptr, B, Sk, Hkv, d, a->dk.stride_b, a->dk.stride_s, a->dk.stride_h, 2),
      span4(a->dv.ptr, B, Sk, Hkv, d, a->dv.stride_b, a->dv.stride_s, a->dv.stride_h, 2),
      lin(a->workspace, (int64_t)need, 1)};
  if (any_bad(in) || any_bad(out)) return FA_ERR_SHAPE;
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 9; ++j)
      if (overlap(out[i], in[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(out[i], out[j])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

size_t bwd_varlen_delta_bytes(const fa_bwd_varlen_args* a) {
  const int64_t n = mul_sat(a->Hq > 0 ? a->Hq : 0, a->total_q > 0 ? a->total_q : 0, 4);
  return n > kMaxExtentBytes ? (size_t)kMaxExtentBytes : align256((size_t)n);
}

fa_status check_bwd_varlen(const fa_bwd_varlen_args* a) {
  if (!a) return FA_ERR_NULL;
  if (a->dtype != FA_BF16) return FA_ERR_DTYPE;
  if (a->nseq < 0 || a->Hq < 1 || a->Hkv < 1 || a->max_seqlen_q < 0 || a->max_seqlen_k < 0 ||
      a->total_q < 0 || a->total_k < 0)
    return FA_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return FA_ERR_HEADDIM;
  if (a->Hq % a->Hkv != 0) return FA_ERR_GQA;
  if (!scale_ok(a->softmax_scale)) return FA_ERR_SCALE;
  if (!a->cu_seqlens_q || !a->cu_seqlens_k) return FA_ERR_NULL;
  // a pointer may be NULL exactly when its tensor has no elements
  if (a->total_q > 0 && (!a->q || !a->o || !a->dout || !a->dq || !a->lse)) return FA_ERR_NULL;
  if (a->total_k > 0 && (!a->k || !a->v || !a->dk || !a->dv)) return FA_ERR_NULL;
  const void* ps[8] = {a->q, a->k, a->v, a->o, a->dout, a->dq, a->dk, a->dv};
  for (int i = 0; i < 8; ++i)
    if (!aligned16(ps[i])) return FA_ERR_ALIGN;
  if (((uintptr_t)a->lse & 3u) || ((uintptr_t)a->cu_seqlens_q & 3u) || ((uintptr_t)a->cu_seqlens_k & 3u))
    return FA_ERR_ALIGN;
  const int64_t st[16] = {a->q_stride_t,  a->q_stride_h,  a->k_stride_t,  a->k_stride_h,
                          a->v_stride_t,  a->v_stride_h,  a->o_stride_t,  a->o_stride_h,
                          a->do_stride_t, a->do_stride_h, a->dq_stride_t, a->dq_stride_h,
                          a->dk_stride_t, a->dk_stride_h, a->dv_stride_t, a->dv_stride_h};
  for (int i = 0; i < 16; ++i)
    if (st[i] < 0 || st[i] % 8 != 0) return FA_ERR_ALIGN;
  const int64_t qtiles = ((int64_t)a->max_seqlen_q + 127) / 128, ktiles = ((int64_t)a->max_seqlen_k + 127) / 128;
  if (varlen_grid_bound(mul_sat(a->Hkv, a->nseq), qtiles, a->Hq / a->Hkv) > 0x7fffffffLL ||
      varlen_grid_bound(mul_sat(a->Hkv, a->nseq), ktiles, 1) > 0x7fffffffLL)
    return FA_ERR_SHAPE;
  if (mul_sat(a->total_q, a->Hq) > 0x7fffffffLL * 16) return FA_ERR_SHAPE;
  if (!fits32(a->max_seqlen_q, a->q_stride_t, 2) || !fits32(a->max_seqlen_q, a->do_stride_t, 2) ||
      !fits32(a->max_seqlen_k, a->k_stride_t, 2) || !fits32(a->max_seqlen_k, a->v_stride_t, 2))
    return FA_ERR_SHAPE;
  const size_t need = bwd_varlen_delta_bytes(a);
  if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if ((uintptr_t)a->workspace & 255u) return FA_ERR_ALIGN;
  // outputs must not overlap each other, the inputs or the workspace
  const int64_t Tq = a->total_q, Tk = a->total_k, Hq = a->Hq, Hkv = a->Hkv, d = a->d;
  const Span in[8] = {
      span4(a->q, 1, Tq, Hq, d, 0, a->q_stride_t, a->q_stride_h, 2),
      span4(a->k, 1, Tk, Hkv, d, 0, a->k_stride_t, a->k_stride_h, 2),
      span4(a->v, 1, Tk, Hkv, d, 0, a->v_stride_t, a->v_stride_h, 2),
      span4(a->o, 1, Tq, Hq, d, 0, a->o_stride_t, a->o_stride_h, 2),
      span4(a->dout, 1, Tq, Hq, d, 0, a->do_stride_t, a->do_stride_h, 2),
      lin(a->lse, mul_sat(Hq, Tq), 4),
      lin(a->cu_seqlens_q, (int64_t)a->nseq + 1, 4),
      lin(a->cu_seqlens_k, (int64_t)a->nseq + 1, 4)};
  const Span out[4] = {
      span4(a->dq, 1, Tq, Hq, d, 0, a->dq_stride_t, a->dq_stride_h, 2),
      span4(a->dk, 1, Tk, Hkv, d, 0, a->dk_stride_t, a->dk_stride_h, 2),
      span4(a->dv, 1, Tk, Hkv, d, 0, a->dv_stride_t, a->dv_stride_h, 2),
      lin(a->workspace, (int64_t)need, 1)};
  if (any_bad(in) || any_bad(out)) return FA_ERR_SHAPE;
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlap(out[i], in[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(out[i], out[j])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

// The tiled bf16 forward.  At d = 128 the two-group kernel (one group's
// softmax runs while the other group's MFMAs run) is faster.  At d = 64 the
// softmax costs about twice the matrix work per tile; the two-group kernel
// still wins once each workgroup's sweep is long enough to amortise its
// start-up over 256 rows (same-box sweeps at H = 16: non-causal from 2048
// keys, causal from 8192) and the query block fills most of those rows (at
// 64 query rows against 8192 keys it ran 20% slower; from 256 rows it was
// between 4% slower and 9% faster).  The one-group kernel (three workgroups
// of 128 rows per CU) is used otherwise and for packed sequences.
//
// At d = 128 and at most 128 query rows (per sequence, for packed inputs)
// the two-group kernel's 256-row workgroups are at least half padding, and
// the one-group kernel (two 128-row workgroups per CU at d = 128) ran 17%
// faster at 64 and 128 rows against 8192 keys (B=16, H=16, both masks); at
// 192-255 rows it ran 18% slower.
hipError_t launch_fwd_tiled(const FwdParams& p, int d, bool causal, bool varlen, hipStream_t stream) {
  if (d == 128 && p.Sq <= 128) return launch_fwd_bf16(p, d, causal, varlen, stream);   // packed: Sq is the longest
  if (d == 128) return launch_fwd_bf16_pp(p, d, causal, varlen, stream);
  // packed d = 64 (longest sequences at least 256 queries and 2048 keys):
  // 16 lengths on [128, 32768], Hq = 32, Hkv = 8, same box: non-causal
  // 921-926 -> 962-967 TFLOP/s with the two-group kernel, causal 985-993 ->
  // 943-948, so packed causal inputs keep the one-group kernel
  const bool pp64 = varlen ? !causal && p.Sk >= 2048 : p.Sk >= (causal ? 8192 : 2048);
  if (d == 64 && p.Sq >= 256 && pp64) return launch_fwd_bf16_pp(p, d, causal, varlen, stream);
  return launch_fwd_bf16(p, d, causal, varlen, stream);
}

// ---- KV-cache attention
int64_t kv_capacity(const fa_fwd_kvcache_args* a) {
  return a->block_table ? (int64_t)a->max_pages_per_seq * a->page_size : (int64_t)a->page_size;
}

int64_t kv_max_len(const fa_fwd_kvcache_args* a) {
  return a->max_seqlen_k > 0 ? (int64_t)a->max_seqlen_k : kv_capacity(a);
}

DecodePlan kvcache_plan(const fa_fwd_kvcache_args* a) {
  return split_plan(a->dtype, a->B, a->Sq, kv_max_len(a), a->Hq, a->Hkv, a->d);
}

bool strides8(int64_t a, int64_t b, int64_t c) {
  return a >= 0 && b >= 0 && c >= 0 && a % 8 == 0 && b % 8 == 0 && c % 8 == 0;
}

fa_status check_kvcache(const fa_fwd_kvcache_args* a) {
  if (!a) return FA_ERR_NULL;
  if (a->dtype != FA_BF16) return FA_ERR_DTYPE;
  if (a->B < 0 || a->Sq < 0 || a->Snew < 0 || a->Hq < 1 || a->Hkv < 1 || a->num_pages < 0 ||
      a->page_size < 1 || a->max_seqlen_k < 0)
    return FA_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return FA_ERR_HEADDIM;
  if (a->Hq % a->Hkv != 0) return FA_ERR_GQA;
  if (!scale_ok(a->softmax_scale)) return FA_ERR_SCALE;
  const bool paged = a->block_table != nullptr;
  if (paged) {
    // a power of two, at least 16 (the decode kernel's DMAs cover up to 8
    // consecutive rows, which must lie in one page)
    if ((a->page_size & (a->page_size - 1)) != 0 || a->page_size < 16) return FA_ERR_SHAPE;
    if (a->max_pages_per_seq < 1 || a->block_table_stride < a->max_pages_per_seq) return FA_ERR_SHAPE;
    if (a->B > 0 && a->num_pages < 1) return FA_ERR_SHAPE;
    if ((uintptr_t)a->block_table & 3u) return FA_ERR_ALIGN;
  } else if (a->num_pages < a->B) {
    return FA_ERR_SHAPE;   // dense cache: page b is sequence b's
  }
  const int64_t cap = kv_capacity(a);
  if (cap > 0x7fffffffLL - 256) return FA_ERR_SHAPE;   // token positions are 32-bit
  if (a->max_seqlen_k > cap || a->Snew > kv_max_len(a)) return FA_ERR_SHAPE;
  if (a->B == 0) return FA_OK;
  if (!a->cache_seqlens || !a->k_cache || !a->v_cache) return FA_ERR_NULL;
  if (a->Sq > 0 && (!a->q.ptr || !a->o.ptr || !a->lse)) return FA_ERR_NULL;
  if (a->Snew > 0 && (!a->k_new.ptr || !a->v_new.ptr)) return FA_ERR_NULL;
  if (!aligned16(a->q.ptr) || !aligned16(a->o.ptr) || !aligned16(a->k_cache) || !aligned16(a->v_cache) ||
      !aligned16(a->k_new.ptr) || !aligned16(a->v_new.ptr) || ((uintptr_t)a->lse & 3u) ||
      ((uintptr_t)a->cache_seqlens & 3u))
    return FA_ERR_ALIGN;
  if (!strides_ok(a->q, 8) || !strides_ok(a->o, 8) || !strides_ok(a->k_new, 8) || !strides_ok(a->v_new, 8) ||
      !strides8(a->k_stride_page, a->k_stride_s, a->k_stride_h) ||
      !strides8(a->v_stride_page, a->v_stride_s, a->v_stride_h))
    return FA_ERR_ALIGN;
  const int64_t tiles = ((int64_t)a->Sq + kBM - 1) / kBM;
  if (mul_sat(tiles, a->Hq, a->B) > 0x7fffffffLL) return FA_ERR_SHAPE;
  // q and o slices, and one page (or a dense cache's rows), are addressed
  // with 32-bit byte offsets
  if (!fits32(a->Sq, a->q.stride_s, 2) || !fits32(a->Sq, a->o.stride_s, 2) ||
      !fits32(a->page_size, a->k_stride_s, 2) || !fits32(a->page_size, a->v_stride_s, 2))
    return FA_ERR_SHAPE;
  const Span so = span4(a->o.ptr, a->B, a->Sq, a->Hq, a->d, a->o.stride_b, a->o.stride_s, a->o.stride_h, 2);
  const Span sl = lin(a->lse, mul_sat(a->B, a->Hq, a->Sq), 4);
  const Span sq = span4(a->q.ptr, a->B, a->Sq, a->Hq, a->d, a->q.stride_b, a->q.stride_s, a->q.stride_h, 2);
  const Span skn = span4(a->k_new.ptr, a->B, a->Snew, a->Hkv, a->d, a->k_new.stride_b, a->k_new.stride_s,
                         a->k_new.stride_h, 2);
  const Span svn = span4(a->v_new.ptr, a->B, a->Snew, a->Hkv, a->d, a->v_new.stride_b, a->v_new.stride_s,
                         a->v_new.stride_h, 2);
  const Span skc = span4(a->k_cache, a->num_pages, a->page_size, a->Hkv, a->d, a->k_stride_page, a->k_stride_s,
                         a->k_stride_h, 2);
  const Span svc = span4(a->v_cache, a->num_pages, a->page_size, a->Hkv, a->d, a->v_stride_page, a->v_stride_s,
                         a->v_stride_h, 2);
  int64_t bt_n = INT64_MAX;
  if (paged) {
    int64_t t;
    if (!__builtin_mul_overflow((int64_t)a->B - 1, a->block_table_stride, &t) &&
        !__builtin_add_overflow(t, (int64_t)a->max_pages_per_seq, &t))
      bt_n = t;
  }
  const Span sbt = paged ? lin(a->block_table, bt_n, 4) : empty_span(nullptr);
  const Span ssl = lin(a->cache_seqlens, a->B, 4);
  const Span all[9] = {so, sl, sq, skn, svn, skc, svc, sbt, ssl};
  if (any_bad(all)) return FA_ERR_SHAPE;
  // outputs: o, lse, and (when appending) the caches
  const Span outs[2] = {so, sl};
  const Span ins[7] = {sq, skn, svn, skc, svc, sbt, ssl};
  for (const Span& o : outs)
    for (const Span& i : ins)
      if (overlap(o, i)) return FA_ERR_ALIAS;
  if (overlap(so, sl)) return FA_ERR_ALIAS;
  if (a->Snew > 0) {
    const Span readers[5] = {sq, skn, svn, sbt, ssl};
    for (const Span& r : readers)
      if (overlap(skc, r) || overlap(svc, r)) return FA_ERR_ALIAS;
  }
  if (a->workspace && a->workspace_bytes > 0) {
    if ((uintptr_t)a->workspace & 255u) return FA_ERR_ALIGN;
    const Span sw = lin(a->workspace, a->workspace_bytes > (size_t)kMaxExtentBytes
                                          ? INT64_MAX : (int64_t)a->workspace_bytes, 1);
    if (sw.bad) return FA_ERR_WORKSPACE;
    for (const Span& x : all)
      if (overlap(sw, x)) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

}  // namespace

extern "C" {

int32_t fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid or unsupported size";
    case FA_ERR_HEADDIM: return "head dimension must be 64 or 128";
    case FA_ERR_DTYPE: return "unsupported dtype for this call";
    case FA_ERR_GQA: return "Hq must be a multiple of Hkv";
    case FA_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_ALIAS: return "an output overlaps another tensor";
    case FA_ERR_HIP: return "HIP runtime error at launch";
    case FA_ERR_SCALE: return "softmax scale must be finite and positive";
    case FA_ERR_SEQLENS: return "cu_seqlens contents are inconsistent (FA_DEBUG check)";
  }
  return "unknown status";
}

size_t fa_fwd_workspace_size(const fa_fwd_args* a) {
  if (!a) return 0;
  const DecodePlan pl = decode_plan(a);
  return pl.eligible ? pl.o_part_bytes + pl.lse_part_bytes : 0;
}

fa_status fa_fwd(const fa_fwd_args* a, hipStream_t stream) {
  const fa_status s = check_fwd(a);
  if (s != FA_OK) return s;
  if (a->B == 0 || a->Sq == 0) return FA_OK;
  FwdParams p = {};
  p.q = a->q.ptr;
  p.k = a->k.ptr;
  p.v = a->v.ptr;
  p.o = a->o.ptr;
  p.lse = a->lse;
  p.q_sb = a->q.stride_b; p.q_ss = a->q.stride_s; p.q_sh = a->q.stride_h;
  p.k_sb = a->k.stride_b; p.k_ss = a->k.stride_s; p.k_sh = a->k.stride_h;
  p.v_sb = a->v.stride_b; p.v_ss = a->v.stride_s; p.v_sh = a->v.stride_h;
  p.o_sb = a->o.stride_b; p.o_ss = a->o.stride_s; p.o_sh = a->o.stride_h;
  p.lse_sb = (int64_t)a->Hq * a->Sq;
  p.lse_sh = a->Sq;
  p.B = a->B; p.Sq = a->Sq; p.Sk = a->Sk; p.Hq = a->Hq; p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.num_m_tiles = (a->Sq + kBM - 1) / kBM;
  p.scale = a->softmax_scale;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  if (a->dtype == FA_FP32) return hip_status(launch_fwd_f32(p, a->d, a->causal != 0, stream));
  if (a->dtype == FA_FP8_E4M3) {
    p.q_descale = a->q_descale;
    p.k_descale = a->k_descale;
    p.v_descale = a->v_descale;
    return hip_status(launch_fwd_fp8(p, a->d, a->causal != 0, stream));
  }
  const DecodePlan pl = decode_plan(a);
  if (pl.eligible && a->workspace && a->workspace_bytes >= pl.o_part_bytes + pl.lse_part_bytes) {
    DecodeParams d = {};
    d.q = p.q; d.k = p.k; d.v = p.v; d.o = p.o; d.lse = p.lse;
    d.o_part = (float*)a->workspace;
    d.lse_part = (float*)((char*)a->workspace + pl.o_part_bytes);
    d.q_sb = p.q_sb; d.q_ss = p.q_ss; d.q_sh = p.q_sh;
    d.k_sb = p.k_sb; d.k_ss = p.k_ss; d.k_sh = p.k_sh;
    d.v_sb = p.v_sb; d.v_ss = p.v_ss; d.v_sh = p.v_sh;
    d.o_sb = p.o_sb; d.o_ss = p.o_ss; d.o_sh = p.o_sh;
    d.lse_sb = p.lse_sb; d.lse_sh = p.lse_sh;
    d.B = p.B; d.Sq = p.Sq; d.Sk = p.Sk; d.Hq = p.Hq; d.Hkv = p.Hkv; d.group = p.group;
    d.causal = a->causal != 0;
    d.nsplit = pl.nsplit;
    d.nrblk = pl.nrblk;
    d.chunk = pl.chunk;
    d.scale = p.scale;
    d.scale_log2 = p.scale_log2;
    return hip_status(launch_decode_bf16(d, a->d, stream));
  }
  return hip_status(launch_fwd_tiled(p, a->d, a->causal != 0, false, stream));
}

fa_status fa_fwd_varlen(const fa_fwd_varlen_args* a, hipStream_t stream) {
  const fa_status s = check_varlen(a);
  if (s != FA_OK) return s;
  if (a->nseq > 0) {
    const fa_status sd = check_seqlens_debug(a->cu_seqlens_q, a->cu_seqlens_k, a->nseq, a->total_q,
                                             a->total_k, a->max_seqlen_q, a->max_seqlen_k, stream);
    if (sd != FA_OK) return sd;
  }
  if (a->nseq == 0 || a->max_seqlen_q == 0 || a->total_q == 0) return FA_OK;
  FwdParams p = {};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.q_ss = a->q_stride_t; p.q_sh = a->q_stride_h;
  p.k_ss = a->k_stride_t; p.k_sh = a->k_stride_h;
  p.v_ss = a->v_stride_t; p.v_sh = a->v_stride_h;
  p.o_ss = a->o_stride_t; p.o_sh = a->o_stride_h;
  p.lse_sb = 0;
  p.lse_sh = a->total_q;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.B = a->nseq; p.Sq = a->max_seqlen_q; p.Sk = a->max_seqlen_k; p.Hq = a->Hq; p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.num_m_tiles = (a->max_seqlen_q + kBM - 1) / kBM;
  p.scale = a->softmax_scale;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  return hip_status(launch_fwd_tiled(p, a->d, a->causal != 0, true, stream));
}

size_t fa_bwd_workspace_size(const fa_bwd_args* a) {
  if (!a) return 0;
  return bwd_delta_bytes(a);
}

fa_status fa_bwd(const fa_bwd_args* a, hipStream_t stream) {
  const fa_status s = check_bwd(a);
  if (s != FA_OK) return s;
  if (a->B == 0 || a->Sq == 0 || a->Sk == 0) {
    // no query rows or no keys: dQ, dK, dV are all zero (a fill kernel, not a
    // memset, so that the call can be captured into a graph)
    const fa_tensor* outs[3] = {&a->dq, &a->dk, &a->dv};
    const int64_t S[3] = {a->Sq, a->Sk, a->Sk};
    const int64_t H[3] = {a->Hq, a->Hkv, a->Hkv};
    for (int i = 0; i < 3; ++i) {
      const fa_tensor& t = *outs[i];
      if (a->B == 0 || S[i] == 0) continue;
      if (launch_zero_bf16(t.ptr, a->B, S[i], H[i], a->d, t.stride_b, t.stride_s, t.stride_h, stream) !=
          hipSuccess)
        return FA_ERR_HIP;
    }
    return FA_OK;
  }
  BwdParams p = {};
  p.q = a->q.ptr; p.k = a->k.ptr; p.v = a->v.ptr; p.o = a->o.ptr; p.dout = a->dout.ptr;
  p.dq = a->dq.ptr; p.dk = a->dk.ptr; p.dv = a->dv.ptr;
  p.lse = a->lse;
  p.delta = (float*)a->workspace;
  p.dq_acc = nullptr;
  p.q_sb = a->q.stride_b; p.q_ss = a->q.stride_s; p.q_sh = a->q.stride_h;
  p.k_sb = a->k.stride_b; p.k_ss = a->k.stride_s; p.k_sh = a->k.stride_h;
  p.v_sb = a->v.stride_b; p.v_ss = a->v.stride_s; p.v_sh = a->v.stride_h;
  p.o_sb = a->o.stride_b; p.o_ss = a->o.stride_s; p.o_sh = a->o.stride_h;
  p.do_sb = a->dout.stride_b; p.do_ss = a->dout.stride_s; p.do_sh = a->dout.stride_h;
  p.dq_sb = a->dq.stride_b; p.dq_ss = a->dq.stride_s; p.dq_sh = a->dq.stride_h;
  p.dk_sb = a->dk.stride_b; p.dk_ss = a->dk.stride_s; p.dk_sh = a->dk.stride_h;
  p.dv_sb = a->dv.stride_b; p.dv_ss = a->dv.stride_s; p.dv_sh = a->dv.stride_h;
  p.B = a->B; p.Sq = a->Sq; p.Sk = a->Sk; p.Hq = a->Hq; p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.causal = a->causal != 0;
  p.scale = a->softmax_scale;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  const int stages = a->stages == FA_BWD_ALL ? (FA_BWD_PREPROCESS | FA_BWD_DKDV | FA_BWD_DQ) : a->stages;
  if (a->dtype == FA_FP8_E4M3) {
    const BwdWorkspace w = bwd_workspace(a);
    p.q_descale = a->q_descale;
    p.k_descale = a->k_descale;
    p.v_descale = a->v_descale;
    p.do8 = (uint8_t*)a->workspace + w.delta;
    p.do_e8m0 = (int*)((char*)a->workspace + w.delta + w.do8);
    return hip_status(launch_bwd_fp8(p, a->d, a->causal != 0, stages, stream));
  }
  return hip_status(launch_bwd_bf16(p, a->d, a->causal != 0, false, stages, stream));
}

fa_status fa_bwd_noalloc(const fa_bwd_args* a, hipStream_t stream) {
  if (!a) return FA_ERR_NULL;
  static_assert(kNoallocScratchBytes == FA_BWD_NOALLOC_MAX_SCRATCH, "scratch size in the header");
  fa_bwd_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  const size_t need = bwd_delta_bytes(&b);
  if (need > kNoallocScratchBytes) return FA_ERR_WORKSPACE;
  if (need > 0) {
    // the library's own per-device scratch array; no allocation
    if (noalloc_scratch(&b.workspace) != hipSuccess) return FA_ERR_HIP;
    b.workspace_bytes = kNoallocScratchBytes;
  }
  return fa_bwd(&b, stream);
}

size_t fa_bwd_varlen_workspace_size(const fa_bwd_varlen_args* a) {
  if (!a) return 0;
  return bwd_varlen_delta_bytes(a);
}

fa_status fa_bwd_varlen(const fa_bwd_varlen_args* a, hipStream_t stream) {
  const fa_status s = check_bwd_varlen(a);
  if (s != FA_OK) return s;
  if (a->nseq > 0) {
    const fa_status sd = check_seqlens_debug(a->cu_seqlens_q, a->cu_seqlens_k, a->nseq, a->total_q,
                                             a->total_k, a->max_seqlen_q, a->max_seqlen_k, stream);
    if (sd != FA_OK) return sd;
  }
  if (a->nseq == 0 || a->total_q == 0 || a->total_k == 0) {
    // no query rows or no keys anywhere: the gradients are zero
    if (a->total_q > 0 &&
        launch_zero_bf16(a->dq, 1, a->total_q, a->Hq, a->d, 0, a->dq_stride_t, a->dq_stride_h, stream) !=
            hipSuccess)
      return FA_ERR_HIP;
    if (a->total_k > 0) {
      if (launch_zero_bf16(a->dk, 1, a->total_k, a->Hkv, a->d, 0, a->dk_stride_t, a->dk_stride_h, stream) !=
              hipSuccess ||
          launch_zero_bf16(a->dv, 1, a->total_k, a->Hkv, a->d, 0, a->dv_stride_t, a->dv_stride_h, stream) !=
              hipSuccess)
        return FA_ERR_HIP;
    }
    return FA_OK;
  }
  BwdParams p = {};
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.dout = a->dout;
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  p.lse = a->lse;
  p.delta = (float*)a->workspace;
  p.dq_acc = nullptr;
  p.q_ss = a->q_stride_t; p.q_sh = a->q_stride_h;
  p.k_ss = a->k_stride_t; p.k_sh = a->k_stride_h;
  p.v_ss = a->v_stride_t; p.v_sh = a->v_stride_h;
  p.o_ss = a->o_stride_t; p.o_sh = a->o_stride_h;
  p.do_ss = a->do_stride_t; p.do_sh = a->do_stride_h;
  p.dq_ss = a->dq_stride_t; p.dq_sh = a->dq_stride_h;
  p.dk_ss = a->dk_stride_t; p.dk_sh = a->dk_stride_h;
  p.dv_ss = a->dv_stride_t; p.dv_sh = a->dv_stride_h;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.total_q = a->total_q;
  p.B = a->nseq; p.Sq = a->max_seqlen_q; p.Sk = a->max_seqlen_k; p.Hq = a->Hq; p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.causal = a->causal != 0;
  p.scale = a->softmax_scale;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  const int stages = FA_BWD_PREPROCESS | FA_BWD_DKDV | FA_BWD_DQ;
  return hip_status(launch_bwd_bf16(p, a->d, a->causal != 0, true, stages, stream));
}

fa_status fa_quantize_fp8(const float* x, int64_t sb, int64_t ss, int64_t sh, int32_t B, int32_t S,
                          int32_t H, int32_t d, int32_t per_tensor, void* codes, float* scales,
                          hipStream_t stream) {
  if (!x || !codes || !scales) return FA_ERR_NULL;
  if (B < 0 || S < 0 || H < 1) return FA_ERR_SHAPE;
  if (d < 16 || d > 256 || d % 16 != 0) return FA_ERR_HEADDIM;
  if (sb < 0 || ss < 0 || sh < 0) return FA_ERR_SHAPE;
  if (((uintptr_t)x & 3u) || ((uintptr_t)codes & 15u) || ((uintptr_t)scales & 3u)) return FA_ERR_ALIGN;
  if (B == 0 || S == 0) return FA_OK;
  const int64_t nb = ((int64_t)S + 127) / 128;
  const Span sx = span4(x, B, S, H, d, sb, ss, sh, 4);
  const Span sc = lin(codes, mul_sat(B, S, H, d), 1);
  const Span ss_ = lin(scales, mul_sat(B, H, nb), 4);
  const Span all[3] = {sx, sc, ss_};
  if (any_bad(all) || mul_sat(B, H, nb) > 0x7fffffffLL || mul_sat(B, S, H, d / 16) > 0x7fffffffLL * 256)
    return FA_ERR_SHAPE;
  if (overlap(sx, sc) || overlap(sx, ss_) || overlap(sc, ss_)) return FA_ERR_ALIAS;
  return hip_status(launch_quantize_fp8(x, sb, ss, sh, B, S, H, d, per_tensor != 0, codes, scales, stream));
}

fa_status fa_merge(const fa_merge_args* a, hipStream_t stream) {
  if (!a) return FA_ERR_NULL;
  if (a->dtype != FA_BF16 && a->dtype != FA_FP32) return FA_ERR_DTYPE;
  if (a->nparts < 1 || a->B < 0 || a->S < 0 || a->H < 1) return FA_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return FA_ERR_HEADDIM;
  const int64_t rows = mul_sat(a->B, a->S, a->H);
  if (rows == 0) return FA_OK;
  if (!a->o_parts || !a->lse_parts || !a->o.ptr || !a->lse) return FA_ERR_NULL;
  const int64_t es = a->dtype == FA_FP32 ? 4 : 2;
  if (((uintptr_t)a->o_parts & (uintptr_t)(es - 1)) || ((uintptr_t)a->lse_parts & 3u) ||
      ((uintptr_t)a->lse & 3u) || ((uintptr_t)a->o.ptr & 1u))
    return FA_ERR_ALIGN;
  if (a->o.stride_b < 0 || a->o.stride_s < 0 || a->o.stride_h < 0) return FA_ERR_SHAPE;
  if (rows > 0x7fffffffLL * 4) return FA_ERR_SHAPE;
  const Span sop = lin(a->o_parts, mul_sat(a->nparts, rows, a->d), es);
  const Span slp = lin(a->lse_parts, mul_sat(a->nparts, rows), 4);
  const Span so = span4(a->o.ptr, a->B, a->S, a->H, a->d, a->o.stride_b, a->o.stride_s, a->o.stride_h, 2);
  const Span sl = lin(a->lse, rows, 4);
  const Span all[4] = {sop, slp, so, sl};
  if (any_bad(all)) return FA_ERR_SHAPE;
  if (overlap(so, sop) || overlap(so, slp) || overlap(sl, sop) || overlap(sl, slp) || overlap(so, sl))
    return FA_ERR_ALIAS;
  MergeParams p = {};
  p.o_parts = a->o_parts;
  p.lse_parts = a->lse_parts;
  p.o = a->o.ptr;
  p.lse = a->lse;
  p.o_sb = a->o.stride_b; p.o_ss = a->o.stride_s; p.o_sh = a->o.stride_h;
  p.nparts = a->nparts; p.B = a->B; p.S = a->S; p.H = a->H;
  return hip_status(launch_merge(p, a->d, a->dtype == FA_FP32, stream));
}

fa_status fa_fwd_mxfp8(const fa_fwd_mxfp8_args* a, hipStream_t stream) {
  if (!a) return FA_ERR_NULL;
  // the dense FP8 rules (shapes, strides in bytes, alignment, aliasing)
  fa_fwd_args f = {};
  f.dtype = FA_FP8_E4M3;
  f.B = a->B; f.Sq = a->Sq; f.Sk = a->Sk; f.Hq = a->Hq; f.Hkv = a->Hkv; f.d = a->d;
  f.causal = a->causal;
  f.softmax_scale = a->softmax_scale;
  f.q = a->q; f.k = a->k; f.v = a->v; f.o = a->o;
  f.lse = a->lse;
  f.q_descale = (const float*)a->q_scale;
  f.k_descale = (const float*)a->k_scale;
  f.v_descale = (const float*)a->v_scale;
  const fa_status s = check_fwd(&f);
  if (s != FA_OK) return s;
  if (a->B == 0 || a->Sq == 0) return FA_OK;
  const int64_t nb = a->d / 32;
  const Span sqs = lin(a->q_scale, mul_sat(a->B, a->Sq, a->Hq, nb), 1);
  const Span sks = lin(a->k_scale, mul_sat(a->B, a->Sk, a->Hkv, nb), 1);
  const Span svs = lin(a->v_scale, mul_sat(a->B, a->Hkv, ((int64_t)a->Sk + 31) / 32, a->d), 1);
  const Span so = span4(a->o.ptr, a->B, a->Sq, a->Hq, a->d, a->o.stride_b, a->o.stride_s, a->o.stride_h, 2);
  const Span sl = lin(a->lse, mul_sat(a->B, a->Hq, a->Sq), 4);
  const Span sc[3] = {sqs, sks, svs};
  if (any_bad(sc)) return FA_ERR_SHAPE;
  for (const Span& x : sc)
    if (overlap(x, so) || overlap(x, sl)) return FA_ERR_ALIAS;
  FwdParams p = {};
  p.q = a->q.ptr; p.k = a->k.ptr; p.v = a->v.ptr; p.o = a->o.ptr; p.lse = a->lse;
  p.q_sb = a->q.stride_b; p.q_ss = a->q.stride_s; p.q_sh = a->q.stride_h;
  p.k_sb = a->k.stride_b; p.k_ss = a->k.stride_s; p.k_sh = a->k.stride_h;
  p.v_sb = a->v.stride_b; p.v_ss = a->v.stride_s; p.v_sh = a->v.stride_h;
  p.o_sb = a->o.stride_b; p.o_ss = a->o.stride_s; p.o_sh = a->o.stride_h;
  p.lse_sb = (int64_t)a->Hq * a->Sq;
  p.lse_sh = a->Sq;
  p.B = a->B; p.Sq = a->Sq; p.Sk = a->Sk; p.Hq = a->Hq; p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.num_m_tiles = (a->Sq + kBM - 1) / kBM;
  p.scale = a->softmax_scale;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  p.q_e8m0 = a->q_scale;
  p.k_e8m0 = a->k_scale;
  p.v_e8m0 = a->v_scale;
  return hip_status(launch_fwd_mxfp8(p, a->d, a->causal != 0, stream));
}

fa_status fa_quantize_mxfp8(const float* x, int64_t sb, int64_t ss, int64_t sh, int32_t B, int32_t S,
                            int32_t H, int32_t d, int32_t axis, void* codes, uint8_t* scales,
                            hipStream_t stream) {
  if (!x || !codes || !scales) return FA_ERR_NULL;
  if (B < 0 || S < 0 || H < 1 || (axis != 0 && axis != 1)) return FA_ERR_SHAPE;
  if (d < 32 || d > 256 || d % 32 != 0) return FA_ERR_HEADDIM;
  if (sb < 0 || ss < 0 || sh < 0) return FA_ERR_SHAPE;
  if (((uintptr_t)x & 3u) || ((uintptr_t)codes & 15u) || ((uintptr_t)scales & 3u)) return FA_ERR_ALIGN;
  if (B == 0 || S == 0) return FA_OK;
  const int64_t nsc = axis == 0 ? mul_sat(B, S, H, d / 32) : mul_sat(B, H, ((int64_t)S + 31) / 32, d);
  const Span sx = span4(x, B, S, H, d, sb, ss, sh, 4);
  const Span sc = lin(codes, mul_sat(B, S, H, d), 1);
  const Span ss_ = lin(scales, nsc, 1);
  const Span all[3] = {sx, sc, ss_};
  if (any_bad(all) || nsc > 0x7fffffffLL * 256) return FA_ERR_SHAPE;
  if (overlap(sx, sc) || overlap(sx, ss_) || overlap(sc, ss_)) return FA_ERR_ALIAS;
  return hip_status(launch_quantize_mxfp8(x, sb, ss, sh, B, S, H, d, axis, codes, scales, stream));
}

size_t fa_fwd_kvcache_workspace_size(const fa_fwd_kvcache_args* a) {
  if (!a) return 0;
  const DecodePlan pl = kvcache_plan(a);
  return pl.eligible ? pl.o_part_bytes + pl.lse_part_bytes : 0;
}

fa_status fa_fwd_kvcache(const fa_fwd_kvcache_args* a, hipStream_t stream) {
  const fa_status s = check_kvcache(a);
  if (s != FA_OK) return s;
  if (a->B == 0) return FA_OK;
  KvCacheParams kv = {};
  kv.seqlens = a->cache_seqlens;
  kv.block_table = a->block_table;
  kv.bt_stride = a->block_table_stride;
  int shift = 0;
  while (a->block_table && (1 << shift) < a->page_size) ++shift;
  kv.page_shift = shift;
  kv.snew = a->Snew;
  kv.k_sp = a->k_stride_page;
  kv.v_sp = a->v_stride_page;
  if (a->Snew > 0) {
    KvAppendParams ap = {};
    ap.k_new = a->k_new.ptr;
    ap.v_new = a->v_new.ptr;
    ap.kn_sb = a->k_new.stride_b; ap.kn_ss = a->k_new.stride_s; ap.kn_sh = a->k_new.stride_h;
    ap.vn_sb = a->v_new.stride_b; ap.vn_ss = a->v_new.stride_s; ap.vn_sh = a->v_new.stride_h;
    ap.k_cache = a->k_cache;
    ap.v_cache = a->v_cache;
    ap.k_ss = a->k_stride_s; ap.k_sh = a->k_stride_h;
    ap.v_ss = a->v_stride_s; ap.v_sh = a->v_stride_h;
    ap.kv = kv;
    ap.B = a->B;
    ap.Hkv = a->Hkv;
    const hipError_t e = launch_kv_append(ap, a->d, stream);
    if (e != hipSuccess) return FA_ERR_HIP;
  }
  if (a->Sq == 0) return FA_OK;
  const int64_t maxlen = kv_max_len(a);
  const float scale_log2 = a->softmax_scale * 1.4426950408889634f;
  const DecodePlan pl = kvcache_plan(a);
  if (pl.eligible && a->workspace && a->workspace_bytes >= pl.o_part_bytes + pl.lse_part_bytes) {
    DecodeParams d = {};
    d.q = a->q.ptr; d.k = a->k_cache; d.v = a->v_cache; d.o = a->o.ptr; d.lse = a->lse;
    d.o_part = (float*)a->workspace;
    d.lse_part = (float*)((char*)a->workspace + pl.o_part_bytes);
    d.q_sb = a->q.stride_b; d.q_ss = a->q.stride_s; d.q_sh = a->q.stride_h;
    d.k_ss = a->k_stride_s; d.k_sh = a->k_stride_h;
    d.v_ss = a->v_stride_s; d.v_sh = a->v_stride_h;
    d.o_sb = a->o.stride_b; d.o_ss = a->o.stride_s; d.o_sh = a->o.stride_h;
    d.lse_sb = (int64_t)a->Hq * a->Sq; d.lse_sh = a->Sq;
    d.B = a->B; d.Sq = a->Sq; d.Sk = (int)maxlen; d.Hq = a->Hq; d.Hkv = a->Hkv; d.group = a->Hq / a->Hkv;
    d.causal = a->causal != 0;
    d.nsplit = pl.nsplit;
    d.nrblk = pl.nrblk;
    d.chunk = pl.chunk;
    d.scale = a->softmax_scale;
    d.scale_log2 = scale_log2;
    d.kv = kv;
    return hip_status(launch_decode_bf16_kvcache(d, a->d, stream));
  }
  FwdParams p = {};
  p.q = a->q.ptr; p.k = a->k_cache; p.v = a->v_cache; p.o = a->o.ptr; p.lse = a->lse;
  p.q_sb = a->q.stride_b; p.q_ss = a->q.stride_s; p.q_sh = a->q.stride_h;
  p.k_ss = a->k_stride_s; p.k_sh = a->k_stride_h;
  p.v_ss = a->v_stride_s; p.v_sh = a->v_stride_h;
  p.o_sb = a->o.stride_b; p.o_ss = a->o.stride_s; p.o_sh = a->o.stride_h;
  p.lse_sb = (int64_t)a->Hq * a->Sq;
  p.lse_sh = a->Sq;
  p.B = a->B; p.Sq = a->Sq; p.Sk = (int)maxlen; p.Hq = a->Hq; p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.num_m_tiles = (a->Sq + kBM - 1) / kBM;
  p.scale = a->softmax_scale;
  p.scale_log2 = scale_log2;
  p.kv = kv;
  const bool causal = a->causal != 0;
  // at most 128 query rows: the one-group kernel, as for the dense forward
  return hip_status(a->d == 128 && a->Sq > 128 ? launch_fwd_bf16_pp_kvcache(p, a->d, causal, stream)
                                               : launch_fwd_bf16_kvcache(p, a->d, causal, stream));
}

}  // extern "C"
