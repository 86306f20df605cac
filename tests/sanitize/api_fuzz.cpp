// Host driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of
// libfa's entry points (test infrastructure).  The kernel launches are
// replaced by stubs that count calls, so every argument check and every
// parameter block runs on the host: each entry point is called with random
// combinations of extreme sizes, strides, flags and (never dereferenced)
// pointers, and with a few hand-made valid argument sets.  Any signed
// overflow, bad shift or out-of-bounds access aborts the run.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>

#include "fa.h"

extern long g_launches;

namespace {

std::mt19937_64 rng(2024);
template <class T, size_t N>
T pick(const T (&v)[N]) {
  return v[rng() % N];
}

const int32_t kI[] = {-2147483647 - 1, -1, 0, 1, 2, 3, 8, 16, 31, 32, 33, 64, 127, 128, 129,
                      256, 1000, 4096, 65535, 1 << 20, 1 << 30, 2147483647};
const int32_t kHead[] = {-1, 0, 1, 2, 4, 8, 32, 1 << 16, 2147483647};
const int32_t kD[] = {0, 16, 32, 64, 96, 128, 256, -64};
const int64_t kStride[] = {-8, 0, 1, 8, 64, 128, 4096, int64_t(1) << 20, int64_t(1) << 31,
                           int64_t(1) << 40, INT64_MAX / 4, INT64_MAX - 7, INT64_MIN};
const uintptr_t kBase = uintptr_t(0x100000000000ull);
uintptr_t ptr() {
  static const uintptr_t off[] = {0, 1, 2, 16, 64, 256, uintptr_t(1) << 24, uintptr_t(1) << 32,
                                  uintptr_t(3) << 40, ~uintptr_t(0) - 15};
  const uintptr_t o = pick(off);
  return o == 0 ? 0 : (o > (uintptr_t(1) << 44) ? o : kBase + o + ((rng() % 64) << 26));
}
fa_tensor tensor() { return fa_tensor{(void*)ptr(), pick(kStride), pick(kStride), pick(kStride)}; }
float scale() {
  static const float v[] = {0.125f, 1.f, 0.f, -1.f, 1e30f, 1e-30f, __builtin_inff(), __builtin_nanf("")};
  return pick(v);
}

// A valid dense layout: contiguous [B,S,H,d] at base + 2^32 * slot.
fa_tensor dense(int slot, int64_t S, int64_t H, int64_t d) {
  return fa_tensor{(void*)(kBase + (uintptr_t(slot) << 32)), S * H * d, H * d, d};
}

}  // namespace

int main() {
  unsetenv("FA_DEBUG");   // the fuzzed pointers must never be read
  long ok[16] = {0}, total = 0;
  for (int it = 0; it < 100000; ++it) {
    {
      fa_fwd_args a;
      memset(&a, 0, sizeof a);
      a.dtype = fa_dtype(rng() % 4);
      a.B = pick(kI), a.Sq = pick(kI), a.Sk = pick(kI), a.Hq = pick(kHead), a.Hkv = pick(kHead);
      a.d = pick(kD), a.causal = int(rng() % 2), a.softmax_scale = scale();
      a.q = tensor(), a.k = tensor(), a.v = tensor(), a.o = tensor();
      a.lse = (float*)ptr();
      a.q_descale = (const float*)ptr(), a.k_descale = (const float*)ptr(), a.v_descale = (const float*)ptr();
      a.workspace = (void*)ptr(), a.workspace_bytes = size_t(pick(kStride));
      fa_fwd_workspace_size(&a);
      ok[fa_fwd(&a, nullptr) == FA_OK]++;
    }
    {
      fa_bwd_args a;
      memset(&a, 0, sizeof a);
      a.dtype = fa_dtype(rng() % 4);
      a.B = pick(kI), a.Sq = pick(kI), a.Sk = pick(kI), a.Hq = pick(kHead), a.Hkv = pick(kHead);
      a.d = pick(kD), a.causal = int(rng() % 2), a.softmax_scale = scale();
      a.q = tensor(), a.k = tensor(), a.v = tensor(), a.o = tensor(), a.dout = tensor();
      a.dq = tensor(), a.dk = tensor(), a.dv = tensor();
      a.lse = (const float*)ptr(), a.workspace = (void*)ptr(), a.workspace_bytes = size_t(pick(kStride));
      a.stages = int(rng() % 9) - 1;
      a.q_descale = (const float*)ptr(), a.k_descale = (const float*)ptr(), a.v_descale = (const float*)ptr();
      fa_bwd_workspace_size(&a);
      ok[2 + (fa_bwd(&a, nullptr) == FA_OK)]++;
      fa_bwd_noalloc(&a, nullptr);
    }
    {
      fa_fwd_varlen_args a;
      memset(&a, 0, sizeof a);
      a.dtype = fa_dtype(rng() % 3);
      a.nseq = pick(kI), a.Hq = pick(kHead), a.Hkv = pick(kHead), a.d = pick(kD);
      a.max_seqlen_q = pick(kI), a.max_seqlen_k = pick(kI), a.total_q = pick(kI), a.total_k = pick(kI);
      a.causal = int(rng() % 2), a.softmax_scale = scale();
      a.q = (void*)ptr(), a.k = (void*)ptr(), a.v = (void*)ptr(), a.o = (void*)ptr();
      int64_t* st = &a.q_stride_t;
      for (int i = 0; i < 8; ++i) st[i] = pick(kStride);
      a.cu_seqlens_q = (const int32_t*)ptr(), a.cu_seqlens_k = (const int32_t*)ptr(), a.lse = (float*)ptr();
      ok[4 + (fa_fwd_varlen(&a, nullptr) == FA_OK)]++;
    }
    {
      fa_bwd_varlen_args a;
      memset(&a, 0, sizeof a);
      a.dtype = fa_dtype(rng() % 3);
      a.nseq = pick(kI), a.Hq = pick(kHead), a.Hkv = pick(kHead), a.d = pick(kD);
      a.max_seqlen_q = pick(kI), a.max_seqlen_k = pick(kI), a.total_q = pick(kI), a.total_k = pick(kI);
      a.causal = int(rng() % 2), a.softmax_scale = scale();
      a.q = (void*)ptr(), a.k = (void*)ptr(), a.v = (void*)ptr(), a.o = (void*)ptr(), a.dout = (void*)ptr();
      a.dq = (void*)ptr(), a.dk = (void*)ptr(), a.dv = (void*)ptr();
      int64_t* st = &a.q_stride_t;
      for (int i = 0; i < 16; ++i) st[i] = pick(kStride);
      a.cu_seqlens_q = (const int32_t*)ptr(), a.cu_seqlens_k = (const int32_t*)ptr(), a.lse = (const float*)ptr();
      a.workspace = (void*)ptr(), a.workspace_bytes = size_t(pick(kStride));
      fa_bwd_varlen_workspace_size(&a);
      ok[6 + (fa_bwd_varlen(&a, nullptr) == FA_OK)]++;
    }
    {
      fa_fwd_kvcache_args a;
      memset(&a, 0, sizeof a);
      a.dtype = fa_dtype(rng() % 3);
      a.B = pick(kI), a.Sq = pick(kI), a.Hq = pick(kHead), a.Hkv = pick(kHead), a.d = pick(kD);
      a.Snew = pick(kI), a.causal = int(rng() % 2), a.softmax_scale = scale();
      a.q = tensor(), a.o = tensor(), a.lse = (float*)ptr();
      a.k_cache = (void*)ptr(), a.v_cache = (void*)ptr();
      a.k_stride_page = pick(kStride), a.k_stride_s = pick(kStride), a.k_stride_h = pick(kStride);
      a.v_stride_page = pick(kStride), a.v_stride_s = pick(kStride), a.v_stride_h = pick(kStride);
      a.num_pages = pick(kI), a.page_size = pick(kI), a.max_pages_per_seq = pick(kI);
      a.max_seqlen_k = pick(kI);
      a.block_table = (const int32_t*)ptr(), a.block_table_stride = pick(kStride);
      a.cache_seqlens = (const int32_t*)ptr(), a.k_new = tensor(), a.v_new = tensor();
      a.workspace = (void*)ptr(), a.workspace_bytes = size_t(pick(kStride));
      fa_fwd_kvcache_workspace_size(&a);
      ok[8 + (fa_fwd_kvcache(&a, nullptr) == FA_OK)]++;
    }
    {
      fa_fwd_mxfp8_args a;
      memset(&a, 0, sizeof a);
      a.B = pick(kI), a.Sq = pick(kI), a.Sk = pick(kI), a.Hq = pick(kHead), a.Hkv = pick(kHead);
      a.d = pick(kD), a.causal = int(rng() % 2), a.softmax_scale = scale();
      a.q = tensor(), a.k = tensor(), a.v = tensor(), a.o = tensor(), a.lse = (float*)ptr();
      a.q_scale = (const uint8_t*)ptr(), a.k_scale = (const uint8_t*)ptr(), a.v_scale = (const uint8_t*)ptr();
      ok[10 + (fa_fwd_mxfp8(&a, nullptr) == FA_OK)]++;
    }
    {
      fa_merge_args a;
      memset(&a, 0, sizeof a);
      a.dtype = fa_dtype(rng() % 3);
      a.nparts = pick(kHead), a.B = pick(kI), a.S = pick(kI), a.H = pick(kHead), a.d = pick(kD);
      a.o_parts = (const void*)ptr(), a.lse_parts = (const float*)ptr(), a.o = tensor(), a.lse = (float*)ptr();
      ok[12 + (fa_merge(&a, nullptr) == FA_OK)]++;
    }
    {
      const int r = fa_quantize_fp8((const float*)ptr(), pick(kStride), pick(kStride), pick(kStride), pick(kI),
                                    pick(kI), pick(kHead), pick(kD), int(rng() % 2), (void*)ptr(),
                                    (float*)ptr(), nullptr);
      const int r2 = fa_quantize_mxfp8((const float*)ptr(), pick(kStride), pick(kStride), pick(kStride),
                                       pick(kI), pick(kI), pick(kHead), pick(kD), int(rng() % 3),
                                       (void*)ptr(), (uint8_t*)ptr(), nullptr);
      ok[14 + (r == FA_OK && r2 == FA_OK)]++;
    }
    ++total;
  }
  // valid argument sets: each must pass and launch
  const long before = g_launches;
  for (int causal = 0; causal < 2; ++causal)
    for (int d = 64; d <= 128; d += 64) {
      fa_fwd_args f;
      memset(&f, 0, sizeof f);
      f.dtype = FA_BF16, f.B = 2, f.Sq = 300, f.Sk = 500, f.Hq = 8, f.Hkv = 2, f.d = d, f.causal = causal;
      f.softmax_scale = 0.125f;
      f.q = dense(1, 300, 8, d), f.k = dense(2, 500, 2, d), f.v = dense(3, 500, 2, d), f.o = dense(4, 300, 8, d);
      f.lse = (float*)(kBase + (uintptr_t(5) << 32));
      if (fa_fwd(&f, nullptr) != FA_OK) return 2;
      fa_bwd_args b;
      memset(&b, 0, sizeof b);
      b.dtype = FA_BF16, b.B = 2, b.Sq = 300, b.Sk = 500, b.Hq = 8, b.Hkv = 2, b.d = d, b.causal = causal;
      b.softmax_scale = 0.125f;
      b.q = f.q, b.k = f.k, b.v = f.v, b.o = dense(4, 300, 8, d), b.dout = dense(6, 300, 8, d);
      b.dq = dense(7, 300, 8, d), b.dk = dense(8, 500, 2, d), b.dv = dense(9, 500, 2, d);
      b.lse = f.lse, b.workspace = (void*)(kBase + (uintptr_t(10) << 32));
      b.workspace_bytes = fa_bwd_workspace_size(&b);
      if (fa_bwd(&b, nullptr) != FA_OK) return 3;
      b.workspace = nullptr, b.workspace_bytes = 0;
      if (fa_bwd_noalloc(&b, nullptr) != FA_OK) return 5;
      // the FP8 backward: e4m3 q, k, v (strides in bytes) with block scales
      fa_bwd_args c = b;
      c.dtype = FA_FP8_E4M3;
      c.q = dense(11, 300, 8, d), c.k = dense(12, 500, 2, d), c.v = dense(13, 500, 2, d);
      c.q_descale = (const float*)(kBase + (uintptr_t(14) << 32));
      c.k_descale = (const float*)(kBase + (uintptr_t(15) << 32));
      c.v_descale = (const float*)(kBase + (uintptr_t(16) << 32));
      c.workspace = (void*)(kBase + (uintptr_t(17) << 32));
      c.workspace_bytes = fa_bwd_workspace_size(&c);
      if (c.workspace_bytes <= fa_bwd_workspace_size(&b)) return 6;
      if (fa_bwd(&c, nullptr) != FA_OK) return 7;
    }
  // FA_DEBUG: the cu_seqlens contents are checked on the host (arrays here
  // are host memory; the runtime stubs copy them)
  {
    const int32_t good_q[4] = {0, 100, 100, 250}, good_k[4] = {0, 70, 300, 310};
    const int32_t bad_start[4] = {1, 100, 100, 250}, bad_order[4] = {0, 120, 100, 250};
    const int32_t bad_end[4] = {0, 100, 100, 249}, bad_max[4] = {0, 10, 200, 250};
    fa_fwd_varlen_args v;
    memset(&v, 0, sizeof v);
    v.dtype = FA_BF16, v.nseq = 3, v.Hq = 8, v.Hkv = 2, v.d = 128, v.max_seqlen_q = 150;
    v.max_seqlen_k = 230, v.total_q = 250, v.total_k = 310, v.softmax_scale = 0.125f;
    v.q = (const void*)(kBase + (uintptr_t(20) << 32)), v.k = (const void*)(kBase + (uintptr_t(21) << 32));
    v.v = (const void*)(kBase + (uintptr_t(22) << 32)), v.o = (void*)(kBase + (uintptr_t(23) << 32));
    v.lse = (float*)(kBase + (uintptr_t(24) << 32));
    v.q_stride_t = 8 * 128, v.q_stride_h = 128, v.o_stride_t = 8 * 128, v.o_stride_h = 128;
    v.k_stride_t = v.v_stride_t = 2 * 128, v.k_stride_h = v.v_stride_h = 128;
    v.cu_seqlens_k = good_k;
    const long l0 = g_launches;
    setenv("FA_DEBUG", "1", 1);
    v.cu_seqlens_q = good_q;
    if (fa_fwd_varlen(&v, nullptr) != FA_OK || g_launches == l0) return 8;
    const int32_t* bad[4] = {bad_start, bad_order, bad_end, bad_max};
    for (const int32_t* b : bad) {
      v.cu_seqlens_q = b;
      const long l1 = g_launches;
      if (fa_fwd_varlen(&v, nullptr) != FA_ERR_SEQLENS || g_launches != l1) return 9;
    }
    setenv("FA_DEBUG", "0", 1);   // off again: contents are not read
    v.cu_seqlens_q = bad_order;
    if (fa_fwd_varlen(&v, nullptr) != FA_OK) return 10;
    unsetenv("FA_DEBUG");
  }
  printf("api fuzz: %ld rounds; accepted fwd %ld bwd %ld varlen %ld bwd_varlen %ld kvcache %ld mx %ld "
         "merge %ld quant %ld; valid-set launches %ld\n",
         total, ok[1], ok[3], ok[5], ok[7], ok[9], ok[11], ok[13], ok[15], g_launches - before);
  return g_launches - before >= 16 ? 0 : 4;
}
