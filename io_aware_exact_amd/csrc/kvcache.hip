// Append step of KV-cache attention for gfx950: new K/V rows are written into
// the cache before the attention kernels read it (the KV-cache entry point of
// the Dao-AILab repository overview, flash_attn_with_kvcache, with an
// appendable and optionally paged cache).
//
// Row i of sequence b ([B, Snew, Hkv, d] bf16) goes to token position
// seqlens[b] + i of that sequence: slot (position mod page size) of the page
// the block table names for it, or, without a block table, row
// seqlens[b] + i of sequence b's own cache.  A pure copy, one 16-byte chunk
// per lane; it is HBM-bound and moves 2 * B * Snew * Hkv * d * 2 bytes each
// way.
#include "device_common.h"
#include "fa_internal.h"

namespace {

constexpr int NTHREADS = 256;

template <int D>
__global__ __launch_bounds__(NTHREADS) void kv_append_kernel(KvAppendParams p) {
  constexpr int CH = D / 8;   // 16-byte chunks per row
  const int64_t rows = (int64_t)p.B * p.kv.snew * p.Hkv;
  const int64_t i = (int64_t)blockIdx.x * NTHREADS + threadIdx.x;
  if (i >= 2 * rows * CH) return;
  const bool is_v = i >= rows * CH;
  const int64_t ii = is_v ? i - rows * CH : i;
  const int64_t r = ii / CH;
  const int c = (int)(ii % CH) * 8;
  const int g = (int)(r % p.Hkv);
  const int64_t bi = r / p.Hkv;
  const int t = (int)(bi % p.kv.snew);
  const int b = (int)(bi / p.kv.snew);
  const int j = p.kv.seqlens[b] + t;
  const __bf16* src = is_v ? (const __bf16*)p.v_new + b * p.vn_sb + t * p.vn_ss + g * p.vn_sh
                           : (const __bf16*)p.k_new + b * p.kn_sb + t * p.kn_ss + g * p.kn_sh;
  __bf16* dst = is_v ? (__bf16*)p.v_cache + g * p.v_sh +
                           kv_token_offset(p.kv.block_table, p.kv.bt_stride, p.kv.page_shift, b, j, p.kv.v_sp, p.v_ss)
                     : (__bf16*)p.k_cache + g * p.k_sh +
                           kv_token_offset(p.kv.block_table, p.kv.bt_stride, p.kv.page_shift, b, j, p.kv.k_sp, p.k_ss);
  *(u32x4*)(dst + c) = *(const u32x4*)(src + c);
}

}  // namespace

hipError_t launch_kv_append(const KvAppendParams& p, int d, hipStream_t stream) {
  const int64_t chunks = 2LL * p.B * p.kv.snew * p.Hkv * (d / 8);
  if (chunks <= 0) return hipSuccess;
  const int64_t nblk = (chunks + NTHREADS - 1) / NTHREADS;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  if (d == 128)
    hipLaunchKernelGGL((kv_append_kernel<128>), dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL((kv_append_kernel<64>), dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}
