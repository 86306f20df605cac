// Exact merge of partial attention results computed over disjoint key sets,
// for gfx950: the per-shard step of sequence-parallel attention (the
// multi-GPU variants of "Flash Attention and Efficient Transformer
// Mechanisms"), where each part is the forward over one shard of the keys.
// A part's (O_p, LSE_p) is a softmax over its own keys, so with
// M = max_p LSE_p and w_p = exp(LSE_p - M):
//     LSE = M + ln sum_p w_p,    O = sum_p w_p O_p / sum_p w_p,
// exact up to rounding; a part with LSE_p = -inf (no visible key) has
// weight 0, and a row with no part that sees a key gets O = 0, LSE = -inf.
// One wave per output row (b, s, h); HBM-bound.
#include "device_common.h"
#include "fa_internal.h"

namespace {

template <int D, bool F32>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, s, h)
  const int64_t nrow = (int64_t)p.B * p.S * p.H;
  if (row >= nrow) return;
  const int lane = threadIdx.x & 63;
  const int h = (int)(row % p.H);
  const int64_t bs = row / p.H;
  const int s = (int)(bs % p.S);
  const int b = (int)(bs / p.S);
  const int64_t part_o = (int64_t)p.B * p.S * p.H * D;   // elements per part
  const int64_t part_l = (int64_t)p.B * p.H * p.S;
  const int64_t lrow = ((int64_t)b * p.H + h) * p.S + s;  // [B,H,S]
  float M = -INFINITY;
  for (int q = 0; q < p.nparts; ++q) M = fmaxf(M, p.lse_parts[q * part_l + lrow]);
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int q = 0; q < p.nparts; ++q) {
      const float w = expf(p.lse_parts[q * part_l + lrow] - M);
      wsum += w;
      const int64_t base = q * part_o + row * D + PER * lane;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float x = F32 ? ((const float*)p.o_parts)[base + e] : (float)((const __bf16*)p.o_parts)[base + e];
        acc[e] = __builtin_fmaf(w, x, acc[e]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  __bf16* orow = (__bf16*)p.o + (int64_t)b * p.o_sb + (int64_t)s * p.o_ss + (int64_t)h * p.o_sh;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[PER * lane + e] = (__bf16)(acc[e] * inv);
  if (lane == 0) p.lse[lrow] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
}

template <int D, bool F32>
hipError_t launch(const MergeParams& p, hipStream_t stream) {
  const int64_t nrow = (int64_t)p.B * p.S * p.H;
  if (nrow <= 0) return hipSuccess;
  const int64_t grid = (nrow + 3) / 4;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((merge_kernel<D, F32>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int d, bool f32, hipStream_t stream) {
  if (d == 128) return f32 ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  return f32 ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
}
