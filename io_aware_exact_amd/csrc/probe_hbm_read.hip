// Measurement probe, not part of the attention path: the HBM read rate that
// a plain streaming kernel reaches on this GPU, the practical ceiling that
// the HBM-bound decode kernel is compared with (as a library GEMM is for the
// MFMA-bound kernels).
//
// Every thread reads 16-byte chunks i, i + S, i + 2S, ... of the buffer
// (S = all threads of the grid), U loads in flight per step, and folds them
// with XOR into one word it writes at the end, so that no load can be
// dropped.  mode 0: ordinary loads, U = 4; modes 1, 2, 3: non-temporal loads
// (the policy the decode kernel's K/V stream uses), U = 4, 8, 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int NT = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int MODE>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (MODE == 1) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int MODE, int U>
__global__ __launch_bounds__(NT) void hbm_read_kernel(const u32x4* __restrict__ src, uint64_t n16,
                                                      uint32_t* __restrict__ out) {
  const uint64_t tid = (uint64_t)blockIdx.x * NT + threadIdx.x;
  const uint64_t S = (uint64_t)gridDim.x * NT;
  u32x4 acc = {0u, 0u, 0u, 0u};
  uint64_t i = tid;
  for (; i + (U - 1) * S < n16; i += U * S) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = ld<MODE>(src + i + u * S);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u];
  }
  for (; i < n16; i += S) acc ^= ld<MODE>(src + i);
  out[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

// buf: device memory of `bytes` bytes (a multiple of 16, 16-byte aligned);
// out: device memory of at least grid * 256 words.  One launch of `grid`
// workgroups of 256 threads on `stream`; 0 on success, else the HIP error
// code.
extern "C" int fa_probe_hbm_read(const void* buf, uint64_t bytes, uint32_t* out, uint64_t out_words, int grid,
                                 int mode, hipStream_t stream) {
  if (!buf || !out || bytes == 0 || bytes % 16 || ((uintptr_t)buf & 15) || grid <= 0 ||
      (uint64_t)grid * NT > out_words || mode < 0 || mode > 3)
    return (int)hipErrorInvalidValue;
  const u32x4* src = (const u32x4*)buf;
  const dim3 g((unsigned)grid), b(NT);
  const uint64_t n16 = bytes / 16;
  if (mode == 0) hipLaunchKernelGGL((hbm_read_kernel<0, 4>), g, b, 0, stream, src, n16, out);
  else if (mode == 1) hipLaunchKernelGGL((hbm_read_kernel<1, 4>), g, b, 0, stream, src, n16, out);
  else if (mode == 2) hipLaunchKernelGGL((hbm_read_kernel<1, 8>), g, b, 0, stream, src, n16, out);
  else hipLaunchKernelGGL((hbm_read_kernel<1, 16>), g, b, 0, stream, src, n16, out);
  return (int)hipGetLastError();
}
