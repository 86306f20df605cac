// Measurement probe, not part of the attention path: the dQ accumulation
// traffic that a backward fusing dQ into the dK/dV kernel would generate.
//
// In that design (the deterministic dQ reduction the Dao-AILab repository
// overview names), each workgroup of the dK/dV kernel owns 128 keys of one
// (batch, head) and visits every 64-row query tile of the head; for each it
// would add a 64 x d fp32 partial of dQ into a global accumulator.  This
// kernel performs exactly those adds, with the dK/dV kernel's grid, order and
// occupancy (512 threads, about the same LDS, so one workgroup per CU), and
// no attention arithmetic: its time is a lower bound on what the fused
// kernel would add to the dK/dV kernel for its dQ partials.
//
//   mode 0: device-scope fp32 atomic adds (unordered, the cheapest correct
//           reduction; the semaphore-ordered one moves the same bytes and
//           also waits for its turn)
//   mode 1: plain load, add, store of every partial (racy: a floor for any
//           read-modify-write scheme, ordered or not)
//   mode 2: plain stores only (the write traffic alone)
//
// Every partial element is 1, so after mode 0 each accumulator element
// equals the number of key tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int NT = 512;
constexpr int BQ = 64;
constexpr int BKV = 128;
constexpr int PAD_BYTES = 128 * 1024;   // LDS held like the dK/dV kernel's

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(NT, 1) void dq_accum_kernel(float* acc, int S, int d, int nkt,
                                                         int mode) {
  __shared__ float pad[PAD_BYTES / 4];
  const int bh = blockIdx.x / nkt;
  const int tid = threadIdx.x;
  // keep the LDS allocation (one word per thread, read back below)
  pad[tid * 61 % (PAD_BYTES / 4)] = (float)tid;
  __syncthreads();
  const float one = pad[tid * 61 % (PAD_BYTES / 4)] >= 0.f ? 1.f : 0.f;
  float* head = acc + (int64_t)bh * S * d;
  const int nqt = S / BQ;
  const int per_tile = BQ * d;                     // elements of one partial
  for (int qt = 0; qt < nqt; ++qt) {
    float* tile = head + (int64_t)qt * per_tile;
    for (int e = 4 * tid; e < per_tile; e += 4 * NT) {
      f32x4* p4 = (f32x4*)(tile + e);
      if (mode == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __hip_atomic_fetch_add(tile + e + j, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (mode == 1) {
        f32x4 v = *p4;
        v += one;
        *p4 = v;
      } else {
        *p4 = (f32x4){one, one, one, one};
      }
    }
  }
}

}  // namespace

// acc: [B*H, S, d] fp32, device memory the caller owns (S a multiple of 128,
// d a multiple of 4).  One launch on `stream`; 0 on success, else the HIP
// error code.
extern "C" int fa_probe_dq_accum(float* acc, int B, int H, int S, int d, int mode,
                                 hipStream_t stream) {
  if (!acc || B <= 0 || H <= 0 || S <= 0 || S % BKV || d <= 0 || d % 4 || mode < 0 || mode > 2)
    return (int)hipErrorInvalidValue;
  const int nkt = S / BKV;
  const long grid = (long)B * H * nkt;
  hipLaunchKernelGGL(dq_accum_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, acc, S, d, nkt,
                     mode);
  return (int)hipGetLastError();
}
