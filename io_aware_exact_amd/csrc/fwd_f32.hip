// fp32 forward of IO-aware exact attention for gfx950 (fp32 in, fp32
// accumulate, fp32 out and LSE): the same tiled computation with an online
// softmax as the bf16 forward ("Flash Attention and Efficient Transformer
// Mechanisms", block computation; Dao-AILab repository overview, online
// softmax with rescaling), with no rounding of Q, K, V or P below fp32.  It
// serves inputs that must not be rounded to bf16; its speed is secondary.
//
// gfx950 mapping: the fp32 matrix instruction v_mfma_f32_32x32x2_f32 (one
// fp32 per lane per operand; A[m][k] in lane m + 32 k, B[k][n] in lane
// n + 32 k; the 16-register accumulator layout of the 32x32 family).
//   * S^T = K Q^T per 32-key block: Q^T stays in registers (D / 2 values per
//     lane); K rows are fed as A rows in the order pi(m) = 2 (4 (m / 8) +
//     m % 4) + (m / 4) % 2, which makes accumulator register i of a lane in
//     half hh hold key 2 i + hh -- exactly the B operand (P^T, keys 2 j + hh)
//     of the j-th step of O^T += V^T P^T.
//   * K and V tiles of 32 keys are staged in LDS (fp32, padded rows), one
//     tile at a time.
#include "device_common.h"
#include "fa_internal.h"

namespace {

constexpr int BM = 128;
constexpr int BN = 32;
constexpr int NTHREADS = 256;

template <int D>
struct F32Tile {
  static constexpr int KSTR = D + 1;     // K rows: 32 rows x 2 columns per read, odd stride
  static constexpr int VSTR = D + 32;    // V rows: 2 rows x 32 columns per read, 32 banks apart
  static constexpr int ND = D / 32;
};

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 1) void fwd_f32_kernel(FwdParams p) {
  using T = F32Tile<D>;
  __shared__ float Ks[BN * T::KSTR];
  __shared__ float Vs[BN * T::VSTR];

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int mt = L % p.num_m_tiles;
  const int rest = L / p.num_m_tiles;
  const int h = rest % p.Hq;
  const int b = rest / p.Hq;
  if (CAUSAL) mt = p.num_m_tiles - 1 - mt;
  const int g = h / p.group;
  const int Lq = p.Sq, Lk = p.Sk;
  const int q0 = mt * BM;
  const int diag = Lk - Lq;

  const float* qb = (const float*)p.q + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
  const float* kb = (const float*)p.k + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const float* vb = (const float*)p.v + (int64_t)b * p.v_sb + (int64_t)g * p.v_sh;
  float* ob = (float*)p.o + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
  float* lseb = p.lse + (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh;

  int kend = Lk;
  if (CAUSAL) kend = min(Lk, q0 + BM + diag);
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int qrow = q0 + wave * 32 + l32;

  // Q^T: lane (n, hh) holds Q[n][2 j + hh], j = 0 .. D/2 - 1
  float qf[D / 2];
#pragma unroll
  for (int j = 0; j < D / 2; ++j) qf[j] = qrow < Lq ? qb[(int64_t)qrow * p.q_ss + 2 * j + hh] : 0.f;
  const int kperm = 2 * (4 * (l32 >> 3) + (l32 & 3)) + ((l32 >> 2) & 1);

  f32x16 oacc[T::ND];
#pragma unroll
  for (int i = 0; i < T::ND; ++i) oacc[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.scale_log2;
  const int wave_last_row = q0 + wave * 32 + 31;
  const int lim = CAUSAL ? min(Lk - 1, qrow + diag) : Lk - 1;

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * BN;
    // stage K and V rows j0 .. j0 + 31 (zero past the end)
    for (int e = tid; e < BN * D; e += NTHREADS) {
      const int r = e / D, c = e % D;
      const bool in = j0 + r < Lk;
      Ks[r * T::KSTR + c] = in ? kb[(int64_t)(j0 + r) * p.k_ss + c] : 0.f;
      Vs[r * T::VSTR + c] = in ? vb[(int64_t)(j0 + r) * p.v_ss + c] : 0.f;
    }
    __syncthreads();
    if (!CAUSAL || j0 <= wave_last_row + diag) {
      f32x16 s = (f32x16){};
#pragma unroll
      for (int j = 0; j < D / 2; ++j) s = mfma_f32(Ks[kperm * T::KSTR + 2 * j + hh], qf[j], s);
      // register i holds key j0 + 2 i + hh
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (j0 + 2 * i + hh > lim) s[i] = -INFINITY;
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_base = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_base) * c2);
      const float nb = -m_base * c2;
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = fast_exp2(__builtin_fmaf(s[i], c2, nb));
        rs += s[i];
      }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < T::ND; ++db) {
        oacc[db] *= alpha;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          oacc[db] = mfma_f32(Vs[(2 * j + hh) * T::VSTR + 32 * db + l32], s[j], oacc[db]);
      }
    }
    __syncthreads();
  }

  const float l_tot = l_run + wave_xor32(l_run);
  if (qrow < Lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = ob + (int64_t)qrow * p.o_ss;
#pragma unroll
    for (int db = 0; db < T::ND; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        f32x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = oacc[db][4 * gi + r] * inv;
        *(f32x4*)(orow + 32 * db + 8 * gi + 4 * hh) = w;
      }
    if (hh == 0) lseb[qrow] = l_tot > 0.f ? m_run * p.scale + logf(l_tot) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const long nblk = (long)p.num_m_tiles * p.Hq * p.B;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  return causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
}
