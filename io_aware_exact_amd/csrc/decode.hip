// Split-KV decode forward of IO-aware exact attention for gfx950 (bf16 in,
// fp32 accumulate), for few query rows per kv head: Sq * (Hq / Hkv) <= 32.
//
// Method.  The same tiled exact attention as the dense forward (blocks of K
// and V are streamed through on-chip memory with an online softmax: "Flash
// Attention and Efficient Transformer Mechanisms", block computation;
// Dao-AILab repository overview, online softmax with rescaling), with the key
// range cut into chunks that run in parallel.  Each chunk p yields a partial
// result over its own keys, O_p (normalised by its own row sum) and LSE_p;
// exact attention over all keys is recovered from the identity
//     LSE = ln sum_p exp(LSE_p),    O = sum_p exp(LSE_p - LSE) O_p,
// which holds because each partial is a softmax over a disjoint key subset.
// This is the KV-cache inference case the repository overview lists
// (flash_attn_with_kvcache), with a dense cache.
//
// gfx950 mapping.  One decode step reads every K and V byte once and does
// ~4 flop per byte, so the kernel is bound by HBM bandwidth; MFMA is still
// the cheapest way to do the dot products.
//   * A workgroup is ONE wave that owns (batch, kv head, key chunk).  The
//     M = Sq * group query rows of the kv head (all query heads of the group,
//     all query positions) form the 32 columns of S^T = K Q^T, so K and V are
//     read once for the whole group; unused columns are zero.
//   * K rows are loaded straight from HBM into the A operand of the 32x32x16
//     bf16 MFMA (16 bytes per lane per load), in the permuted row order that
//     makes accumulator registers 0..7 / 8..15 hold 8 consecutive keys, so
//     the probabilities are directly the B operand of O^T += V^T P^T.
//   * V rows go HBM -> registers -> a wave-private LDS tile (coalesced
//     16-byte loads, whole rows per 16 lanes) and come back as V^T through
//     the LDS transposing read.  The next block's K and V loads are issued
//     before the current block's MFMAs (32 keys, 16 KB per wave in flight).
//   * A second kernel combines the partials of every row.
//   * KV-cache attention (an appended, possibly paged cache) runs the same
//     kernel with KVC = true: each sequence's length is its cached count plus
//     the appended rows, and every K/V row is addressed through the block
//     table (page, slot); rows past the end read the last valid row instead,
//     and their scores are masked.
#include "device_common.h"
#include "fa_internal.h"

namespace {

constexpr int BNK = 32;   // keys per iteration (one MFMA block)

template <int D>
struct DecTile {
  static constexpr int VSTR = D + 32;        // V row stride in LDS (elements): 4 rows of
                                             // a transposing read fall on disjoint banks
  static constexpr int NC = D / 16;          // 16-wide d chunks (K^T Q)
  static constexpr int ND = D / 32;          // 32-row d blocks of O^T
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int RPP = 64 / CH;        // V rows per wave load pass
  static constexpr int NP = BNK / RPP;       // V load passes per block
  static constexpr int BUF = BNK * VSTR;     // elements of one V buffer
};

__device__ __forceinline__ int row_perm(int l32) {
  return 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
}

// LDS writes of this wave are visible to its later LDS reads and vice versa.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, bool KVC>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  using T = DecTile<D>;
  __shared__ __attribute__((aligned(16))) __bf16 Vs[T::BUF];

  const int split = blockIdx.x % p.nsplit;
  const int rest = blockIdx.x / p.nsplit;
  const int g = rest % p.Hkv;
  const int b = rest / p.Hkv;
  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int Lk = KVC ? p.kv.seqlens[b] + p.kv.snew : p.Sk;
  const int diag = Lk - p.Sq;
  const int nrows = p.Sq * p.group;

  const int kbeg = split * p.chunk;
  const int kend = min(Lk, kbeg + p.chunk);
  const int nblk = kend > kbeg ? (kend - kbeg + BNK - 1) / BNK : 0;

  // ---- Q^T fragments: column n is query row (head-in-group n / Sq, position n % Sq)
  const int n = l32;
  const int hi = n / p.Sq, qi = n % p.Sq;
  const int h = g * p.group + hi;
  bf16x8 qf[T::NC];
  if (n < nrows) {
    const __bf16* qrow = (const __bf16*)p.q + (int64_t)b * p.q_sb + (int64_t)qi * p.q_ss + (int64_t)h * p.q_sh;
#pragma unroll
    for (int c = 0; c < T::NC; ++c) qf[c] = *(const bf16x8*)(qrow + 16 * c + 8 * hh);
  } else {
#pragma unroll
    for (int c = 0; c < T::NC; ++c) qf[c] = (bf16x8){};
  }
  const int lim = (p.causal ? min(Lk - 1, qi + diag) : Lk - 1);

  // ---- K (direct to MFMA operands) and V (via LDS) streaming; keys past the
  // end of the cache read as zero and are masked
  const __bf16* kb = (const __bf16*)p.k + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const __bf16* vb = (const __bf16*)p.v + (int64_t)b * p.v_sb + (int64_t)g * p.v_sh;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)((int64_t)Lk * p.k_ss * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)((int64_t)Lk * p.v_ss * 2));
  const int kp = row_perm(l32);
  const int vrow = lane / T::CH;
  const int vcol = (lane % T::CH) * 8;
  bf16x8 kf[T::NC];
  u32x4 vreg[T::NP];
  // KV cache.  Without a block table the sequence's cache is one dense
  // region, read exactly like the dense path.  With pages of >= 32 tokens a
  // block (32 keys from a multiple of 32) lies in one page: its page number
  // comes from a window of block-table entries held one per lane, and its
  // rows are read through a buffer resource over the page's rows that hold
  // tokens (rows past the end read as zero, as in the dense path).  Smaller
  // pages: every row's page comes from the window by a cross-lane permute,
  // and rows past the end read the last row (finite; their scores are
  // masked).  Lk >= 1 whenever a block is loaded.
  const __bf16* kcb = (const __bf16*)p.k + (int64_t)g * p.k_sh;
  const __bf16* vcb = (const __bf16*)p.v + (int64_t)g * p.v_sh;
  const bool paged = KVC && p.kv.block_table != nullptr;
  const int shift = p.kv.page_shift;
  const int32_t* btrow = paged ? p.kv.block_table + (int64_t)b * p.kv.bt_stride : nullptr;
  const int last_page_no = paged && Lk > 0 ? (Lk - 1) >> shift : 0;
  PageWindow win;
  __amdgpu_buffer_rsrc_t rkc = rk, rvc = rv;
  if (KVC && !paged) {
    rkc = make_rsrc(kcb + (int64_t)b * p.kv.k_sp, (uint32_t)((int64_t)Lk * p.k_ss * 2));
    rvc = make_rsrc(vcb + (int64_t)b * p.kv.v_sp, (uint32_t)((int64_t)Lk * p.v_ss * 2));
  }
  auto load_rows = [&](const __amdgpu_buffer_rsrc_t& rkk, const __amdgpu_buffer_rsrc_t& rvv, int r0) {
    const uint32_t kr = (uint32_t)(r0 + kp);
#pragma unroll
    for (int c = 0; c < T::NC; ++c)
      kf[c] = __builtin_bit_cast(bf16x8, buf_load16(rkk, (kr * (uint32_t)p.k_ss + 16 * c + 8 * hh) * 2));
#pragma unroll
    for (int u = 0; u < T::NP; ++u) {
      const uint32_t r = (uint32_t)(r0 + vrow + u * T::RPP);
      vreg[u] = buf_load16(rvv, (r * (uint32_t)p.v_ss + vcol) * 2);
    }
  };
  auto gload = [&](int j0) {
    if constexpr (KVC) {
      if (!paged) {
        load_rows(rkc, rvc, j0);
      } else if (shift >= 5) {
        const int pn = j0 >> shift;
        win.cover(btrow, pn, pn, last_page_no, lane);
        const int64_t page = win.uniform(pn);
        const int first_tok = pn << shift;
        const int rows = min(Lk - first_tok, 1 << shift);
        const __amdgpu_buffer_rsrc_t rkp = make_rsrc(kcb + page * p.kv.k_sp, (uint32_t)(rows * p.k_ss * 2));
        const __amdgpu_buffer_rsrc_t rvp = make_rsrc(vcb + page * p.kv.v_sp, (uint32_t)(rows * p.v_ss * 2));
        load_rows(rkp, rvp, j0 - first_tok);
      } else {
        win.cover(btrow, j0 >> shift, min(j0 + BNK - 1, Lk - 1) >> shift, last_page_no, lane);
        const int mask = (1 << shift) - 1;
        const int jk = min(j0 + kp, Lk - 1);
        const __bf16* kr = kcb + (int64_t)win.per_lane(jk >> shift) * p.kv.k_sp + (int64_t)(jk & mask) * p.k_ss;
#pragma unroll
        for (int c = 0; c < T::NC; ++c) kf[c] = *(const bf16x8*)(kr + 16 * c + 8 * hh);
#pragma unroll
        for (int u = 0; u < T::NP; ++u) {
          const int jv = min(j0 + vrow + u * T::RPP, Lk - 1);
          vreg[u] = *(const u32x4*)(vcb + (int64_t)win.per_lane(jv >> shift) * p.kv.v_sp +
                                    (int64_t)(jv & mask) * p.v_ss + vcol);
        }
      }
    } else {
      load_rows(rk, rv, j0);
    }
  };
  const int trG = lane >> 4;
  const int tr_row = 8 * (trG >> 1) + ((lane >> 2) & 3);
  const int tr_col = 16 * (trG & 1) + 4 * (lane & 3);

  f32x16 oacc[T::ND];
#pragma unroll
  for (int i = 0; i < T::ND; ++i) oacc[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.scale_log2;

  if (nblk > 0) gload(kbeg);
  for (int t = 0; t < nblk; ++t) {
    const int j0 = kbeg + t * BNK;
    // stage this block's V rows and consume its K operands, then issue the
    // next block's loads into the same registers
#pragma unroll
    for (int u = 0; u < T::NP; ++u) *(u32x4*)(Vs + (vrow + u * T::RPP) * T::VSTR + vcol) = vreg[u];
    f32x16 s = (f32x16){};
#pragma unroll
    for (int c = 0; c < T::NC; ++c) s = mfma32(kf[c], qf[c], s);
    if (t + 1 < nblk) gload(j0 + BNK);
    wave_lds_sync();
    // register i holds key j0 + 16 (i / 8) + 8 hh + i % 8; keys past the
    // chunk belong to the next chunk, keys past lim are masked or missing
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kj = j0 + 16 * (i >> 3) + 8 * hh + (i & 7);
      if (kj > lim || kj >= kend) s[i] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, wave_xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_base) * c2);
    const float nb = -m_base * c2;
    float rs = 0.f;
    bf16x8 pf[2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = fast_exp2(__builtin_fmaf(s[8 * half + e], c2, nb));
        rs += pv;
        pf[half][e] = (__bf16)pv;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < T::ND; ++i) oacc[i] *= alpha;
    const __bf16* vbase = Vs + tr_row * T::VSTR + tr_col;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < T::ND; ++db) {
        const __bf16* vp = vbase + 16 * c * T::VSTR + 32 * db;
        const bf16x8 vf = cat_bf16(lds_read_tr16(vp), lds_read_tr16(vp + 4 * T::VSTR));
        oacc[db] = mfma32(vf, pf[c], oacc[db]);
      }
    // the next iteration's writes come after these reads
    wave_lds_sync();
  }

  // ---- partial result of this chunk: O_p = O / l (fp32), LSE_p
  const float l_tot = l_run + wave_xor32(l_run);
  if (n < nrows) {
    const int64_t row = ((int64_t)b * p.Hq + h) * p.Sq + qi;     // [B,Hq,Sq]
    float* op = p.o_part + (row * p.nsplit + split) * D;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < T::ND; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        f32x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = oacc[db][4 * gi + r] * inv;
        *(f32x4*)(op + 32 * db + 8 * gi + 4 * hh) = w;
      }
    if (hh == 0) p.lse_part[row * p.nsplit + split] = l_tot > 0.f ? m_run * p.scale + logf(l_tot) : -INFINITY;
  }
}

// One wave per query row: LSE = ln sum_p exp(LSE_p), O = sum_p exp(LSE_p - LSE) O_p.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nrow = (int64_t)p.B * p.Hq * p.Sq;
  if (row >= nrow) return;
  const int lane = threadIdx.x & 63;
  const float* lp = p.lse_part + row * p.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, lp[s]);
  const int qi = (int)(row % p.Sq);
  const int64_t bh = row / p.Sq;
  const int h = (int)(bh % p.Hq);
  const int b = (int)(bh / p.Hq);
  __bf16* orow = (__bf16*)p.o + (int64_t)b * p.o_sb + (int64_t)qi * p.o_ss + (int64_t)h * p.o_sh;
  constexpr int PER = D / 64;   // d elements per lane
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    const float* op = p.o_part + row * p.nsplit * D;
    for (int s = 0; s < p.nsplit; ++s) {
      const float w = expf(lp[s] - M);
      wsum += w;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = __builtin_fmaf(w, op[s * D + PER * lane + e], acc[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[PER * lane + e] = (__bf16)(acc[e] * inv);
  if (lane == 0) p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + qi] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
}

template <int D, bool KVC>
hipError_t launch(const DecodeParams& p, hipStream_t stream) {
  const long nblk = (long)p.B * p.Hkv * p.nsplit;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_split_kernel<D, KVC>), dim3((unsigned)nblk), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long nrow = (long)p.B * p.Hq * p.Sq;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)((nrow + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, int d, hipStream_t stream) {
  return d == 128 ? launch<128, false>(p, stream) : launch<64, false>(p, stream);
}

hipError_t launch_decode_bf16_kvcache(const DecodeParams& p, int d, hipStream_t stream) {
  return d == 128 ? launch<128, true>(p, stream) : launch<64, true>(p, stream);
}
