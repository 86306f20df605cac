// Split-KV decode forward of IO-aware exact attention for gfx950 (bf16 in,
// fp32 accumulate), for few query rows per kv head (Sq * (Hq / Hkv) up to a
// few 32-row tiles).
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
//   * A workgroup is ONE wave that owns (batch, kv head, row block, key
//     chunk).  The M = Sq * group query rows of the kv head (all query heads
//     of the group, all query positions) form the columns of S^T = K Q^T, 32
//     per row block, so K and V are read once per 32 rows of the group;
//     unused columns are zero.
//   * K and V tiles of 32 keys go from HBM straight into a 2-stage,
//     wave-private LDS ring by DMA (buffer_load ... lds), stored swizzled so
//     that the K A-operand reads (16 consecutive rows per 16 lanes, in the
//     permuted row order that makes accumulator registers 0..7 / 8..15 hold
//     8 consecutive keys, so the probabilities are directly the B operand of
//     O^T += V^T P^T) and the V^T transposing reads are free of bank
//     conflicts.  While one block is consumed the next is in flight, with no
//     registers held for it; explicit vmcnt waits let the younger block's
//     DMA stay outstanding.
//   * A second kernel combines the partials of every row.
//   * KV-cache attention (an appended, possibly paged cache) runs the same
//     kernel with KVC = 1 or 2: each sequence's length is its cached count plus
//     the appended rows; each DMA covers a few consecutive rows inside one
//     page (pages hold at least 16 tokens) and reads them through that page's
//     buffer resource, found in a window of block-table entries.
#include <type_traits>

#include "device_common.h"
#include "fa_internal.h"

namespace {

constexpr int BNK = 32;   // keys per iteration (one MFMA block)

template <int D>
struct DecTile {
  static constexpr int NC = D / 16;          // 16-wide d chunks (K^T Q)
  static constexpr int ND = D / 32;          // 32-row d blocks of O^T
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

// s_waitcnt immediate waiting until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left at their maxima).
#define VMCNT_IMM(n) ((((n) >> 4) << 14) | 0x0F70 | ((n) & 15))

// ---------------------------------------------------------------------------
// Split-KV decode.  K and V tiles of 32 keys go from HBM straight into an
// NST-stage wave-private LDS ring (buffer_load ... lds, no staging
// registers), so NST - 1 blocks are in flight while one is consumed.  Tiles
// are stored swizzled (swz): the K A-operand reads (16 consecutive rows per
// 16 lanes) and the V transposing reads are both free of bank conflicts.
// Each lane of a 1 KB DMA fetches the logical chunk that belongs at its
// physical slot.  KV cache: a DMA covers RPI consecutive rows, inside one
// page for pages of >= 16 tokens, so each DMA takes the page's buffer
// resource (rows past the sequence end read as zero).
// KVC: 0 the dense tensors; a KV cache of 1 one region per sequence (no
// block table) or 2 pages (each its own instance, which folds away the
// other's load path).
template <int D, int KVC, int NST>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  using T = DecTile<D>;
  constexpr int TILE = BNK * D;            // elements of one K or V tile
  constexpr int RPI = 512 / D;             // rows per 1 KB DMA
  constexpr int NLD = BNK / RPI;           // DMAs per tile
  // one array per stage, so that the compiler can tell a stage being read
  // from the stages whose DMA is still in flight
  __shared__ __attribute__((aligned(16))) __bf16 smem0[2 * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 smem1[2 * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 smem2[NST > 2 ? 2 * TILE : 8];
  static_assert(NST == 2 || NST == 3, "stages");

  // uniform indices, kept scalar: a buffer resource built from a value the
  // compiler takes as per-lane would put every load in a waterfall loop
  const int split = __builtin_amdgcn_readfirstlane(blockIdx.x % p.nsplit);
  const int rest = __builtin_amdgcn_readfirstlane(blockIdx.x / p.nsplit);
  const int rblk = __builtin_amdgcn_readfirstlane(rest % p.nrblk);
  const int rest2 = __builtin_amdgcn_readfirstlane(rest / p.nrblk);
  const int g = __builtin_amdgcn_readfirstlane(rest2 % p.Hkv);
  const int b = __builtin_amdgcn_readfirstlane(rest2 / p.Hkv);
  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int Lk = KVC ? p.kv.seqlens[b] + p.kv.snew : p.Sk;
  const int diag = Lk - p.Sq;
  const int nrows = p.Sq * p.group;

  const int kbeg = split * p.chunk;
  const int kend = min(Lk, kbeg + p.chunk);
  const int nblk = kend > kbeg ? (kend - kbeg + BNK - 1) / BNK : 0;

  // ---- Q^T fragments: column l32 of row block rblk is query row n (head in
  // the group n / Sq, position n % Sq)
  const int n = 32 * rblk + l32;
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

  // ---- DMA addressing: lane's row within a 1 KB group and its logical column
  const int lrow_in = lane / (64 / RPI);
  const int lpc = lane % (64 / RPI);
  uint32_t koff[NLD], voff[NLD];
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int row = RPI * u + lrow_in;
    const int col = swz<D>(row, 8 * lpc) - row * D;
    koff[u] = (uint32_t)(row * p.k_ss + col) * 2;
    voff[u] = (uint32_t)(row * p.v_ss + col) * 2;
  }
  constexpr bool paged = KVC == 2;
  const int shift = p.kv.page_shift;
  const int32_t* btrow = paged ? p.kv.block_table + (int64_t)b * p.kv.bt_stride : nullptr;
  const int last_page_no = paged && Lk > 0 ? (Lk - 1) >> shift : 0;
  PageWindow win;
  const __bf16* kseq = (const __bf16*)uniform_ptr(
      (const __bf16*)p.k + (KVC ? (int64_t)b * p.kv.k_sp : (int64_t)b * p.k_sb) + (int64_t)g * p.k_sh);
  const __bf16* vseq = (const __bf16*)uniform_ptr(
      (const __bf16*)p.v + (KVC ? (int64_t)b * p.kv.v_sp : (int64_t)b * p.v_sb) + (int64_t)g * p.v_sh);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kseq, (uint32_t)((int64_t)Lk * p.k_ss * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vseq, (uint32_t)((int64_t)Lk * p.v_ss * 2));
  const __bf16* kcb = (const __bf16*)p.k + (int64_t)g * p.k_sh;   // paged: page bases
  const __bf16* vcb = (const __bf16*)p.v + (int64_t)g * p.v_sh;
  auto kstage = [&](auto st_c) -> __bf16* {
    constexpr int ST = decltype(st_c)::value;
    return ST == 0 ? smem0 : ST == 1 ? smem1 : smem2;
  };
  auto vstage = [&](auto st_c) -> __bf16* { return kstage(st_c) + TILE; };
  auto issue = [&](auto st, int j0) {
    if (paged) {
      win.cover(btrow, j0 >> shift, min(j0 + BNK - 1, Lk - 1) >> shift, last_page_no, lane);
#pragma unroll
      for (int u = 0; u < NLD; ++u) {
        const int pn = min(j0 + RPI * u, Lk - 1) >> shift;
        const int64_t page = win.uniform(pn);
        const int first_tok = pn << shift;
        const int rows = max(0, min(Lk - first_tok, 1 << shift));
        const uint32_t rel = (uint32_t)(j0 - first_tok);
        buf_load16_lds_stream(make_rsrc(kcb + page * p.kv.k_sp, (uint32_t)(rows * p.k_ss * 2)),
                              rel * (uint32_t)p.k_ss * 2 + koff[u], kstage(st) + RPI * u * D);
        buf_load16_lds_stream(make_rsrc(vcb + page * p.kv.v_sp, (uint32_t)(rows * p.v_ss * 2)),
                              rel * (uint32_t)p.v_ss * 2 + voff[u], vstage(st) + RPI * u * D);
      }
    } else {
      const uint32_t kb0 = (uint32_t)j0 * (uint32_t)p.k_ss * 2, vb0 = (uint32_t)j0 * (uint32_t)p.v_ss * 2;
#pragma unroll
      for (int u = 0; u < NLD; ++u) {
        buf_load16_lds_stream(rk, kb0 + koff[u], kstage(st) + RPI * u * D);
        buf_load16_lds_stream(rv, vb0 + voff[u], vstage(st) + RPI * u * D);
      }
    }
  };

  // ---- operand addresses within a stage (swizzled; see device_common.h)
  const int kp = row_perm(l32);
  int aoff[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) aoff[c] = swz<D>(kp, 16 * c + 8 * hh);
  const int trG = lane >> 4;
  const int tr_row = 8 * (trG >> 1) + ((lane >> 2) & 3);
  const int tr_col = 16 * (trG & 1) + 4 * (lane & 3);
  int toff[2][T::ND];
#pragma unroll
  for (int db = 0; db < T::ND; ++db) {
    toff[0][db] = swz<D>(tr_row, 32 * db + tr_col);
    toff[1][db] = swz<D>(tr_row + 4, 32 * db + tr_col);
  }

  f32x16 oacc[T::ND];
#pragma unroll
  for (int i = 0; i < T::ND; ++i) oacc[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.scale_log2;

  if (nblk > 0) issue(std::integral_constant<int, 0>{}, kbeg);
  if (nblk > 1) issue(std::integral_constant<int, 1>{}, kbeg + BNK);
  if (NST > 2 && nblk > 2) issue(std::integral_constant<int, NST - 1>{}, kbeg + 2 * BNK);
  // block t in stage ST = t mod NST
  auto block = [&](auto st_c, int t) {
    const int j0 = kbeg + t * BNK;
    // block t has landed once at most the younger blocks' DMAs are pending
    const int younger = min(NST - 1, nblk - 1 - t);
    if (NST == 3 && younger == 2) __builtin_amdgcn_s_waitcnt(VMCNT_IMM(4 * NLD));
    else if (younger >= 1) __builtin_amdgcn_s_waitcnt(VMCNT_IMM(2 * NLD));
    else __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
    wave_lds_sync();
    const __bf16* Ks = kstage(st_c);
    const __bf16* Vs = vstage(st_c);
    f32x16 s = (f32x16){};
#pragma unroll
    for (int c = 0; c < T::NC; ++c) s = mfma32(*(const bf16x8*)(Ks + aoff[c]), qf[c], s);
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
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < T::ND; ++db) {
        const bf16x8 vf = cat_bf16(lds_read_tr16(Vs + toff[0][db] + 16 * c * D),
                                   lds_read_tr16(Vs + toff[1][db] + 16 * c * D));
        oacc[db] = mfma32(vf, pf[c], oacc[db]);
      }
    // this stage's reads are done before the DMA refills it
    wave_lds_sync();
    if (t + NST < nblk) issue(st_c, j0 + NST * BNK);
  };
  // Unrolled by 2 NST: the compiler's own wait before a stage's first LDS
  // read is exact except at the loop head, where merging the entry and
  // back-edge paths makes it wait for every DMA in flight.
  for (int t = 0; t < nblk; t += 2 * NST) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int tr = t + r * NST;
      if (tr < nblk) block(std::integral_constant<int, 0>{}, tr);
      if (tr + 1 < nblk) block(std::integral_constant<int, 1>{}, tr + 1);
      if (NST > 2 && tr + 2 < nblk) block(std::integral_constant<int, NST - 1>{}, tr + 2);
    }
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

constexpr int kDecodeStages = 2;   // DMA stages per wave (3 measured slower)

template <int D, int KVC>
hipError_t launch(const DecodeParams& p, hipStream_t stream) {
  if (p.nrblk < 1 || p.nsplit < 1) return hipErrorInvalidValue;
  const long nblk = (long)p.B * p.Hkv * p.nrblk * p.nsplit;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_split_kernel<D, KVC, kDecodeStages>), dim3((unsigned)nblk), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long nrow = (long)p.B * p.Hq * p.Sq;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)((nrow + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, int d, hipStream_t stream) {
  return d == 128 ? launch<128, 0>(p, stream) : launch<64, 0>(p, stream);
}

hipError_t launch_decode_bf16_kvcache(const DecodeParams& p, int d, hipStream_t stream) {
  if (!p.kv.block_table) return d == 128 ? launch<128, 1>(p, stream) : launch<64, 1>(p, stream);
  return d == 128 ? launch<128, 2>(p, stream) : launch<64, 2>(p, stream);
}
