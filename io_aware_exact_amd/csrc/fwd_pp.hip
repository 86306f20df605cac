// Forward kernel of IO-aware exact attention for gfx950 with two wave groups
// in ping-pong (bf16 in, fp32 accumulate, bf16 out, fp32 LSE).
//
// Method: as the tiled forward ("Flash Attention and Efficient Transformer
// Mechanisms", block computation; Dao-AILab repository overview, online
// softmax with rescaling).  The schedule follows the idea of hiding the
// low-throughput softmax under matrix products ("FlashAttention-3: Fast and
// Accurate Attention with Asynchrony and Low-precision", second
// contribution), built for CDNA4 from barriers instead of asynchronous
// tensor cores:
//   * a workgroup of 8 waves owns 256 query rows (32 per wave); waves 0-3
//     (group A) and 4-7 (group B) share the four SIMDs pairwise;
//   * work alternates in phases separated by workgroup barriers: in every
//     phase one group issues MFMAs -- P V for tile t-1 and the scores of tile
//     t -- while the other runs the softmax of its newest scores, so the two
//     waves of a SIMD always have different pipes to use;
//   * group A takes the MFMA role in even phases, B in odd ones; phase f reads
//     K of tile f/2 and V of tile f/2 - 1; K_{t+1} and V_t are loaded in
//     phase 2t into the free LDS stages, straight from HBM by LDS DMA (or,
//     for KV caches with pages below 64 tokens, through registers written at
//     the end of phase 2t+1), and are in LDS when phase 2t+1 ends.
// Operand layouts, the transposed score orientation, lazy rescaling and
// masking are those of the one-group forward kernel.
#include <type_traits>

#include "device_common.h"
#include "fa_internal.h"

namespace {

constexpr int BM = 256;
constexpr int BN = 64;
constexpr int NT = 512;

// DMA: K and V tiles go from HBM straight into swizzled LDS stages (swz in
// device_common.h, no padding); otherwise through registers into padded rows.
template <int D, bool DMA>
struct PpTile {
  static constexpr int KSTR = DMA ? D : D + 8;    // K rows: 16 rows x 16 bytes per 16 lanes
  static constexpr int VSTR = DMA ? D : D + 32;   // V rows: read transposed, 4 rows x 64 bytes
  static constexpr int NC = D / 16;
  static constexpr int ND = D / 32;
  static constexpr int CH = D / 8;
  static constexpr int RPP = NT / CH;
  static constexpr int NP = BN / RPP;
  static constexpr int KSTAGE = BN * KSTR;
  static constexpr int VSTAGE = BN * VSTR;
};

// Workgroup barrier between phases.  The instruction scheduler may not move
// work across it: register-only work (the exponentials) would otherwise
// drift into the neighbouring phase and the two groups would no longer
// alternate.  It waits for this wave's LDS accesses only, not for loads in
// flight (a fenced barrier would also wait for the LDS DMAs issued in the
// phase); tiles that must have landed are waited for explicitly.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// KVC: 0 the dense or packed tensors; a KV cache of 1 one region per
// sequence (no block table), 2 pages of at least 64 tokens, 3 smaller pages
// (each layout its own instance, which folds away the paths it cannot take)
template <int D, bool CAUSAL, bool VARLEN, int KVC>
__global__ __launch_bounds__(NT, 1) void fwd_bf16_pp_kernel(FwdParams p) {
  // dense and packed tensors and KV caches whose 64-key tiles each lie in one
  // region (no block table, or pages of >= 64 tokens): tiles by LDS DMA;
  // smaller pages (a page per row) through registers
  constexpr bool DMA = KVC <= 2;
  using T = PpTile<D, DMA>;
  // one array per stage: the compiler then knows that a DMA into one stage
  // does not write the others, and makes reads of the others wait for it
  __shared__ __attribute__((aligned(16))) __bf16 ks0[T::KSTAGE];
  __shared__ __attribute__((aligned(16))) __bf16 ks1[T::KSTAGE];
  __shared__ __attribute__((aligned(16))) __bf16 vs0[T::VSTAGE];
  __shared__ __attribute__((aligned(16))) __bf16 vs1[T::VSTAGE];

  // Dense: consecutive query tiles of one head share an XCD.  Packed
  // sequences: runs of query tiles of the query heads of one (sequence, kv
  // head) per XCD (varlen_order).  Causal: heaviest tiles first.
  int mt, h, b;
  if (VARLEN) {
    int row, t;
    if (!varlen_order(blockIdx.x, p.Hkv * p.B, kFwdPpVarlenRun * p.group, row, t)) return;
    mt = t / p.group;
    if (mt >= p.num_m_tiles) return;   // padding of the last run
    h = (row % p.Hkv) * p.group + (t - mt * p.group);
    b = row / p.Hkv;
    if (CAUSAL) mt = p.num_m_tiles - 1 - mt;
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    mt = L % p.num_m_tiles;
    const int rest = L / p.num_m_tiles;
    h = rest % p.Hq;
    b = rest / p.Hq;
    if (CAUSAL) mt = p.num_m_tiles - 1 - mt;
  }
  const int g = h / p.group;
  int Lq = p.Sq, Lk = p.Sk;
  int64_t qtok = 0, ktok = 0;
  if (VARLEN) {
    const int qs = p.cu_q[b], ks = p.cu_k[b];
    Lq = p.cu_q[b + 1] - qs;
    Lk = p.cu_k[b + 1] - ks;
    qtok = qs;
    ktok = ks;
  }
  if (KVC) Lk = p.kv.seqlens[b] + p.kv.snew;   // cached tokens plus the appended ones
  const int q0 = mt * BM;
  if (q0 >= Lq) return;   // workgroup-uniform: no barrier is reached
  const int diag = Lk - Lq;

  const __bf16* qb = (const __bf16*)p.q + (VARLEN ? qtok * p.q_ss : (int64_t)b * p.q_sb) + (int64_t)h * p.q_sh;
  // KV cache: the head's base, rows through the block table
  const __bf16* kb = (const __bf16*)p.k + (KVC ? 0 : VARLEN ? ktok * p.k_ss : (int64_t)b * p.k_sb) + (int64_t)g * p.k_sh;
  const __bf16* vb = (const __bf16*)p.v + (KVC ? 0 : VARLEN ? ktok * p.v_ss : (int64_t)b * p.v_sb) + (int64_t)g * p.v_sh;
  __bf16* ob = (__bf16*)p.o + (VARLEN ? qtok * p.o_ss : (int64_t)b * p.o_sb) + (int64_t)h * p.o_sh;
  float* lseb = p.lse + (VARLEN ? qtok : (int64_t)b * p.lse_sb) + (int64_t)h * p.lse_sh;

  int kend = Lk;
  if (CAUSAL) kend = min(Lk, q0 + BM + diag);
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                  // 0: group A, 1: group B
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- Q^T fragments (B operand of S^T = K Q^T), resident for the sweep
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)((int64_t)Lq * p.q_ss * 2));
  const int qrow = q0 + wave * 32 + l32;
  bf16x8 qf[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c)
    qf[c] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(qrow * p.q_ss + 16 * c + 8 * hh) * 2));

  const int kperm = 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
  const int trG = lane >> 4;
  const int tr_row = 8 * (trG >> 1) + ((lane >> 2) & 3);
  const int tr_col = 16 * (trG & 1) + 4 * (lane & 3);

  // ---- K/V staging through registers into two LDS stages each
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)((int64_t)Lk * p.k_ss * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)((int64_t)Lk * p.v_ss * 2));
  const int lrow = tid / T::CH;
  const int lcol = (tid % T::CH) * 8;
  const uint32_t koff = (uint32_t)(lrow * p.k_ss + lcol) * 2;
  const uint32_t voff = (uint32_t)(lrow * p.v_ss + lcol) * 2;
  u32x4 kreg[T::NP], vreg[T::NP];
  // stages are chosen at compile time (St: std::integral_constant)
  auto kstage = [&](auto St) -> __bf16* { return decltype(St)::value ? ks1 : ks0; };
  auto vstage = [&](auto St) -> __bf16* { return decltype(St)::value ? vs1 : vs0; };
  // KV cache.  Without a block table the sequence's cache is one dense
  // region, read like the dense path.  With pages of >= 64 tokens a tile (64
  // keys from a multiple of 64) lies in one page, found in a window of
  // block-table entries held one per lane and read through a buffer resource
  // over the page's rows that hold tokens (rows past the end read as zero).
  // Smaller pages: each row's page comes from the window by a cross-lane
  // permute, and rows past the end read the last row (finite; masked).
  constexpr bool paged = KVC >= 2;
  const int shift = p.kv.page_shift;
  const int32_t* btrow = paged ? p.kv.block_table + (int64_t)b * p.kv.bt_stride : nullptr;
  const int last_page_no = paged && Lk > 0 ? (Lk - 1) >> shift : 0;
  PageWindow win;
  __amdgpu_buffer_rsrc_t rkc = rk, rvc = rv;
  if (KVC && !paged) {
    rkc = make_rsrc(kb + (int64_t)b * p.kv.k_sp, (uint32_t)((int64_t)Lk * p.k_ss * 2));
    rvc = make_rsrc(vb + (int64_t)b * p.kv.v_sp, (uint32_t)((int64_t)Lk * p.v_ss * 2));
  }
  // one operand (K or V) of the tile at key j0
  auto gload_one = [&](u32x4 (&regs)[T::NP], const __amdgpu_buffer_rsrc_t& rd, uint32_t off,
                       const __bf16* base, int64_t sp, int64_t ss, int j0) {
    if constexpr (KVC) {
      if (!paged) {
#pragma unroll
        for (int u = 0; u < T::NP; ++u) regs[u] = buf_load16(rd, off + (uint32_t)(j0 + u * T::RPP) * (uint32_t)ss * 2);
      } else if (KVC == 2) {
        const int pn = j0 >> shift;
        win.cover(btrow, pn, pn, last_page_no, lane);
        const int64_t page = win.uniform(pn);
        const int first_tok = pn << shift;
        const int rows = min(Lk - first_tok, 1 << shift);
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(base + page * sp, (uint32_t)(rows * ss * 2));
#pragma unroll
        for (int u = 0; u < T::NP; ++u)
          regs[u] = buf_load16(rp, off + (uint32_t)(j0 - first_tok + u * T::RPP) * (uint32_t)ss * 2);
      } else {
        win.cover(btrow, j0 >> shift, min(j0 + BN - 1, Lk - 1) >> shift, last_page_no, lane);
        const int mask = (1 << shift) - 1;
#pragma unroll
        for (int u = 0; u < T::NP; ++u) {
          const int j = min(j0 + lrow + u * T::RPP, Lk - 1);
          regs[u] = *(const u32x4*)(base + (int64_t)win.per_lane(j >> shift) * sp + (int64_t)(j & mask) * ss + lcol);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < T::NP; ++u) regs[u] = buf_load16(rd, off + (uint32_t)(j0 + u * T::RPP) * (uint32_t)ss * 2);
    }
  };
  auto gload_k = [&](int j0) __attribute__((always_inline)) { gload_one(kreg, KVC ? rkc : rk, koff, kb, p.kv.k_sp, p.k_ss, j0); };
  auto gload_v = [&](int j0) __attribute__((always_inline)) { gload_one(vreg, KVC ? rvc : rv, voff, vb, p.kv.v_sp, p.v_ss, j0); };
  auto lstore_k = [&](auto st) __attribute__((always_inline)) {
    __bf16* Ks = kstage(st);
#pragma unroll
    for (int u = 0; u < T::NP; ++u) *(u32x4*)(Ks + (lrow + u * T::RPP) * T::KSTR + lcol) = kreg[u];
  };
  auto lstore_v = [&](auto st) __attribute__((always_inline)) {
    __bf16* Vs = vstage(st);
#pragma unroll
    for (int u = 0; u < T::NP; ++u) *(u32x4*)(Vs + (lrow + u * T::RPP) * T::VSTR + lcol) = vreg[u];
  };
  // LDS DMA: each wave fills rows [8 w, 8 w + 8) of a tile, one 1 KB block
  // (RPI rows) per load, every lane fetching the logical chunk that belongs
  // at its physical place in the swizzled row.  The data is in LDS once
  // vmcnt has drained (waited for before the barrier that ends phase 2t+1).
  constexpr int RPI = 512 / D;
  constexpr int NLD = 8 / RPI;
  uint32_t kdoff[NLD], vdoff[NLD];
  if constexpr (DMA) {
    const int lrow_in = lane / (64 / RPI), lpc = lane % (64 / RPI);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int row = 8 * wave + RPI * u + lrow_in;
      const int col = swz<D>(row, 8 * lpc) - row * D;   // logical column of this chunk
      kdoff[u] = (uint32_t)(row * p.k_ss + col) * 2;
      vdoff[u] = (uint32_t)(row * p.v_ss + col) * 2;
    }
  }
  // the buffer resource and first-row byte offset of the tile at key j0:
  // dense, packed and unpaged caches read one region; with pages of >= 64
  // tokens the tile lies in one page, read through a resource over that
  // page's rows that hold tokens
  auto tile_src = [&](int j0, const __amdgpu_buffer_rsrc_t& rd, const __bf16* base, int64_t sp, int64_t ss,
                      __amdgpu_buffer_rsrc_t& r, uint32_t& off) __attribute__((always_inline)) {
    if constexpr (KVC == 2) {
      const int pn = j0 >> shift;
      win.cover(btrow, pn, pn, last_page_no, lane);
      const int64_t page = win.uniform(pn);
      const int first_tok = pn << shift;
      const int rows = min(Lk - first_tok, 1 << shift);
      r = make_rsrc(base + page * sp, (uint32_t)(rows * ss * 2));
      off = (uint32_t)(j0 - first_tok) * (uint32_t)ss * 2;
    } else {
      r = rd;
      off = (uint32_t)j0 * (uint32_t)ss * 2;
    }
  };
  auto dma_k = [&](int j0, auto st) __attribute__((always_inline)) {
    __amdgpu_buffer_rsrc_t r;
    uint32_t off;
    tile_src(j0, KVC ? rkc : rk, kb, p.kv.k_sp, p.k_ss, r, off);
#pragma unroll
    for (int u = 0; u < NLD; ++u) buf_load16_lds(r, off + kdoff[u], kstage(st) + (8 * wave + RPI * u) * D);
  };
  auto dma_v = [&](int j0, auto st) __attribute__((always_inline)) {
    __amdgpu_buffer_rsrc_t r;
    uint32_t off;
    tile_src(j0, KVC ? rvc : rv, vb, p.kv.v_sp, p.v_ss, r, off);
#pragma unroll
    for (int u = 0; u < NLD; ++u) buf_load16_lds(r, off + vdoff[u], vstage(st) + (8 * wave + RPI * u) * D);
  };
  // operand addresses in the swizzled stages: per-lane bases plus constants
  // (the chunk permutation depends on the row modulo 16 only)
  int aoff[T::NC], toff[2][T::ND];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) aoff[c] = DMA ? swz<D>(kperm, 16 * c + 8 * hh) : kperm * T::KSTR + 8 * hh + 16 * c;
#pragma unroll
  for (int db = 0; db < T::ND; ++db) {
    toff[0][db] = DMA ? swz<D>(tr_row, 32 * db + tr_col) : tr_row * T::VSTR + tr_col + 32 * db;
    toff[1][db] = DMA ? swz<D>(tr_row + 4, 32 * db + tr_col) : (tr_row + 4) * T::VSTR + tr_col + 32 * db;
  }

  f32x16 oacc[T::ND];
#pragma unroll
  for (int i = 0; i < T::ND; ++i) oacc[i] = (f32x16){};
  f32x16 sacc[2] = {(f32x16){}, (f32x16){}};
  bf16x8 pf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) pf[c] = (bf16x8){};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c2 = p.scale_log2;
  const float lazy_margin = 8.f / c2;   // 2^8 growth of the probabilities, in score units
  const int wave_first_row = q0 + wave * 32;

  // O^T += V^T P^T for the tile whose V is in stage st
  auto pv_product = [&](auto st) __attribute__((always_inline)) {
    const __bf16* vs = vstage(st);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int db = 0; db < T::ND; ++db) {
        const bf16x8 vf = cat_bf16(lds_read_tr16(vs + toff[0][db] + 16 * c * T::VSTR),
                                   lds_read_tr16(vs + toff[1][db] + 16 * c * T::VSTR));
        oacc[db] = mfma32(vf, pf[c], oacc[db]);
      }
    }
    // keep the transposing reads one MFMA group ahead of the products
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * T::ND, 0);
#pragma unroll
    for (int i = 0; i < 3 * T::ND; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, T::ND, 0);
  };
  // S^T = K Q^T for the tile whose K is in stage st
  auto scores = [&](auto st) __attribute__((always_inline)) {
    const __bf16* ks = kstage(st);
    sacc[0] = (f32x16){};
    sacc[1] = (f32x16){};
#pragma unroll
    for (int c = 0; c < T::NC; ++c) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8 kf = *(const bf16x8*)(ks + aoff[c] + 32 * kb2 * T::KSTR);
        sacc[kb2] = mfma32(kf, qf[c], sacc[kb2]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * T::NC - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // mask, running max, lazy rescale, exponentials and row sum of tile t.
  // O = O_acc / l is the same for any running max that keeps the
  // exponentials finite, so m, l and O_acc are rescaled only when some row's
  // max grew by more than 2^8 in exp2 units.
  auto softmax = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * BN;
    const bool need_mask = (j0 + BN > Lk) || (CAUSAL && j0 + BN - 1 > wave_first_row + diag);
    if (need_mask) {
      const int lim = CAUSAL ? min(Lk - 1, qrow + diag) : Lk - 1;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kj = j0 + 32 * kb2 + 16 * (i >> 3) + 8 * hh + (i & 7);
          if (kj > lim) sacc[kb2][i] = -INFINITY;
        }
    }
    float rs = 0.f;
    auto exponentials = [&](float nb) __attribute__((always_inline)) {
      rs = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = fast_exp2(__builtin_fmaf(sacc[kb2][8 * half + e], c2, nb));
            rs += pv;
            pf[2 * kb2 + half][e] = (__bf16)pv;
          }
        }
    };
    // Once every row of the wave has an m, the exponentials are first taken
    // against it without forming the tile max: if every lane's partial row
    // sum is still at most 2^8, no probability exceeds 2^8 and the tile is
    // done.  Only otherwise is the tile max formed, m, l and O_acc rescaled
    // (lazily, as above) and the exponentials redone.
    bool exact = true;
    if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY) == 0) {
      exponentials(-m_run * c2);
      exact = __builtin_amdgcn_ballot_w64(!(rs <= 256.f)) != 0;
    }
    if (exact) {
      float mx = sacc[0][0];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb2][i]);
      mx = fmaxf(mx, wave_xor32(mx));
      const bool grow = mx > m_run + lazy_margin;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = grow ? fast_exp2((m_run - mx) * c2) : 1.f;
        if (grow) m_run = mx;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < T::ND; ++i) oacc[i] *= alpha;
      }
      exponentials((m_run == -INFINITY) ? 0.f : -m_run * c2);
    }
    l_run += rs;
    __asm__ volatile("" : "+v"(l_run));   // the row sum belongs to this phase
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // K_{t+1} and V_t (Par = t mod 2): issued in phase 2t into the stages
  // last read in phase 2t-1, in LDS after phase 2t+1
  auto issue = [&](int t, auto Par) __attribute__((always_inline)) {
    constexpr int par = decltype(Par)::value;
    using Next = std::integral_constant<int, 1 - par>;
    const bool more = t + 1 < ntiles;
    if constexpr (DMA) {
      if (more) dma_k((t + 1) * BN, Next{});
      dma_v(t * BN, Par);
    } else {
      (void)Next{};
      if (more) gload_k((t + 1) * BN);
      gload_v(t * BN);
    }
  };
  auto land = [&](int t, auto Par) __attribute__((always_inline)) {
    constexpr int par = decltype(Par)::value;
    using Next = std::integral_constant<int, 1 - par>;
    if constexpr (DMA) {
      (void)Next{};
      wait_vmem();
    } else {
      if (t + 1 < ntiles) lstore_k(Next{});
      lstore_v(Par);
    }
  };

  if (ntiles > 0) {
    if constexpr (DMA) {
      dma_k(0, S0{});
    } else {
      gload_k(0);
      lstore_k(S0{});
    }
  }
  wait_vmem();  // Q fragments (and K_0) have landed on every path into the loop
  __syncthreads();

  // A wave sees tile t iff t < nt_w (monotone in t under the causal mask).
  int nt_w = ntiles;
  if (CAUSAL) {
    const int last_key = wave_first_row + 31 + diag;
    nt_w = last_key < 0 ? 0 : min(ntiles, last_key / BN + 1);
  }
  const bool is_a = grp == 0;

  // The two groups run separate programs with the same number of barriers;
  // the loops are unrolled by two so that every stage is known at compile
  // time.  Phases 2t and 2t+1 of group A, t >= 1 (Par = t mod 2):
  auto iter_a = [&](int t, auto Par) __attribute__((always_inline)) {
    using Prev = std::integral_constant<int, 1 - decltype(Par)::value>;
    issue(t, Par);
    __builtin_amdgcn_sched_barrier(0);   // loads first, ahead of the products
    if (t - 1 < nt_w) pv_product(Prev{});
    if (t < nt_w) scores(Par);
    phase_barrier();                                     // phase 2t
    if (t < nt_w) softmax(t);
    land(t, Par);
    phase_barrier();                                     // phase 2t+1
  };
  // and of group B
  auto iter_b = [&](int t, auto Par) __attribute__((always_inline)) {
    using Prev = std::integral_constant<int, 1 - decltype(Par)::value>;
    issue(t, Par);
    if (t - 1 < nt_w) softmax(t - 1);
    phase_barrier();                                     // phase 2t
    if (t - 1 < nt_w) pv_product(Prev{});
    if (t < nt_w) scores(Par);
    land(t, Par);
    phase_barrier();                                     // phase 2t+1
  };
  if (ntiles > 0) {
    const int last = ntiles - 1;
    if (is_a) {
      issue(0, S0{});
      __builtin_amdgcn_sched_barrier(0);
      if (nt_w > 0) scores(S0{});
      phase_barrier();                                   // phase 0
      if (nt_w > 0) softmax(0);
      land(0, S0{});
      phase_barrier();                                   // phase 1
      int t = 1;
      for (; t + 1 < ntiles; t += 2) {
        iter_a(t, S1{});
        iter_a(t + 1, S0{});
      }
      if (t < ntiles) iter_a(t, S1{});
      if (last < nt_w) {
        if (last & 1) pv_product(S1{});
        else pv_product(S0{});
      }
      phase_barrier();                                   // phase 2n
    } else {
      issue(0, S0{});
      phase_barrier();                                   // phase 0
      if (nt_w > 0) scores(S0{});
      land(0, S0{});
      phase_barrier();                                   // phase 1
      int t = 1;
      for (; t + 1 < ntiles; t += 2) {
        iter_b(t, S1{});
        iter_b(t + 1, S0{});
      }
      if (t < ntiles) iter_b(t, S1{});
      if (last < nt_w) softmax(last);
      phase_barrier();                                   // phase 2n
      if (last < nt_w) {                                 // phase 2n+1
        if (last & 1) pv_product(S1{});
        else pv_product(S0{});
      }
    }
  }

  // ---- epilogue: normalise, write O (bf16) and LSE (natural log)
  const float l_tot = l_run + wave_xor32(l_run);
  if (qrow < Lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(ob, (uint32_t)((int64_t)Lq * p.o_ss * 2));
    const uint32_t orow = (uint32_t)(qrow * p.o_ss) * 2;
#pragma unroll
    for (int db = 0; db < T::ND; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(oacc[db][4 * gi + r] * inv);
        buf_store8(__builtin_bit_cast(u32x2, w), ro, orow + (uint32_t)(32 * db + 8 * gi + 4 * hh) * 2);
      }
    if (hh == 0) lseb[qrow] = l_tot > 0.f ? m_run * p.scale + logf(l_tot) : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool VARLEN, int KVC = 0>
hipError_t launch(FwdParams p, hipStream_t stream) {
  const int rows = p.Sq;   // dense: Sq; varlen: max query length
  p.num_m_tiles = (rows + BM - 1) / BM;
  const long nblk = VARLEN ? varlen_grid(p.Hkv * p.B, p.num_m_tiles * p.group, kFwdPpVarlenRun * p.group)
                           : (long)p.num_m_tiles * p.Hq * p.B;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_pp_kernel<D, CAUSAL, VARLEN, KVC>), dim3((unsigned)nblk), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// d = 128 and d = 64, dense or packed.
hipError_t launch_fwd_bf16_pp(const FwdParams& p, int d, bool causal, bool varlen, hipStream_t stream) {
  if (d == 64) {
    if (causal) return varlen ? launch<64, true, true>(p, stream) : launch<64, true, false>(p, stream);
    return varlen ? launch<64, false, true>(p, stream) : launch<64, false, false>(p, stream);
  }
  if (d != 128) return hipErrorInvalidValue;
  if (causal) return varlen ? launch<128, true, true>(p, stream) : launch<128, true, false>(p, stream);
  return varlen ? launch<128, false, true>(p, stream) : launch<128, false, false>(p, stream);
}

// KV-cache attention (d = 128): the cache pages are read through the block
// table, each sequence's length is its cached count plus the appended rows.
hipError_t launch_fwd_bf16_pp_kvcache(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d != 128) return hipErrorInvalidValue;
  if (!p.kv.block_table) return causal ? launch<128, true, false, 1>(p, stream) : launch<128, false, false, 1>(p, stream);
  if (p.kv.page_shift >= 6) return causal ? launch<128, true, false, 2>(p, stream) : launch<128, false, false, 2>(p, stream);
  return causal ? launch<128, true, false, 3>(p, stream) : launch<128, false, false, 3>(p, stream);
}
