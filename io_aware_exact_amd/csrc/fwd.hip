// Forward kernel of IO-aware exact attention for gfx950 (bf16 in, fp32
// accumulate, bf16 out, fp32 LSE), one group of four waves per workgroup.
// Serves d = 64, where the softmax outweighs the matrix work per tile, for
// packed sequences, KV caches and dense inputs with short key sweeps, and
// d = 128 inputs of at most 128 query rows per sequence; other d = 128
// inputs and long dense d = 64 sweeps run the two-group kernel of fwd_pp.hip.
//
// Method (pages on IO-aware exact attention): blocks of Q, K and V are moved
// from HBM into on-chip memory and partial outputs are computed there
// ("Flash Attention and Efficient Transformer Mechanisms", block
// computation); the softmax is evaluated online with a running row maximum
// and rescaling of earlier partial results (Dao-AILab repository overview,
// core contributions), so the Sq x Sk score matrix is never written out
// ("Dao and colleagues: IO-aware exact attention with FlashAttention",
// summary).  The result is exact attention up to floating-point rounding.
//
// gfx950 mapping.
//   * A workgroup of 4 waves owns BM = 128 query rows of one (batch, head);
//     each wave owns 32 rows for the whole KV sweep, so the forward needs no
//     cross-wave reduction.
//   * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16
//     MFMA: K rows are the A operand (read from LDS), Q^T is the B operand
//     held in VGPRs for the whole sweep.  In the accumulator layout every lane
//     then owns ONE query row (column n = lane % 32) and 16 of the 32 keys of a
//     block, so row max and row sum are in-lane, plus one exchange with lane
//     l ^ 32 for the max.
//   * K rows are loaded into the A operand in a permuted order chosen so that
//     accumulator registers 0..7 / 8..15 of a lane hold 8 consecutive keys:
//     after the exponentials they are directly the B operand (P^T) of
//     O^T += V^T P^T, with no register shuffle and no LDS round trip.
//   * V^T, the A operand of that product, is read from the row-major V tile
//     with the LDS transposing load (ds_read_b64_tr_b16).
//   * K/V tiles of BN = 64 keys are double-buffered in LDS; the next tile
//     is issued before the current tile's MFMAs, straight from HBM into the
//     other (swizzled) buffer by LDS DMA, or for KV caches with pages below
//     64 tokens through registers (16 bytes per lane) written to it after
//     them.  One barrier per tile.
//   * exp2 with the softmax scale and log2(e) folded into one FMA.
//   * Causal: tiles entirely above the diagonal are skipped (the loop stops at
//     the last visible key), waves skip tiles none of their rows can see, and
//     element masks are applied only on tiles that cross the diagonal or the
//     sequence end.  Heavy (late) query tiles are dispatched first.
//   * Workgroup ids are remapped so that consecutive tiles of one kv head land
//     on the same XCD (dispatch is round-robin over the 8 XCDs, each with its
//     own L2), letting the head's K/V tiles be served from that L2.
#include "device_common.h"
#include "fa_internal.h"

namespace {

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NTHREADS = 256;

// DMA: tiles go from HBM straight into swizzled LDS stages (swz in
// device_common.h, rows of D elements); otherwise through registers into
// padded rows.
template <int D, bool DMA>
struct FwdTile {
  // LDS row strides (elements) of the padded layout.  K is read in rows of
  // 16 bytes per lane by 16 lanes at once: a stride of 4 banks (mod 64)
  // spreads 16 rows over all 64 banks.  V is read transposed, 4 rows x 64
  // bytes per 32 lanes: a stride of 16 banks (mod 64) puts the 4 rows on
  // disjoint banks.
  static constexpr int KSTR = DMA ? D : D + 8;
  static constexpr int VSTR = DMA ? D : D + 32;
  static constexpr int NC = D / 16;     // 16-wide chunks of d (QK^T)
  static constexpr int ND = D / 32;     // 32-row blocks of d (O^T)
  static constexpr int CH = D / 8;      // 16-byte chunks per row
  static constexpr int RPP = NTHREADS / CH;  // rows per load pass
  static constexpr int NP = BN / RPP;        // load passes per tile
  static constexpr int STAGE = BN * (KSTR + VSTR);
  static constexpr int LDS_ELEMS = 2 * STAGE;
};

// KVC: 0 the dense or packed tensors; a KV cache of 1 one region per
// sequence (no block table), 2 pages of at least 64 tokens, 3 smaller pages
// (each layout its own instance, which folds away the paths it cannot take).
// d=64: three workgroups per CU fit in LDS; the bound keeps every instance
// within the registers of three waves per SIMD.
template <int D, bool CAUSAL, bool VARLEN, int KVC>
__global__ __launch_bounds__(NTHREADS, D == 64 ? 3 : 2) void fwd_bf16_kernel(FwdParams p) {
  // dense and packed tensors and KV caches whose 64-key tiles each lie in one
  // region: tiles by LDS DMA; smaller pages (a page per row) through registers
  constexpr bool DMA = KVC <= 2;
  using T = FwdTile<D, DMA>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[T::LDS_ELEMS];

  // ---- which (batch, head, query tile).  Dense: consecutive tiles of one
  // head share an XCD (L2 reuse of its K/V); causal tiles heaviest first.
  // Packed sequences: runs of query tiles of the query heads of one
  // (sequence, kv head) per XCD, rows rotated over the XCDs (varlen_order).
  int mt, h, b;
  if (VARLEN) {
    int row, t;
    if (!varlen_order(blockIdx.x, p.Hkv * p.B, kFwdVarlenRun * p.group, row, t)) return;
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
  if (q0 >= Lq) return;
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- Q^T fragments (B operand of S^T = K Q^T), resident for the sweep.
  // Rows past the sequence end read as zero (buffer bounds check).
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)((int64_t)Lq * p.q_ss * 2));
  const int qrow = q0 + wave * 32 + l32;
  bf16x8 qf[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c)
    qf[c] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(qrow * p.q_ss + 16 * c + 8 * hh) * 2));

  // K row read by this lane for A-operand row m = l32 (see file comment)
  const int kperm = 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
  // transposing-read coordinates for V^T
  const int trG = lane >> 4;
  const int tr_r = lane & 3;
  const int tr_e = (lane >> 2) & 3;
  const int tr_row = 8 * (trG >> 1) + tr_e;
  const int tr_col = 16 * (trG & 1) + 4 * tr_r;

  // global -> register staging of one K/V tile; rows past the sequence end
  // read as zero (their scores are masked, their P entries are zero)
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)((int64_t)Lk * p.k_ss * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)((int64_t)Lk * p.v_ss * 2));
  const int lrow = tid / T::CH;
  const int lcol = (tid % T::CH) * 8;
  const uint32_t koff = (uint32_t)(lrow * p.k_ss + lcol) * 2;
  const uint32_t voff = (uint32_t)(lrow * p.v_ss + lcol) * 2;
  u32x4 kreg[T::NP], vreg[T::NP];
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
  auto load_rows = [&](const __amdgpu_buffer_rsrc_t& rkk, const __amdgpu_buffer_rsrc_t& rvv, int r0) {
#pragma unroll
    for (int u = 0; u < T::NP; ++u) {
      const uint32_t r = (uint32_t)(r0 + u * T::RPP);
      kreg[u] = buf_load16(rkk, koff + r * (uint32_t)p.k_ss * 2);
      vreg[u] = buf_load16(rvv, voff + r * (uint32_t)p.v_ss * 2);
    }
  };
  auto gload = [&](int j0) {
    if constexpr (KVC) {
      if (!paged) {
        load_rows(rkc, rvc, j0);
      } else if (KVC == 2) {
        const int pn = j0 >> shift;
        win.cover(btrow, pn, pn, last_page_no, lane);
        const int64_t page = win.uniform(pn);
        const int first_tok = pn << shift;
        const int rows = min(Lk - first_tok, 1 << shift);
        load_rows(make_rsrc(kb + page * p.kv.k_sp, (uint32_t)(rows * p.k_ss * 2)),
                  make_rsrc(vb + page * p.kv.v_sp, (uint32_t)(rows * p.v_ss * 2)), j0 - first_tok);
      } else {
        win.cover(btrow, j0 >> shift, min(j0 + BN - 1, Lk - 1) >> shift, last_page_no, lane);
        const int mask = (1 << shift) - 1;
#pragma unroll
        for (int u = 0; u < T::NP; ++u) {
          const int j = min(j0 + lrow + u * T::RPP, Lk - 1);
          const int64_t page = win.per_lane(j >> shift);
          kreg[u] = *(const u32x4*)(kb + page * p.kv.k_sp + (int64_t)(j & mask) * p.k_ss + lcol);
          vreg[u] = *(const u32x4*)(vb + page * p.kv.v_sp + (int64_t)(j & mask) * p.v_ss + lcol);
        }
      }
    } else {
      load_rows(rk, rv, j0);
    }
  };
  auto lstore = [&](__bf16* Ks) {
    __bf16* Vs = Ks + BN * T::KSTR;
#pragma unroll
    for (int u = 0; u < T::NP; ++u) {
      *(u32x4*)(Ks + (lrow + u * T::RPP) * T::KSTR + lcol) = kreg[u];
      *(u32x4*)(Vs + (lrow + u * T::RPP) * T::VSTR + lcol) = vreg[u];
    }
  };
  // LDS DMA: each wave fills rows [16 w, 16 w + 16) of the K and V tiles,
  // one 1 KB block (RPI rows) per load, every lane fetching the logical
  // chunk that belongs at its physical place in the swizzled row.
  constexpr int RPI = 512 / D;
  constexpr int RPW = BN / 4;
  constexpr int NLD = RPW / RPI;
  uint32_t kdoff[NLD], vdoff[NLD];
  if constexpr (DMA) {
    const int lrow_in = lane / (64 / RPI), lpc = lane % (64 / RPI);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int row = RPW * wave + RPI * u + lrow_in;
      const int col = swz<D>(row, 8 * lpc) - row * D;   // logical column of this chunk
      kdoff[u] = (uint32_t)(row * p.k_ss + col) * 2;
      vdoff[u] = (uint32_t)(row * p.v_ss + col) * 2;
    }
  }
  // buffer resources and first-row byte offsets of the tile at key j0:
  // one region, or (pages of >= 64 tokens) the tile's page
  auto dma = [&](int j0, __bf16* Ks) {
    __amdgpu_buffer_rsrc_t r_k = KVC ? rkc : rk, r_v = KVC ? rvc : rv;
    uint32_t ok = (uint32_t)j0 * (uint32_t)p.k_ss * 2, ov = (uint32_t)j0 * (uint32_t)p.v_ss * 2;
    if constexpr (KVC == 2) {
      const int pn = j0 >> shift;
      win.cover(btrow, pn, pn, last_page_no, lane);
      const int64_t page = win.uniform(pn);
      const int first_tok = pn << shift;
      const int rows = min(Lk - first_tok, 1 << shift);
      r_k = make_rsrc(kb + page * p.kv.k_sp, (uint32_t)(rows * p.k_ss * 2));
      r_v = make_rsrc(vb + page * p.kv.v_sp, (uint32_t)(rows * p.v_ss * 2));
      ok = (uint32_t)(j0 - first_tok) * (uint32_t)p.k_ss * 2;
      ov = (uint32_t)(j0 - first_tok) * (uint32_t)p.v_ss * 2;
    }
    __bf16* Vs = Ks + BN * T::KSTR;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      buf_load16_lds(r_k, ok + kdoff[u], Ks + (RPW * wave + RPI * u) * D);
      buf_load16_lds(r_v, ov + vdoff[u], Vs + (RPW * wave + RPI * u) * D);
    }
  };
  // operand addresses: per-lane bases plus constants (in the swizzled layout
  // the chunk permutation depends on the row modulo 16 only)
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
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c2 = p.scale_log2;
  const float lazy_margin = 8.f / c2;   // 2^8 growth of the probabilities, in score units

  if (ntiles > 0) {
    if constexpr (DMA) {
      dma(0, smem);
    } else {
      gload(0);
      lstore(smem);
    }
  }
  wait_vmem();  // Q fragments (and tile 0) have landed on every path into the loop
  __syncthreads();

  const int wave_last_row = q0 + wave * 32 + 31;
  // One tile, with its stage and the other stage as restrict pointers: the
  // compiler then knows that the DMA filling `nxt` writes nothing this tile
  // reads, and issues the reads without waiting for it.
  auto tile = [&](int t, const __bf16* __restrict__ cur, __bf16* __restrict__ nxt) __attribute__((always_inline)) {
    const int j0 = t * BN;
    const bool more = t + 1 < ntiles;
    if (more) {
      if constexpr (DMA) dma(j0 + BN, nxt);
      else gload(j0 + BN);
    }

    // Non-causal: always true, but kept opaque to the compiler, which
    // otherwise schedules the loop into more registers than three waves per
    // SIMD allow once the softmax has its two paths.
    const bool wave_active = CAUSAL ? j0 <= wave_last_row + diag : __builtin_amdgcn_readfirstlane(ntiles) > 0;
    if (wave_active) {
      const __bf16* Ks = cur;
      const __bf16* Vs = cur + BN * T::KSTR;
      // ---- S^T = K Q^T for two 32-key blocks
      f32x16 sacc[2] = {(f32x16){}, (f32x16){}};
      // per-lane bases plus compile-time constants (folded into the LDS
      // instructions' offset fields)
#pragma unroll
      for (int c = 0; c < T::NC; ++c) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const bf16x8 kf = *(const bf16x8*)(Ks + aoff[c] + 32 * kb2 * T::KSTR);
          sacc[kb2] = mfma32(kf, qf[c], sacc[kb2]);
        }
      }
      // ---- mask (only on tiles crossing the diagonal or the sequence end)
      const bool need_mask = (j0 + BN > Lk) || (CAUSAL && j0 + BN - 1 > q0 + wave * 32 + diag);
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
      // ---- online softmax: running max, rescale, exponentials, row sum.
      // The running max m only has to bound the scores well enough that
      // exp2((s - m) c2) stays finite; the result O = O_acc / l is the same
      // for any m.  So m, l and O_acc are rescaled only when some row's max
      // grew by more than 2^8 in exp2 units (probabilities then stay <= 256,
      // fine for fp32 sums and bf16 operands); after the first tiles this
      // almost never happens and the 64 O_acc multiplies are skipped.
      // Once every row of the wave has an m, the exponentials are first
      // taken against it without forming the tile max; if every lane's
      // partial row sum is still at most 2^8, no probability exceeds 2^8 and
      // the tile is done.  Only otherwise is the tile max formed and the
      // exponentials redone.
      float rs = 0.f;
      bf16x8 pf[4];
      auto exponentials = [&](float nb) {
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
      // ---- O^T += V^T P^T
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int db = 0; db < T::ND; ++db) {
          const bf16x8 vf = cat_bf16(lds_read_tr16(Vs + toff[0][db] + 16 * c * T::VSTR),
                                     lds_read_tr16(Vs + toff[1][db] + 16 * c * T::VSTR));
          oacc[db] = mfma32(vf, pf[c], oacc[db]);
        }
      }
    }
    if (more) {
      if constexpr (DMA) wait_vmem();
      else lstore(nxt);
    }
    __syncthreads();
  };
  for (int t = 0; t < ntiles; ++t) {
    __bf16* cur = smem + (t & 1) * T::STAGE;
    tile(t, cur, smem + ((t & 1) ^ 1) * T::STAGE);
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
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const long nblk = VARLEN ? varlen_grid(p.Hkv * p.B, p.num_m_tiles * p.group, kFwdVarlenRun * p.group)
                           : (long)p.num_m_tiles * p.Hq * p.B;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, VARLEN, KVC>), dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

// KV-cache instances, one per cache layout (no block table, pages of at
// least 64 tokens, smaller pages)
template <int D>
hipError_t launch_kvcache(const FwdParams& p, bool causal, hipStream_t stream) {
  if (!p.kv.block_table) return causal ? launch<D, true, false, 1>(p, stream) : launch<D, false, false, 1>(p, stream);
  if (p.kv.page_shift >= 6) return causal ? launch<D, true, false, 2>(p, stream) : launch<D, false, false, 2>(p, stream);
  return causal ? launch<D, true, false, 3>(p, stream) : launch<D, false, false, 3>(p, stream);
}

}  // namespace

// d = 64, and d = 128 with at most 128 query rows per sequence (otherwise
// d = 128 and long dense d = 64 sweeps run the ping-pong kernel)
hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, bool varlen, hipStream_t stream) {
  if (d == 128) {
    if (causal) return varlen ? launch<128, true, true>(p, stream) : launch<128, true, false>(p, stream);
    return varlen ? launch<128, false, true>(p, stream) : launch<128, false, false>(p, stream);
  }
  if (d != 64) return hipErrorInvalidValue;
  if (causal) return varlen ? launch<64, true, true>(p, stream) : launch<64, true, false>(p, stream);
  return varlen ? launch<64, false, true>(p, stream) : launch<64, false, false>(p, stream);
}

// KV-cache attention with the one-group kernel (d = 64, and d = 128 with at
// most 128 query rows; other d = 128 inputs use the ping-pong kernel).
hipError_t launch_fwd_bf16_kvcache(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 64) return launch_kvcache<64>(p, causal, stream);
  if (d == 128) return launch_kvcache<128>(p, causal, stream);
  return hipErrorInvalidValue;
}
