// FP8 (OCP E4M3) forward of IO-aware exact attention for gfx950, and the
// block quantiser that prepares its inputs.
//
// Method ("FlashAttention-3: Fast and Accurate Attention with Asynchrony and
// Low-precision", summary, third contribution and results): the forward's two
// products run on FP8 matrix units for roughly twice the 16-bit throughput,
// and block-wise scaling of the FP8 inputs is what keeps the error well below
// per-tensor quantisation.  The tiling and the online softmax are those of the
// bf16 forward ("Flash Attention and Efficient Transformer Mechanisms", block
// computation; Dao-AILab repository overview, online softmax with rescaling).
//
// Scales.  Q, K and V each carry one fp32 scale per (batch, head, 128-token
// block): the real value of a code is e4m3(code) * scale.  With tiles of 128
// query rows and 64 keys, a workgroup has one Q scale sq and each key tile J
// one K scale sk_J and one V scale sv_J, so
//   * the scores are s = (scale * sq * sk_J) * (q8 . k8): the whole factor,
//     times log2(e), is the per-tile constant of the exp2 FMA;
//   * p = exp2(s - m) is stored in e4m3 with a power-of-two prescale that
//     rides in the exp2 FMA constant, so that small probabilities keep 3
//     mantissa bits; m is a lazily moved reference (see LAZY), so p may
//     exceed 1 by up to 2^LAZY;
//   * per-block scales: V's scale rides in the P V product.  With sv_ref the
//     head's largest V scale, sv_J / sv_ref = 2^k r (k <= 0 an integer, r in
//     [1, 2)); p is stored as 2^7 r p (log2 r joins the exp2 constant) and
//     2^(k - 7) is the instruction's E8M0 scale of the P operand, exact; the
//     accumulator holds O_acc = sum p v8 sv_J / sv_ref, the row sum
//     l = sum 2^7 p (each tile's sum of stored values times 1/r), and the
//     epilogue writes O = sv_ref 2^7 O_acc / l.  No rescale happens when the
//     V block changes;
//   * MX scales: p is stored as 2^8 p and the V block scales are the E8M0
//     scales of the V operand.
//
// gfx950 mapping.  As in the bf16 forward (S^T = K Q^T with query rows in the
// MFMA columns, 4 waves x 32 rows, 2-stage LDS ring of 64-key tiles), with the
// 32x32x64 f8f6f4 MFMA (format E4M3, unit block scales).  Each lane's 32
// operand bytes are one k-slice of 32; A and B use the same byte order.
//   * S^T: lane (row m, half hh) of K and of Q^T holds d = 64 c + 32 hh + j.
//   * O^T += V^T P^T over 64 keys: byte 8 r + e of a lane in half hh is key
//     16 r + 8 hh + e.  With the permuted K row order these are exactly the
//     accumulator registers 8 (r % 2) + e of score block r / 2, and V^T is
//     read from the row-major V tile with the 8-bit LDS transposing read
//     (ds_read_b64_tr_b8: within 16 lanes, lane i gets byte i % 8 of the
//     rows addressed by lanes i / 8 + 2 e, e = 0..7).
//
// MX variant (MX = true): the scales are gfx950's native block scales, one
// E8M0 power of two per 32 elements along each product's reduction
// dimension (Q and K: along d; V: along the keys), passed per lane to the
// scaled MFMA.  The scores and P V come out in true units, so no scale
// enters the softmax or the rescale.  The instruction's two 32-element
// scale blocks (checked with an in-bounds probe) are bytes 0-15 of both lane
// halves (scale from the half-0 lane of the row) and bytes 16-31 of both
// halves (scale from the half-1 lane).  Hence:
//   * P V: with the key order above, bytes 0-15 of the two halves are keys
//     0-31 of the tile and bytes 16-31 keys 32-63, so the V scale of lane
//     half hh is that of key block 2 t + hh, with no change of layout;
//   * S^T: Q and K fragments are loaded so that bytes 0-15 of half hh hold
//     d = 64 c + 16 hh + i and bytes 16-31 hold d = 64 c + 32 + 16 hh + i,
//     which makes the blocks d = 64 c .. 64 c + 31 (scale of d block 2 c,
//     from half 0) and 64 c + 32 .. 64 c + 63 (d block 2 c + 1, half 1).
#include "device_common.h"
#include "fa_internal.h"

namespace {

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NTHREADS = 256;
constexpr int QBLK = 128;          // tokens per quantisation block
// Probabilities are stored in e4m3 as 2^P_LOG2 p (MX) or 2^P_LOG2_BLK r p
// with r in [1, 2) (per-block scales, see the kernel); values down to
// 2^-(6 + P_LOG2) keep 3 mantissa bits.
constexpr float P_LOG2 = 8.f;
constexpr float P_LOG2_BLK = 7.f;
// The running maximum m is a reference, moved (and the accumulators rescaled)
// only when a tile's maximum exceeds it by more than LAZY (exp2 units): the
// largest stored value is then below 2^8 * 2^LAZY = 445.7 <= 448, in both
// paths.
constexpr float LAZY = 0.8f;

typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// With per-lane E8M0 scales (low byte of sa for A's block, of sb for B's).
__device__ __forceinline__ f32x16 mfma_mx(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2*)(p));
}

// Four fp32 values -> four e4m3 codes in one word, a in the low byte
// (hardware rounding to nearest even; inputs here lie in [0, 256]).
__device__ __forceinline__ int pack4_fp8(float a, float b, float c, float d) {
  // the second conversion overwrites the upper half the first one keeps, so
  // the kept value can be any dead register (a's bits: no zeroing move)
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <int D>
struct Fp8Tile {
  // LDS row strides in bytes.  K rows are read 16 bytes per lane, 16 lanes
  // at once, rows {0-3, 8-11} and {4-7, 12-15} of a block: a stride of 36
  // (d = 128) or 20 (d = 64) banks puts them on distinct banks of the 64.
  // V is read transposed, 8 rows x 32 bytes per 32 lanes: a stride of 40 or
  // 24 banks (8 times an odd number, mod 64) puts the 8 rows on disjoint
  // banks, where D + 16 made two of them share 4 banks on every read.
  static constexpr int STR = D + 16;
  static constexpr int STR_V = D + 32;
  static constexpr int NC = D / 64;       // 64-wide d chunks of S^T
  static constexpr int ND = D / 32;       // 32-row d blocks of O^T
  static constexpr int CH = D / 16;       // 16-byte chunks per row
  static constexpr int RPP = NTHREADS / CH;
  static constexpr int NP = BN / RPP;
  static constexpr int STAGE = BN * (STR + STR_V);
};

template <int D, bool CAUSAL, bool MX>
__global__ __launch_bounds__(NTHREADS, MX ? 2 : 3) void fwd_fp8_kernel(FwdParams p) {
  using T = Fp8Tile<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];

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

  const uint8_t* qb = (const uint8_t*)p.q + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
  const uint8_t* kb = (const uint8_t*)p.k + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const uint8_t* vb = (const uint8_t*)p.v + (int64_t)b * p.v_sb + (int64_t)g * p.v_sh;
  __bf16* ob = (__bf16*)p.o + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
  float* lseb = p.lse + (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh;
  const int nqb = (Lq + QBLK - 1) / QBLK, nkb = (Lk + QBLK - 1) / QBLK;
  const float sq = MX ? 1.f : p.q_descale[((int64_t)b * p.Hq + h) * nqb + q0 / QBLK];
  const float* ksc = MX ? nullptr : p.k_descale + ((int64_t)b * p.Hkv + g) * nkb;
  const float* vsc = MX ? nullptr : p.v_descale + ((int64_t)b * p.Hkv + g) * nkb;
  constexpr int NB32 = D / 32;   // MX blocks per row along d

  int kend = Lk;
  if (CAUSAL) kend = min(Lk, q0 + BM + diag);
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- Q^T fragments (B operand): 32 bytes of row qrow per 64-wide d chunk
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)((int64_t)Lq * p.q_ss));
  const int qrow = q0 + wave * 32 + l32;
  i32x8 qf[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) {
    const uint32_t off = (uint32_t)(qrow * p.q_ss + 64 * c);
    const u32x4 lo = buf_load16(rq, off + (MX ? 16 * hh : 32 * hh)),
                hi = buf_load16(rq, off + (MX ? 32 + 16 * hh : 32 * hh + 16));
    qf[c] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }

  // MX: E8M0 scales of this lane's Q^T blocks (row qrow, d block 2c + hh)
  int qsc[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) qsc[c] = 127;
  if (MX && qrow < Lq) {
    const uint8_t* qs = p.q_e8m0 + (((int64_t)b * Lq + qrow) * p.Hq + h) * NB32;
#pragma unroll
    for (int c = 0; c < T::NC; ++c) qsc[c] = qs[2 * c + hh];
  }

  const int kperm = 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
  // transposing-read source coordinates of this lane (see file comment)
  const int G = lane >> 4, u = lane & 15;
  const int tr_row = 8 * (G >> 1) + (u >> 1);
  const int tr_col = 16 * (G & 1) + 8 * (u & 1);
  // byte offsets within a 64-wide d chunk of this lane's two 16-byte halves
  const int dlo = MX ? 16 * hh : 32 * hh, dhi = MX ? 32 + 16 * hh : 32 * hh + 16;

  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)((int64_t)Lk * p.k_ss));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)((int64_t)Lk * p.v_ss));
  const int lrow = tid / T::CH;
  const int lcol = (tid % T::CH) * 16;
  u32x4 kreg[T::NP], vreg[T::NP];
  // MX: scales of the next tile, loaded with it.  K: the d-block scales of
  // this lane's A row in score blocks 0 and 1 (one word for d = 128, a
  // half-word for d = 64); V: the key-block-hh scale of d row 32 db + l32.
  // Indices past the sequence end are clamped (their codes read as zero).
  uint32_t ksn[2] = {0u, 0u}, vsn[T::ND];
  // per-block path: the K and V scales of the next tile, loaded with it so
  // that their latency is hidden like the tile's (non-causal instances; the
  // causal ones measured slower this way and load them in the tile)
  float skn = 1.f, svn = 1.f;
  const int nkb32 = (Lk + 31) / 32;
  auto gload = [&](int j0) {
#pragma unroll
    for (int w = 0; w < T::NP; ++w) {
      const uint32_t r = (uint32_t)(j0 + lrow + w * T::RPP);
      kreg[w] = buf_load16(rk, r * (uint32_t)p.k_ss + lcol);
      vreg[w] = buf_load16(rv, r * (uint32_t)p.v_ss + lcol);
    }
    if constexpr (!MX && !CAUSAL) {
      skn = ksc[j0 / QBLK];
      svn = vsc[j0 / QBLK];
    }
    if constexpr (MX) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int tok = min(j0 + 32 * kb2 + kperm, Lk - 1);
        const uint8_t* ks = p.k_e8m0 + (((int64_t)b * Lk + tok) * p.Hkv + g) * NB32;
        ksn[kb2] = NB32 == 4 ? *(const uint32_t*)ks : (uint32_t)*(const uint16_t*)ks;
      }
      const int kblk = min((j0 >> 5) + hh, nkb32 - 1);
      const uint8_t* vs = p.v_e8m0 + (((int64_t)b * p.Hkv + g) * nkb32 + kblk) * D + l32;
#pragma unroll
      for (int db = 0; db < T::ND; ++db) vsn[db] = vs[32 * db];
    }
  };
  auto lstore = [&](int st) {
    uint8_t* Ks = smem + st * T::STAGE;
    uint8_t* Vs = Ks + BN * T::STR;
#pragma unroll
    for (int w = 0; w < T::NP; ++w) {
      *(u32x4*)(Ks + (lrow + w * T::RPP) * T::STR + lcol) = kreg[w];
      *(u32x4*)(Vs + (lrow + w * T::RPP) * T::STR_V + lcol) = vreg[w];
    }
  };
  uint32_t ksc_t[2] = {0u, 0u}, vsc_t[T::ND];   // MX scales of the tile in LDS
  float sk_t = 1.f, sv_t = 1.f;                  // per-block scales of the tile in LDS
  auto take_scales = [&]() {
    if constexpr (!MX && !CAUSAL) {
      sk_t = skn;
      sv_t = svn;
    }
    if constexpr (MX) {
      ksc_t[0] = ksn[0];
      ksc_t[1] = ksn[1];
#pragma unroll
      for (int db = 0; db < T::ND; ++db) vsc_t[db] = vsn[db];
    }
  };

  f32x16 oacc[T::ND];
#pragma unroll
  for (int i = 0; i < T::ND; ++i) oacc[i] = (f32x16){};
  float m_run = -INFINITY;   // running max in log2 units of the scaled scores
  constexpr float PL = MX ? P_LOG2 : P_LOG2_BLK;
  float l_run = 0.f;         // sum of 2^PL p
  float nbm = PL;            // PL - m_run (PL while m_run is -inf), kept with m_run
  const float cq = p.scale_log2 * sq;
  // per-block path: the head's largest V scale, the reference of O_acc
  float sv_ref = 1.f;
  if (!MX) {
    float m = 0.f;
    for (int i = lane; i < nkb; i += 64) m = fmaxf(m, vsc[i]);
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) m = fmaxf(m, __shfl_xor(m, w, 64));
    sv_ref = m > 0.f ? m : 1.f;
  }
  const float inv_sv_ref = __builtin_amdgcn_rcpf(sv_ref);

  if (ntiles > 0) {
    gload(0);
    lstore(0);
    take_scales();
  }
  wait_vmem();
  __syncthreads();

  const int wave_last_row = q0 + wave * 32 + 31;
  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    const int j0 = t * BN;
    const bool more = t + 1 < ntiles;
    if (more) gload(j0 + BN);
    // Non-causal: always true, but kept opaque to the compiler.  Knowing it,
    // the compiler schedules the loop into 199 registers (two waves per
    // SIMD); as a branch it fits 165 (three waves per SIMD).
    const bool wave_active = CAUSAL ? j0 <= wave_last_row + diag : __builtin_amdgcn_readfirstlane(ntiles) > 0;
    if (wave_active) {
      const uint8_t* Ks = smem + st * T::STAGE;
      const uint8_t* Vs = Ks + BN * T::STR;
      const float c2 = MX ? p.scale_log2 : cq * (CAUSAL ? ksc[j0 / QBLK] : sk_t);
      // per-block path: sv_J / sv_ref = 2^kv r, r in [1, 2)
      int pbyte = 127;            // E8M0 scale of the P operand
      float log2r = 0.f, inv_r = 1.f;
      if (!MX) {
        // wave-uniform: the bit manipulation below then runs on the scalar unit
        const uint32_t rb = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)__builtin_bit_cast(uint32_t, (CAUSAL ? vsc[j0 / QBLK] : sv_t) * inv_sv_ref));
        const int kv = max(-119, min(0, (int)(rb >> 23) - 127));
        const float r = __builtin_bit_cast(float, (rb & 0x7FFFFFu) | 0x3F800000u);
        pbyte = 127 + kv - (int)P_LOG2_BLK;
        log2r = __builtin_amdgcn_logf(r);
        inv_r = __builtin_amdgcn_rcpf(r);
      }
      const uint8_t* kbase = Ks + kperm * T::STR;
      f32x16 sacc[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int c = 0; c < T::NC; ++c)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const uint8_t* kp = kbase + 32 * kb2 * T::STR + 64 * c;
          const u32x4 lo = *(const u32x4*)(kp + dlo), hi = *(const u32x4*)(kp + dhi);
          const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          if constexpr (MX)
            sacc[kb2] = mfma_mx(kf, qf[c], sacc[kb2], (int)(ksc_t[kb2] >> (8 * (2 * c + hh))), qsc[c]);
          else
            sacc[kb2] = mfma_fp8(kf, qf[c], sacc[kb2]);
        }
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
      float mx = sacc[0][0];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb2][i]);
      mx = fmaxf(mx, wave_xor32(mx)) * c2;
      // move the reference only when the tile's maximum exceeds it by more
      // than LAZY (first tile: always).  A new reference sits log2 r above
      // the maximum, so that the largest stored value, 2^PL r exp2(mx - m),
      // is exactly 2^PL: a row dominated by one key then carries no e4m3
      // rounding on that key's probability.
      const bool grow = mx > m_run + LAZY;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // rare after the first tiles
        const float m_new = mx + log2r;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
        if (grow) m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < T::ND; ++i) oacc[i] *= alpha;
        nbm = (m_run == -INFINITY ? 0.f : -m_run) + PL;
      }
      // stored value 2^PL r exp2(s c2 - m): the prescale and log2 r ride in
      // the FMA constant
      const float nb = nbm + log2r;
      float rs = 0.f;
      i32x8 pf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = fast_exp2(__builtin_fmaf(sacc[r >> 1][8 * (r & 1) + e], c2, nb));
          rs += pv[e];
        }
        pf[2 * r] = pack4_fp8(pv[0], pv[1], pv[2], pv[3]);
        pf[2 * r + 1] = pack4_fp8(pv[4], pv[5], pv[6], pv[7]);
      }
      l_run += MX ? rs : rs * inv_r;
      // O_hat^T += V8^T P8^T (64 keys per MFMA)
      const uint8_t* vbase = Vs + tr_row * T::STR_V + tr_col;
#pragma unroll
      for (int db = 0; db < T::ND; ++db) {
        i32x8 vf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2 x = lds_read_tr8(vbase + 16 * r * T::STR_V + 32 * db);
          vf[2 * r] = x[0];
          vf[2 * r + 1] = x[1];
        }
        if constexpr (MX)
          oacc[db] = mfma_mx(vf, pf, oacc[db], (int)vsc_t[db], 127);
        else
          oacc[db] = mfma_mx(vf, pf, oacc[db], 127, pbyte);
      }
    }
    if (more) {
      lstore(st ^ 1);
      take_scales();
    }
    __syncthreads();
  }

  // ---- epilogue: O = sv_ref 2^PL O_acc / l (MX: O_acc / l, l in units of
  // 2^PL), LSE = ln 2 (m - PL) + ln l
  const float l_tot = l_run + wave_xor32(l_run);
  if (qrow < Lq) {
    const float inv = l_tot > 0.f ? (MX ? 1.f : sv_ref * exp2f(PL)) / l_tot : 0.f;
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
    if (hh == 0) lseb[qrow] = l_tot > 0.f ? (m_run - PL) * 0.6931471805599453f + logf(l_tot) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Quantiser: x fp32 [B,S,H,d] (strided) -> e4m3 codes [B,S,H,d] contiguous and
// fp32 scales [B,H,ceil(S/128)].

// fp32 -> OCP E4M3 code: nearest value, ties to the even code, saturating to
// +-448; NaN -> 0x7F.  Written from the format definition (1 sign bit,
// 4 exponent bits with bias 7, 3 mantissa bits, subnormal step 2^-9).
__device__ __forceinline__ uint32_t encode_e4m3(float y) {
  const uint32_t uy = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (uy >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a != a) return 0x7Fu;
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);   // 0..8, exact product
  const uint32_t ua = __builtin_bit_cast(uint32_t, a);
  const uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);             // round 23 -> 3 mantissa bits
  return sign | ((r >> 20) - (120u << 3));
}

struct QuantParams {
  const float* x;
  int64_t sb, ss, sh;
  uint8_t* codes;
  float* scales;
  int B, S, H, d, nb;
};

// one workgroup per (b, h, block): amax over 128 tokens x d
__global__ __launch_bounds__(256) void quant_amax_kernel(QuantParams p, int per_tensor) {
  const int blk = blockIdx.x % p.nb;
  const int bh = blockIdx.x / p.nb;
  const int h = bh % p.H, b = bh / p.H;
  const int s0 = blk * QBLK, s1 = min(p.S, s0 + QBLK);
  float m = 0.f;
  const int n = (s1 - s0) * p.d;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int s = s0 + i / p.d, c = i % p.d;
    m = fmaxf(m, fabsf(p.x[(int64_t)b * p.sb + (int64_t)s * p.ss + (int64_t)h * p.sh + c]));
  }
  __shared__ float red[256];
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float amax = red[0];
    p.scales[blockIdx.x] = per_tensor ? amax : (amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f);
  }
}

// per-tensor: one workgroup turns the block maxima into the tensor scale
__global__ __launch_bounds__(256) void quant_tensor_scale_kernel(QuantParams p) {
  const int n = p.B * p.H * p.nb;
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, p.scales[i]);
  __shared__ float red[256];
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  const float amax = red[0];
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  for (int i = threadIdx.x; i < n; i += 256) p.scales[i] = s;
}

// one thread per 16 consecutive elements of a (b, s, h) row
__global__ __launch_bounds__(256) void quant_encode_kernel(QuantParams p) {
  const int per_row = p.d / 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.S * p.H * per_row;
  if (idx >= total) return;
  const int c16 = (int)(idx % per_row);
  int64_t r = idx / per_row;
  const int h = (int)(r % p.H);
  r /= p.H;
  const int s = (int)(r % p.S);
  const int b = (int)(r / p.S);
  const float sc = p.scales[((int64_t)b * p.H + h) * p.nb + s / QBLK];
  const float* xr = p.x + (int64_t)b * p.sb + (int64_t)s * p.ss + (int64_t)h * p.sh + 16 * c16;
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) word |= encode_e4m3(__fdiv_rn(xr[4 * w + e], sc)) << (8 * e);
    out[w] = word;
  }
  *(u32x4*)(p.codes + (((int64_t)b * p.S + s) * p.H + h) * p.d + 16 * c16) = out;
}

// ---------------------------------------------------------------------------
// MX quantiser: E4M3 codes with one E8M0 scale per 32 consecutive elements.
// The shared exponent is the smallest e with amax <= 448 * 2^e, i.e.
// floor(log2(amax)) - 8 plus one when amax's significand exceeds 1.75, so no
// element saturates; clamped to [-127, 127], 0 for a zero block.  The codes
// encode x * 2^-e, exact in fp32 outside subnormal results.

// Shared exponent from the bit pattern of amax = max |x| (an integer max of
// the magnitude bits orders finite values the same way, subnormals included).
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits) {
  if (amax_bits == 0u) return 0;
  const int E = (int)(amax_bits >> 23);
  const int fl = E > 0 ? E - 127                                          // normal
                       : (31 - __builtin_clz(amax_bits & 0x7FFFFFu)) - 149;   // subnormal
  // significand above 1.75 = 448 / 2^8: one more (subnormals are clamped anyway)
  const int up = (E > 0 && (amax_bits & 0x7FFFFFu) > 0x600000u) ? 1 : 0;
  return min(127, max(-127, fl - 8 + up));
}

struct MxQuantParams {
  const float* x;
  int64_t sb, ss, sh;
  uint8_t* codes;
  uint8_t* scales;
  int B, S, H, d, nb;   // nb: token blocks (axis 1)
};

// Blocks along d: one thread per (b, s, h, 32-element block).
__global__ __launch_bounds__(256) void quant_mx_d_kernel(MxQuantParams p) {
  const int nbd = p.d / 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.S * p.H * nbd;
  if (idx >= total) return;
  const int blk = (int)(idx % nbd);
  int64_t r = idx / nbd;
  const int h = (int)(r % p.H);
  r /= p.H;
  const int s = (int)(r % p.S);
  const int b = (int)(r / p.S);
  const float* xr = p.x + (int64_t)b * p.sb + (int64_t)s * p.ss + (int64_t)h * p.sh + 32 * blk;
  float v[32];
  uint32_t amax = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = xr[i];
    amax = max(amax, __builtin_bit_cast(uint32_t, v[i]) & 0x7FFFFFFFu);
  }
  const int e = mx_exponent(amax);
  uint8_t* out = p.codes + (((int64_t)b * p.S + s) * p.H + h) * p.d + 32 * blk;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    u32x4 q;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) word |= encode_e4m3(ldexpf(v[16 * w + 4 * j + c], -e)) << (8 * c);
      q[j] = word;
    }
    *(u32x4*)(out + 16 * w) = q;
  }
  p.scales[idx] = (uint8_t)(e + 127);   // [B,S,H,d/32]
}

// Blocks along the tokens: one thread per (b, h, token block, d column).
__global__ __launch_bounds__(256) void quant_mx_s_kernel(MxQuantParams p) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.H * p.nb * p.d;
  if (idx >= total) return;
  const int c = (int)(idx % p.d);
  int64_t r = idx / p.d;
  const int blk = (int)(r % p.nb);
  r /= p.nb;
  const int h = (int)(r % p.H);
  const int b = (int)(r / p.H);
  const int s0 = 32 * blk, s1 = min(p.S, s0 + 32);
  const float* xc = p.x + (int64_t)b * p.sb + (int64_t)h * p.sh + c;
  uint32_t amax = 0u;
  for (int s = s0; s < s1; ++s) amax = max(amax, __builtin_bit_cast(uint32_t, xc[(int64_t)s * p.ss]) & 0x7FFFFFFFu);
  const int e = mx_exponent(amax);
  for (int s = s0; s < s1; ++s)
    p.codes[(((int64_t)b * p.S + s) * p.H + h) * p.d + c] = (uint8_t)encode_e4m3(ldexpf(xc[(int64_t)s * p.ss], -e));
  p.scales[idx] = (uint8_t)(e + 127);   // [B,H,nb,d]
}

template <int D, bool CAUSAL, bool MX = false>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const long nblk = (long)p.num_m_tiles * p.Hq * p.B;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, MX>), dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  return causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
}

hipError_t launch_quantize_fp8(const float* x, int64_t sb, int64_t ss, int64_t sh, int B, int S,
                               int H, int d, int per_tensor, void* codes, float* scales,
                               hipStream_t stream) {
  QuantParams p = {x, sb, ss, sh, (uint8_t*)codes, scales, B, S, H, d, (S + QBLK - 1) / QBLK};
  const long nblk = (long)B * H * p.nb;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_amax_kernel, dim3((unsigned)nblk), dim3(256), 0, stream, p, per_tensor);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (per_tensor) {
    hipLaunchKernelGGL(quant_tensor_scale_kernel, dim3(1), dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long n16 = (long)B * S * H * (d / 16);
  const long grid = (n16 + 255) / 256;
  if (grid > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_encode_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_mxfp8(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch<128, true, true>(p, stream) : launch<128, false, true>(p, stream);
  return causal ? launch<64, true, true>(p, stream) : launch<64, false, true>(p, stream);
}

hipError_t launch_quantize_mxfp8(const float* x, int64_t sb, int64_t ss, int64_t sh, int B, int S,
                                 int H, int d, int axis, void* codes, uint8_t* scales,
                                 hipStream_t stream) {
  MxQuantParams p = {x, sb, ss, sh, (uint8_t*)codes, scales, B, S, H, d, (S + 31) / 32};
  const long n = axis == 0 ? (long)B * S * H * (d / 32) : (long)B * H * p.nb * d;
  if (n <= 0) return hipSuccess;
  const long grid = (n + 255) / 256;
  if (grid > 0x7fffffffL) return hipErrorInvalidValue;
  if (axis == 0)
    hipLaunchKernelGGL(quant_mx_d_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(quant_mx_s_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}
