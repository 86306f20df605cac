// FP8 (OCP E4M3) backward of IO-aware exact attention for gfx950.
//
// Method.  The recomputation-based backward ("Dao and colleagues: IO-aware
// exact attention with FlashAttention", summary: tiling plus recomputation;
// Dao-AILab repository overview: deterministic backward passes) with its
// matrix products on FP8 matrix units, extending the FP8 forward of
// "FlashAttention-3: Fast and Accurate Attention with Asynchrony and
// Low-precision" (summary, third contribution) to the gradients.  With
// P = exp(scale Q K^T - LSE) and D_i = sum_c dO_ic O_ic:
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),
//     dK = scale dS^T Q,   dQ = scale dS K.
//
// Operands and scales.  Q, K and V are the forward's E4M3 codes with one fp32
// scale per (batch, head, 128-token block).  The other operands are
// quantised here:
//   * dO: one power-of-two scale per (batch, head, 128-row block), the
//     smallest under which no element saturates, computed by the preprocess
//     kernel, which also forms D from the quantised dO (so that the rows of
//     dS still sum to zero);
//   * P: stored as 2^8 p (as in the FP8 forward), unit scale 2^-8 in the
//     matrix instruction;
//   * dS: one power-of-two scale per 32 elements along each product's
//     reduction dimension (gfx950's native E8M0 block scaling), computed in
//     registers from the block's largest magnitude: the 32 values of a block
//     sit in one lane and the lane 32 apart, so one exchange finds it.
// The fp32 scales fold into per-tile constants: sq * sk into the exp2
// constant of the scores, sv (and the dO scale, applied by the instruction)
// into dP, sq into dS for dK^T += Q^T dS, and sk into dS for
// dQ^T += K^T dS^T; dV and dK come out in true units.
//
// gfx950 mapping.  v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3, per-lane E8M0
// block scales) for all five products; each lane's 32 operand bytes of a
// 64-element k-slice hold, for a d-reduction, d = 64 c + 32 hh + j, and for a
// token reduction, token 16 r + 8 hh + e at byte 8 r + e (the order in which
// the score accumulators of a 64-token tile lie when the A-operand rows are
// fed permuted); the column-wise operands (dO^T, Q^T, K^T) come from the
// 8-bit LDS transposing read.  The instruction's two 32-element scale blocks
// are bytes 0-15 of both lane halves (scale from the half-0 lane) and bytes
// 16-31 (scale from the half-1 lane), i.e. tokens 0-31 and 32-63 of a tile.
//   * bwd_fp8_preprocess: one workgroup per (batch, head, 128 query rows).
//   * bwd_dkdv_fp8: the bf16 kernel's structure: 128 keys of one (batch, kv
//     head), each 32-key group split between a P-wave (K resident,
//     S = Q K^T, P, dV^T += dO^T P) and a dS-wave (V resident, dP = dO V^T,
//     dS, dK^T += Q^T dS) that runs one query tile behind and receives P in
//     fp32 through LDS (the dS-wave has the longer VALU part, so P reaches
//     it ready to use); Q and dO tiles of 64 rows through a 3-stage ring.
//   * bwd_dq_fp8: 128 query rows of one (batch, head); Q^T and dO^T
//     resident, K and V tiles of 64 keys through a 2-stage ring; dQ is a
//     fixed-order sum over the key tiles (no atomics), at the price of
//     recomputing S and dP.
#include "device_common.h"
#include "fa_internal.h"

namespace {

constexpr int QBLK = 128;                 // tokens per fp32 scale block of q, k, v (and of dO)
constexpr float LOG2E = 1.4426950408889634f;
constexpr int UNIT = 127;                 // E8M0 byte of 2^0
constexpr int P_BYTE = 127 - 8;           // E8M0 byte of 2^-8: P is stored as 2^8 p

typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_mx(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2*)(p));
}

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Four fp32 values (each within +-448) -> four e4m3 codes in one word, a in
// the low byte; the hardware rounds to nearest even.
__device__ __forceinline__ int pack4_fp8(float a, float b, float c, float d) {
  // the second conversion overwrites the upper half the first one keeps, so
  // the kept value can be any dead register (a's bits: no zeroing move)
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// The smallest e with amax <= 448 * 2^e: a power-of-two scale under which no
// element of the block saturates E4M3 (the block maximum lands in
// (224, 448] * 2^e).  Clamped to [-126, 126], so that 2^-e is a normal float
// and e + 127 a valid E8M0 byte; 0 for an all-zero block.
__device__ __forceinline__ int fit_exponent(float amax) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, amax);
  if (bits == 0u) return 0;
  const int up = (bits & 0x7FFFFFu) > 0x600000u ? 1 : 0;   // significand above 1.75
  return min(126, max(-126, (int)(bits >> 23) - 127 - 8 + up));
}

// 2^e as a float, for e in [-126, 127].
__device__ __forceinline__ float exp2i(int e) {
  return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

// A-operand row order that makes accumulator registers 0..7 / 8..15 of a
// lane cover 8 consecutive rows (as in the bf16 kernels).
__device__ __forceinline__ int row_perm(int l32) {
  return 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
}

// Scores (or dS) of a 64-token tile, two 32-token blocks of 16 accumulator
// registers each, scaled by per-block factors and packed as a B operand:
// byte 8 r + e of half hh is token 16 r + 8 hh + e, i.e. register
// 8 (r % 2) + e of block r / 2.
__device__ __forceinline__ i32x8 pack_tile(const float (&v)[2][16], float f0, float f1) {
  i32x8 out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float f = r < 2 ? f0 : f1;
    const float* x = &v[r >> 1][8 * (r & 1)];
    out[2 * r] = pack4_fp8(x[0] * f, x[1] * f, x[2] * f, x[3] * f);
    out[2 * r + 1] = pack4_fp8(x[4] * f, x[5] * f, x[6] * f, x[7] * f);
  }
  return out;
}

typedef short s16x2 __attribute__((ext_vector_type(2)));
// Four fp32 values divided by s, a power of two, -> four e4m3 codes, with
// the division done by the scaled conversion itself (v_cvt_scalef32_pk_fp8:
// it divides by 2^exponent(s); checked with an in-bounds probe against the
// plain conversion of x / s).  As pack4_fp8, the first conversion's kept
// upper half is a dead register.
__device__ __forceinline__ int pack4_fp8_scaled(float a, float b, float c, float d, float s) {
  const s16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(s16x2, a), a, b, s, false);
  return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c, d, s, true));
}
// pack_tile with the values of block 0 divided by f0, block 1 by f1
__device__ __forceinline__ i32x8 pack_tile_scaled(const float (&v)[2][16], float f0, float f1) {
  i32x8 out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float f = r < 2 ? f0 : f1;
    const float* x = &v[r >> 1][8 * (r & 1)];
    out[2 * r] = pack4_fp8_scaled(x[0], x[1], x[2], x[3], f);
    out[2 * r + 1] = pack4_fp8_scaled(x[4], x[5], x[6], x[7], f);
  }
  return out;
}

// E4M3 codes of dS for one lane (two 32-token blocks, 16 values each), with
// one power-of-two scale per block: returns the packed operand and, in
// `sbyte`, the E8M0 byte this lane passes to the instruction (block 0 from
// the half-0 lanes, block 1 from the half-1 lanes).
__device__ __forceinline__ i32x8 quantise_ds(const float (&v)[2][16], int hh, int& sbyte) {
  float m0 = 0.f, m1 = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    m0 = fmaxf(m0, fabsf(v[0][i]));
    m1 = fmaxf(m1, fabsf(v[1][i]));
  }
  m0 = fmaxf(m0, wave_xor32(m0));
  m1 = fmaxf(m1, wave_xor32(m1));
  const int e0 = fit_exponent(m0), e1 = fit_exponent(m1);
  sbyte = (hh ? e1 : e0) + 127;
  return pack_tile_scaled(v, exp2i(e0), exp2i(e1));
}

// ---------------------------------------------------------------------------
// Per (batch, head, 128-row block): the power-of-two dO scale, the E4M3 codes
// of dO ([B,Hq,Sq,d] in the workspace) and D_i = sum_c dq(dO)_ic O_ic in
// fp32 from the values the products will see.
template <int D>
__global__ __launch_bounds__(256) void bwd_fp8_preprocess_kernel(BwdParams p) {
  constexpr int HALF = D / 2;                  // elements per thread (two threads per row)
  const int nqb = (p.Sq + QBLK - 1) / QBLK;
  const int blk = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb;             // b * Hq + h
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int row = blk * QBLK + (tid >> 1);
  const bool valid = row < p.Sq;
  float g[HALF];
  float amax = 0.f;
  if (valid) {
    const __bf16* gp = (const __bf16*)p.dout + (int64_t)b * p.do_sb + (int64_t)row * p.do_ss +
                       (int64_t)h * p.do_sh + half * HALF;
#pragma unroll
    for (int c = 0; c < HALF / 8; ++c) {
      const bf16x8 x = *(const bf16x8*)(gp + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        g[8 * c + e] = (float)x[e];
        amax = fmaxf(amax, fabsf(g[8 * c + e]));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < HALF; ++i) g[i] = 0.f;
  }
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) amax = fmaxf(amax, __shfl_xor(amax, w, 64));
  __shared__ float red[4];
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = fit_exponent(amax);
  const float inv = exp2i(-e), sc = exp2i(e);
  float dsum = 0.f;
  if (valid) {
    const __bf16* op = (const __bf16*)p.o + (int64_t)b * p.o_sb + (int64_t)row * p.o_ss +
                       (int64_t)h * p.o_sh + half * HALF;
    uint8_t* dst = p.do8 + ((int64_t)bh * p.Sq + row) * D + half * HALF;
#pragma unroll
    for (int c = 0; c < HALF / 16; ++c) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* x = g + 16 * c + 4 * j;
        w[j] = (uint32_t)pack4_fp8(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
      }
      *(u32x4*)(dst + 16 * c) = w;
      const bf16x8 o0 = *(const bf16x8*)(op + 16 * c), o1 = *(const bf16x8*)(op + 16 * c + 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float d0 = __builtin_amdgcn_cvt_f32_fp8((int)w[j], 0) * sc;
        const float d1 = __builtin_amdgcn_cvt_f32_fp8((int)w[j], 1) * sc;
        const float d2 = __builtin_amdgcn_cvt_f32_fp8((int)w[j], 2) * sc;
        const float d3 = __builtin_amdgcn_cvt_f32_fp8((int)w[j], 3) * sc;
        const int i = 4 * j;
        dsum = __builtin_fmaf(d0, (float)(i < 8 ? o0[i] : o1[i - 8]), dsum);
        dsum = __builtin_fmaf(d1, (float)(i + 1 < 8 ? o0[i + 1] : o1[i - 7]), dsum);
        dsum = __builtin_fmaf(d2, (float)(i + 2 < 8 ? o0[i + 2] : o1[i - 6]), dsum);
        dsum = __builtin_fmaf(d3, (float)(i + 3 < 8 ? o0[i + 3] : o1[i - 5]), dsum);
      }
    }
  }
  dsum += __shfl_xor(dsum, 1, 64);
  if (valid && half == 0) p.delta[(int64_t)bh * p.Sq + row] = dsum;
  if (tid == 0) p.do_e8m0[(int64_t)bh * nqb + blk] = e + 127;
}

// ---------------------------------------------------------------------------
// dK, dV for 128 keys of one (batch, kv head); see the file comment.
template <int D>
struct DkdvFp8Tile {
  static constexpr int NT = 512;               // 8 waves: 4 key groups x 2 roles
  static constexpr int BKV = 128;              // keys per workgroup: one scale block
  static constexpr int BQ = 64;                // query rows per streamed tile
  static constexpr int NC = D / 64;            // 64-wide d chunks
  static constexpr int ND = D / 32;            // 32-row d blocks of dK^T, dV^T
  static constexpr int STR = D + 16;           // LDS row stride in bytes
  static constexpr int TILE = BQ * STR;        // bytes of one Q or dO tile
  static constexpr int STATS = 2 * BQ * 4 + 16;   // LSE (log2), D * sq, sq, dO scale byte
  static constexpr int STAGE_BYTES = 2 * TILE + STATS;
  static constexpr int NSTAGE = 3;             // P-wave's tile, dS-wave's tile, next tile
  static constexpr int PEX_SLOT = 4 * 2 * 64 * 16 * 4;   // fp32 P of 4 key groups x 2 blocks
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES + 2 * PEX_SLOT;
  static constexpr int CH = D / 16;            // 16-byte chunks per row
  static constexpr int LD_THREADS = BQ * CH;   // threads loading one chunk of Q and of dO
  static_assert(STAGE_BYTES % 16 == 0 && LD_THREADS <= NT, "tile layout");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_fp8_kernel(BwdParams p) {
  using T = DkdvFp8Tile<D>;
  __shared__ __attribute__((aligned(16))) char smem[T::LDS_BYTES];

  // consecutive key tiles of one kv head share an XCD
  const int nkt = (p.Sk + T::BKV - 1) / T::BKV;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = L % nkt;
  const int rest = L / nkt;
  const int g = rest % p.Hkv;
  const int b = rest / p.Hkv;
  const int Lq = p.Sq, Lk = p.Sk;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int kgrp = wave & 3;
  const bool pwave = wave < 4;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int diag = Lk - Lq;
  const int k0 = kt * T::BKV;
  const int kw0 = k0 + 32 * kgrp;
  const int key = kw0 + l32;

  // ---- resident K (P-wave) or V (dS-wave) row of this lane: B operand of
  // Q K^T / dO V^T, 32 bytes (d = 64 c + 32 hh + j) per 64-wide chunk
  const uint8_t* kvb = pwave ? (const uint8_t*)p.k + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh
                             : (const uint8_t*)p.v + (int64_t)b * p.v_sb + (int64_t)g * p.v_sh;
  const int64_t kv_ss = pwave ? p.k_ss : p.v_ss;
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc(uniform_ptr(kvb), (uint32_t)((int64_t)Lk * kv_ss));
  i32x8 bf[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) {
    const uint32_t off = (uint32_t)(key * kv_ss + 64 * c + 32 * hh);
    bf[c] = cat8(buf_load16(rkv, off), buf_load16(rkv, off + 16));
  }
  const int nkb = (Lk + QBLK - 1) / QBLK, nqb = (Lq + QBLK - 1) / QBLK;
  // fp32 scale of this workgroup's 128 keys: sk (P-wave) or sv (dS-wave)
  const float skv = (pwave ? p.k_descale : p.v_descale)[((int64_t)b * p.Hkv + g) * nkb + kt];

  // ---- query tiles: every head of the group, from the first tile that can
  // see this workgroup's keys
  const int nqt = (Lq + T::BQ - 1) / T::BQ;
  int qt0 = 0;
  if (CAUSAL) qt0 = max(0, k0 - diag) / T::BQ;
  const int per_head = max(0, nqt - qt0);
  const int niter = per_head * p.group;

  auto stage = [&](int st) { return (uint8_t*)(smem + st * T::STAGE_BYTES); };
  // register-staged loads: one 16-byte chunk of Q and of dO per loading
  // thread, LSE / D by threads 0..127, the tile's scales by every thread
  const int lrow = tid / T::CH, lcol = 16 * (tid % T::CH);
  int ld_h = 0, ld_qt = 0;
  __amdgpu_buffer_rsrc_t rq, rdo;
  const float* lse_h = nullptr;
  const float* del_h = nullptr;
  const float* sq_h = nullptr;
  const int* sdo_h = nullptr;
  auto set_head = [&](int hi) {
    const int h = p.group * g + hi;
    const int64_t bh = (int64_t)b * p.Hq + h;
    rq = make_rsrc(uniform_ptr((const uint8_t*)p.q + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh),
                   (uint32_t)((int64_t)Lq * p.q_ss));
    rdo = make_rsrc(uniform_ptr(p.do8 + bh * Lq * D), (uint32_t)((int64_t)Lq * D));
    lse_h = p.lse + bh * Lq;
    del_h = p.delta + bh * Lq;
    sq_h = p.q_descale + bh * nqb;
    sdo_h = p.do_e8m0 + bh * nqb;
  };
  if (niter > 0) set_head(0);
  u32x4 qreg = {0u, 0u, 0u, 0u}, doreg = {0u, 0u, 0u, 0u};
  float sval = 0.f, sqv = 1.f;
  int edo = UNIT;
  auto gload = [&]() {
    const int q0 = (qt0 + ld_qt) * T::BQ;
    if (tid < T::LD_THREADS) {
      qreg = buf_load16(rq, (uint32_t)((q0 + lrow) * p.q_ss + lcol));
      doreg = buf_load16(rdo, (uint32_t)((q0 + lrow) * D + lcol));
    }
    if (tid < 2 * T::BQ) {
      const int r = q0 + (tid & (T::BQ - 1));
      if (tid < T::BQ) sval = r < Lq ? lse_h[r] : INFINITY;
      else sval = r < Lq ? del_h[r] : 0.f;
    }
    sqv = sq_h[q0 / QBLK];
    edo = sdo_h[q0 / QBLK];
    if (++ld_qt == per_head) {
      ld_qt = 0;
      if (++ld_h < p.group) set_head(ld_h);
    }
  };
  // LSE is stored as a log2 value minus 8, so that exp2 gives 2^8 p, the
  // value the E4M3 P operand holds (no visible key or padding row: +inf, so
  // the probabilities are zero); D is stored times the tile's Q scale and
  // 2^-8, which the dS side needs with the 2^8 p it receives
  auto lstore = [&](int st) {
    uint8_t* Qs = stage(st);
    uint8_t* Os = Qs + T::TILE;
    float* stats = (float*)(Os + T::TILE);
    if (tid < T::LD_THREADS) {
      *(u32x4*)(Qs + lrow * T::STR + lcol) = qreg;
      *(u32x4*)(Os + lrow * T::STR + lcol) = doreg;
    }
    if (tid < T::BQ) stats[tid] = (sval == -INFINITY) ? INFINITY : __builtin_fmaf(sval, LOG2E, -8.f);
    else if (tid < 2 * T::BQ) stats[tid] = sval * sqv * (1.f / 256.f);
    else if (tid == 2 * T::BQ) stats[2 * T::BQ] = sqv;
    else if (tid == 2 * T::BQ + 1) ((int*)stats)[2 * T::BQ + 1] = edo;
  };
  // fp32 P of key group kgrp, query block qb, in exchange slot sl: four
  // 16-byte words per lane, lane-interleaved
  auto pex = [&](int sl, int qb) {
    return (u32x4*)(smem + T::NSTAGE * T::STAGE_BYTES + sl * T::PEX_SLOT) + ((kgrp * 2 + qb) * 4) * 64 + lane;
  };

  f32x16 acc[T::ND];
#pragma unroll
  for (int i = 0; i < T::ND; ++i) acc[i] = (f32x16){};
  const float c2 = p.scale_log2;
  const int prow = row_perm(l32);
  // 8-bit transposing-read coordinates (rows of the tile are the k index)
  const int G = lane >> 4, u = lane & 15;
  const int tr_row = 8 * (G >> 1) + (u >> 1);
  const int tr_col = 16 * (G & 1) + 8 * (u & 1);

  if (niter > 0) {
    gload();
    lstore(0);
  }
  wait_vmem();
  __syncthreads();

  int st_cur = 0, st_prev = 2, st_next = 1;
  int pw_qt = 0;
  for (int it = 0; it <= niter; ++it) {
    const bool more = it + 1 < niter;
    if (more) gload();
    const bool work = pwave ? it < niter : it > 0;
    if (work) {
      const int t = pwave ? it : it - 1;
      const uint8_t* Qs = stage(pwave ? st_cur : st_prev);
      const uint8_t* Os = Qs + T::TILE;
      const float* stats = (const float*)(Os + T::TILE);
      const float sq_t = stats[2 * T::BQ];
      const int edo_t = ((const int*)stats)[2 * T::BQ + 1];
      const uint8_t* As = pwave ? Qs : Os;   // A rows: Q for S, dO for dP
      const uint8_t* Ts = pwave ? Os : Qs;   // transposed: dO^T for dV, Q^T for dK
      // ---- S = Q K^T or dP = dO V^T for both query blocks
      f32x16 s2[2] = {(f32x16){}, (f32x16){}};
      const int sa = pwave ? UNIT : edo_t;
#pragma unroll
      for (int c = 0; c < T::NC; ++c)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const uint8_t* ap = As + (prow + 32 * qb) * T::STR + 64 * c + 32 * hh;
          s2[qb] = mfma_mx(cat8(*(const u32x4*)ap, *(const u32x4*)(ap + 16)), bf[c], s2[qb], sa, UNIT);
        }
      float v[2][16];
      int sb_byte = P_BYTE;
      if (pwave) {
        const int q0 = (qt0 + pw_qt) * T::BQ;
        const float c2t = c2 * sq_t * skv;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int qr0 = q0 + 32 * qb;
          const f32x4* l4 = (const f32x4*)(stats + 32 * qb + 8 * hh);
          const f32x4 la = l4[0], lb = l4[1], lc = l4[4], ld = l4[5];
          const float lrow_v[16] = {la[0], la[1], la[2], la[3], lb[0], lb[1], lb[2], lb[3],
                                    lc[0], lc[1], lc[2], lc[3], ld[0], ld[1], ld[2], ld[3]};
          const bool need_mask = (kw0 + 31 >= Lk) || (CAUSAL && qr0 + diag < kw0 + 31);
#pragma unroll
          for (int i = 0; i < 16; ++i) v[qb][i] = fast_exp2(__builtin_fmaf(s2[qb][i], c2t, -lrow_v[i]));
          if (need_mask) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int iq = qr0 + ((i < 8) ? 8 * hh + i : 16 + 8 * hh + (i - 8));
              if (key >= Lk || (CAUSAL && key > iq + diag)) v[qb][i] = 0.f;
            }
          }
          // v = 2^8 P, passed in fp32
          u32x4* pe = pex(t & 1, qb);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            pe[64 * j] = __builtin_bit_cast(u32x4, (f32x4){v[qb][4 * j], v[qb][4 * j + 1], v[qb][4 * j + 2], v[qb][4 * j + 3]});
        }
      } else {
        // dS * sq = 2^8 P (dP sv sq 2^-8 - D sq 2^-8), 2^8 P from the P-wave
        const float f = skv * sq_t * (1.f / 256.f);
        const float* dels = stats + T::BQ;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const f32x4* d4 = (const f32x4*)(dels + 32 * qb + 8 * hh);
          const f32x4 da = d4[0], db = d4[1], dc = d4[4], dd = d4[5];
          const float drow_v[16] = {da[0], da[1], da[2], da[3], db[0], db[1], db[2], db[3],
                                    dc[0], dc[1], dc[2], dc[3], dd[0], dd[1], dd[2], dd[3]};
          const u32x4* pe = pex(t & 1, qb);
          f32x4 p4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) p4[j] = __builtin_bit_cast(f32x4, pe[64 * j]);
#pragma unroll
          for (int i = 0; i < 16; ++i) v[qb][i] = p4[i >> 2][i & 3] * __builtin_fmaf(s2[qb][i], f, -drow_v[i]);
        }
      }
      // ---- B operand of the second product: 2^8 P (P-wave) or dS (dS-wave)
      const i32x8 ob = pwave ? pack_tile(v, 1.f, 1.f) : quantise_ds(v, hh, sb_byte);
      const int ta = pwave ? edo_t : UNIT;   // scale of dO^T (P-wave) or Q^T (dS-wave)
      // ---- acc += Ts^T ob (64 query rows per instruction)
      const uint8_t* tbase = Ts + tr_row * T::STR + tr_col;
#pragma unroll
      for (int db = 0; db < T::ND; ++db) {
        i32x8 tf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2 x = lds_read_tr8(tbase + 16 * r * T::STR + 32 * db);
          tf[2 * r] = x[0];
          tf[2 * r + 1] = x[1];
        }
        acc[db] = mfma_mx(tf, ob, acc[db], ta, sb_byte);
      }
    }
    // the next tile goes to stage (it + 1) % 3, last read by the dS-wave in
    // iteration it - 1; P slot it % 2 is read in iteration it + 1
    if (more) lstore(st_next);
    __syncthreads();
    const int st_free = st_prev;
    st_prev = st_cur;
    st_cur = st_next;
    st_next = st_free;
    if (++pw_qt == per_head) pw_qt = 0;
  }

  // ---- epilogue: dV (P-wave) or dK = scale * dK (dS-wave), bf16, one key row per lane
  if (key < Lk) {
    __bf16* out = pwave ? (__bf16*)p.dv + (int64_t)b * p.dv_sb + (int64_t)g * p.dv_sh + (int64_t)key * p.dv_ss
                        : (__bf16*)p.dk + (int64_t)b * p.dk_sb + (int64_t)g * p.dk_sh + (int64_t)key * p.dk_ss;
    const float f = pwave ? 1.f : p.scale;
#pragma unroll
    for (int db = 0; db < T::ND; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(acc[db][4 * gi + r] * f);
        *(bf16x4*)(out + 32 * db + 8 * gi + 4 * hh) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ for 128 query rows of one (batch, query head); see the file comment.
template <int D>
struct DqFp8Tile {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int NC = D / 64;
  static constexpr int ND = D / 32;
  static constexpr int STR = D + 16;
  static constexpr int CH = D / 16;
  static constexpr int RPP = 256 / CH;         // tile rows per load pass
  static constexpr int NP = BN / RPP;          // passes per tile
  static constexpr int STAGE = 2 * BN * STR;   // K and V tiles
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_fp8_kernel(BwdParams p) {
  using T = DqFp8Tile<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];

  const int nmt = (p.Sq + T::BM - 1) / T::BM;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int mt = L % nmt;
  const int rest = L / nmt;
  const int h = rest % p.Hq;
  const int b = rest / p.Hq;
  if (CAUSAL) mt = nmt - 1 - mt;   // heaviest tiles first
  const int g = h / p.group;
  const int Lq = p.Sq, Lk = p.Sk;
  const int diag = Lk - Lq;
  const int q0 = mt * T::BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int qrow = q0 + 32 * wave + l32;
  const int64_t bh = (int64_t)b * p.Hq + h;
  const int nqb = (Lq + QBLK - 1) / QBLK, nkb = (Lk + QBLK - 1) / QBLK;

  // ---- resident Q^T and dO^T rows of this lane (B operands)
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(uniform_ptr((const uint8_t*)p.q + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh),
                (uint32_t)((int64_t)Lq * p.q_ss));
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(uniform_ptr(p.do8 + bh * Lq * D), (uint32_t)((int64_t)Lq * D));
  i32x8 qf[T::NC], of[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) {
    const uint32_t oq = (uint32_t)(qrow * p.q_ss + 64 * c + 32 * hh);
    const uint32_t od = (uint32_t)(qrow * D + 64 * c + 32 * hh);
    qf[c] = cat8(buf_load16(rq, oq), buf_load16(rq, oq + 16));
    of[c] = cat8(buf_load16(rdo, od), buf_load16(rdo, od + 16));
  }
  float lse2 = INFINITY, dlt = 0.f;
  if (qrow < Lq) {
    const float lv = p.lse[bh * Lq + qrow];
    lse2 = (lv == -INFINITY) ? INFINITY : lv * LOG2E;
    dlt = p.delta[bh * Lq + qrow];
  }
  const float sq = p.q_descale[bh * nqb + q0 / QBLK];   // 128 rows: one scale block
  const int edo = p.do_e8m0[bh * nqb + q0 / QBLK];
  const float c2 = p.scale_log2 * sq;
  const float* ksc = p.k_descale + ((int64_t)b * p.Hkv + g) * nkb;
  const float* vsc = p.v_descale + ((int64_t)b * p.Hkv + g) * nkb;

  int kend = Lk;
  if (CAUSAL) kend = min(Lk, q0 + T::BM + diag);
  const int ntiles = kend > 0 ? (kend + T::BN - 1) / T::BN : 0;
  const int wrow0 = q0 + 32 * wave;
  int nt_w = wrow0 < Lq ? ntiles : 0;   // tiles this wave sees: t < nt_w
  if (CAUSAL) {
    const int last_key = wrow0 + 31 + diag;
    nt_w = last_key < 0 ? 0 : min(nt_w, last_key / T::BN + 1);
  }

  // ---- K and V tiles: register-staged into a 2-stage LDS ring
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(uniform_ptr((const uint8_t*)p.k + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh),
                (uint32_t)((int64_t)Lk * p.k_ss));
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(uniform_ptr((const uint8_t*)p.v + (int64_t)b * p.v_sb + (int64_t)g * p.v_sh),
                (uint32_t)((int64_t)Lk * p.v_ss));
  const int lrow = tid / T::CH, lcol = 16 * (tid % T::CH);
  u32x4 kreg[T::NP], vreg[T::NP];
  // the K and V scales of the tile being loaded travel with it, so their
  // load latency is hidden like the tile's
  float sk_n = 1.f, sv_n = 1.f;
  auto gload = [&](int j0) {
#pragma unroll
    for (int w = 0; w < T::NP; ++w) {
      const uint32_t r = (uint32_t)(j0 + lrow + w * T::RPP);
      kreg[w] = buf_load16(rk, r * (uint32_t)p.k_ss + lcol);
      vreg[w] = buf_load16(rv, r * (uint32_t)p.v_ss + lcol);
    }
    sk_n = ksc[j0 / QBLK];
    sv_n = vsc[j0 / QBLK];
  };
  auto lstore = [&](int st) {
    uint8_t* Ks = smem + st * T::STAGE;
    uint8_t* Vs = Ks + T::BN * T::STR;
#pragma unroll
    for (int w = 0; w < T::NP; ++w) {
      *(u32x4*)(Ks + (lrow + w * T::RPP) * T::STR + lcol) = kreg[w];
      *(u32x4*)(Vs + (lrow + w * T::RPP) * T::STR + lcol) = vreg[w];
    }
  };

  const int kperm = row_perm(l32);
  const int G = lane >> 4, u = lane & 15;
  const int tr_row = 8 * (G >> 1) + (u >> 1);
  const int tr_col = 16 * (G & 1) + 8 * (u & 1);
  f32x16 dq[T::ND];
#pragma unroll
  for (int i = 0; i < T::ND; ++i) dq[i] = (f32x16){};

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  float sk_c = sk_n, sv_c = sv_n;   // scales of the tile in LDS
  wait_vmem();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    const int j0 = t * T::BN;
    const bool more = t + 1 < ntiles;
    if (more) gload(j0 + T::BN);
    if (t < nt_w) {
      const uint8_t* Ks = smem + st * T::STAGE;
      const uint8_t* Vs = Ks + T::BN * T::STR;
      const float sk = sk_c, sv = sv_c;
      // ---- S^T = K Q^T and dP^T = V dO^T (keys in the rows, queries in the lanes)
      f32x16 sacc[2] = {(f32x16){}, (f32x16){}}, dacc[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int c = 0; c < T::NC; ++c)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const int off = (kperm + 32 * kb2) * T::STR + 64 * c + 32 * hh;
          sacc[kb2] = mfma_mx(cat8(*(const u32x4*)(Ks + off), *(const u32x4*)(Ks + off + 16)), qf[c],
                              sacc[kb2], UNIT, UNIT);
          dacc[kb2] = mfma_mx(cat8(*(const u32x4*)(Vs + off), *(const u32x4*)(Vs + off + 16)), of[c],
                              dacc[kb2], UNIT, edo);
        }
      // ---- dS * sk = P (dP sv sk - D sk); keys past lim get P = 0
      const float c2t = c2 * sk, f = sv * sk, dsk = dlt * sk;
      const bool need_mask = (j0 + T::BN > Lk) || (CAUSAL && j0 + T::BN - 1 > wrow0 + diag);
      const int lim = CAUSAL ? min(Lk - 1, qrow + diag) : Lk - 1;
      // Keys past lim get P = 0.  Register i of block kb2 holds key j0 +
      // 32 kb2 + 16 (i >> 3) + 8 hh + (i & 7), so the test is a constant
      // against one per-lane threshold, and it runs only on tiles that need
      // it: need_mask is wave-uniform, and saying so, with the unmasked loop
      // written out separately, gives a branch instead of selects on every
      // element of every tile.
      float v[2][16];
      if (__builtin_amdgcn_readfirstlane((int)need_mask) != 0) {
        const int thr = lim - j0 - 8 * hh;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float pv = fast_exp2(__builtin_fmaf(sacc[kb2][i], c2t, -lse2));
            if (32 * kb2 + 16 * (i >> 3) + (i & 7) > thr) pv = 0.f;
            v[kb2][i] = pv * __builtin_fmaf(dacc[kb2][i], f, -dsk);
          }
      } else {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            v[kb2][i] = fast_exp2(__builtin_fmaf(sacc[kb2][i], c2t, -lse2)) * __builtin_fmaf(dacc[kb2][i], f, -dsk);
      }
      int sbyte;
      const i32x8 ds8 = quantise_ds(v, hh, sbyte);
      // ---- dQ^T += K^T dS^T (64 keys per instruction; K^T by transposing reads)
      const uint8_t* kbase = Ks + tr_row * T::STR + tr_col;
#pragma unroll
      for (int db = 0; db < T::ND; ++db) {
        i32x8 kf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2 x = lds_read_tr8(kbase + 16 * r * T::STR + 32 * db);
          kf[2 * r] = x[0];
          kf[2 * r + 1] = x[1];
        }
        dq[db] = mfma_mx(kf, ds8, dq[db], UNIT, sbyte);
      }
    }
    if (more) lstore(st ^ 1);
    sk_c = sk_n;
    sv_c = sv_n;
    __syncthreads();
  }

  if (qrow < Lq) {
    __bf16* dqb = (__bf16*)p.dq + (int64_t)b * p.dq_sb + (int64_t)h * p.dq_sh + (int64_t)qrow * p.dq_ss;
#pragma unroll
    for (int db = 0; db < T::ND; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(dq[db][4 * gi + r] * p.scale);
        *(bf16x4*)(dqb + 32 * db + 8 * gi + 4 * hh) = w;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdParams& p, int stages, hipStream_t stream) {
  if (stages & 1) {
    const long nblk = (long)p.B * p.Hq * ((p.Sq + QBLK - 1) / QBLK);
    if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
    if (nblk > 0) {
      hipLaunchKernelGGL((bwd_fp8_preprocess_kernel<D>), dim3((unsigned)nblk), dim3(256), 0, stream, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if ((stages & 2) && p.Sk > 0) {
    const long nblk = (long)((p.Sk + 127) / 128) * p.Hkv * p.B;
    if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_fp8_kernel<D, CAUSAL>), dim3((unsigned)nblk), dim3(DkdvFp8Tile<D>::NT), 0,
                       stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & 4) {
    const long nblk = (long)((p.Sq + 127) / 128) * p.Hq * p.B;
    if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dq_fp8_kernel<D, CAUSAL>), dim3((unsigned)nblk), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_fp8(const BwdParams& p, int d, bool causal, int stages, hipStream_t stream) {
  if (d == 128) return causal ? launch<128, true>(p, stages, stream) : launch<128, false>(p, stages, stream);
  return causal ? launch<64, true>(p, stages, stream) : launch<64, false>(p, stages, stream);
}
