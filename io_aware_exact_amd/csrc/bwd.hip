// Backward kernels of IO-aware exact attention for gfx950 (bf16 in, fp32
// accumulate, bf16 gradients).
//
// Method.  The backward recomputes the attention probabilities from the
// saved row log-sum-exp instead of reading a stored probability matrix
// ("Dao and colleagues: IO-aware exact attention with FlashAttention",
// summary: tiling plus recomputation), and its reductions are deterministic
// (Dao-AILab repository overview: deterministic backward passes).  With
// P = exp(scale Q K^T - LSE) and D_i = sum_c dO_ic O_ic, the calculus
// derivative of exact attention is
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),
//     dK = scale dS^T Q,   dQ = scale dS K.
//
// gfx950 mapping (32x32x16 bf16 MFMA, operand layouts in device_common.h).
//   * bwd_preprocess: D = rowsum(dO o O) in fp32, one 16-lane group per row.
//   * bwd_dkdv: a workgroup of 8 waves owns 128 keys of one (batch, kv head);
//     each 32-key group has a P-wave (K rows in VGPRs as the B operand of
//     S = Q K^T, the dV^T accumulator) and a dS-wave (V rows for dP = dO V^T,
//     the dK^T accumulator) that shares its SIMD; P goes from one to the
//     other through LDS.  Query tiles of 64 rows (Q, dO, LSE, D) of every
//     query head of the group stream through a double-buffered LDS ring.
//     Query rows are fed to the A operand in a permuted order so that
//     accumulator registers 0..7 / 8..15 of a lane hold 8 consecutive
//     queries: P and dS are then directly the B operands of dV^T += dO^T P
//     and dK^T += Q^T dS (dO^T and Q^T come from the LDS transposing read).
//     Each key's gradient is a sum in a fixed order over (query head, query
//     tile): no atomics.
//   * bwd_dq: a workgroup of 4 waves owns 128 query rows; each wave keeps
//     Q^T, dO^T, LSE and D of its 32 rows in registers and sweeps the K/V
//     tiles (double-buffered in LDS) in order, computing S^T = K Q^T,
//     dP^T = V dO^T, dS^T, and dQ^T += K^T dS^T.  dQ is therefore a
//     fixed-order sum as well; the price is recomputing S and dP a second
//     time (7 products instead of the method's 5).
//   * Causal: key tiles above the diagonal are skipped on both sides, element
//     masks only on tiles crossing it.  Rows past the sequence end read as
//     zero (buffer bounds checks) and their LSE is taken as +inf, so their
//     probabilities are exactly zero.
#include "device_common.h"
#include "fa_internal.h"

namespace {

constexpr int NTHREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;

// A-operand row order that makes accumulator registers 0..7 / 8..15 of a
// lane cover 8 consecutive rows (see the forward kernel).
__device__ __forceinline__ int row_perm(int l32) {
  return 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
}

// Row (within a 32-row block) held by accumulator register i of a lane in
// half hh, when the A operand rows were fed in row_perm order.
__device__ __forceinline__ int perm_row_of_reg(int i, int hh) {
  return (i < 8) ? 8 * hh + i : 16 + 8 * hh + (i - 8);
}

// ---------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic (fp32), written to delta[b][h][i].
template <int D>
__global__ __launch_bounds__(NTHREADS) void bwd_preprocess_kernel(BwdParams p) {
  constexpr int LPR = D / 8;                 // lanes per row (16 B each)
  constexpr int RPB = NTHREADS / LPR;        // rows per block
  const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
  const long nrows = (long)p.B * p.Sq * p.Hq;
  const int c = (threadIdx.x % LPR) * 8;
  float acc = 0.f;
  long b = 0, i = 0, h = 0;
  if (row < nrows) {
    h = row % p.Hq;
    const long t = row / p.Hq;
    i = t % p.Sq;
    b = t / p.Sq;
    const bf16x8 o = *(const bf16x8*)((const __bf16*)p.o + b * p.o_sb + i * p.o_ss + h * p.o_sh + c);
    const bf16x8 g = *(const bf16x8*)((const __bf16*)p.dout + b * p.do_sb + i * p.do_ss + h * p.do_sh + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, 64);
  if (row < nrows && (threadIdx.x % LPR) == 0) p.delta[(b * p.Hq + h) * p.Sq + i] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV for 128 keys of one (batch, kv head), with the work of each 32-key
// group split between two waves on the same SIMD: the P-wave keeps K and the
// dV^T accumulator (S = Q K^T, P = exp2(S c - LSE log2 e), dV^T += dO^T P) and
// the dS-wave keeps V and the dK^T accumulator (dP = dO V^T, dS = P o (dP - D),
// dK^T += Q^T dS), receiving P through LDS.  Each wave then holds one resident
// operand and one accumulator, which lets two waves share a SIMD; the MFMA
// work is unchanged.  The dS-wave runs one query tile behind the P-wave, so
// in every iteration both roles have MFMA and VALU work and one barrier
// suffices: iteration t has the P-wave on tile t and the dS-wave on tile
// t - 1, whose P the P-wave left in LDS during iteration t - 1.
template <int D>
struct DkdvTile {
  static constexpr int NT = 512;               // 8 waves: 4 key groups x 2 roles
  static constexpr int BKV = 128;              // keys per workgroup (32 per key group)
  static constexpr int BQ = 64;                // query rows per streamed tile (2 blocks of 32)
  static constexpr int NC = D / 16;
  static constexpr int ND = D / 32;
  static constexpr int TILE = BQ * D;          // elements of one Q or dO tile (swizzled rows)
  static constexpr int STAGE_BYTES = 2 * TILE * 2 + 2 * BQ * 4;
  static constexpr int NSTAGE = 3;             // tile t (P-wave), t - 1 (dS-wave), t + 1 (loading)
  static constexpr int PEX_SLOT = 4 * 2 * 64 * 16 * 2;   // bf16 P of 4 key groups x 2 blocks
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES + 2 * PEX_SLOT;
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdParams p) {
  using T = DkdvTile<D>;
  __shared__ __attribute__((aligned(16))) char smem[T::LDS_BYTES];

  // Dense: consecutive key tiles of one kv head share an XCD.  Packed
  // sequences: runs of key tiles of one (sequence, kv head) per XCD, lowest
  // key tiles (the heaviest when causal) first.
  int kt, g, b;
  if (VARLEN) {
    int row;
    if (!varlen_order(blockIdx.x, p.Hkv * p.B, kDkdvVarlenRun, row, kt)) return;
    g = row % p.Hkv;
    b = row / p.Hkv;
  } else {
    const int nkt = (p.Sk + T::BKV - 1) / T::BKV;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    kt = L % nkt;
    const int rest = L / nkt;
    g = rest % p.Hkv;
    b = rest / p.Hkv;
  }
  int Lq = p.Sq, Lk = p.Sk;
  int64_t qtok = 0, ktok = 0;
  if (VARLEN) {
    const int qs = p.cu_q[b], ks = p.cu_k[b];
    Lq = p.cu_q[b + 1] - qs;
    Lk = p.cu_k[b + 1] - ks;
    qtok = qs;
    ktok = ks;
  }
  if (kt * T::BKV >= Lk) return;   // workgroup-uniform: past this sequence's keys

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int kgrp = wave & 3;                // key group (shared by the two roles)
  const bool pwave = wave < 4;              // role: P-wave (else dS-wave)
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int diag = Lk - Lq;
  const int k0 = kt * T::BKV;
  const int kw0 = k0 + 32 * kgrp;           // first key of this key group
  const int key = kw0 + l32;                // key owned by this lane (C column)

  // ---- resident operand: K (P-wave) or V (dS-wave), B operand of Q K^T / dO V^T
  const __bf16* kvb = pwave ? (const __bf16*)p.k + (VARLEN ? ktok * p.k_ss : (int64_t)b * p.k_sb) + (int64_t)g * p.k_sh
                            : (const __bf16*)p.v + (VARLEN ? ktok * p.v_ss : (int64_t)b * p.v_sb) + (int64_t)g * p.v_sh;
  const int64_t kv_ss = pwave ? p.k_ss : p.v_ss;
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc(kvb, (uint32_t)((int64_t)Lk * kv_ss * 2));
  bf16x8 bf[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c)
    bf[c] = __builtin_bit_cast(bf16x8, buf_load16(rkv, (uint32_t)(key * kv_ss + 16 * c + 8 * hh) * 2));

  // ---- query tiles to visit: every head of the group, tiles from the first
  // one that can see this workgroup's keys
  const int nqt = (Lq + T::BQ - 1) / T::BQ;
  int qt0 = 0;
  if (CAUSAL) qt0 = max(0, k0 - diag) / T::BQ;
  const int per_head = max(0, nqt - qt0);
  const int niter = per_head * p.group;

  auto stage = [&](int st) { return (__bf16*)(smem + st * T::STAGE_BYTES); };
  // Q and dO tiles go from HBM straight into the swizzled LDS stage: each
  // wave fills rows [8 w, 8 w + 8) of both tiles, one 1 KB block (RPI rows)
  // per load, every lane fetching the logical chunk that belongs at its
  // physical position in the block.  The per-lane part of every address is
  // fixed; a tile adds its first row.  The tile to load next is tracked as
  // (head in group, query tile) counters, so no division is needed, and the
  // buffer resources change only when the head does.
  constexpr int RPI = 512 / D;               // rows per 1 KB block
  constexpr int NLD = 8 / RPI;               // blocks per wave per tile
  const int lrow_in = lane / (64 / RPI);     // row of this lane within a block
  const int lpc = lane % (64 / RPI);         // physical 16-byte chunk
  uint32_t qoff[NLD], dooff[NLD];
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int row = 8 * (wave & 7) + RPI * u + lrow_in;                // row of the tile
    const int col = swz<D>(row, 8 * lpc) - row * D;                     // logical column (elements)
    qoff[u] = (uint32_t)(row * p.q_ss + col) * 2;
    dooff[u] = (uint32_t)(row * p.do_ss + col) * 2;
  }
  int ld_h = 0, ld_qt = 0;                   // next tile to load: head in group, tile in head
  __amdgpu_buffer_rsrc_t rq, rdo;
  const float* lse_h = nullptr;
  const float* del_h = nullptr;
  auto set_head = [&](int hi) {
    const int h = p.group * g + hi;
    const __bf16* qb = (const __bf16*)p.q + (VARLEN ? qtok * p.q_ss : (int64_t)b * p.q_sb) + (int64_t)h * p.q_sh;
    const __bf16* db = (const __bf16*)p.dout + (VARLEN ? qtok * p.do_ss : (int64_t)b * p.do_sb) + (int64_t)h * p.do_sh;
    rq = make_rsrc(qb, (uint32_t)((int64_t)Lq * p.q_ss * 2));
    rdo = make_rsrc(db, (uint32_t)((int64_t)Lq * p.do_ss * 2));
    // LSE and D: [B, Hq, Sq] dense, [Hq, Tq] packed
    const int64_t rowbase = VARLEN ? (int64_t)h * p.total_q + qtok : ((int64_t)b * p.Hq + h) * Lq;
    lse_h = p.lse + rowbase;
    del_h = p.delta + rowbase;
  };
  if (niter > 0) set_head(0);
  float sval = 0.f;
  // loads the tile (ld_h, ld_qt) into stage st and advances the counters
  auto gload = [&](int st) {
    const int q0 = (qt0 + ld_qt) * T::BQ;
    __bf16* Qs = stage(st);
    __bf16* Os = Qs + T::TILE;
    const uint32_t qbase = (uint32_t)q0 * (uint32_t)p.q_ss * 2;
    const uint32_t dobase = (uint32_t)q0 * (uint32_t)p.do_ss * 2;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      buf_load16_lds(rq, qbase + qoff[u], Qs + (8 * (wave & 7) + RPI * u) * D);
      buf_load16_lds(rdo, dobase + dooff[u], Os + (8 * (wave & 7) + RPI * u) * D);
    }
    // threads 0..63 fetch LSE, threads 64..127 fetch D (used only when the
    // stage is completed, so no wait here)
    if (tid < 2 * T::BQ) {
      const int r = q0 + (tid & (T::BQ - 1));
      if (tid < T::BQ) sval = r < Lq ? lse_h[r] : INFINITY;
      else sval = r < Lq ? del_h[r] : 0.f;
    }
    if (++ld_qt == per_head) {
      ld_qt = 0;
      if (++ld_h < p.group) set_head(ld_h);
    }
  };
  // LSE is stored as a log2 value; no visible key (LSE = -inf) or padding
  // (+inf) makes the probabilities zero
  auto lstore_stats = [&](int st) {
    float* stats = (float*)(stage(st) + 2 * T::TILE);
    if (tid < T::BQ) stats[tid] = (sval == -INFINITY) ? INFINITY : sval * LOG2E;
    else if (tid < 2 * T::BQ) stats[tid] = sval;
  };
  // bf16 P of key group kgrp, query block qb, in P-exchange slot sl, stored
  // lane-interleaved (16 consecutive lanes write 256 contiguous bytes)
  auto pex = [&](int sl, int qb) {
    return (u32x4*)(smem + T::NSTAGE * T::STAGE_BYTES + sl * T::PEX_SLOT) + ((kgrp * 2 + qb) * 2) * 64 + lane;
  };

  f32x16 acc[T::ND];
#pragma unroll
  for (int i = 0; i < T::ND; ++i) acc[i] = (f32x16){};
  const float c2 = p.scale_log2;
  const int prow = row_perm(l32);
  const int trG = lane >> 4;
  const int tr_row = 8 * (trG >> 1) + ((lane >> 2) & 3);
  const int tr_col = 16 * (trG & 1) + 4 * (lane & 3);

  // The chunk permutation of a swizzled tile depends on the row modulo 16
  // only, so every operand address is a per-lane base plus a constant:
  // swz(r + 16 k, c) = swz(r, c) + 16 k D.  The per-lane parts are added to
  // the tile base once per iteration; the constants fold into the LDS
  // instructions' offset fields.
  int aoff[T::NC], toff[2][T::ND];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) aoff[c] = swz<D>(prow, 16 * c + 8 * hh);
#pragma unroll
  for (int dbk = 0; dbk < T::ND; ++dbk) {
    toff[0][dbk] = swz<D>(tr_row, 32 * dbk + tr_col);
    toff[1][dbk] = swz<D>(tr_row + 4, 32 * dbk + tr_col);
  }

  if (niter > 0) {
    gload(0);
    lstore_stats(0);
  }
  wait_vmem();
  __syncthreads();

  // stages of the P-wave's tile (it % 3), the dS-wave's tile ((it - 1) % 3)
  // and the tile being loaded ((it + 1) % 3); the P-wave's query tile
  int st_cur = 0, st_prev = 2, st_next = 1;
  int pw_qt = 0;

  // Every block is computed: query blocks that see none of this key group's
  // keys (past the end, where LSE = +inf; above the causal diagonal; keys
  // past Lk) get P = 0 from the masks, so their contributions vanish, and
  // the MFMAs need no data-dependent branches.
  for (int it = 0; it <= niter; ++it) {
    const bool more = it + 1 < niter;
    if (more) gload(st_next);
    // P-wave on tile it; dS-wave on tile it - 1
    const bool work = pwave ? it < niter : it > 0;
    if (work) {
      const int t = pwave ? it : it - 1;
      const __bf16* Qs = stage(pwave ? st_cur : st_prev);
      const __bf16* Os = Qs + T::TILE;
      const float* stats = (const float*)(Os + T::TILE);
      const __bf16* As = pwave ? Qs : Os;   // A operand rows: Q for S, dO for dP
      const __bf16* Ts = pwave ? Os : Qs;   // transposed: dO^T for dV, Q^T for dK
      // ---- S = Q K^T or dP = dO V^T for both query blocks, two interleaved chains
      f32x16 s2[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int c = 0; c < T::NC; ++c) {
        const __bf16* ap = As + aoff[c];
        const bf16x8 a0 = *(const bf16x8*)(ap);
        const bf16x8 a1 = *(const bf16x8*)(ap + 32 * D);
        s2[0] = mfma32(a0, bf[c], s2[0]);
        s2[1] = mfma32(a1, bf[c], s2[1]);
      }
      // keep the operand reads four MFMAs ahead of the products (left to
      // itself the compiler issues them two ahead and waits on each pair)
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * T::NC - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // ---- B operands of the second product: P (P-wave) or dS (dS-wave)
      bf16x8 ob[2][2];
      if (pwave) {
        const int q0 = (qt0 + pw_qt) * T::BQ;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int qr0 = q0 + 32 * qb;
          const f32x4* l4 = (const f32x4*)(stats + 32 * qb + 8 * hh);
          const f32x4 la = l4[0], lb = l4[1], lc = l4[4], ld = l4[5];
          const float lrow_v[16] = {la[0], la[1], la[2], la[3], lb[0], lb[1], lb[2], lb[3],
                                    lc[0], lc[1], lc[2], lc[3], ld[0], ld[1], ld[2], ld[3]};
          const bool need_mask = (kw0 + 31 >= Lk) || (CAUSAL && qr0 + diag < kw0 + 31);
          f32x16 pv;
#pragma unroll
          for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(__builtin_fmaf(s2[qb][i], c2, -lrow_v[i]));
          if (need_mask) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int iq = qr0 + perm_row_of_reg(i, hh);
              if (key >= Lk || (CAUSAL && key > iq + diag)) pv[i] = 0.f;
            }
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) ob[qb][i >> 3][i & 7] = (__bf16)pv[i];
          u32x4* pe = pex(t & 1, qb);
          pe[0] = __builtin_bit_cast(u32x4, ob[qb][0]);
          pe[64] = __builtin_bit_cast(u32x4, ob[qb][1]);
        }
      } else {
        const float* dels = stats + T::BQ;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const f32x4* d4 = (const f32x4*)(dels + 32 * qb + 8 * hh);
          const f32x4 da = d4[0], db = d4[1], dc = d4[4], dd = d4[5];
          const float drow_v[16] = {da[0], da[1], da[2], da[3], db[0], db[1], db[2], db[3],
                                    dc[0], dc[1], dc[2], dc[3], dd[0], dd[1], dd[2], dd[3]};
          const u32x4* pe = pex(t & 1, qb);
          const bf16x8 p0 = __builtin_bit_cast(bf16x8, pe[0]);
          const bf16x8 p1 = __builtin_bit_cast(bf16x8, pe[64]);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float pvv = (float)(i < 8 ? p0[i] : p1[i - 8]);
            ob[qb][i >> 3][i & 7] = (__bf16)(pvv * (s2[qb][i] - drow_v[i]));
          }
        }
      }
      // ---- acc += Ts^T ob for both query blocks
      const __bf16* tb[2][T::ND];
#pragma unroll
      for (int dbk = 0; dbk < T::ND; ++dbk) {
        tb[0][dbk] = Ts + toff[0][dbk];
        tb[1][dbk] = Ts + toff[1][dbk];
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
          for (int dbk = 0; dbk < T::ND; ++dbk) {
            const int rb = (32 * qb + 16 * kc) * D;
            const bf16x8 ta = cat_bf16(lds_read_tr16(tb[0][dbk] + rb), lds_read_tr16(tb[1][dbk] + rb));
            acc[dbk] = mfma32(ta, ob[qb][kc], acc[dbk]);
          }
        }
      }
      // the transposing reads two MFMAs ahead of the products (the
      // compiler's own schedule issues nearly all of them first)
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 4 * T::ND - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // gload filled stage (it + 1) % 3, last read by the dS-wave in
    // iteration it - 1; P slot it % 2 is read in iteration it + 1; both are
    // complete and visible after the wait and barrier below
    if (more) lstore_stats(st_next);
    wait_vmem();
    __syncthreads();
    const int st_free = st_prev;
    st_prev = st_cur;
    st_cur = st_next;
    st_next = st_free;
    if (++pw_qt == per_head) pw_qt = 0;
  }

  // ---- epilogue: dV (P-wave) or dK = scale * dK (dS-wave), bf16, one key row per lane
  if (key < Lk) {
    __bf16* out = pwave ? (__bf16*)p.dv + (VARLEN ? ktok * p.dv_ss : (int64_t)b * p.dv_sb) + (int64_t)g * p.dv_sh +
                              (int64_t)key * p.dv_ss
                        : (__bf16*)p.dk + (VARLEN ? ktok * p.dk_ss : (int64_t)b * p.dk_sb) + (int64_t)g * p.dk_sh +
                              (int64_t)key * p.dk_ss;
    const float f = pwave ? 1.f : p.scale;
#pragma unroll
    for (int dbk = 0; dbk < T::ND; ++dbk)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(acc[dbk][4 * gi + r] * f);
        *(bf16x4*)(out + 32 * dbk + 8 * gi + 4 * hh) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ for 128 query rows of one (batch, query head).  Tile t's MFMA block
// computes dQ^T += K_{t-1}^T dS_{t-1}^T together with S^T and dP^T of tile
// t, and the VALU block that follows forms dS^T of tile t: one MFMA block and
// one VALU block per tile.  K and V tiles come straight from HBM into
// swizzled LDS stages (LDS DMA), K in three stages (K_{t-1} is still read in
// iteration t), V in two.
template <int D>
struct DqTile {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int NC = D / 16;
  static constexpr int ND = D / 32;
  static constexpr int TILE = BN * D;         // swizzled rows, no padding
  static constexpr int KSTAGES = 3;
  static constexpr int VSTAGES = 2;
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NTHREADS, 2) void bwd_dq_kernel(BwdParams p) {
  using T = DqTile<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[(T::KSTAGES + T::VSTAGES) * T::TILE];

  // Dense: consecutive query tiles of one head share an XCD.  Packed
  // sequences: runs of query tiles of the query heads of one (sequence, kv
  // head) per XCD, which all read that K/V.  Causal: heaviest tiles first.
  const int nmt = (p.Sq + T::BM - 1) / T::BM;
  int mt, h, b;
  if (VARLEN) {
    int row, t;
    if (!varlen_order(blockIdx.x, p.Hkv * p.B, kDqVarlenRun * p.group, row, t)) return;
    mt = t / p.group;
    if (mt >= nmt) return;   // padding of the last run
    h = (row % p.Hkv) * p.group + (t - mt * p.group);
    b = row / p.Hkv;
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    mt = L % nmt;
    const int rest = L / nmt;
    h = rest % p.Hq;
    b = rest / p.Hq;
  }
  if (CAUSAL) mt = nmt - 1 - mt;
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
  const int diag = Lk - Lq;
  const int q0 = mt * T::BM;
  if (q0 >= Lq) return;   // workgroup-uniform: past this sequence's rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int qrow = q0 + 32 * wave + l32;

  const __bf16* qb = (const __bf16*)p.q + (VARLEN ? qtok * p.q_ss : (int64_t)b * p.q_sb) + (int64_t)h * p.q_sh;
  const __bf16* dob = (const __bf16*)p.dout + (VARLEN ? qtok * p.do_ss : (int64_t)b * p.do_sb) + (int64_t)h * p.do_sh;
  const __bf16* kb = (const __bf16*)p.k + (VARLEN ? ktok * p.k_ss : (int64_t)b * p.k_sb) + (int64_t)g * p.k_sh;
  const __bf16* vb = (const __bf16*)p.v + (VARLEN ? ktok * p.v_ss : (int64_t)b * p.v_sb) + (int64_t)g * p.v_sh;

  // ---- resident Q^T, dO^T fragments (B operands), LSE and D of this row
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)((int64_t)Lq * p.q_ss * 2));
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dob, (uint32_t)((int64_t)Lq * p.do_ss * 2));
  bf16x8 qf[T::NC], of[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) {
    qf[c] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(qrow * p.q_ss + 16 * c + 8 * hh) * 2));
    of[c] = __builtin_bit_cast(bf16x8, buf_load16(rdo, (uint32_t)(qrow * p.do_ss + 16 * c + 8 * hh) * 2));
  }
  float lse2 = INFINITY, dlt = 0.f;
  if (qrow < Lq) {
    // LSE and D: [B, Hq, Sq] dense, [Hq, Tq] packed
    const int64_t ri = (VARLEN ? (int64_t)h * p.total_q + qtok : ((int64_t)b * p.Hq + h) * Lq) + qrow;
    const float v = p.lse[ri];
    lse2 = (v == -INFINITY) ? INFINITY : v * LOG2E;
    dlt = p.delta[ri];
  }

  int kend = Lk;
  if (CAUSAL) kend = min(Lk, q0 + T::BM + diag);
  const int ntiles = kend > 0 ? (kend + T::BN - 1) / T::BN : 0;
  // tiles this wave sees: t < nt_w (monotone under the causal mask)
  const int wrow0 = q0 + 32 * wave;
  int nt_w = wrow0 < Lq ? ntiles : 0;
  if (CAUSAL) {
    const int last_key = wrow0 + 31 + diag;
    nt_w = last_key < 0 ? 0 : min(nt_w, last_key / T::BN + 1);
  }

  // ---- K/V tiles: HBM -> swizzled LDS stage by DMA; each wave fills rows
  // [16 w, 16 w + 16) of both tiles, one 1 KB block (RPI rows) per load,
  // every lane fetching the logical chunk that belongs at its physical place
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)((int64_t)Lk * p.k_ss * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)((int64_t)Lk * p.v_ss * 2));
  constexpr int RPI = 512 / D;               // rows per 1 KB block
  constexpr int RPW = T::BN / 4;             // tile rows filled by each wave
  constexpr int NLD = RPW / RPI;             // blocks per wave per tile
  const int lrow_in = lane / (64 / RPI);
  const int lpc = lane % (64 / RPI);
  auto kstage = [&](int s) { return smem + s * T::TILE; };
  auto vstage = [&](int s) { return smem + (T::KSTAGES + s) * T::TILE; };
  auto dma = [&](int t) {
    const int j0 = t * T::BN;
    __bf16* Ks = kstage(t % 3);
    __bf16* Vs = vstage(t & 1);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int row = RPW * wave + RPI * u + lrow_in;
      const int col = swz<D>(row, 8 * lpc) - row * D;                 // logical column of this chunk
      const uint32_t r = (uint32_t)(j0 + row);
      buf_load16_lds(rk, (r * (uint32_t)p.k_ss + col) * 2, Ks + (RPW * wave + RPI * u) * D);
      buf_load16_lds(rv, (r * (uint32_t)p.v_ss + col) * 2, Vs + (RPW * wave + RPI * u) * D);
    }
  };

  f32x16 dq[T::ND];
#pragma unroll
  for (int i = 0; i < T::ND; ++i) dq[i] = (f32x16){};
  bf16x8 dsb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dsb[i] = (bf16x8){};
  const float c2 = p.scale_log2;
  const int prow = row_perm(l32);
  const int trG = lane >> 4;
  const int tr_row = 8 * (trG >> 1) + ((lane >> 2) & 3);
  const int tr_col = 16 * (trG & 1) + 4 * (lane & 3);
  // swizzled operand addresses: per-lane bases plus constants (the chunk
  // permutation depends on the row modulo 16 only)
  int aoff[T::NC], toff[2][T::ND];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) aoff[c] = swz<D>(prow, 16 * c + 8 * hh);
#pragma unroll
  for (int dbk = 0; dbk < T::ND; ++dbk) {
    toff[0][dbk] = swz<D>(tr_row, 32 * dbk + tr_col);
    toff[1][dbk] = swz<D>(tr_row + 4, 32 * dbk + tr_col);
  }

  // dQ^T += K^T dS^T of tile t (K^T by transposing reads)
  auto dq_product = [&](int t) {
    const __bf16* Ks = kstage(t % 3);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int dbk = 0; dbk < T::ND; ++dbk) {
        const bf16x8 ka = cat_bf16(lds_read_tr16(Ks + toff[0][dbk] + 16 * c * D),
                                   lds_read_tr16(Ks + toff[1][dbk] + 16 * c * D));
        dq[dbk] = mfma32(ka, dsb[c], dq[dbk]);
      }
    // the transposing reads two MFMAs ahead of the products
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * T::ND - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  if (ntiles > 0) dma(0);
  wait_vmem();   // Q, dO fragments and tile 0 have landed
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * T::BN;
    // The K^T reads of tile t - 1 are issued before the DMA of tile t + 1:
    // the compiler cannot tell the transposing reads from a read of the
    // stage being filled, and would wait for the whole DMA first.
    if (t >= 1 && t - 1 < nt_w) dq_product(t - 1);
    // tile t + 1 goes to K stage (t+1)%3 and V stage (t+1)&1, last read in
    // iteration t - 1
    if (t + 1 < ntiles) dma(t + 1);
    if (t < nt_w) {
      const __bf16* Ks = kstage(t % 3);
      const __bf16* Vs = vstage(t & 1);
      const bool need_mask = (j0 + T::BN > Lk) || (CAUSAL && j0 + T::BN - 1 > wrow0 + diag);
      const int lim = CAUSAL ? min(Lk - 1, qrow + diag) : Lk - 1;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        f32x16 s = (f32x16){}, dp = (f32x16){};
        if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < T::NC; ++c) {
          const int off = aoff[c] + 32 * kb2 * D;
          s = mfma32(*(const bf16x8*)(Ks + off), qf[c], s);
          dp = mfma32(*(const bf16x8*)(Vs + off), of[c], dp);
        }
        if constexpr (D == 128) {
          // d=128: fence the 16 products and keep their operand reads four
          // MFMAs ahead (left to itself the compiler waits on each read; at
          // d=64 its own schedule is faster)
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int i = 0; i < 2 * T::NC - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // Keys past lim (sequence end, causal diagonal) get P = 0.  Register
        // i of this lane holds key j0 + 32 kb2 + 8 hh + r_i with r_i a
        // constant, so the test is r_i > thr for one per-lane threshold: one
        // compare and one select per element, with no per-element index
        // arithmetic, and only on tiles that need a mask.
        // need_mask is wave-uniform; saying so gives a real branch (the
        // compiler would otherwise select on every element of every tile)
        if (__builtin_amdgcn_readfirstlane((int)need_mask) != 0) {
          const int thr = lim - j0 - 32 * kb2 - 8 * hh;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float pv = fast_exp2(__builtin_fmaf(s[i], c2, -lse2));
            if (perm_row_of_reg(i, 0) > thr) pv = 0.f;
            dsb[2 * kb2 + (i >> 3)][i & 7] = (__bf16)(pv * (dp[i] - dlt));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float pv = fast_exp2(__builtin_fmaf(s[i], c2, -lse2));
            dsb[2 * kb2 + (i >> 3)][i & 7] = (__bf16)(pv * (dp[i] - dlt));
          }
        }
      }
    }
    wait_vmem();
    __syncthreads();
  }
  if (ntiles > 0 && ntiles - 1 < nt_w) dq_product(ntiles - 1);

  if (qrow < Lq) {
    __bf16* dqb = (__bf16*)p.dq + (VARLEN ? qtok * p.dq_ss : (int64_t)b * p.dq_sb) + (int64_t)h * p.dq_sh +
                  (int64_t)qrow * p.dq_ss;
#pragma unroll
    for (int dbk = 0; dbk < T::ND; ++dbk)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(dq[dbk][4 * gi + r] * p.scale);
        *(bf16x4*)(dqb + 32 * dbk + 8 * gi + 4 * hh) = w;
      }
  }
}

// Zero fill of a strided bf16 [B,S,H,d] tensor, 8 elements per thread.
__global__ __launch_bounds__(256) void zero_bf16_kernel(__bf16* ptr, int64_t S, int64_t H, int64_t d,
                                                       int64_t sb, int64_t ss, int64_t sh, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t per_row = d / 8;
  const int64_t c = (i % per_row) * 8;
  int64_t r = i / per_row;
  const int64_t h = r % H;
  r /= H;
  const int64_t s = r % S;
  const int64_t b = r / S;
  *(u32x4*)(ptr + b * sb + s * ss + h * sh + c) = (u32x4){0u, 0u, 0u, 0u};
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_bwd(const BwdParams& p, int stages, hipStream_t stream) {
  if (stages & 1) {
    // packed rows [Tq, Hq, d] are the dense layout with B = 1, Sq = Tq, and D
    // [Hq, Tq] is its [B, Hq, Sq]
    BwdParams pp = p;
    if (VARLEN) {
      pp.B = 1;
      pp.Sq = p.total_q;
    }
    constexpr int RPB = NTHREADS / (D / 8);
    const long rows = (long)pp.B * pp.Sq * pp.Hq;
    const long nblk = (rows + RPB - 1) / RPB;
    if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_preprocess_kernel<D>), dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, pp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & 2) && p.Sk > 0) {
    const int nkt = (p.Sk + DkdvTile<D>::BKV - 1) / DkdvTile<D>::BKV;
    const long nblk = VARLEN ? varlen_grid(p.Hkv * p.B, nkt, kDkdvVarlenRun)
                             : (long)nkt * p.Hkv * p.B;
    if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)nblk), dim3(DkdvTile<D>::NT), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & 4) {
    const int nmt = (p.Sq + DqTile<D>::BM - 1) / DqTile<D>::BM;
    const long nblk = VARLEN ? varlen_grid(p.Hkv * p.B, nmt * p.group, kDqVarlenRun * p.group)
                             : (long)nmt * p.Hq * p.B;
    if (nblk > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, bool varlen, int stages,
                           hipStream_t stream) {
  if (d == 128) {
    if (causal) return varlen ? launch_bwd<128, true, true>(p, stages, stream) : launch_bwd<128, true, false>(p, stages, stream);
    return varlen ? launch_bwd<128, false, true>(p, stages, stream) : launch_bwd<128, false, false>(p, stages, stream);
  }
  if (causal) return varlen ? launch_bwd<64, true, true>(p, stages, stream) : launch_bwd<64, true, false>(p, stages, stream);
  return varlen ? launch_bwd<64, false, true>(p, stages, stream) : launch_bwd<64, false, false>(p, stages, stream);
}

hipError_t launch_zero_bf16(void* ptr, int64_t B, int64_t S, int64_t H, int64_t d, int64_t sb,
                            int64_t ss, int64_t sh, hipStream_t stream) {
  const int64_t n8 = B * S * H * (d / 8);
  if (n8 <= 0) return hipSuccess;
  const int64_t grid = (n8 + 255) / 256;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (__bf16*)ptr, S, H, d,
                     sb, ss, sh, n8);
  return hipGetLastError();
}
