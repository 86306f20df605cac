// Internal launch descriptors shared by the host entry points and kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Packed-sequence workgroup orders (varlen_order in device_common.h): query
// or key tiles per XCD run, per query head of a kv group.
constexpr int kFwdVarlenRun = 4;      // fwd_bf16_kernel (128-row tiles, 2 workgroups per CU)
constexpr int kFwdPpVarlenRun = 2;    // fwd_bf16_pp_kernel (256-row tiles, 1 per CU)
constexpr int kDkdvVarlenRun = 8;     // bwd_dkdv_kernel (128 keys, 1 per CU)
constexpr int kDqVarlenRun = 4;       // bwd_dq_kernel (128 rows, 2 per CU)

// A KV cache read by token position (KV-cache attention).  Token j of
// sequence b is slot j & (2^page_shift - 1) of page
// block_table[b * bt_stride + (j >> page_shift)]; with no block table,
// sequence b owns page b and the slot is j.  The token and head strides are
// the k_ss/k_sh and v_ss/v_sh of the launch parameters.
struct KvCacheParams {
  const int32_t* seqlens;      // [B] tokens cached before the append
  const int32_t* block_table;  // [B, bt_stride] page indices, or NULL
  int64_t bt_stride;
  int page_shift;
  int snew;                    // tokens appended per sequence (part of every length)
  int64_t k_sp, v_sp;          // element strides between pages
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_ss, q_sh;   // element strides; for varlen q_sb is unused
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t lse_sb, lse_sh;     // dense: [B,Hq,Sq]; varlen: lse_sh = total_q
  const int32_t* cu_q;        // varlen only
  const int32_t* cu_k;
  const float* q_descale;     // fp8 only
  const float* k_descale;
  const float* v_descale;
  const uint8_t* q_e8m0;      // MX fp8 only: [B,Sq,Hq,d/32], [B,Sk,Hkv,d/32], [B,Hkv,ceil(Sk/32),d]
  const uint8_t* k_e8m0;
  const uint8_t* v_e8m0;
  int B, Sq, Sk, Hq, Hkv, group;   // varlen: B = nseq, Sq/Sk = max lengths
  int num_m_tiles;
  float scale;                // softmax scale
  float scale_log2;           // scale * log2(e)
  KvCacheParams kv;           // KV-cache kernels only (then Sk bounds every length)
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const float* lse;
  float* delta;               // workspace [B,Hq,Sq]: rowsum(dO * O)
  float* dq_acc;              // workspace [B,Hq,Sq,d] fp32
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t do_sb, do_ss, do_sh;
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  int64_t dv_sb, dv_ss, dv_sh;
  const int* cu_q;            // packed sequences: token offsets [B + 1] (else NULL)
  const int* cu_k;
  int total_q;                // packed sequences: Tq (LSE and D are [Hq, Tq])
  int B, Sq, Sk, Hq, Hkv, group;
  int causal;
  float scale;
  float scale_log2;
  // FP8 backward only: per-block fp32 scales of the E4M3 q, k, v codes
  // ([B,Hq,ceil(Sq/128)], [B,Hkv,ceil(Sk/128)]), and the workspace's
  // quantised dO: codes [B,Hq,Sq,d] and one power-of-two scale per
  // (batch, head, 128-row block) stored as its E8M0 byte [B,Hq,ceil(Sq/128)]
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  uint8_t* do8;
  int* do_e8m0;
};

// Split-KV decode: partial results per (row, split) in the caller's workspace.
struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* o_part;              // [B,Hq,Sq,nsplit,d] fp32, each normalised by its own row sum
  float* lse_part;            // [B,Hq,Sq,nsplit] fp32
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t lse_sb, lse_sh;
  int B, Sq, Sk, Hq, Hkv, group;
  int causal;
  int nsplit, chunk;          // keys [s*chunk, (s+1)*chunk) form split s
  int nrblk;                  // blocks of 32 of the Sq * group query rows of a kv head
  float scale;
  float scale_log2;
  KvCacheParams kv;           // KV-cache kernels only (then Sk bounds every length)
};

// Append of new K/V rows into a KV cache: row i of sequence b goes to token
// position seqlens[b] + i.
struct KvAppendParams {
  const void* k_new;
  const void* v_new;
  int64_t kn_sb, kn_ss, kn_sh, vn_sb, vn_ss, vn_sh;
  void* k_cache;
  void* v_cache;
  int64_t k_ss, k_sh, v_ss, v_sh;
  KvCacheParams kv;
  int B, Hkv;
};

// Merge of partial results over key shards: parts [nparts, B, S, H, d]
// (bf16 or fp32, contiguous) and [nparts, B, H, S] fp32.
struct MergeParams {
  const void* o_parts;
  const float* lse_parts;
  void* o;
  float* lse;                 // [B, H, S] contiguous
  int64_t o_sb, o_ss, o_sh;
  int nparts, B, S, H;
};
hipError_t launch_merge(const MergeParams& p, int d, bool f32, hipStream_t stream);

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, bool varlen,
                           hipStream_t stream);
hipError_t launch_fwd_bf16_pp(const FwdParams& p, int d, bool causal, bool varlen,
                              hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_mxfp8(const FwdParams& p, int d, bool causal, hipStream_t stream);
// MX fp8 quantiser: axis 0 blocks of 32 along d, axis 1 blocks of 32 tokens.
hipError_t launch_quantize_mxfp8(const float* x, int64_t sb, int64_t ss, int64_t sh, int B, int S,
                                 int H, int d, int axis, void* codes, uint8_t* scales,
                                 hipStream_t stream);
hipError_t launch_quantize_fp8(const float* x, int64_t sb, int64_t ss, int64_t sh, int B, int S,
                               int H, int d, int per_tensor, void* codes, float* scales,
                               hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams& p, int d, hipStream_t stream);
// KV-cache attention: the same kernels reading a paged (or dense) cache with
// per-sequence lengths seqlens[b] + snew.
hipError_t launch_decode_bf16_kvcache(const DecodeParams& p, int d, hipStream_t stream);
hipError_t launch_fwd_bf16_kvcache(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_bf16_pp_kvcache(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_kv_append(const KvAppendParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, bool varlen, int stages,
                           hipStream_t stream);
hipError_t launch_bwd_fp8(const BwdParams& p, int d, bool causal, int stages, hipStream_t stream);
// Zero a bf16 [B,S,H,d] tensor with element strides (d contiguous).
hipError_t launch_zero_bf16(void* ptr, int64_t B, int64_t S, int64_t H, int64_t d, int64_t sb,
                            int64_t ss, int64_t sh, hipStream_t stream);

// Scratch for the no-allocation entry points: a fixed per-device array of
// kNoallocScratchBytes in the library's device code.  noalloc_scratch returns
// its address on the current device (looked up once per device).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** ptr);
