/*
 * fa.h -- C ABI of libfa.so: IO-aware exact attention on AMD Instinct MI355X
 * (gfx950).
 *
 * What the calls compute.  Exact softmax attention, O = softmax(scale * Q K^T
 * [+ causal mask]) V, evaluated tile by tile with a running row maximum and
 * row sum so that the Sq x Sk score matrix never reaches device memory, and
 * its backward, which rebuilds the probabilities from the saved row
 * log-sum-exp instead of storing them.  Sources (pages on IO-aware exact
 * attention):
 *   - "Dao and colleagues: IO-aware exact attention with FlashAttention",
 *     research record, fields "summary" and "boundary": exact attention by
 *     tiling plus recomputation, the full attention matrix is never
 *     materialised, arithmetic stays quadratic;
 *   - "Flash Attention and Efficient Transformer Mechanisms": blocks of Q, K
 *     and V are read from high-bandwidth memory into on-chip memory and
 *     partial outputs are computed there, and the result is that of
 *     standard attention, not an approximation of it;
 *   - Dao-AILab repository overview: online softmax with rescaling, tiled
 *     attention staged through on-chip memory, a dense entry point, a packed
 *     variable-length entry point and a KV-cache (decode) entry point,
 *     deterministic backward passes;
 *   - "FlashAttention-3: Fast and Accurate Attention with Asynchrony and
 *     Low-precision" (summary, third contribution): an FP8 forward with
 *     block-wise scaling.
 *
 * Conventions (readings; the pages fix none of them):
 *   - dense tensors are [B, S, H, d] with element strides for B, S and H and
 *     a contiguous last dimension; packed (varlen) tensors are [T, H, d];
 *   - query head h uses kv head h / (Hq / Hkv) (grouped-query attention);
 *   - causal masking is bottom-right aligned: query row i sees key j iff
 *     j <= i + (Sk - Sq); a row that sees no key gets O = 0, LSE = -inf;
 *   - LSE is the natural-log log-sum-exp of the scaled, masked scores, fp32,
 *     laid out [B, Hq, Sq] (dense) or [Hq, T_q] (varlen), contiguous;
 *   - inputs are bf16 (or OCP e4m3 for the FP8 forward, or fp32 for the fp32
 *     forward); accumulation is fp32; outputs O, dQ, dK, dV are bf16 (fp32
 *     for the fp32 forward), rounded to nearest even.
 *
 * Ownership.  Every pointer is a DEVICE pointer owned by the caller; a
 * tensor pointer may be NULL exactly when that tensor has no elements.  The
 * library never allocates, frees or keeps a pointer past the enqueued work,
 * and never synchronises the stream: all work is enqueued on `stream`.
 * Outputs are fully overwritten.
 *
 * Errors.  Arguments are checked on the host before anything is enqueued; a
 * failed check returns a nonzero fa_status and has no side effect.  A failed
 * kernel launch returns FA_ERR_HIP.  Faults inside kernels are asynchronous
 * and surface at the caller's next synchronisation.  The contents of
 * cu_seqlens arrays live on the device and are trusted (they must be
 * non-decreasing, start at 0 and stay within the packed tensors).
 *
 * Debug checks.  When the environment variable FA_DEBUG is set to a value
 * other than "0" at the time of a call, the packed-sequence calls
 * (fa_fwd_varlen, fa_bwd_varlen) also check the cu_seqlens contents: they
 * synchronise `stream`, copy both arrays to the host and return
 * FA_ERR_SEQLENS, with nothing enqueued, unless each starts at 0, never
 * decreases, ends at its total (total_q, total_k) and has no step above its
 * max_seqlen.  This is the one case in which the library synchronises.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 2

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* a size is <= 0 or out of the supported range */
  FA_ERR_HEADDIM = 3,     /* d is not 64 or 128 */
  FA_ERR_DTYPE = 4,       /* unsupported dtype for this call */
  FA_ERR_GQA = 5,         /* Hq is not a multiple of Hkv */
  FA_ERR_ALIGN = 6,       /* a pointer or stride is not 16-byte aligned */
  FA_ERR_WORKSPACE = 7,   /* workspace missing or smaller than required */
  FA_ERR_ALIAS = 8,       /* an output overlaps an input or another output */
  FA_ERR_HIP = 9,         /* the HIP runtime reported an error at launch */
  FA_ERR_SCALE = 10,      /* softmax scale is not a finite number > 0 */
  FA_ERR_SEQLENS = 11     /* FA_DEBUG only: cu_seqlens contents are inconsistent */
} fa_status;

typedef enum { FA_BF16 = 0, FA_FP32 = 1, FA_FP8_E4M3 = 2 } fa_dtype;

/* A dense [B, S, H, d] tensor: base pointer and element strides of the B, S
 * and H dimensions (the d dimension has stride 1).  Strides must be
 * multiples of 8 elements for bf16 and of 16 for fp8 (16-byte rows). */
typedef struct {
  void* ptr;
  int64_t stride_b, stride_s, stride_h;
} fa_tensor;

/* Dense forward.  q [B,Sq,Hq,d], k and v [B,Sk,Hkv,d] in `dtype`; o
 * [B,Sq,Hq,d] fp32 for FA_FP32, else bf16; lse [B,Hq,Sq] fp32 contiguous
 * (required).  FA_FP32 computes everything in fp32 (no rounding of the
 * inputs or the probabilities); it is meant for checking, not speed.
 * FP8 only: q_descale [B,Hq,ceil(Sq/128)], k_descale and v_descale
 * [B,Hkv,ceil(Sk/128)], fp32 contiguous: the real value of an element is its
 * e4m3 value times the scale of its (batch, head, 128-token block).
 * softmax_scale must be finite and > 0 (1/sqrt(d) is the usual choice).
 *
 * Split-KV decode path (KV-cache inference: the repository overview's
 * flash_attn_with_kvcache entry point, here over a dense cache).  When the
 * M = Sq * (Hq / Hkv) query rows of one kv head fit one 32-wide tile (M <= 32,
 * e.g. one new token per sequence), or up to four such tiles that number
 * fewer than the group's query heads (ceil(M / 32) < Hq / Hkv, M <= 128),
 * fa_fwd_workspace_size returns a nonzero size; given a workspace of at least that many bytes (256-byte aligned, not
 * overlapping any tensor), fa_fwd cuts the keys into chunks that run in
 * parallel, each producing a partial (O_p, LSE_p), and merges them exactly:
 * LSE = ln sum_p exp(LSE_p), O = sum_p exp(LSE_p - LSE) O_p.  Without a
 * workspace the same call runs the tiled kernel (same result up to rounding
 * order, much slower for these shapes).  The workspace holds no state between
 * calls. */
typedef struct {
  fa_dtype dtype;
  int32_t B, Sq, Sk, Hq, Hkv, d;
  int32_t causal;
  float softmax_scale;
  fa_tensor q, k, v, o;
  float* lse;
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  void* workspace;
  size_t workspace_bytes;
} fa_fwd_args;

/* Packed variable-length forward (bf16).  Sequence z owns query rows
 * cu_seqlens_q[z] .. cu_seqlens_q[z+1]-1 of q [Tq,Hq,d] and key rows
 * cu_seqlens_k[z] .. cu_seqlens_k[z+1]-1 of k, v [Tk,Hkv,d]; it attends only
 * to its own keys (causal alignment per sequence).  cu_seqlens_* are int32
 * device arrays of nseq+1 entries; max_seqlen_q bounds every query length.
 * o [Tq,Hq,d] bf16; lse [Hq,Tq] fp32 contiguous; total_q = Tq. */
typedef struct {
  fa_dtype dtype;
  int32_t nseq, Hq, Hkv, d, max_seqlen_q, max_seqlen_k, total_q, total_k;
  int32_t causal;
  float softmax_scale;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_stride_t, q_stride_h, k_stride_t, k_stride_h;
  int64_t v_stride_t, v_stride_h, o_stride_t, o_stride_h;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  float* lse;
} fa_fwd_varlen_args;

/* Dense backward.  Inputs: q, k, v, the forward output o, its gradient dout
 * [B,Sq,Hq,d], and the forward's lse [B,Hq,Sq].  Outputs dq [B,Sq,Hq,d], dk
 * and dv [B,Sk,Hkv,d] (bf16; for GQA, dk/dv sum over the query heads of each
 * kv head).  workspace: at least fa_bwd_workspace_size bytes, 256-byte
 * aligned.  The result is bitwise reproducible run to run.
 *
 * dtype FA_BF16: q, k, v, o, dout bf16.
 * dtype FA_FP8_E4M3 (the FP8 forward's gradient; "FlashAttention-3: Fast
 * and Accurate Attention with Asynchrony and Low-precision", summary, third
 * contribution, carried to the backward): q, k, v are the E4M3 codes and
 * q_descale, k_descale, v_descale the per-block fp32 scales of fa_fwd's FP8
 * path (strides in bytes; the gradient is taken with respect to the
 * dequantised values); o and dout are bf16.  All five products run on the
 * FP8 matrix instruction: dO is rounded to E4M3 with one power-of-two scale
 * per (batch, head, 128-row block) (kept in the workspace, with D computed
 * from it), P to E4M3 after a 2^8 prescale, and dS to E4M3 with one
 * power-of-two scale per 32 elements along each product's reduction
 * dimension.  The workspace is then D, the dO codes [B,Hq,Sq,d] and their
 * scales.
 *
 * stages: 0 (or FA_BWD_ALL) runs the whole backward.  Otherwise a bitmask of
 * FA_BWD_PREPROCESS (D = rowsum(dO o O) into the workspace), FA_BWD_DKDV and
 * FA_BWD_DQ, run in that order; the last two read D from the workspace, so
 * running them without FA_BWD_PREPROCESS is meaningful only after a call that
 * ran it with the same inputs and workspace (otherwise the gradients are
 * garbage; nothing faults).  Lets a caller time or overlap the stages. */
#define FA_BWD_ALL 0
#define FA_BWD_PREPROCESS 1
#define FA_BWD_DKDV 2
#define FA_BWD_DQ 4
typedef struct {
  fa_dtype dtype;
  int32_t B, Sq, Sk, Hq, Hkv, d;
  int32_t causal;
  float softmax_scale;
  fa_tensor q, k, v, o, dout, dq, dk, dv;
  const float* lse;
  void* workspace;
  size_t workspace_bytes;
  int32_t stages;
  const float* q_descale;   /* FP8 only: [B,Hq,ceil(Sq/128)] */
  const float* k_descale;   /* FP8 only: [B,Hkv,ceil(Sk/128)] */
  const float* v_descale;   /* FP8 only: [B,Hkv,ceil(Sk/128)] */
} fa_bwd_args;

/* Packed variable-length backward (bf16), the gradient of fa_fwd_varlen.
 * Layouts are those of fa_fwd_varlen_args: q, o, dout and dq are [Tq,Hq,d],
 * k, v, dk and dv are [Tk,Hkv,d] (token and head strides in elements, d
 * contiguous), lse is the forward's [Hq,Tq] fp32 (contiguous), cu_seqlens_*
 * are int32 device arrays of nseq+1 entries, max_seqlen_* bound every
 * sequence length, total_q = Tq and total_k = Tk.  Sequence z's gradients
 * involve only its own rows (causal alignment per sequence); for GQA, dk and
 * dv sum over the query heads of each kv head.  workspace: at least
 * fa_bwd_varlen_workspace_size bytes, 256-byte aligned (D = rowsum(dO o O),
 * [Hq,Tq] fp32).  A pointer may be NULL exactly when its tensor has no
 * elements.  Bitwise reproducible run to run; each sequence's gradients are
 * bitwise those of fa_bwd on that sequence alone.  Same errors as fa_bwd. */
typedef struct {
  fa_dtype dtype;
  int32_t nseq, Hq, Hkv, d, max_seqlen_q, max_seqlen_k, total_q, total_k;
  int32_t causal;
  float softmax_scale;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  int64_t q_stride_t, q_stride_h, k_stride_t, k_stride_h, v_stride_t, v_stride_h;
  int64_t o_stride_t, o_stride_h, do_stride_t, do_stride_h;
  int64_t dq_stride_t, dq_stride_h, dk_stride_t, dk_stride_h, dv_stride_t, dv_stride_h;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const float* lse;
  void* workspace;
  size_t workspace_bytes;
} fa_bwd_varlen_args;

/* KV-cache attention (bf16): the repository overview's KV-cache entry point
 * (flash_attn_with_kvcache), with a cache that is appended to and may be
 * paged.  Layouts and rules are readings; the pages give none.
 *
 * Cache.  k_cache and v_cache are [num_pages, page_size, Hkv, d] with
 * element strides *_stride_page, *_stride_s and *_stride_h (d contiguous,
 * strides multiples of 8).  Token j of sequence b is slot j % page_size of
 * page block_table[b * block_table_stride + j / page_size]; page_size must be
 * a power of two of at least 16 and block_table an int32 device array with
 * max_pages_per_seq used columns per row.  With block_table NULL the cache is
 * dense: page b is all of sequence b's cache (num_pages >= B, page_size =
 * the capacity, any value >= 1).  cache_seqlens [B] int32 (device) counts
 * the tokens each sequence already has in the cache.
 *
 * Append.  When Snew > 0, k_new and v_new [B, Snew, Hkv, d] are written
 * first, at token positions cache_seqlens[b] .. cache_seqlens[b] + Snew - 1
 * of each sequence (the caller provides those pages in block_table).
 * cache_seqlens itself is not modified.
 *
 * Attention.  q [B, Sq, Hq, d] attends to the L_b = cache_seqlens[b] + Snew
 * tokens of its sequence, causal alignment bottom-right against L_b (query
 * row i sees key j iff j <= i + L_b - Sq); o [B, Sq, Hq, d] bf16, lse
 * [B, Hq, Sq] fp32 contiguous.  Sq may be 0 (append only).
 *
 * max_seqlen_k bounds every L_b (0: the capacity, max_pages_per_seq *
 * page_size, or page_size for a dense cache); it sizes the grid and the
 * split plan.  For the decode shapes of fa_fwd (Sq * (Hq / Hkv) <= 32, or up
 * to 128 in fewer 32-row tiles than Hq / Hkv), fa_fwd_kvcache_workspace_size
 * is nonzero and with that workspace (256-byte aligned) the keys are cut into
 * chunks that run in parallel and are merged exactly, as in fa_fwd's decode
 * path; otherwise (or without a workspace) the tiled forward kernels read
 * the cache pages directly (chunked prefill against a cache).
 *
 * Device contents are trusted: every L_b <= max_seqlen_k, and the block
 * table holds valid page indices for tokens 0 .. L_b - 1.  o and lse must
 * not overlap the inputs or the cache; k_new / v_new must not overlap the
 * cache.  Deterministic. */
typedef struct {
  fa_dtype dtype;
  int32_t B, Sq, Hq, Hkv, d, Snew;
  int32_t causal;
  float softmax_scale;
  fa_tensor q, o;
  float* lse;
  void* k_cache;
  void* v_cache;
  int64_t k_stride_page, k_stride_s, k_stride_h;
  int64_t v_stride_page, v_stride_s, v_stride_h;
  int32_t num_pages, page_size, max_pages_per_seq, max_seqlen_k;
  const int32_t* block_table;
  int64_t block_table_stride;
  const int32_t* cache_seqlens;
  fa_tensor k_new, v_new;
  void* workspace;
  size_t workspace_bytes;
} fa_fwd_kvcache_args;

/* MX FP8 forward: gfx950's native block scaling (OCP microscaling).  q, k
 * and v hold OCP E4M3 codes (fa_tensor strides in bytes, 16-byte rows); each
 * block of 32 consecutive elements along a product's reduction dimension
 * carries one E8M0 scale byte (real value 2^(byte - 127); 255 is not
 * allowed):
 *   q_scale [B, Sq, Hq, d/32] and k_scale [B, Sk, Hkv, d/32]: blocks along d;
 *   v_scale [B, Hkv, ceil(Sk/32), d]: blocks of 32 keys for each d column;
 * all uint8, contiguous, 4-byte aligned (fa_quantize_mxfp8 writes them).
 * Both products run on the scaled MFMA with these per-block scales; the
 * probabilities are rounded to E4M3 after a 2^8 prescale, as in fa_fwd's
 * FP8 path.  o [B,Sq,Hq,d] bf16, lse [B,Hq,Sq] fp32.  d is 64 or 128; the
 * other rules and errors are fa_fwd's. */
typedef struct {
  int32_t B, Sq, Sk, Hq, Hkv, d;
  int32_t causal;
  float softmax_scale;
  fa_tensor q, k, v, o;
  float* lse;
  const uint8_t* q_scale;
  const uint8_t* k_scale;
  const uint8_t* v_scale;
} fa_fwd_mxfp8_args;

/* Exact merge of partial attention results over disjoint key sets: the
 * per-shard step of sequence-parallel attention, where part p is the forward
 * of the same queries over shard p of the keys (e.g. fa_fwd on that shard).
 * o_parts [nparts, B, S, H, d] (dtype FA_BF16 or FA_FP32) and lse_parts
 * [nparts, B, H, S] fp32 are contiguous; o [B, S, H, d] bf16 (strides as
 * fa_tensor), lse [B, H, S] fp32 contiguous.  With M = max_p LSE_p and
 * w_p = exp(LSE_p - M): LSE = M + ln sum_p w_p, O = sum_p w_p O_p / sum_p w_p;
 * a part with LSE_p = -inf has weight 0 and a row where every part has
 * LSE_p = -inf gets O = 0, LSE = -inf.  d is 64 or 128; outputs must not
 * overlap the parts.  Deterministic (parts are summed in order). */
typedef struct {
  fa_dtype dtype;
  int32_t nparts, B, S, H, d;
  const void* o_parts;
  const float* lse_parts;
  fa_tensor o;
  float* lse;
} fa_merge_args;

/* Returns FA_ABI_VERSION. */
int32_t fa_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* fa_status_string(fa_status status);

/* Workspace bytes the split-KV decode path of fa_fwd uses for these
 * arguments; 0 when the decode path does not apply (then pass none). */
size_t fa_fwd_workspace_size(const fa_fwd_args* args);

/* Workspace bytes fa_bwd needs for these arguments. */
size_t fa_bwd_workspace_size(const fa_bwd_args* args);

/* Dense forward; see fa_fwd_args.  dtype FA_BF16, or FA_FP8_E4M3 (FP8
 * forward, "FlashAttention-3 ..." third contribution: both products run on
 * FP8 MFMA with fp32 accumulation; q/k/v are OCP E4M3 codes with strides in
 * bytes, the three descale arrays are required, the probabilities are
 * rounded to E4M3 after a 2^8 prescale; no decode path and no backward). */
fa_status fa_fwd(const fa_fwd_args* args, hipStream_t stream);

/* Packed variable-length forward; see fa_fwd_varlen_args. */
fa_status fa_fwd_varlen(const fa_fwd_varlen_args* args, hipStream_t stream);

/* Dense backward; see fa_bwd_args. */
fa_status fa_bwd(const fa_bwd_args* args, hipStream_t stream);

/* Dense backward that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid allocation).  Arguments, checks and
 * results are fa_bwd's (bitwise the same gradients), except that
 * args->workspace and args->workspace_bytes are ignored: the scratch fa_bwd
 * keeps there (fa_bwd_workspace_size bytes: D = rowsum(dO o O), 4 bytes per
 * query row and head, rounded up to 256 bytes; for FP8 also the dO codes and
 * scales) lives in a fixed array of FA_BWD_NOALLOC_MAX_SCRATCH bytes in the
 * library's device code, one per GPU, held until the process ends.  Calls
 * needing more (bf16: B * Hq * Sq > 8,388,608 query rows x heads) return
 * FA_ERR_WORKSPACE.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents: calls that overlap in time on one GPU
 * (several streams or host threads) race on it and must be serialised by
 * the caller, and a call whose stages skip FA_BWD_PREPROCESS uses the
 * scratch left by the previous call on that GPU.  The first call on a
 * device looks up the array's address there (FA_ERR_HIP if that fails). */
#define FA_BWD_NOALLOC_MAX_SCRATCH (32u << 20)
fa_status fa_bwd_noalloc(const fa_bwd_args* args, hipStream_t stream);

/* Workspace bytes fa_bwd_varlen needs for these arguments. */
size_t fa_bwd_varlen_workspace_size(const fa_bwd_varlen_args* args);

/* Packed variable-length backward; see fa_bwd_varlen_args. */
fa_status fa_bwd_varlen(const fa_bwd_varlen_args* args, hipStream_t stream);

/* Workspace bytes the split-KV path of fa_fwd_kvcache uses for these
 * arguments; 0 when it does not apply. */
size_t fa_fwd_kvcache_workspace_size(const fa_fwd_kvcache_args* args);

/* KV-cache attention with append; see fa_fwd_kvcache_args. */
fa_status fa_fwd_kvcache(const fa_fwd_kvcache_args* args, hipStream_t stream);

/* FP8 quantiser (input preparation for the FP8 forward; "FlashAttention-3:
 * Fast and Accurate Attention with Asynchrony and Low-precision", third
 * contribution and the block versus per-tensor error comparison).
 * d must be a multiple of 16 and at most 256; x 4-byte aligned, codes
 * 16-byte aligned; x, codes and scales must not overlap.
 * x [B,S,H,d] fp32 with element strides (d contiguous) -> codes [B,S,H,d]
 * e4m3 contiguous and scales [B,H,ceil(S/128)] fp32 contiguous.
 * per_tensor = 0: one scale per (batch, head, 128-token block),
 *   scale = amax/448 over the block (1 for an all-zero block);
 * per_tensor = 1: one scale amax/448 over the whole tensor, written to every
 *   entry of `scales` so the FP8 forward reads the same layout.
 * code = nearest e4m3 value of the fp32 quotient x/scale, ties to the even
 * code, saturating to +-448.  Deterministic. */
fa_status fa_quantize_fp8(const float* x, int64_t stride_b, int64_t stride_s,
                          int64_t stride_h, int32_t B, int32_t S, int32_t H,
                          int32_t d, int32_t per_tensor, void* codes,
                          float* scales, hipStream_t stream);

/* Merge of partial results over key shards; see fa_merge_args. */
fa_status fa_merge(const fa_merge_args* args, hipStream_t stream);

/* MX FP8 forward; see fa_fwd_mxfp8_args. */
fa_status fa_fwd_mxfp8(const fa_fwd_mxfp8_args* args, hipStream_t stream);

/* MX FP8 quantiser (input preparation for fa_fwd_mxfp8).  x [B,S,H,d] fp32
 * with element strides (d contiguous, 4-byte aligned) -> codes [B,S,H,d] e4m3
 * contiguous (16-byte aligned) and E8M0 scale bytes (4-byte aligned):
 *   axis 0: blocks of 32 along d (for q and k), scales [B,S,H,d/32];
 *   axis 1: blocks of 32 tokens along S for each (b, h, d column) (for v),
 *           scales [B,H,ceil(S/32),d]; the last block may be partial.
 * Per block, e is the smallest exponent with amax <= 448 * 2^e (so no
 * element saturates), clamped to [-127, 127], and 0 for an all-zero block;
 * the scale byte is e + 127 and the codes are the nearest e4m3 values of
 * x * 2^-e, ties to the even code.  d is a multiple of 32, at most
 * 256.  x, codes and scales must not overlap.  Deterministic. */
fa_status fa_quantize_mxfp8(const float* x, int64_t stride_b, int64_t stride_s,
                            int64_t stride_h, int32_t B, int32_t S, int32_t H,
                            int32_t d, int32_t axis, void* codes,
                            uint8_t* scales, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
