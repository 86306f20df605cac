// Device-side vector types and small helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define FA_LDS __attribute__((address_space(3)))

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand layout (lane l, element e):
//   A[m][k]: m = l % 32, k = 8 * (l / 32) + e
//   B[k][n]: n = l % 32, k = 8 * (l / 32) + e
//   C[m][n]: n = l % 32, m = 8 * (i / 4) + 4 * (l / 32) + (i % 4) for reg i
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transposing read of 4 x 16-bit values.  Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte rows addressed by lanes
// 16 * (l / 16) + i / 4 + 4 * e, for e = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(p));
}

__device__ __forceinline__ bf16x8 cat_bf16(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float wave_xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// A wave-uniform pointer made explicitly scalar.  64-bit products of uniform
// values may be computed on the vector unit; a buffer resource built from
// such a value would make the compiler wrap every load in a waterfall loop.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Raw buffer resource over [base, base + bytes).  Loads past the end return
// zero and stores past the end are dropped (the bounds check covers the
// per-lane offset), which is how tile tails are handled without clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ void buf_store8(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

// 16 bytes per lane from a buffer straight into LDS: lane i of the wave
// writes bytes [16 i, 16 i + 16) after the wave-uniform LDS address `lds`
// (one 1 KB block per wave); lanes past the buffer end write zeros.  The data
// is in LDS once vmcnt has drained.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)lds, 16, off, 0, 0, 0);
}

// The same for data read exactly once (a KV cache streamed by the decode):
// the nontemporal policy (nt) keeps it from displacing reusable lines in
// the L2 and the last-level cache; a plain read-bandwidth test streams
// about 12% faster with it.
__device__ __forceinline__ void buf_load16_lds_stream(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)lds, 16, off, 0, 0, 2);
}

// s_waitcnt vmcnt(0): all outstanding vector-memory loads have returned.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Element index of (row, col) in a row-major LDS tile of bf16 rows of D
// elements (D = 64 or 128, no padding) whose 16-byte chunks are XOR-permuted
// per row.  The permutation keeps both access patterns of the kernels free of
// bank conflicts on the 64 four-byte LDS banks:
//   (1) 16 lanes each reading 16 bytes at one column of 16 consecutive rows
//       (MFMA operands taken row-wise);
//   (2) 32 lanes of the transposing read covering 4 consecutive rows, the
//       first a multiple of 4, x 64 contiguous bytes (operands taken
//       column-wise).
// For D = 128 a row spans all banks: chunk c of row r goes to c ^ f(r) with
// f(r) = 4 (r mod 4) + (r / 4 mod 4), distinct over 16 consecutive rows and
// moving each of 4 consecutive rows to its own group of 4 chunks.  For D = 64
// two rows share the banks (odd rows on the upper half) and
// f(r) = 4 (r / 2 mod 2) + (r / 4 mod 4) does the same within each half.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  static_assert(D == 64 || D == 128, "head dimension");
  const int f = D == 128 ? 4 * (row & 3) + ((row >> 2) & 3) : 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
  return row * D + ((((col >> 3) ^ f)) << 3) + (col & 7);
}

// Workgroup orders.  The hardware deals workgroup w of a dispatch to XCD
// w % 8, and each XCD has its own L2.
//
// Dense shapes: map dispatch index w of n to a logical tile index so that
// logical neighbours share an XCD (each XCD gets one contiguous range).
__device__ __forceinline__ int xcd_remap(int w, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = w & 7, s = w >> 3;
  return x * q + (x < r ? x : r) + s;
}

// Packed sequences: the work is `rows` rows of tiles (a row is one sequence
// and head, whose tiles read one operand stream).  Each XCD takes runs of
// `run` consecutive tiles of one row, so the workgroups resident on it read
// the same stream through its L2; the rows of a run group are dealt over the
// eight XCDs with a rotation that advances with the group, so that the
// heaviest rows do not all land on one XCD.  A contiguous range per XCD (as
// above) would hand whole long sequences to one XCD.  The grid holds
// varlen_grid(rows, ntiles, run) workgroups; returns false on its padding.
__host__ __device__ __forceinline__ long varlen_grid(int rows, int ntiles, int run) {
  return 8L * ((rows + 7) / 8) * run * ((ntiles + run - 1) / run);
}
__device__ __forceinline__ bool varlen_order(int w, int rows, int run, int& row, int& tile) {
  const int x = w & 7, n = w >> 3;
  const int r8 = (rows + 7) >> 3;
  const int k = n % run;
  const int rest = n / run;
  const int grp = rest / r8;
  row = (rest - grp * r8) * 8 + ((x + grp) & 7);
  tile = grp * run + k;
  return row < rows;
}

// Page and slot of token j of sequence b in a KV cache of pages: page
// block_table[b * bt_stride + (j >> page_shift)], slot j & (page size - 1);
// without a block table sequence b owns page b and the slot is j.
__device__ __forceinline__ void kv_page_slot(const int32_t* block_table, int64_t bt_stride,
                                             int page_shift, int b, int j, int64_t& page, int& slot) {
  page = b;
  slot = j;
  if (block_table) {
    page = block_table[(int64_t)b * bt_stride + (j >> page_shift)];
    slot = j & ((1 << page_shift) - 1);
  }
}

// Element offset page * page_stride + slot * token_stride of that token.
__device__ __forceinline__ int64_t kv_token_offset(const int32_t* block_table, int64_t bt_stride,
                                                   int page_shift, int b, int j,
                                                   int64_t page_stride, int64_t token_stride) {
  int64_t page;
  int slot;
  kv_page_slot(block_table, bt_stride, page_shift, b, j, page, slot);
  return page * page_stride + (int64_t)slot * token_stride;
}

// A window of up to 64 consecutive page numbers of one sequence's block-table
// row, one per lane of a wave: lane i holds the page of page number base + i
// (clamped to the sequence's last page, so no entry past it is read).  A
// refill is one vector load; lookups are a lane read (same page number across
// the wave) or a cross-lane permute (per-lane page numbers).
struct PageWindow {
  int base = -1;
  int pages = 0;
  // make page numbers first..last available (uniform; last - first < 64)
  __device__ __forceinline__ void cover(const int32_t* row, int first, int last, int max_page_no,
                                        int lane) {
    if (base < 0 || first < base || last >= base + 64) {
      base = first;
      pages = row[min(first + lane, max_page_no)];
      // Wait here, on this rare path: otherwise the compiler waits before
      // every later read of the window, for all loads then in flight (the
      // tile loads just issued included).
      wait_vmem();
    }
  }
  __device__ __forceinline__ int uniform(int page_no) const {
    return __builtin_amdgcn_readlane(pages, page_no - base);
  }
  // every lane of the wave must take part
  __device__ __forceinline__ int per_lane(int page_no) const {
    return __builtin_amdgcn_ds_bpermute((page_no - base) << 2, pages);
  }
};
