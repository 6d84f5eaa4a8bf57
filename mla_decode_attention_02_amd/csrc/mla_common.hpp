// Shared device-side definitions of the MLA decode kernels (gfx950 only).
//
// Notation: a cached row is 576 bf16/fp16 values (512 latent + 64 rope); V is
// its first 512 columns; a page holds 64 consecutive tokens of one request
// (page "FlashMLA: 高性能GPU注意力机制计算库 文件结构分析", section "项目主要功能").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mla {

constexpr int kDK = 576;
constexpr int kDV = 512;
constexpr int kPage = 64;
constexpr int kRowChunks = kDK * 2 / 16;          // 72 sixteen-byte chunks per row
constexpr int kPageBytes = kPage * kDK * 2;       // 73728 bytes per page
constexpr int kPageSlots = kPage * kRowChunks;    // 4608 chunks per page
constexpr int kThreads = 256;                     // 4 waves of 64
constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running maxima are only raised when a row's maximum grows by more than this
// (in log2 units); until then probabilities are at most 2^kRescaleSlack.
constexpr float kRescaleSlack = 8.0f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

// Kernel parameters (element strides; innermost dimension contiguous).
struct DecodeParams {
  const void* q;
  int64_t q_s0, q_s1, q_s2;
  const void* k;
  int64_t k_s0, k_s1;
  const int32_t* block_table;
  int64_t bt_s;
  const int32_t* seqlens;
  const int32_t* sched;          // null: every wave derives the schedule from seqlens
  const int32_t* split_offsets;  // null exactly when sched is
  int sched_f;                   // the scheduler's per-piece overhead F (pages)
  int batch, s_q, h_q, rows, num_parts, causal;
  float scale_log2;         // softmax_scale * log2(e)
  void* out;
  int64_t o_s0, o_s1, o_s2;
  float* lse;               // [batch * rows]
  float* part_o;            // [slots, rows, 512] fp32
  float* part_lse;          // [slots, rows]
  int kv_fp8;               // k_cache holds fp8 e4m3 codes (else the dtype of q)
  int qk8;                  // fp8 cache and fp8 query codes for the Q.K^T product
  const float* k_scale;     // fp8: per-page scale (K = code * scale), or null for 1
  int* counters;            // [m_blocks, batch] arrivals per row tile of a split request
  int* req_slots;           // [batch][2] first piece slot and piece count per request,
                            // written by the split-KV kernel when it derives the
                            // schedule itself, read by the combine
  int fuse_max;             // requests cut into 2 .. fuse_max pieces are merged in the
                            // split-KV kernel (0: never)
};

// Kernel parameters of paged multi-head / grouped-query decode (element
// strides).  The units of work are (request, KV head) pairs, unit u = b * h_kv
// + g; unit u has rows = s_q * group query rows (row r: token r / group, query
// head g * group + r % group).
struct MhaParams {
  const void* q;
  int64_t q_s0, q_s1, q_s2;
  const void* k;
  int64_t k_s0, k_s1, k_s2;  // page, slot, head
  const void* v;
  int64_t v_s0, v_s1, v_s2;
  const int32_t* block_table;
  int64_t bt_s;
  const int32_t* seqlens;
  const int32_t* sched;          // null: every wave derives the schedule from seqlens
  const int32_t* split_offsets;  // null exactly when sched is
  int sched_f;                   // the scheduler's per-piece overhead F (pages)
  int batch, s_q, h_q, h_kv, group, rows, num_parts, causal;
  float scale_log2;         // softmax_scale * log2(e)
  void* out;
  int64_t o_s0, o_s1, o_s2;
  float* lse;               // [batch, s_q, h_q]
  float* part_o;            // [slots, rows, d_v] fp32
  float* part_lse;          // [slots, rows]
  int kv_fp8;               // caches hold fp8 e4m3 codes (bf16 q)
  const float* k_scale;     // fp8: [num_pages, h_kv] scales of K (null: 1)
  const float* v_scale;     // fp8: [num_pages, h_kv] scales of V (null: 1)
};

// Arguments of the merge of context-parallel shards (strides in elements).
struct MergeParams {
  const void* part_out;     // shard r, request b, token, head: r*p_s0 + b*p_s1 + t*p_s2 + h*p_s3
  int64_t p_s0, p_s1, p_s2, p_s3;
  const float* part_lse;    // shard r: r*lse_s + b*rows + row
  int64_t lse_s;
  int num_shards, batch, s_q, h_q;
  void* out;
  int64_t o_s0, o_s1, o_s2;
  float* lse;               // [batch * rows]
};

// ---------------------------------------------------------------- dtypes --
template <typename T> struct Dt;

template <> struct Dt<__bf16> {
  __device__ static inline f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
  // two floats -> packed pair, round to nearest even
  __device__ static inline uint32_t pack2(float x, float y) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
  }
  // packed pair -> two floats (exact)
  __device__ static inline void unpack2(uint32_t u, float& x, float& y) {
    x = __uint_as_float(u << 16);
    y = __uint_as_float(u & 0xFFFF0000u);
  }
};

template <> struct Dt<_Float16> {
  __device__ static inline f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 v = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static inline void unpack2(uint32_t u, float& x, float& y) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 v = __builtin_bit_cast(f16x2, u);
    x = (float)v[0];
    y = (float)v[1];
  }
};

// --------------------------------------------------------------- helpers --
// LDS image of one page (73728 bytes):
//   value region  [64 rows][64 chunks of 16 B]  bytes      0 .. 65535  (columns 0..511)
//   rope region   [64 rows][ 8 chunks of 16 B]  bytes  65536 .. 73727  (columns 512..575)
// Chunks are XOR-swizzled within a row so that the reads of the kernels hit
// the 64 four-byte LDS banks without conflicts.  On gfx950 a 16-byte-per-lane
// LDS read is served 16 lanes per clock, in the lane sets {0-7, 24-31},
// {8-15, 16-23}, {32-39, 56-63} and {40-47, 48-55} (measured); a set is
// conflict-free when its 16 accesses fall into 16 distinct 16-byte bank
// groups (address bits 4..7).  The score reads of a 16-row tile put rows
// r and r+8 of lane groups g and g^1 into one set, so the value-region key is
// (row & 7) << 1: rows 0..7 land on even groups, and g^1 moves rows 8..15 to
// the odd ones.  The same key keeps the transposed value reads (4 rows x 2
// chunks per 16 lanes) at their full rate; the rope region uses a 3-bit key
// for its 128-byte rows.
constexpr int kRopeOff = 64 * 1024;

__device__ __forceinline__ int swz_v(int row) { return (row & 7) << 1; }
__device__ __forceinline__ int swz_r(int row) { return (row >> 1) & 7; }

// Byte offset of the 16-byte chunk holding columns 8c..8c+7 (c < 64) of `row`.
__device__ __forceinline__ int voff(int row, int c) { return row * 1024 + ((c ^ swz_v(row)) << 4); }
// Byte offset of rope chunk c (c < 8, columns 512 + 8c ..) of `row`.
__device__ __forceinline__ int roff(int row, int c) { return kRopeOff + row * 128 + ((c ^ swz_r(row)) << 4); }

// Score-operand chunk ks*4 + g of `row` (ks compile-time, 0 <= g < 4): the
// constant part of the swizzled offset is split off so that it folds into the
// instruction's immediate offset.
template <int KS>
__device__ __forceinline__ int kchunk_off(int row, int g) {
  if constexpr (KS < 16) {
    return row * 1024 + (KS >> 2) * 256 + ((((KS & 3) * 4 + g) ^ swz_v(row)) << 4);
  } else {
    return kRopeOff + row * 128 + ((((KS - 16) * 4 + g) ^ swz_r(row)) << 4);
  }
}

// Workgroup barrier that orders LDS reads and writes only: unlike
// __syncthreads() it does not wait for outstanding global loads (the next page
// in flight in registers).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wave index as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Uniform loads through the constant address space become scalar loads.
template <typename T>
__device__ __forceinline__ T ldu(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Maximum across lanes l, l^16, l^32, l^48 (one value per 16-lane row group).
__device__ __forceinline__ float max_across_groups(float x) {
  uint32_t u = __float_as_uint(x);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  u = __float_as_uint(x);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}

__device__ __forceinline__ float sum_across_groups(float x) {
  uint32_t u = __float_as_uint(x);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  u = __float_as_uint(x);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// One page in flight, staged in registers: 18 x 16 bytes per lane.
struct PageStage {
  u32x4 v[18];
};

typedef __amdgpu_buffer_rsrc_t BufRsrc;

// Buffer descriptor over one page: base address in scalar registers, loads
// then need only a 32-bit per-lane offset; reads past `bytes` return zero.
__device__ __forceinline__ BufRsrc page_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, 0x00020000);
}

// Cache policy of the page loads: 0 = default, 2 = non-temporal (the page is
// streamed through once; measured +16% sustained HBM bandwidth on this part).
template <int kAux>
__device__ __forceinline__ u32x4 buf_load16(BufRsrc r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kAux));
}

// Issue the loads of one 64x576 page (HBM -> registers).  Wave w fetches value
// rows 16w..16w+15 (one 1 KiB row per instruction, fully coalesced) and rope
// rows 16w..16w+15 (8 rows per instruction).  Lane l fetches the source chunk
// that belongs in LDS slot l of its row, i.e. chunk l ^ swizzle(row).  The row
// offset is part of the per-lane offset, which is what the descriptor's range
// check sees: rows past the descriptor's end read as zeros.
template <int kAux>
__device__ __forceinline__ void stage_load(PageStage& st, BufRsrc page, int row_bytes, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int key = (j & 7) << 1;                          // == swz_v(16 * wave + j)
    st.v[j] = buf_load16<kAux>(page, ((lane ^ key) << 4) + (wave * 16 + j) * row_bytes, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave * 2 + i) * 8 + (lane >> 3);
    const int voff = r * row_bytes + 1024 + (((lane & 7) ^ swz_r(r)) << 4);
    st.v[16 + i] = buf_load16<kAux>(page, voff, 0);
  }
}

// Physical page numbers of one request, fetched 64 at a time with a single
// vector load (lane i holds entry base + i) and read with v_readlane, so the
// page loop never waits on a scalar memory round trip (whose counter it would
// share with the LDS reads).  A refill costs one memory round trip per 64 pages.
struct BlockWindow {
  const int32_t* bt;
  int hi, base, cur, lane;
  __device__ __forceinline__ void init(const int32_t* bt_, int lo, int hi_, int lane_) {
    bt = bt_;
    hi = hi_;
    base = lo;
    lane = lane_;
    cur = lo + lane < hi ? bt[lo + lane] : 0;
    asm volatile("" : "+v"(cur));
  }
  __device__ __forceinline__ int phys(int pg) {
    if (pg >= base + 64) {
      base += 64;
      cur = base + lane < hi ? bt[base + lane] : 0;
      // consume the refill here, so the wait for it stays on this rare path and
      // is not merged into every step (where page loads are in flight)
      asm volatile("" : "+v"(cur));
    }
    return __builtin_amdgcn_readlane(cur, pg - base);
  }
};

// ------------------------------------------------------------ half pages --
// LDS image of half a page (32 consecutive tokens, 36864 bytes), filled by
// direct HBM -> LDS loads (LDS-DMA, no register staging):
//   value region  [32 rows][64 chunks of 16 B]  bytes      0 .. 32767
//   rope region   [32 rows][ 8 chunks of 16 B]  bytes  32768 .. 36863
// with the same in-row swizzles as the full-page image.  Once the score pass
// over a half page is done, its rope region is reused for the probabilities
// P[64 rows][32 keys], stored key-group major: the 16 bytes of keys 8c..8c+7
// of row r at 1024 c + 16 r, so that each 16-lane group of an operand read
// covers 256 contiguous bytes.
constexpr int kHalfRows = 32;
constexpr int kHalfBytes = kHalfRows * kDK * 2;     // 36864
constexpr int kHalfRopeOff = kHalfRows * 1024;      // 32768

// Score-operand chunk ks*4 + g of half-page row `row` (ks compile-time).
template <int KS>
__device__ __forceinline__ int hchunk_off(int row, int g) {
  if constexpr (KS < 16) {
    return row * 1024 + (KS >> 2) * 256 + ((((KS & 3) * 4 + g) ^ swz_v(row)) << 4);
  } else {
    return kHalfRopeOff + row * 128 + ((((KS - 16) * 4 + g) ^ swz_r(row)) << 4);
  }
}

// Byte offset of 16-byte chunk c (keys 8c .. 8c+7) of row `row` of the P tile.
__device__ __forceinline__ int pchunk_off(int row, int c) { return kHalfRopeOff + c * 1024 + row * 16; }

// One LDS-DMA instruction: every lane moves 16 bytes from the page at
// (voff + soff) to LDS address dst + 16 * lane.
template <int kAux>
__device__ __forceinline__ void dma16(BufRsrc page, MLA_LDS char* dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(page, (MLA_LDS void*)dst, 16, voff, soff, 0, kAux);
}

// Rope rows 8i .. 8i+7 of half page `half` (one instruction; lane l takes row
// 8i + l/8, slot l%8).  The row offset is in the per-lane offset, so the
// descriptor's range check covers it.
template <int kAux>
__device__ __forceinline__ void dma_rope_rows8(BufRsrc page, MLA_LDS char* hb, int half, int i, int row_bytes,
                                               int lane) {
  const int r = i * 8 + (lane >> 3);
  const int voff = (half * kHalfRows + r) * row_bytes + 1024 + (((lane & 7) ^ swz_r(r)) << 4);
  dma16<kAux>(page, hb + kHalfRopeOff + i * 1024, voff, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (its older LDS-DMA loads have landed), then a workgroup barrier that also
// orders LDS accesses.  The vmcnt wait is the builtin, so that the compiler's
// own wait placement knows which loads are still in flight after it.
template <int N>
__device__ __forceinline__ void dma_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  // s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4] (7 = no wait),
  // lgkmcnt [11:8] (15 = no wait)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Write a staged page into an LDS page buffer (contiguous 1 KiB per instruction).
__device__ __forceinline__ void stage_store(const PageStage& st, MLA_LDS char* buf, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 16; ++j) *(MLA_LDS u32x4*)(buf + (wave * 16 + j) * 1024 + lane * 16) = st.v[j];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    *(MLA_LDS u32x4*)(buf + kRopeOff + (wave * 2 + i) * 1024 + lane * 16) = st.v[16 + i];
}

// Compile-time unrolled loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Keys visible to query token `tok` of a request with n cached tokens.
__device__ __forceinline__ int visible_count(int n, int s_q, int tok, int causal) {
  if (!causal) return n;
  int c = n - s_q + tok + 1;
  return c < 0 ? 0 : (c > n ? n : c);
}

__device__ __forceinline__ u32x4 ld_lds16(const MLA_LDS char* p) {
  return *(const MLA_LDS u32x4*)p;
}

// Transposed LDS read: within each 16-lane group, lane i receives column i of
// the 4 x 16 block of 16-bit values whose row r, columns 4c..4c+3 are addressed
// by lane 4r + c.
__device__ __forceinline__ u32x2 ld_lds_tr(const MLA_LDS char* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

}  // namespace mla
