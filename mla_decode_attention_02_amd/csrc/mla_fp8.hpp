// Pieces shared by the split-KV kernels over an fp8 e4m3 cache (gfx950).
//
// The cache holds e4m3 codes and one fp32 scale per page (K = scale * code).
// Pages stay codes in LDS and operands are converted to bf16 as they are read:
// every e4m3 value is a bf16 value, so the conversion is exact (pages
// "DeepSeek开源FlashMLA全解析：性能革命背后的技术密码", section "1.2 计算模式创新：
// 混合精度矩阵乘法", and "云上AI推理新突破：FlashMLA赋能DeepSeek-V2-Lite提速16%",
// section "3. 动态精度缩放", for fp8 keys with a scale and 16-bit softmax and
// value products).
//
// LDS image of cached rows: row r at r * 576 bytes, 36 chunks of 16 bytes,
// chunk c of row r at slot c ^ rot8(r), rot8(r) = 2 * (bit 2 of r xor bit 4
// of r) (which stays inside the row's aligned group of four chunks), so that
// the 16-byte score-operand reads of 16 rows and the transposed reads of 8
// rows meet distinct bank groups.
#pragma once

#include "mla_splitkv.hpp"

namespace mla {

constexpr int kRow8 = kDK;                   // bytes of a cached row of codes
constexpr int kPage8 = kPage * kRow8;        // 36864 bytes of a page image
constexpr int kSlots8 = kPage8 / 16;         // 2304 sixteen-byte slots
constexpr int kDma8 = kPage8 / 1024 / 4;     // LDS-DMA instructions per wave and page (9)

__device__ __forceinline__ int rot8(int r) { return ((r >> 1) ^ (r >> 3)) & 2; }

// Eight e4m3 codes (one 8-byte word) -> eight bf16 values.
__device__ __forceinline__ u32x4 codes8_to_bf16(u32x2 w) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

// Q fragments in the contraction order of the 16-byte K reads: fragment 2m
// holds columns 64m + 16g .. +8 and fragment 2m + 1 columns 64m + 16g + 8 .. +8.
__device__ __forceinline__ void load_q_frag8(const DecodeParams& p, int b, int row, int g, u32x4 (&qf)[18]) {
  if (row < p.rows) {
    const int tok = row / p.h_q;
    const int head = row - tok * p.h_q;
    const __bf16* base = (const __bf16*)p.q + b * p.q_s0 + tok * p.q_s1 + head * p.q_s2 + 16 * g;
#pragma unroll
    for (int m = 0; m < 9; ++m) {
      qf[2 * m] = *(const u32x4*)(base + 64 * m);
      qf[2 * m + 1] = *(const u32x4*)(base + 64 * m + 8);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 18; ++k) qf[k] = u32x4{0, 0, 0, 0};
  }
}

// ---------------------------------------------------- fp8 query codes --
// Q taken into fp8 for an fp8 query-key product (page "DeepSeek开源FlashMLA全解析：
// 性能革命背后的技术密码", section "1.2 计算模式创新：混合精度矩阵乘法", and page
// "云上AI推理新突破：FlashMLA赋能DeepSeek-V2-Lite提速16%", section "3. 动态精度缩放":
// q and k in fp8 for Q.K^T, the softmax and P.V in 16 bits).  Each query row
// has its own power-of-two scale 2^k, the smallest with max|q| * 2^-k <= 448
// (the largest e4m3 value; k = 0 for a row of zeros), so the scaling is exact
// and the e4m3 rounding (to nearest, ties to even) the only one.
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Operand layout of the 16x16x128 fp8 MFMA as used here: within a lane group
// g (lanes 16g .. 16g+15, one row each), step m covers the 16-column chunks
// 8m + g (bytes 0..15 of the lane's eight registers) and 8m + 4 + g (bytes
// 16..31); the same for the Q and K operands (the unit pairs byte j of a lane
// group in both, whatever columns it stands for).  So each of a step's two
// 16-byte K reads takes four consecutive chunks across the lane groups, the
// order of the 16-bit score reads.  Step 4 holds chunks 32 .. 35 (columns
// 512 .. 575) in its first half and zeros in its second.
constexpr int kQ8Steps = 5;
// first column of half h (0, 1) of step m for lane group g
__device__ __forceinline__ int q8_col(int m, int h, int g) { return 128 * m + 64 * h + 16 * g; }

__device__ __forceinline__ int q8_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  (void)frexpf(amax, &e);                    // amax = f * 2^e, f in [0.5, 1)
  int k = e - 9;                             // amax * 2^-k in [256, 512)
  if (ldexpf(amax, -k) > 448.f) ++k;
  return k;
}

// Codes of query row `row` for lane group g (zeros past the rows), and the
// row's scale 2^k.  Two passes over the row (the maximum, then the codes):
// holding the whole row's raw values between them would cost 80 registers.
__device__ __forceinline__ void load_q_codes8(const DecodeParams& p, int b, int row, int g, i32x8 (&qc)[kQ8Steps],
                                              float& qscale) {
  const bool live = row < p.rows;
  const int tok = live ? row / p.h_q : 0;
  const int head = live ? row - tok * p.h_q : 0;
  const __bf16* base = (const __bf16*)p.q + b * p.q_s0 + tok * p.q_s1 + head * p.q_s2;
  // eight columns: h = 0, 1 the first half of step m, h = 2, 3 the second
  auto raw = [&](int m, int h) {
    const bool in = live && (m < kQ8Steps - 1 || h < 2);
    return in ? *(const u32x4*)(base + q8_col(m, h >> 1, g) + 8 * (h & 1)) : u32x4{0, 0, 0, 0};
  };
  auto val = [](uint32_t w, int hi) { return __uint_as_float(hi ? (w & 0xFFFF0000u) : (w << 16)); };
  float amax = 0.f;
#pragma unroll
  for (int m = 0; m < kQ8Steps; ++m)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 w = raw(m, h);
#pragma unroll
      for (int d = 0; d < 4; ++d) amax = fmaxf(amax, fmaxf(fabsf(val(w[d], 0)), fabsf(val(w[d], 1))));
    }
  amax = max_across_groups(amax);            // the four lane groups of the row
  const int k = q8_exponent(amax);
  qscale = ldexpf(1.f, k);
#pragma unroll
  for (int m = 0; m < kQ8Steps; ++m)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 w = raw(m, h);
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2) {
        // dword 2h + d2 of the operand: four columns of raw(m, h)
        const uint32_t w0 = w[2 * d2], w1 = w[2 * d2 + 1];
        int c = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(val(w0, 0), -k), ldexpf(val(w0, 1), -k), 0, false);
        c = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(val(w1, 0), -k), ldexpf(val(w1, 1), -k), c, true);
        qc[m][2 * h + d2] = c;
      }
    }
}

__device__ __forceinline__ u32x2 ld_lds_tr8(const MLA_LDS char* p) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS v2i*)p);
  return __builtin_bit_cast(u32x2, v);
}

}  // namespace mla
