// Split-KV MLA decode over an fp8 e4m3 cache, up to 16 query rows (bf16 q).
//
// The cache holds e4m3 codes and a scale c per page (K = c * codes).  Pages
// stream HBM -> LDS as codes (36 KiB a page, by LDS-DMA, three pages ahead
// into four buffers named at compile time) and stay codes in LDS; operands
// are converted to bf16 when they are read (every e4m3 value is a bf16 value,
// so the conversion is exact).  The scale enters as S = c * (q . codes) and
// as the value operand c * P, the softmax denominator summing the unscaled P,
// so any finite scale is applied without rounding c * code.
//
// Waves: wave w = 2 kh + ch takes keys 32 kh .. +32 of every page (its own
// online softmax) and output columns 256 ch .. +256.  The two waves of a key
// half (siblings ch = 0, 1) each form one of its two 16-key score tiles, S^T
// for keys 32 kh + 16 ch .. +16, from 16x16x32 MFMAs over the 16 rows (Q
// fragments in registers, K operands from 16-byte LDS reads, each feeding two
// MFMAs: the contraction runs over the 576 columns in the order in which a
// lane's 16 codes arrive, and the Q fragments are loaded in that order), and
// swap tiles through LDS, so no score is formed twice and both run the same
// softmax over the 32 keys; P . V uses 16x16x32 MFMAs over the 32 keys, the V^T
// operand from one 8-bit transposed LDS read per 16 columns (within a 16-lane
// group, lane 2r + h addresses key row r, columns 8h .. 8h+7, and lane i
// receives column i of the eight rows).  The two key halves merge once per
// chunk through LDS.
//
// LDS image of a page: 64 rows of 576 bytes, 36 chunks of 16 bytes, chunk c of
// row r at slot c ^ rot(r), rot(r) = 2 * (bit 2 of r xor bit 4 of r) (which
// stays inside the row's aligned group of four chunks), so that the 16-byte
// score-operand reads of 16 rows and the transposed reads of 8 rows meet
// distinct bank groups.
#include "mla_fp8.hpp"

namespace mla {

// kQ8: the query rows are taken into fp8 too (load_q_codes8) and each score
// tile comes from five 16x16x128 fp8 MFMAs on the cached codes, with the
// operand layout of the 64-row fp8 kernel (the page images share it).
template <bool kQ8>
__global__ __launch_bounds__(kThreads, 1) void splitkv_fp8_kernel(DecodeParams p) {
  typedef __bf16 T;
  __shared__ __attribute__((aligned(1024))) char b0_raw[kPage8];
  __shared__ __attribute__((aligned(1024))) char b1_raw[kPage8];
  __shared__ __attribute__((aligned(1024))) char b2_raw[kPage8];
  __shared__ __attribute__((aligned(1024))) char b3_raw[kPage8];
  // page scale of each buffer, landed by LDS-DMA (each wave fills its own 64
  // floats; all read the first): one array per buffer, so that the compiler
  // can tell a read of one from the loads in flight into another
  __shared__ float sc0_raw[kWaves * 64];
  __shared__ float sc1_raw[kWaves * 64];
  __shared__ float sc2_raw[kWaves * 64];
  __shared__ float sc3_raw[kWaves * 64];
  __shared__ float ml_s[2][16][2];           // key half 1: (m, l) of each row, per column half
  __shared__ f32x4 sx_s[kWaves][64];         // each wave's 16-key score tile, for its sibling
  __shared__ MergeLds<16> merge_s;
  auto buf = [&](auto ic) -> MLA_LDS char* {
    constexpr int i = decltype(ic)::value & 3;
    if constexpr (i == 0) return (MLA_LDS char*)b0_raw;
    else if constexpr (i == 1) return (MLA_LDS char*)b1_raw;
    else if constexpr (i == 2) return (MLA_LDS char*)b2_raw;
    else return (MLA_LDS char*)b3_raw;
  };
  auto sbuf = [&](auto ic) -> MLA_LDS float* {
    constexpr int i = decltype(ic)::value & 3;
    if constexpr (i == 0) return (MLA_LDS float*)sc0_raw;
    else if constexpr (i == 1) return (MLA_LDS float*)sc1_raw;
    else if constexpr (i == 2) return (MLA_LDS float*)sc2_raw;
    else return (MLA_LDS float*)sc3_raw;
  };

  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int kh = wave >> 1, ch = wave & 1;
  const int row_bytes = (int)p.k_s1;          // fp8: elements are bytes
  const bool scaled = p.k_scale != nullptr;
  // per-lane read offsets within a page image
  const int krot = rot8(li);                  // K rows 32kh + 16kt + li: rot depends on li and kt
  const int vs = li >> 1, vh = li & 1;        // transposed reads: key slot row vs, column half vh
  const int vrow = 32 * kh + (vs < 4 ? 4 * g + vs : 12 + 4 * g + vs);
  const int vrot = rot8(vrow);
  // this lane's source offset within a page for each of the wave's DMA
  // instructions (instruction j = 9 w + i covers slots 64 j .. 64 j + 63 of
  // the image, lane l slot 64 j + l, i.e. row q / 36, slot q % 36, holding
  // source chunk slot ^ rot(row)): computed once, since the division by 36
  // and the 32-bit products cost ~100 cycles per instruction if rebuilt for
  // every page
  int doff[kDma8];
#pragma unroll
  for (int i = 0; i < kDma8; ++i) {
    const int q = (wave * kDma8 + i) * 64 + lane;
    const int r = q / 36;
    doff[i] = r * row_bytes + (((q - r * 36) ^ rot8(r)) << 4);
  }

  for_each_chunk(p, [&](const Chunk& c) {
    BlockWindow bw;
    bw.init(p.block_table + (int64_t)c.b * p.bt_s, c.lo, c.hi, lane);
    u32x4 qf[kQ8 ? 1 : 18];
    i32x8 qc[kQ8 ? kQ8Steps : 1];
    float qscale = 1.f;                       // 2^k of the row's fp8 codes
    if constexpr (kQ8) load_q_codes8(p, c.b, li, g, qc, qscale);
    else load_q_frag8(p, c.b, li, g, qf);
    const int cnt = li < p.rows ? visible_count(c.n, p.s_q, li / p.h_q, p.causal) : 0;
    const int npg = c.hi - c.lo;

    // LDS-DMA of page s of the chunk into buffer ic (offsets doff above).
    // Rows past the request's length are out of the descriptor's range and
    // land as zeros.  Every wave also lands the page's scale in its own slot.
    // Past the chunk the descriptors are empty, so every step issues the same
    // loads.
    auto issue = [&](auto ic, int s) {
      MLA_LDS char* bp = buf(ic);
      const bool real = s < npg;
      const int pg = c.lo + s;
      const int phys = real ? bw.phys(pg) : 0;
      const int valid = real ? min(kPage, c.n - pg * kPage) : 0;
      const BufRsrc pr = page_rsrc((const char*)p.k + (int64_t)phys * p.k_s0,
                                   valid > 0 ? (valid - 1) * row_bytes + kRow8 : 0);
#pragma unroll
      for (int i = 0; i < kDma8; ++i) dma16<kNarrowAux>(pr, bp + (wave * kDma8 + i) * 1024, doff[i], 0);
      const BufRsrc sr = page_rsrc((const char*)p.k_scale, scaled && real ? 0x7FFFFFFF : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (MLA_LDS void*)(sbuf(ic) + wave * 64), 4, 0, phys * 4, 0, 0);
    };

    float m_run = -INFINITY, l_part = 0.f;
    f32x4 o[16];
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
    issue(std::integral_constant<int, 2>{}, 2);

    auto step = [&](auto Hc, int s) {
      constexpr int H = decltype(Hc)::value;
      dma_barrier<2 * (kDma8 + 1)>();              // page s landed; all waves done with s - 1
      issue(std::integral_constant<int, H + 3>{}, s + 3);
      const MLA_LDS char* kb = buf(Hc);
      // The operand reads of a step are issued early and together: with one
      // wave per SIMD nothing else hides the LDS latency.  First the V
      // operands of the whole step (they do not depend on the scores), then
      // the K operands of this wave's score tile.
      const MLA_LDS char* vp = kb + vrow * kRow8 + vh * 8;
      u32x2 vw[16];
#pragma unroll
      for (int ct = 0; ct < 16; ++ct) vw[ct] = ld_lds_tr8(vp + (((16 * ch + ct) ^ vrot) << 4));
      // S^T of this wave's 16-key tile kt = ch (keys 32kh + 16ch + 4g .. +4 of row
      // li; rot8 of row 32kh + 16ch + li is krot ^ 2ch); the sibling wave (same
      // key half, other column half) forms the other tile, and the two swap
      // tiles through LDS
      const MLA_LDS char* rp = kb + (32 * kh + 16 * ch + li) * kRow8;
      const int rrot = krot ^ (2 * ch);
      f32x4 own = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kQ8) {
        // K operand of step m: chunks 8m + g and 8m + 4 + g of the key's row
        // (swizzled); the second half of step 4 lies past the row: zeros
        auto kop = [&](int m) {
          const u32x4 lo = ld_lds16(rp + (((8 * m + g) ^ rrot) << 4));
          const u32x4 hi = m < kQ8Steps - 1 ? ld_lds16(rp + (((8 * m + 4 + g) ^ rrot) << 4)) : u32x4{0, 0, 0, 0};
          return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        };
        i32x8 ka[kQ8Steps];
#pragma unroll
        for (int m = 0; m < kQ8Steps; ++m) ka[m] = kop(m);
#pragma unroll
        for (int m = 0; m < kQ8Steps; ++m)
          own = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka[m], qc[m], own, 0, 0, 0, 127, 0, 127);
      } else {
        u32x4 k0[9];
#pragma unroll
        for (int m = 0; m < 9; ++m) k0[m] = ld_lds16(rp + (((4 * m + g) ^ rrot) << 4));
#pragma unroll
        for (int m = 0; m < 9; ++m) {
          own = Dt<T>::mfma32(codes8_to_bf16(u32x2{k0[m][0], k0[m][1]}), qf[2 * m], own);
          own = Dt<T>::mfma32(codes8_to_bf16(u32x2{k0[m][2], k0[m][3]}), qf[2 * m + 1], own);
        }
      }
      const float ksc = scaled ? sbuf(Hc)[0] : 1.f;
      sx_s[wave][lane] = own;
      lds_barrier();
      const f32x4 sib = sx_s[wave ^ 1][lane];
      f32x4 sc[2];
      sc[0] = ch == 0 ? own : sib;
      sc[1] = ch == 0 ? sib : own;
      // online softmax of row li over this wave's 32 keys
      float x[8] = {sc[0][0], sc[0][1], sc[0][2], sc[0][3], sc[1][0], sc[1][1], sc[1][2], sc[1][3]};
      const int key0 = (c.lo + s) * kPage + 32 * kh + 4 * g;
      const float sl = p.scale_log2 * ksc * qscale;          // qscale: 2^k (exact), or 1
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = (key0 + (j >> 2) * 16 + (j & 3) < cnt) ? x[j] * sl : -INFINITY;
        mx = fmaxf(mx, x[j]);
      }
      mx = max_across_groups(mx);
      float alpha = 1.f;
      if (mx > m_run + kRescaleSlack) {
        alpha = __builtin_amdgcn_exp2f(m_run - mx);
        m_run = mx;
      }
      const float msub = (m_run == -INFINITY) ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = __builtin_amdgcn_exp2f(x[j] - msub);
        rs += x[j];
      }
      l_part = l_part * alpha + rs;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int ct = 0; ct < 16; ++ct) o[ct] *= alpha;
      }
      // P^T operand: k-slots 8g .. 8g+7 = keys 4g..4g+3 and 16+4g..16+4g+3
      const u32x4 pf = u32x4{Dt<T>::pack2(x[0] * ksc, x[1] * ksc), Dt<T>::pack2(x[2] * ksc, x[3] * ksc),
                             Dt<T>::pack2(x[4] * ksc, x[5] * ksc), Dt<T>::pack2(x[6] * ksc, x[7] * ksc)};
      // O^T += V^T . P^T over columns 256ch + 16ct .. +16
#pragma unroll
      for (int ct = 0; ct < 16; ++ct) o[ct] = Dt<T>::mfma32(codes8_to_bf16(vw[ct]), pf, o[ct]);
    };
    int s0 = 0;
    for (; s0 + 4 <= npg; s0 += 4) static_for<0, 4>([&](auto Hc) { step(Hc, s0 + decltype(Hc)::value); });
    static_for<0, 3>([&](auto Hc) {
      const int s = s0 + decltype(Hc)::value;
      if (s < npg) step(Hc, s);
    });
    dma_barrier<0>();                              // loads past the chunk drained, buffers free

    // merge of the two key halves: waves of key half 1 hand (m, l, O) over
    // through LDS (page buffers 0 and 1), the waves of key half 0 finish
    const float lw = sum_across_groups(l_part);
    float* xo = (float*)(ch == 0 ? b0_raw : b1_raw);       // [16 rows][256 + 4] floats
    constexpr int kXs = 260;
    if (kh == 1) {
#pragma unroll
      for (int ct = 0; ct < 16; ++ct) *(f32x4*)(xo + li * kXs + 16 * ct + 4 * g) = o[ct];
      if (g == 0) {
        ml_s[ch][li][0] = m_run;
        ml_s[ch][li][1] = lw;
      }
    }
    lds_barrier();
    if (kh == 0 && li < p.rows) {
      const float m1 = ml_s[ch][li][0], l1 = ml_s[ch][li][1];
      const float M = fmaxf(m_run, m1);
      const float f0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
      const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
      const float L = lw * f0 + l1 * f1;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      const float lse = lse_of(M, L);
      if (c.nsplit == 1) {
#pragma unroll
        for (int ct = 0; ct < 16; ++ct) {
          const f32x4 v = (o[ct] * f0 + *(const f32x4*)(xo + li * kXs + 16 * ct + 4 * g) * f1) * inv;
          store_out4<T>(p, c.b, li, 256 * ch + 16 * ct + 4 * g, v);
        }
        if (ch == 0 && g == 0) p.lse[(int64_t)c.b * p.rows + li] = lse;
      } else {
        const int64_t slot = c.slot0 + c.split;
        float* dst = p.part_o + (slot * p.rows + li) * kDV + 256 * ch + 4 * g;
#pragma unroll
        for (int ct = 0; ct < 16; ++ct)
          *(f32x4*)(dst + 16 * ct) = (o[ct] * f0 + *(const f32x4*)(xo + li * kXs + 16 * ct + 4 * g) * f1) * inv;
        if (ch == 0 && g == 0) p.part_lse[slot * p.rows + li] = lse;
      }
    }
    lds_barrier();                                 // merge buffers read before the next chunk's loads
    if (c.nsplit > 1 && c.nsplit <= p.fuse_max) fused_merge<T, 16, kThreads>(p, c, 0, merge_s);
  });
}

hipError_t launch_splitkv_fp8(const DecodeParams& p, hipStream_t st) {
  if (p.qk8) hipLaunchKernelGGL(splitkv_fp8_kernel<true>, dim3(p.num_parts, 1), dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(splitkv_fp8_kernel<false>, dim3(p.num_parts, 1), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
