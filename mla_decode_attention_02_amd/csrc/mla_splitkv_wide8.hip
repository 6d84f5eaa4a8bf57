// Split-KV MLA decode over an fp8 e4m3 cache, wide tile (64 query rows per
// workgroup, bf16 q).
//
// The workgroup keeps the roles of the 16-bit wide kernel: 8 waves, two per
// SIMD; score waves 0..3 own query rows 16w .. +16, form S^T over the 32 keys
// of half page t, run the online softmax and hand P(t) and alpha(t) over
// through LDS; output waves 4..7 accumulate O^T += V^T . P^T over output
// columns 128c .. +128 of all 64 rows on half page t-1; one workgroup barrier
// per step; half page t+2 is loaded during step t into one of four buffers
// named at compile time.  What the fp8 cache changes:
//   * a half page is 32 rows of 576 codes, an 18 KiB image in the fp8 layout
//     (row r at 576 r, chunk c at slot c ^ rot8(r)); each score wave moves five
//     1 KiB pieces of it per step, and the last two of the twenty pieces land
//     zeros in the buffer's 2 KiB tail, so that every wave has the same number
//     of loads in flight;
//   * score operands: 16-byte reads of 16 codes of a key row, each converted
//     to two bf16 operands feeding two MFMAs (half the LDS bytes per MFMA of
//     the 16-bit kernel), with Q fragments loaded in the matching order;
//   * value operands: one 8-bit transposed read per 16 output columns,
//     converted to bf16;
//   * the page scale c (K = c * code) enters as S = c (q . codes) and as the
//     probabilities written for the output waves, c P, while the softmax
//     denominator sums P; each score wave lands the scale of every half page
//     in LDS with its pieces.
#include "mla_fp8.hpp"

namespace mla {

constexpr int kHalf8 = kHalfRows * kRow8;       // 18432 bytes of a half-page image
constexpr int kHalfSlots8 = kHalf8 / 16;        // 1152 sixteen-byte slots
constexpr int kDmaW8 = 5;                       // cache pieces per score wave and half page
constexpr int kHalfBuf8 = 4 * kDmaW8 * 1024;    // 20 KiB: the image and the tail of the padding pieces
static_assert(kHalfBuf8 >= kHalf8 && kHalfSlots8 <= 4 * kDmaW8 * 64, "half-page pieces");

// kQ8: the query rows are taken into fp8 too (load_q_codes8) and S^T = K.Q^T
// runs on the 16x16x128 fp8 MFMA straight from the cached codes in LDS (five
// steps of 128 columns, the last half zero); the probabilities and P.V are
// the same as without it.
template <bool kQ8>
__global__ __launch_bounds__(512, 1) void splitkv_wide_fp8_kernel(DecodeParams p) {
  typedef __bf16 T;
  __shared__ __attribute__((aligned(1024))) char hb0_raw[kHalfBuf8];
  __shared__ __attribute__((aligned(1024))) char hb1_raw[kHalfBuf8];
  __shared__ __attribute__((aligned(1024))) char hb2_raw[kHalfBuf8];
  __shared__ __attribute__((aligned(1024))) char hb3_raw[kHalfBuf8];
  // page scale of the half page in each buffer: each score wave lands its own
  // 64 copies and reads its own
  __shared__ float sc0_raw[4 * 64];
  __shared__ float sc1_raw[4 * 64];
  __shared__ float sc2_raw[4 * 64];
  __shared__ float sc3_raw[4 * 64];
  __shared__ __attribute__((aligned(1024))) char pb_raw[2][4096];   // c P(t), key-slot-group major
  __shared__ float alpha_s[2][64];
  __shared__ float l_s[64];
  __shared__ float m_s[64];
  __shared__ MergeLds<64> merge_s;
  auto hbuf = [&](auto ic) -> MLA_LDS char* {
    constexpr int i = decltype(ic)::value & 3;
    if constexpr (i == 0) return (MLA_LDS char*)hb0_raw;
    else if constexpr (i == 1) return (MLA_LDS char*)hb1_raw;
    else if constexpr (i == 2) return (MLA_LDS char*)hb2_raw;
    else return (MLA_LDS char*)hb3_raw;
  };
  auto sbuf = [&](auto ic) -> MLA_LDS float* {
    constexpr int i = decltype(ic)::value & 3;
    if constexpr (i == 0) return (MLA_LDS float*)sc0_raw;
    else if constexpr (i == 1) return (MLA_LDS float*)sc1_raw;
    else if constexpr (i == 2) return (MLA_LDS float*)sc2_raw;
    else return (MLA_LDS float*)sc3_raw;
  };
  auto pbuf = [&](auto ic) -> MLA_LDS char* {
    constexpr int i = decltype(ic)::value & 1;
    return (MLA_LDS char*)pb_raw[i];
  };
  // P.V runs over the 32 keys of a half page in a permuted order: k-slots
  // 8c .. 8c+7 hold keys 4c .. 4c+3 and 16+4c .. 16+4c+3, the eight scores one
  // lane of a score wave owns, so that lane writes them with one 16-byte store.
  auto poff = [](int row, int c) { return c * 1024 + row * 16; };

  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int mrow0 = blockIdx.y * 64;
  const int row_bytes = (int)p.k_s1;          // fp8: elements are bytes
  const bool scaled = p.k_scale != nullptr;

  auto half_pages = [&](const Chunk& c) {
    const int end = min(c.n, c.hi * kPage);
    return (end - c.lo * kPage + kHalfRows - 1) / kHalfRows;
  };

  if (wave < 4) {
    // -------------------------------------------------------- score waves --
    const int srow = wave * 16 + li;
    const int krot = rot8(li);                  // rows li and 16 + li: rot8(16 + li) = krot ^ 2
    // Source offset, within a half page, of the 16-byte slot this lane lands
    // with each of the wave's pieces: piece j = 5 wave + i covers image slots
    // 64 j .. 64 j + 63, slot q holding chunk (q % 36) ^ rot8(q / 36) of row
    // q / 36.  Pieces 18 and 19 (wave 3, i = 3, 4) lie past the image and
    // load through an empty descriptor.
    int doff[kDmaW8];
#pragma unroll
    for (int i = 0; i < kDmaW8; ++i) {
      const int q = (wave * kDmaW8 + i) * 64 + lane;
      const int r = q / 36;
      doff[i] = r * row_bytes + (((q - r * 36) ^ rot8(r)) << 4);
    }
    int doff2[kDmaW8];                          // the same for the second half of a page
#pragma unroll
    for (int i = 0; i < kDmaW8; ++i) doff2[i] = doff[i] + kHalfRows * row_bytes;
    const bool pad_wave = wave == 3;
    const BufRsrc none = page_rsrc((const char*)p.k, 0);
    // the page scales (no memory access without them)
    const BufRsrc scales = page_rsrc((const char*)p.k_scale, scaled ? 0x7FFFFFFF : 0);
    for_each_chunk(p, [&](const Chunk& c) {
      BlockWindow bw;
      bw.init(p.block_table + (int64_t)c.b * p.bt_s, c.lo, c.hi, lane);
      const int nh = half_pages(c);
      const int qrow = mrow0 + srow;
      u32x4 qf[kQ8 ? 1 : 18];
      i32x8 qc[kQ8 ? kQ8Steps : 1];
      float qscale = 1.f;                       // 2^k of the row's fp8 codes
      if constexpr (kQ8) load_q_codes8(p, c.b, qrow, g, qc, qscale);
      else load_q_frag8(p, c.b, qrow, g, qf);
      const int cnt = qrow < p.rows ? visible_count(c.n, p.s_q, qrow / p.h_q, p.causal) : 0;
      float m_run = -INFINITY;   // running max of row srow, log2 units
      float l_part = 0.f;        // this lane's share of its running sum

      // Sources of half page hh: the page's rows (past the end of the request
      // out of the descriptor's range, so they land as zeros) and the offset
      // of its scale.  Past the chunk the row descriptor is empty, which keeps
      // the count of loads in flight uniform.
      struct HalfSrc {
        BufRsrc rows;
        int scale_off;
      };
      auto half_src = [&](int hh) {
        const bool real = hh < nh;
        const int pg = c.lo + (hh >> 1);
        const int phys = real ? bw.phys(pg) : 0;
        const int valid = real ? page_valid_rows(c.n, pg) : 0;
        HalfSrc h;
        h.rows = page_rsrc((const char*)p.k + (int64_t)phys * p.k_s0, valid > 0 ? (valid - 1) * row_bytes + kRow8 : 0);
        h.scale_off = phys * 4;                 // page 0's scale past the chunk (never used)
        return h;
      };
      // load i of half page hh into buffer ic: pieces 0..4, then the scale
      auto load = [&](auto ic, int hh, const HalfSrc& h, auto i_c) {
        constexpr int i = decltype(i_c)::value;
        // With the fp8 score product the loads sit one per MFMA step; the
        // scheduling barriers keep the compiler from gathering them (the
        // offsets are loop-invariant), which measured 2-4 % faster there and
        // no faster with the bf16 score product.
        if constexpr (kQ8) __builtin_amdgcn_sched_barrier(0);
        if constexpr (i < kDmaW8) {
          const BufRsrc src = (i >= 3 && pad_wave) ? none : h.rows;
          const int off = kQ8 ? ((hh & 1) ? doff2[i] : doff[i]) : doff[i] + (hh & 1) * kHalfRows * row_bytes;
          dma16<kWideAux>(src, hbuf(ic) + (wave * kDmaW8 + i) * 1024, off, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(scales, (MLA_LDS void*)(sbuf(ic) + wave * 64), 4, 0,
                                                   h.scale_off, 0, 0);
        }
        if constexpr (kQ8) __builtin_amdgcn_sched_barrier(0);
      };
      {
        const HalfSrc h0 = half_src(0), h1 = half_src(1);
        static_for<0, kDmaW8 + 1>([&](auto i) { load(std::integral_constant<int, 0>{}, 0, h0, i); });
        static_for<0, kDmaW8 + 1>([&](auto i) { load(std::integral_constant<int, 1>{}, 1, h1, i); });
      }
      dma_barrier<kDmaW8 + 1>();                                           // X(-1)

      // step t < nh: S(t), softmax, c P(t) and alpha(t); loads of half page t+2
      auto step = [&](auto Hc, int t) {
        constexpr int H = decltype(Hc)::value;
        const MLA_LDS char* kb = hbuf(Hc);
        const HalfSrc hs = half_src(t + 2);
        // S^T for keys li (tile 0) and 16 + li (tile 1) x 16 rows
        const MLA_LDS char* rp0 = kb + li * kRow8;
        const MLA_LDS char* rp1 = rp0 + 16 * kRow8;
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kQ8) {
          // K operand of step m: chunks 8m + g and 8m + 4 + g of the key's row
          // (swizzled); the second half of step 4 lies past the row: zeros
          auto kop = [&](const MLA_LDS char* rp, int rot, int m) {
            const u32x4 lo = ld_lds16(rp + (((8 * m + g) ^ rot) << 4));
            const u32x4 hi = m < kQ8Steps - 1 ? ld_lds16(rp + (((8 * m + 4 + g) ^ rot) << 4)) : u32x4{0, 0, 0, 0};
            return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          };
          // both tiles' operands two steps ahead of their MFMAs (a ring of three)
          i32x8 ka[3], kb1[3];
          static_for<0, 2>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            ka[m] = kop(rp0, krot, m);
            kb1[m] = kop(rp1, krot ^ 2, m);
          });
          static_for<0, kQ8Steps>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            if constexpr (m + 2 < kQ8Steps) {
              ka[(m + 2) % 3] = kop(rp0, krot, m + 2);
              kb1[(m + 2) % 3] = kop(rp1, krot ^ 2, m + 2);
            }
            s0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka[m % 3], qc[m], s0, 0, 0, 0, 127, 0, 127);
            s1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kb1[m % 3], qc[m], s1, 0, 0, 0, 127, 0, 127);
            load(std::integral_constant<int, H + 2>{}, t + 2, hs, mc);            // pieces 0 .. 4
            if constexpr (m == 0) load(std::integral_constant<int, H + 2>{}, t + 2, hs,
                                       std::integral_constant<int, kDmaW8>{});    // the scale
          });
        } else {
          u32x4 k0[9], k1[9];
#pragma unroll
          for (int m = 0; m < 9; ++m) k0[m] = ld_lds16(rp0 + (((4 * m + g) ^ krot) << 4));
          static_for<0, 9>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            s0 = Dt<T>::mfma32(codes8_to_bf16(u32x2{k0[m][0], k0[m][1]}), qf[2 * m], s0);
            s0 = Dt<T>::mfma32(codes8_to_bf16(u32x2{k0[m][2], k0[m][3]}), qf[2 * m + 1], s0);
            k1[m] = ld_lds16(rp1 + (((4 * m + g) ^ krot ^ 2) << 4));
            if constexpr (m <= kDmaW8) load(std::integral_constant<int, H + 2>{}, t + 2, hs, mc);
          });
#pragma unroll
          for (int m = 0; m < 9; ++m) {
            s1 = Dt<T>::mfma32(codes8_to_bf16(u32x2{k1[m][0], k1[m][1]}), qf[2 * m], s1);
            s1 = Dt<T>::mfma32(codes8_to_bf16(u32x2{k1[m][2], k1[m][3]}), qf[2 * m + 1], s1);
          }
        }
        // online softmax of row srow over keys 4g+r (tile 0) and 16+4g+r (tile 1);
        // the scale multiplies before the maximum (it may be of either sign)
        const float ksc = scaled ? sbuf(Hc)[wave * 64] : 1.f;
        const float sl = p.scale_log2 * ksc * qscale;          // qscale: 2^k (exact), or 1
        float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        const int key0 = (2 * c.lo + t) * kHalfRows + 4 * g;
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
        MLA_LDS char* pb = pbuf(Hc);
        *(MLA_LDS u32x4*)(pb + poff(srow, g)) =
            u32x4{Dt<T>::pack2(x[0] * ksc, x[1] * ksc), Dt<T>::pack2(x[2] * ksc, x[3] * ksc),
                  Dt<T>::pack2(x[4] * ksc, x[5] * ksc), Dt<T>::pack2(x[6] * ksc, x[7] * ksc)};
        if (g == 0) alpha_s[H & 1][srow] = alpha;
        dma_barrier<kDmaW8 + 1>();                                         // X(t)
      };
      int t0 = 0;
      for (; t0 + 4 <= nh; t0 += 4) static_for<0, 4>([&](auto Hc) { step(Hc, t0 + decltype(Hc)::value); });
      static_for<0, 3>([&](auto Hc) {
        const int t = t0 + decltype(Hc)::value;
        if (t < nh) step(Hc, t);
      });
      {
        const float lw = sum_across_groups(l_part);
        if (g == 0) {
          l_s[srow] = lw;
          m_s[srow] = m_run;
        }
      }
      lds_barrier();                                                        // X(nh)
      if (c.nsplit > 1 && c.nsplit <= p.fuse_max) fused_merge<T, 64, 512>(p, c, mrow0, merge_s);
    });
  } else {
    // ------------------------------------------------------- output waves --
    const int cw = wave - 4;                                  // columns cw*128 .. +128
    for_each_chunk(p, [&](const Chunk& c) {
      const int nh = half_pages(c);
      f32x4 o[8][4];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) o[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      lds_barrier();                                                        // X(-1)

      // step t >= 1: O *= alpha(t-1); O^T += V^T . (c P)^T over half page t-1
      auto step = [&](auto Hc, int t) {
        constexpr int H = decltype(Hc)::value;
        const MLA_LDS char* prv = hbuf(std::integral_constant<int, H + 3>{});   // half page t-1
        MLA_LDS char* pb = pbuf(std::integral_constant<int, H + 1>{});          // c P(t-1)
        int ln = lane;                 // opaque: read offsets are rebuilt, not kept live
        asm volatile("" : "+v"(ln));
        const int lg = ln >> 4, ll = ln & 15;
        // transposed reads: within a 16-lane group, lane 2s + h addresses key
        // slot s (slots 0..3 = keys 4lg .. +3, slots 4..7 = keys 16+4lg .. +3),
        // columns 8h .. 8h+7 of a 16-column chunk; lane ll receives column ll
        const int vs = ll >> 1, vh = ll & 1;
        const int vrow = vs < 4 ? 4 * lg + vs : 12 + 4 * lg + vs;
        const MLA_LDS char* vp = prv + vrow * kRow8 + vh * 8;
        const int vrot = rot8(vrow);
        auto load_v = [&](int ct) { return ld_lds_tr8(vp + (((8 * cw + ct) ^ vrot) << 4)); };
        float a4[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) a4[rt] = alpha_s[(H + 1) & 1][rt * 16 + ll];
        u32x4 pf[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) pf[rt] = ld_lds16(pb + poff(rt * 16 + ll, lg));
        u32x2 vw[8];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) vw[ct] = load_v(ct);
        const bool resc = (a4[0] != 1.f) | (a4[1] != 1.f) | (a4[2] != 1.f) | (a4[3] != 1.f);
        if (__any(resc)) {
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) o[ct][rt] *= a4[rt];
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          if (ct + 4 < 8) vw[ct + 4] = load_v(ct + 4);
          const u32x4 vf = codes8_to_bf16(vw[ct]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) o[ct][rt] = Dt<T>::mfma32(vf, pf[rt], o[ct][rt]);
        }
      };
      auto stepx = [&](auto Hc, int t) {
        if (t >= 1) step(Hc, t);
        lds_barrier();                                                      // X(t)
      };
      int t0 = 0;
      for (; t0 + 4 <= nh + 1; t0 += 4) static_for<0, 4>([&](auto Hc) { stepx(Hc, t0 + decltype(Hc)::value); });
      static_for<0, 3>([&](auto Hc) {
        const int t = t0 + decltype(Hc)::value;
        if (t <= nh) stepx(Hc, t);
      });
      // epilogue: normalise, write the final output or an fp32 partial
      int eln = lane;
      asm volatile("" : "+v"(eln));
      const int eli = eln & 15, eg = eln >> 4;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int rl = rt * 16 + eli;
        const int row = mrow0 + rl;
        if (row >= p.rows) continue;
        const float l = l_s[rl];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float lse = lse_of(m_s[rl], l);
        if (c.nsplit == 1) {
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
            store_out4<T>(p, c.b, row, cw * 128 + ct * 16 + 4 * eg, o[ct][rt] * inv);
          if (cw == 0 && eg == 0) p.lse[(int64_t)c.b * p.rows + row] = lse;
        } else {
          const int64_t slot = c.slot0 + c.split;
          float* dst = p.part_o + (slot * p.rows + row) * kDV + cw * 128 + 4 * eg;
#pragma unroll
          for (int ct = 0; ct < 8; ++ct) *(f32x4*)(dst + ct * 16) = o[ct][rt] * inv;
          if (cw == 0 && eg == 0) p.part_lse[slot * p.rows + row] = lse;
        }
      }
      if (c.nsplit > 1 && c.nsplit <= p.fuse_max) fused_merge<T, 64, 512>(p, c, mrow0, merge_s);
    });
  }
}

hipError_t launch_splitkv_wide_fp8(const DecodeParams& p, int m_blocks, hipStream_t st) {
  if (p.qk8) hipLaunchKernelGGL(splitkv_wide_fp8_kernel<true>, dim3(p.num_parts, m_blocks), dim3(512), 0, st, p);
  else hipLaunchKernelGGL(splitkv_wide_fp8_kernel<false>, dim3(p.num_parts, m_blocks), dim3(512), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
