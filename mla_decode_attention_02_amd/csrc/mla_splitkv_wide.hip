// Split-KV MLA decode attention, wide tile (64 query rows per workgroup).
// Built with MFMA accumulators in AGPR form (the default).
#include "mla_splitkv.hpp"

namespace mla {

// ------------------------------------------------------------------ wide --
// 64 query rows per workgroup, 8 waves (two per SIMD) in two roles, so that on
// every SIMD the MFMAs of one role overlap the softmax arithmetic and LDS
// traffic of the other (the MI355X counterpart of the seesaw schedule's two
// alternating warpgroups).  Keys are processed in half pages of 32; step t
// scores half page t and accumulates half page t-1.
//   * score waves 0..3, (rg, kg) = (w >> 1, w & 1): raw scores S^T for query
//     rows rg*32 .. +32 (two 16-row tiles, Q fragments in registers) and keys
//     kg*16 .. +16 of half page t; each K fragment read from LDS feeds two
//     MFMAs.  The scores go to one of two fp32 tiles in LDS.  These waves also
//     issue all the HBM -> LDS loads, spread over their MFMA stream.
//   * output waves 4..7, (rh, ch) = (c >> 1, c & 1): O^T for rows rh*32 .. +32
//     and columns ch*256 .. +256 (128 fp32 registers per lane).  Each runs the
//     online softmax of its 32 rows itself (the two waves of a row half do the
//     same arithmetic), so the probabilities go straight from its registers
//     into the MFMA operand and no wave waits for another's P.
// One workgroup barrier per step (scores of t written, loads of t+1 landed).
// Half pages stream HBM -> LDS by direct (LDS-DMA) loads into four buffers
// named at compile time (the step loop is unrolled by four, so the compiler
// can tell the LDS reads of one buffer from the loads in flight into
// another); the loads of half page t+2 are issued during step t.
template <typename T>
__global__ __launch_bounds__(512, 1) void splitkv_wide_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char hb0_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char hb1_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char hb2_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char hb3_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char s_raw[2][64 * 32 * 4];   // S(t), fp32 [row][32 keys]
  static_assert(4 * kHalfBytes + 2 * 64 * 32 * 4 <= 163840, "LDS budget of one workgroup");
  auto hbuf = [&](auto ic) -> MLA_LDS char* {
    constexpr int i = decltype(ic)::value & 3;
    if constexpr (i == 0) return (MLA_LDS char*)hb0_raw;
    else if constexpr (i == 1) return (MLA_LDS char*)hb1_raw;
    else if constexpr (i == 2) return (MLA_LDS char*)hb2_raw;
    else return (MLA_LDS char*)hb3_raw;
  };
  auto stile = [&](auto ic) -> MLA_LDS char* {
    constexpr int i = decltype(ic)::value & 1;
    return (MLA_LDS char*)s_raw[i];
  };
  // 16-byte chunk c (keys 4c .. 4c+3) of row `row` of a score tile
  auto schunk = [](int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); };

  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int mrow0 = blockIdx.y * 64;
  const int row_bytes = (int)(p.k_s1 * 2);
  const int page_bytes = (kPage - 1) * row_bytes + kDK * 2;

  // Half pages of a chunk: its pages, less a last half that lies wholly past
  // the end of the request.
  auto half_pages = [&](const Chunk& c) {
    const int end = min(c.n, c.hi * kPage);
    return (end - c.lo * kPage + kHalfRows - 1) / kHalfRows;
  };

  // The role test is the outermost branch: each role walks the partition's
  // chunks in its own loop, so the loop invariants of one role are not kept
  // alive in the other.  Both loops meet at the same barriers.
  if (wave < 4) {
    // -------------------------------------------------------- score waves --
    const int rg = wave >> 1, kg = wave & 1;
    const int krow = kg * 16 + li;                            // K row read by this lane
    for_each_chunk(p, [&](const Chunk& c) {
      BlockWindow bw;
      bw.init(p.block_table + (int64_t)c.b * p.bt_s, c.lo, c.hi, lane);
      const int nh = half_pages(c);
      u32x4 qf[2][18];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) load_q_frag<T>(p, c.b, mrow0 + rg * 32 + rt * 16 + li, g, qf[rt]);
      // Loads of half page hh: this wave moves value rows 8w .. 8w+7 (piece
      // i < 8) and rope rows 8w .. 8w+7 (piece 8).  Past the end of the chunk
      // an empty descriptor keeps the count of loads in flight uniform
      // (every lane out of range, no memory access).
      auto page_desc = [&](int hh) {
        const bool real = hh < nh;
        return page_of(p, real ? bw.phys(c.lo + (hh >> 1)) : 0, real ? page_bytes : 0);
      };
      auto piece = [&](auto ic, int hh, BufRsrc pg, int i) {
        MLA_LDS char* hb = hbuf(ic);
        const int half = hh & 1;
        int ln = lane;                 // opaque: offsets are rebuilt, not kept live
        asm volatile("" : "+v"(ln));
        if (i < 8) {
          const int r = 8 * wave + i;
          dma16<kWideAux>(pg, hb + r * 1024, (ln ^ swz_v(r)) << 4, (half * kHalfRows + r) * row_bytes);
        } else {
          dma_rope_rows8<kWideAux>(pg, hb, half, wave, row_bytes, ln);
        }
      };
      {
        const BufRsrc pg0 = page_desc(0), pg1 = page_desc(1);
#pragma unroll
        for (int i = 0; i < 9; ++i) piece(std::integral_constant<int, 0>{}, 0, pg0, i);
#pragma unroll
        for (int i = 0; i < 9; ++i) piece(std::integral_constant<int, 1>{}, 1, pg1, i);
      }
      dma_barrier<9>();                                                     // X(-1)

      // step t < nh: S(t) into score tile t&1; loads of half page t+2
      auto step = [&](auto Hc, int t) {
        constexpr int H = decltype(Hc)::value;
        MLA_LDS char* cur = hbuf(Hc);
        const BufRsrc pg = page_desc(t + 2);
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        // S^T over the 576-deep contraction; K reads run kAhead steps ahead
        constexpr int kAhead = 6;
        u32x4 kf[kAhead + 1];
        static_for<0, kAhead>([&](auto kc) {
          constexpr int ks = decltype(kc)::value;
          kf[ks] = ld_lds16(cur + hchunk_off<ks>(krow, g));
        });
        static_for<0, 18>([&](auto ksc) {
          constexpr int ks = decltype(ksc)::value;
          if constexpr (ks + kAhead < 18) kf[(ks + kAhead) % (kAhead + 1)] = ld_lds16(cur + hchunk_off<ks + kAhead>(krow, g));
          if constexpr (ks % 2 == 0) piece(std::integral_constant<int, H + 2>{}, t + 2, pg, ks / 2);
          s0 = Dt<T>::mfma32(kf[ks % (kAhead + 1)], qf[0][ks], s0);
          s1 = Dt<T>::mfma32(kf[ks % (kAhead + 1)], qf[1][ks], s1);
        });
        MLA_LDS char* st = stile(Hc);
        const int row0 = rg * 32 + li;
        *(MLA_LDS f32x4*)(st + schunk(row0, kg * 4 + g)) = s0;
        *(MLA_LDS f32x4*)(st + schunk(row0 + 16, kg * 4 + g)) = s1;
        dma_barrier<9>();                                                   // X(t)
      };
      // whole groups of four steps, then the tail: every step of the loop body
      // runs, so the compiler sees which buffer each load in flight targets
      int t0 = 0;
      for (; t0 + 4 <= nh; t0 += 4) static_for<0, 4>([&](auto Hc) { step(Hc, t0 + decltype(Hc)::value); });
      static_for<0, 3>([&](auto Hc) {
        const int t = t0 + decltype(Hc)::value;
        if (t < nh) step(Hc, t);
      });
      lds_barrier();                                                        // X(nh)
    });
  } else {
    // ------------------------------------------------------- output waves --
    const int cw = wave - 4;
    const int rh = cw >> 1, ch = cw & 1;      // rows rh*32 .. +32, columns ch*256 .. +256
    for_each_chunk(p, [&](const Chunk& c) {
      const int nh = half_pages(c);
      int cnt[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int qrow = mrow0 + rh * 32 + rt * 16 + li;
        cnt[rt] = qrow < p.rows ? visible_count(c.n, p.s_q, qrow / p.h_q, p.causal) : 0;
      }
      float m_run[2] = {-INFINITY, -INFINITY};   // running max per row, log2 units
      float l_part[2] = {0.f, 0.f};              // this lane's share of the running sums
      f32x4 o[16][2];
#pragma unroll
      for (int ct = 0; ct < 16; ++ct)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) o[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      lds_barrier();                                                        // X(-1)

      // step t >= 1: softmax of half page t-1 for this wave's 32 rows, then
      // O^T += V^T . P^T over it
      auto step = [&](auto Hc, int t) {
        constexpr int H = decltype(Hc)::value;
        MLA_LDS char* st = stile(std::integral_constant<int, H + 1>{});   // S(t-1)
        MLA_LDS char* prv = hbuf(std::integral_constant<int, H + 3>{});   // half page t-1
        // Lane-dependent read addresses are rebuilt here from an opaque copy of
        // the lane index: cheaper than keeping them alive across the loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lg = ln >> 4, ll = ln & 15;
        const int vrow = 8 * lg + (ll >> 2);                  // value row (lo) of the transposed reads
        const int vbase = vrow * 1024 + ch * 512 + (ll & 1) * 8;
        const int vkey = swz_v(vrow);                         // vrow + 4 uses vkey ^ 8
        const int vh = (ll >> 1) & 1;
        auto load_v = [&](int ct) {
          const int x = ((2 * ct + vh) ^ vkey) << 4;
          const u32x2 lo4 = ld_lds_tr(prv + vbase + x);
          const u32x2 hi4 = ld_lds_tr(prv + vbase + 4096 + (x ^ 128));
          return u32x4{lo4[0], lo4[1], hi4[0], hi4[1]};
        };
        // scores of rows rh*32 + rt*16 + ll, keys 8lg .. 8lg+7
        f32x4 sv[2][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int row = rh * 32 + rt * 16 + ll;
          sv[rt][0] = *(MLA_LDS f32x4*)(st + schunk(row, 2 * lg));
          sv[rt][1] = *(MLA_LDS f32x4*)(st + schunk(row, 2 * lg + 1));
        }
        constexpr int kVAhead = 6;
        u32x4 vf[kVAhead + 1];
#pragma unroll
        for (int ct = 0; ct < kVAhead; ++ct) vf[ct] = load_v(ct);
        // online softmax; the lane's 8 probabilities per row tile are the
        // P^T operand of that tile as they stand
        const int key0 = (2 * c.lo + t - 1) * kHalfRows + 8 * lg;
        // whole half page visible to both row tiles of this lane: no masking
        const bool full = key0 + 8 <= min(cnt[0], cnt[1]);
        u32x4 pf[2];
        float alpha[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          float x[8] = {sv[rt][0][0], sv[rt][0][1], sv[rt][0][2], sv[rt][0][3],
                        sv[rt][1][0], sv[rt][1][1], sv[rt][1][2], sv[rt][1][3]};
          if (!full) {
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = (key0 + j < cnt[rt]) ? x[j] : -INFINITY;
          }
          float mx = x[0];
#pragma unroll
          for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
          // scores are raw dot products: scale_log2 > 0 commutes with the max
          mx = max_across_groups(mx) * p.scale_log2;
          alpha[rt] = 1.f;
          if (mx > m_run[rt] + kRescaleSlack) {
            alpha[rt] = __builtin_amdgcn_exp2f(m_run[rt] - mx);
            m_run[rt] = mx;
          }
          const float msub = (m_run[rt] == -INFINITY) ? 0.f : m_run[rt];
          float rs = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], p.scale_log2, -msub));
            rs += x[j];
          }
          l_part[rt] = l_part[rt] * alpha[rt] + rs;
          pf[rt] = u32x4{Dt<T>::pack2(x[0], x[1]), Dt<T>::pack2(x[2], x[3]), Dt<T>::pack2(x[4], x[5]),
                         Dt<T>::pack2(x[6], x[7])};
        }
        // alpha is per row = per lane column of the accumulator tiles
        if (__any((alpha[0] != 1.f) | (alpha[1] != 1.f))) {
#pragma unroll
          for (int ct = 0; ct < 16; ++ct)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) o[ct][rt] *= alpha[rt];
        }
#pragma unroll
        for (int ct = 0; ct < 16; ++ct) {
          if (ct + kVAhead < 16) vf[(ct + kVAhead) % (kVAhead + 1)] = load_v(ct + kVAhead);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) o[ct][rt] = Dt<T>::mfma32(vf[ct % (kVAhead + 1)], pf[rt], o[ct][rt]);
        }
      };
      // step t in 0 .. nh; every step ends with X(t)
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
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float l = sum_across_groups(l_part[rt]);
        const int row = mrow0 + rh * 32 + rt * 16 + li;
        if (row >= p.rows) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float lse = lse_of(m_run[rt], l);
        if (c.nsplit == 1) {
#pragma unroll
          for (int ct = 0; ct < 16; ++ct)
            store_out4<T>(p, c.b, row, ch * 256 + ct * 16 + 4 * g, o[ct][rt] * inv);
          if (ch == 0 && g == 0) p.lse[(int64_t)c.b * p.rows + row] = lse;
        } else {
          const int64_t slot = c.slot0 + c.split;
          float* dst = p.part_o + (slot * p.rows + row) * kDV + ch * 256 + 4 * g;
#pragma unroll
          for (int ct = 0; ct < 16; ++ct) *(f32x4*)(dst + ct * 16) = o[ct][rt] * inv;
          if (ch == 0 && g == 0) p.part_lse[slot * p.rows + row] = lse;
        }
      }
    });
  }
}

hipError_t launch_splitkv_wide(const DecodeParams& p, int dtype, int m_blocks, hipStream_t st) {
  if (dtype == 0) hipLaunchKernelGGL(splitkv_wide_kernel<__bf16>, dim3(p.num_parts, m_blocks), dim3(512), 0, st, p);
  else hipLaunchKernelGGL(splitkv_wide_kernel<_Float16>, dim3(p.num_parts, m_blocks), dim3(512), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
