// Split-KV MLA decode attention, wide tile (64 query rows per workgroup).
// Built with MFMA accumulators in AGPR form (the default).
#include "mla_splitkv.hpp"

namespace mla {

// ------------------------------------------------------------------ wide --
// 64 query rows per workgroup, 8 waves (two per SIMD) in two roles, so that on
// every SIMD the MFMAs of one role overlap the softmax arithmetic and LDS
// traffic of the other (the MI355X counterpart of the seesaw schedule's two
// alternating warpgroups).  Keys are processed in half pages of 32.
//   * score waves 0..3, (rg, kg) = (w >> 1, w & 1): raw scores S^T for query
//     rows rg*32 .. +32 (two 16-row tiles, Q fragments in registers) and keys
//     kg*16 .. +16 of half page t; each K fragment read from LDS feeds two
//     MFMAs.  The scores go to an fp32 tile in LDS.  These waves also issue
//     all the HBM -> LDS loads, spread over their MFMA stream.
//   * output waves 4..7: wave c owns the softmax of rows 16c .. 16c+15 (all 32
//     keys of the half page, so no cross-wave maximum exchange), writes their
//     probabilities P(t) and rescale factors to LDS, and accumulates
//     O^T += V^T . P^T for output columns 128c .. +128 of all 64 rows.
// Step t has two workgroup barriers: X(t) after the scores S(t) are written,
// Y(t) after P(t) is written.  Between Y(t-1) and X(t) the output waves form
// P(t-1).V(t-1) while the score waves finish S(t); between X(t) and Y(t) the
// output waves run the softmax of t while the score waves start S(t+1).
// Half pages stream HBM -> LDS by direct (LDS-DMA) loads into four buffers
// named at compile time (the step loop is unrolled by four, so the compiler
// can tell the LDS reads of one buffer from the loads in flight into
// another); the loads of half page t+2 are issued during step t and waited
// for at X(t+1).
template <typename T>
__global__ __launch_bounds__(512, 1) void splitkv_wide_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char hb0_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char hb1_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char hb2_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char hb3_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char s_raw[64 * 32 * 4];   // S(t), fp32 [row][32 keys]
  __shared__ float alpha_s[64];
  __shared__ float l_s[64];
  __shared__ float m_s[64];
  auto hbuf = [&](auto ic) -> MLA_LDS char* {
    constexpr int i = decltype(ic)::value & 3;
    if constexpr (i == 0) return (MLA_LDS char*)hb0_raw;
    else if constexpr (i == 1) return (MLA_LDS char*)hb1_raw;
    else if constexpr (i == 2) return (MLA_LDS char*)hb2_raw;
    else return (MLA_LDS char*)hb3_raw;
  };
  MLA_LDS char* const stile = (MLA_LDS char*)s_raw;
  // 16-byte chunk c (keys 4c .. 4c+3) of row `row` of the score tile
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
        if (i < 8) {
          const int r = 8 * wave + i;
          dma16<kWideAux>(pg, hb + r * 1024, (lane ^ swz_v(r)) << 4, (half * kHalfRows + r) * row_bytes);
        } else {
          dma_rope_rows8<kWideAux>(pg, hb, half, wave, row_bytes, lane);
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
          if constexpr (ks == 10) {
            // Y(t-1): the output waves have published P(t-1); nothing of this
            // wave depends on it, so no wait for outstanding LDS reads
            if (t >= 1) asm volatile("s_barrier" ::: "memory");
          }
          s0 = Dt<T>::mfma32(kf[ks % (kAhead + 1)], qf[0][ks], s0);
          s1 = Dt<T>::mfma32(kf[ks % (kAhead + 1)], qf[1][ks], s1);
        });
        // raw scores to the tile (the softmax of t-1 has read the previous ones)
        const int row0 = rg * 32 + li;
        *(MLA_LDS f32x4*)(stile + schunk(row0, kg * 4 + g)) = s0;
        *(MLA_LDS f32x4*)(stile + schunk(row0 + 16, kg * 4 + g)) = s1;
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
      asm volatile("s_barrier" ::: "memory");                               // Y(nh-1)
      lds_barrier();                                                        // E
    });
  } else {
    // ------------------------------------------------------- output waves --
    const int cw = wave - 4;                                  // columns cw*128 .. +128
    const int srow = cw * 16 + li;                            // softmax row of this lane
    for_each_chunk(p, [&](const Chunk& c) {
      const int nh = half_pages(c);
      const int qrow = mrow0 + srow;
      const int cnt = qrow < p.rows ? visible_count(c.n, p.s_q, qrow / p.h_q, p.causal) : 0;
      float m_run = -INFINITY;   // running max of row srow, log2 units
      float l_part = 0.f;        // this lane's share of its running sum
      f32x4 o[8][4];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) o[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      lds_barrier();                                                        // X(-1)

      // O *= alpha(t-1); O^T[col][row] += V^T . P^T over half page t-1
      auto pv = [&](auto Pc) {
        MLA_LDS char* prv = hbuf(Pc);
        // Lane-dependent read addresses are rebuilt here from an opaque copy of
        // the lane index: cheaper than keeping ~64 of them (16 per buffer)
        // alive in registers across the step loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lg = ln >> 4, ll = ln & 15;
        const int vrow = 8 * lg + (ll >> 2);                  // value row (lo) of the transposed reads
        const int vbase = vrow * 1024 + cw * 256 + (ll & 1) * 8;
        const int vkey = swz_v(vrow);                         // vrow + 4 uses vkey ^ 8
        const int vh = (ll >> 1) & 1;
        auto load_v = [&](int ct) {
          const int x = ((2 * ct + vh) ^ vkey) << 4;
          const u32x2 lo4 = ld_lds_tr(prv + vbase + x);
          const u32x2 hi4 = ld_lds_tr(prv + vbase + 4096 + (x ^ 128));
          return u32x4{lo4[0], lo4[1], hi4[0], hi4[1]};
        };
        // every operand read of the step is issued before the first MFMA
        float a4[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) a4[rt] = alpha_s[rt * 16 + ll];
        u32x4 pf[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) pf[rt] = ld_lds16(prv + pchunk_off(rt * 16 + ll, lg));
        u32x4 vf[8];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) vf[ct] = load_v(ct);
        const bool resc = (a4[0] != 1.f) | (a4[1] != 1.f) | (a4[2] != 1.f) | (a4[3] != 1.f);
        if (__any(resc)) {
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) o[ct][rt] *= a4[rt];
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) o[ct][rt] = Dt<T>::mfma32(vf[ct], pf[rt], o[ct][rt]);
      };
      // step t accumulates half page t-1 and, for t < nh, runs the softmax of t
      auto step = [&](auto Hc, int t) {
        constexpr int H = decltype(Hc)::value;
        if (t >= 1) pv(std::integral_constant<int, H + 3>{});
        if (t == nh) return;
        lds_barrier();                                                      // X(t)
        // softmax of row srow over keys 8g .. 8g+7 of half page t
        const f32x4 sa = *(MLA_LDS f32x4*)(stile + schunk(srow, 2 * g));
        const f32x4 sb = *(MLA_LDS f32x4*)(stile + schunk(srow, 2 * g + 1));
        float x[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
        const int key0 = (2 * c.lo + t) * kHalfRows + 8 * g;
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[j] = (key0 + j < cnt) ? x[j] * p.scale_log2 : -INFINITY;
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
        const u32x4 pk = {Dt<T>::pack2(x[0], x[1]), Dt<T>::pack2(x[2], x[3]), Dt<T>::pack2(x[4], x[5]),
                          Dt<T>::pack2(x[6], x[7])};
        *(MLA_LDS u32x4*)(hbuf(Hc) + pchunk_off(srow, g)) = pk;
        if (g == 0) alpha_s[srow] = alpha;
        lds_barrier();                                                      // Y(t)
      };
      int t0 = 0;
      for (; t0 + 4 <= nh + 1; t0 += 4) static_for<0, 4>([&](auto Hc) { step(Hc, t0 + decltype(Hc)::value); });
      static_for<0, 3>([&](auto Hc) {
        const int t = t0 + decltype(Hc)::value;
        if (t <= nh) step(Hc, t);
      });
      {
        const float lw = sum_across_groups(l_part);
        if (g == 0) {
          l_s[srow] = lw;
          m_s[srow] = m_run;
        }
      }
      lds_barrier();                                                        // E
      // epilogue: normalise, write the final output or an fp32 partial
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int rl = rt * 16 + li;
        const int row = mrow0 + rl;
        if (row >= p.rows) continue;
        const float l = l_s[rl];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float lse = lse_of(m_s[rl], l);
        if (c.nsplit == 1) {
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
            store_out4<T>(p, c.b, row, cw * 128 + ct * 16 + 4 * g, o[ct][rt] * inv);
          if (cw == 0 && g == 0) p.lse[(int64_t)c.b * p.rows + row] = lse;
        } else {
          const int64_t slot = c.slot0 + c.split;
          float* dst = p.part_o + (slot * p.rows + row) * kDV + cw * 128 + 4 * g;
#pragma unroll
          for (int ct = 0; ct < 8; ++ct) *(f32x4*)(dst + ct * 16) = o[ct][rt] * inv;
          if (cw == 0 && g == 0) p.part_lse[slot * p.rows + row] = lse;
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
