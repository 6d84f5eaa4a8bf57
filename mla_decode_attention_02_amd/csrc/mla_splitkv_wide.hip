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
//   * score waves 0..3: wave w owns query rows 16w .. 16w+15 (Q fragments in
//     registers) and forms S^T over all 32 keys of half page t, so the row
//     maximum needs no other wave; it runs the online softmax and writes the
//     probabilities P(t) (bf16/fp16) and rescale factors alpha(t) to LDS.
//     These waves also issue all the HBM -> LDS loads, spread over their MFMA
//     stream.
//   * output waves 4..7: wave c accumulates O^T += V^T . P^T for output columns
//     128c .. +128 of all 64 rows on half page t-1, after scaling by
//     alpha(t-1).  They issue no global memory operation in the loop.
// One workgroup barrier per step (P(t) written, loads of t+1 landed).  Half
// pages stream HBM -> LDS by direct (LDS-DMA) loads into four buffers named at
// compile time (the step loop is unrolled by four, so the compiler can tell
// the LDS reads of one buffer from the loads in flight into another); P and
// alpha are double-buffered; the loads of half page t+2 are issued in step t.
template <typename T>
__global__ __launch_bounds__(512, 1) void splitkv_wide_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char hb0_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char hb1_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char hb2_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char hb3_raw[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) char pb_raw[2][4096];   // P(t), key-slot-group major
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
  auto pbuf = [&](auto ic) -> MLA_LDS char* {
    constexpr int i = decltype(ic)::value & 1;
    return (MLA_LDS char*)pb_raw[i];
  };
  // The contraction of P.V over the 32 keys of a half page runs in a permuted
  // key order: k-slots 8c .. 8c+7 hold keys 4c .. 4c+3 and 16+4c .. 16+4c+3, the
  // eight scores one lane of a score wave owns (key c of the two 16-key score
  // tiles), so that lane writes its probabilities with a single 16-byte store.
  // Byte offset of the 16 bytes of slot group c of row `row` in a P tile:
  auto poff = [](int row, int c) { return c * 1024 + row * 16; };

  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int mrow0 = blockIdx.y * 64;
  const int row_bytes = (int)(p.k_s1 * 2);

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
    const int srow = wave * 16 + li;                          // tile row of this lane
    // This lane's source offsets for the wave's nine loads of a half page
    // (value rows 8w .. 8w+7, then rope rows 8w .. 8w+7), for either half of
    // a page: computed once, so a load costs no address arithmetic in the
    // MFMA stream.
    int dof[2][9];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * wave + i;
        dof[h][i] = ((lane ^ swz_v(r)) << 4) + (h * kHalfRows + r) * row_bytes;
      }
      const int rr = 8 * wave + (lane >> 3);
      dof[h][8] = (h * kHalfRows + rr) * row_bytes + 1024 + (((lane & 7) ^ swz_r(rr)) << 4);
    }
    for_each_chunk(p, [&](const Chunk& c) {
      BlockWindow bw;
      bw.init(p.block_table + (int64_t)c.b * p.bt_s, c.lo, c.hi, lane);
      const int nh = half_pages(c);
      const int qrow = mrow0 + srow;
      u32x4 qf[18];
      load_q_frag<T>(p, c.b, qrow, g, qf);
      const int cnt = qrow < p.rows ? visible_count(c.n, p.s_q, qrow / p.h_q, p.causal) : 0;
      float m_run = -INFINITY;   // running max of row srow, log2 units
      float l_part = 0.f;        // this lane's share of its running sum
      // Loads of half page hh: this wave moves value rows 8w .. 8w+7 (piece
      // i < 8) and rope rows 8w .. 8w+7 (piece 8).  Past the end of the chunk
      // an empty descriptor keeps the count of loads in flight uniform
      // (every lane out of range, no memory access).  With loop-invariant
      // offsets the compiler would gather the loads at one point of the step,
      // which stalls the MFMA stream; the scheduling barriers keep each one
      // where it is issued.
      auto page_desc = [&](int hh) {
        const bool real = hh < nh;
        const int pg = c.lo + (hh >> 1);
        return page_of(p, real ? bw.phys(pg) : 0, real ? page_valid_rows(c.n, pg) : 0);
      };
      auto piece = [&](auto ic, int hh, BufRsrc pg, int i) {
        MLA_LDS char* hb = hbuf(ic);
        const int half = hh & 1;
        __builtin_amdgcn_sched_barrier(0);
        if (i < 8) dma16<kWideAux>(pg, hb + (8 * wave + i) * 1024, half ? dof[1][i] : dof[0][i], 0);
        else dma16<kWideAux>(pg, hb + kHalfRopeOff + wave * 1024, half ? dof[1][8] : dof[0][8], 0);
        __builtin_amdgcn_sched_barrier(0);
      };
      {
        const BufRsrc pg0 = page_desc(0), pg1 = page_desc(1);
#pragma unroll
        for (int i = 0; i < 9; ++i) piece(std::integral_constant<int, 0>{}, 0, pg0, i);
#pragma unroll
        for (int i = 0; i < 9; ++i) piece(std::integral_constant<int, 1>{}, 1, pg1, i);
      }
      dma_barrier<9>();                                                     // X(-1)

      // step t < nh: S(t), softmax, P(t) and alpha(t); loads of half page t+2
      auto step = [&](auto Hc, int t) {
        constexpr int H = decltype(Hc)::value;
        MLA_LDS char* cur = hbuf(Hc);
        const BufRsrc pg = page_desc(t + 2);
        // S^T for the 32 keys (two 16-key tiles) x 16 rows; K reads run kAhead
        // contraction steps ahead of the MFMAs
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        constexpr int kAhead = 4;
        u32x4 kf[kAhead + 1][2];
        static_for<0, kAhead>([&](auto kc) {
          constexpr int ks = decltype(kc)::value;
          kf[ks][0] = ld_lds16(cur + hchunk_off<ks>(li, g));
          kf[ks][1] = ld_lds16(cur + hchunk_off<ks>(16 + li, g));
        });
        static_for<0, 18>([&](auto ksc) {
          constexpr int ks = decltype(ksc)::value;
          if constexpr (ks + kAhead < 18) {
            kf[(ks + kAhead) % (kAhead + 1)][0] = ld_lds16(cur + hchunk_off<ks + kAhead>(li, g));
            kf[(ks + kAhead) % (kAhead + 1)][1] = ld_lds16(cur + hchunk_off<ks + kAhead>(16 + li, g));
          }
          if constexpr (ks % 2 == 0) piece(std::integral_constant<int, H + 2>{}, t + 2, pg, ks / 2);
          s0 = Dt<T>::mfma32(kf[ks % (kAhead + 1)][0], qf[ks], s0);
          s1 = Dt<T>::mfma32(kf[ks % (kAhead + 1)][1], qf[ks], s1);
        });
        // online softmax of row srow over keys 4g+r (tile 0) and 16+4g+r (tile 1)
        float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        const int key0 = (2 * c.lo + t) * kHalfRows + 4 * g;
        if (!(key0 + 20 <= cnt)) {   // some key of this lane not visible
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = (key0 + (j >> 2) * 16 + (j & 3) < cnt) ? x[j] : -INFINITY;
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
        // scores are raw dot products: scale_log2 > 0 commutes with the max
        mx = max_across_groups(mx) * p.scale_log2;
        float alpha = 1.f;
        if (mx > m_run + kRescaleSlack) {
          alpha = __builtin_amdgcn_exp2f(m_run - mx);
          m_run = mx;
        }
        const float msub = (m_run == -INFINITY) ? 0.f : m_run;
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], p.scale_log2, -msub));
          rs += x[j];
        }
        l_part = l_part * alpha + rs;
        // one store: two stores to this tile would be merged into a single
        // instruction that waits for every load in flight
        MLA_LDS char* pb = pbuf(Hc);
        *(MLA_LDS u32x4*)(pb + poff(srow, g)) =
            u32x4{Dt<T>::pack2(x[0], x[1]), Dt<T>::pack2(x[2], x[3]), Dt<T>::pack2(x[4], x[5]),
                  Dt<T>::pack2(x[6], x[7])};
        if (g == 0) alpha_s[H & 1][srow] = alpha;
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

      // step t >= 1: O *= alpha(t-1); O^T += V^T . P^T over half page t-1
      auto step = [&](auto Hc, int t) {
        constexpr int H = decltype(Hc)::value;
        MLA_LDS char* prv = hbuf(std::integral_constant<int, H + 3>{});   // half page t-1
        MLA_LDS char* pb = pbuf(std::integral_constant<int, H + 1>{});    // P(t-1)
        // Lane-dependent read addresses are rebuilt here from an opaque copy of
        // the lane index: cheaper than keeping them alive across the loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lg = ln >> 4, ll = ln & 15;
        // slots 8lg .. 8lg+7 = keys 4lg .. 4lg+3 (lo) and 16+4lg .. 16+4lg+3 (hi)
        const int vrow = 4 * lg + (ll >> 2);                  // value row (lo) of the transposed reads
        const int vbase = vrow * 1024 + cw * 256 + (ll & 1) * 8;
        const int vkey = swz_v(vrow);                         // the same for vrow + 16
        const int vh = (ll >> 1) & 1;
        auto load_v = [&](int ct) {
          const int x = ((2 * ct + vh) ^ vkey) << 4;
          const u32x2 lo4 = ld_lds_tr(prv + vbase + x);
          const u32x2 hi4 = ld_lds_tr(prv + vbase + 16 * 1024 + x);
          return u32x4{lo4[0], lo4[1], hi4[0], hi4[1]};
        };
        float a4[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) a4[rt] = alpha_s[(H + 1) & 1][rt * 16 + ll];
        u32x4 pf[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) pf[rt] = ld_lds16(pb + poff(rt * 16 + ll, lg));
        u32x4 vf[8];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) vf[ct] = load_v(ct);
        const bool resc = (a4[0] != 1.f) | (a4[1] != 1.f) | (a4[2] != 1.f) | (a4[3] != 1.f);
        if (__any(resc)) {
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) o[ct][rt] *= a4[rt];
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          if (ct + 4 < 8) vf[ct + 4] = load_v(ct + 4);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) o[ct][rt] = Dt<T>::mfma32(vf[ct], pf[rt], o[ct][rt]);
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
      // epilogue: normalise, write the final output or an fp32 partial.  The
      // lane's row and column come from an opaque copy of the lane index, so
      // that their address arithmetic is done here: hoisted to the kernel
      // start, the per-row-tile addresses were spilled to scratch, and each
      // reload waited for every store issued before it.
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

hipError_t launch_splitkv_wide(const DecodeParams& p, int dtype, int m_blocks, hipStream_t st) {
  if (dtype == 0) hipLaunchKernelGGL(splitkv_wide_kernel<__bf16>, dim3(p.num_parts, m_blocks), dim3(512), 0, st, p);
  else hipLaunchKernelGGL(splitkv_wide_kernel<_Float16>, dim3(p.num_parts, m_blocks), dim3(512), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
