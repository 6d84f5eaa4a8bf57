// Split-KV MLA decode attention, narrow tile (up to 16 query rows per workgroup).
// Built with MFMA accumulators in VGPR form: the per-wave output rescale runs on
// them with plain VALU instructions, without AGPR round trips.
#include "mla_splitkv.hpp"

namespace mla {

// ---------------------------------------------------------------- narrow --
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void splitkv_narrow_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char kbuf0_raw[kPageBytes];
  __shared__ __attribute__((aligned(1024))) char kbuf1_raw[kPageBytes];
  __shared__ float m_w[kWaves][16];
  __shared__ float l_w[kWaves][16];
  __shared__ MergeLds<16> merge_s;
  MLA_LDS char* kbuf0 = (MLA_LDS char*)kbuf0_raw;
  MLA_LDS char* kbuf1 = (MLA_LDS char*)kbuf1_raw;
  constexpr int kMergeStride = kDV + 4;   // floats per row of the merge buffer
  static_assert(2 * 16 * kMergeStride * 4 <= kPageBytes, "merge buffer fits two waves per page buffer");

  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int row_bytes = (int)(p.k_s1 * 2);

  for_each_chunk(p, [&](const Chunk& c) {
    BlockWindow bw;
    bw.init(p.block_table + (int64_t)c.b * p.bt_s, c.lo, c.hi, lane);
    u32x4 qf[18];
    load_q_frag<T>(p, c.b, li, g, qf);
    const int cnt = li < p.rows ? visible_count(c.n, p.s_q, li / p.h_q, p.causal) : 0;
    float m_run = -INFINITY, l_part = 0.f;
    f32x4 o[32];
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int krow = wave * 16 + li;                       // key row of the score operand
    const int vrow = wave * 16 + 4 * g + (li >> 2);        // value row of the transposed reads
    const int vbase = vrow * 1024 + (li & 1) * 8;
    const int vkey = swz_v(vrow);
    const int vh = (li >> 1) & 1;

    // two pages in flight in registers while a third is read from LDS
    PageStage st[2];
    stage_load<kNarrowAux>(st[0], page_of(p, bw.phys(c.lo), page_valid_rows(c.n, c.lo)), row_bytes, wave, lane);
    if (c.lo + 1 < c.hi) stage_load<kNarrowAux>(st[1], page_of(p, bw.phys(c.lo + 1), page_valid_rows(c.n, c.lo + 1)), row_bytes, wave, lane);
    stage_store(st[0], kbuf0, wave, lane);
    lds_barrier();
    page_loop(c.lo, c.hi, kbuf0, kbuf1, [&](auto par, MLA_LDS char* cur, MLA_LDS char* nxt, int pg) {
      constexpr int P = decltype(par)::value;   // st[P] held page pg, st[P ^ 1] holds pg + 1
      if (pg + 2 < c.hi) stage_load<kNarrowAux>(st[P], page_of(p, bw.phys(pg + 2), page_valid_rows(c.n, pg + 2)), row_bytes, wave, lane);

      // S^T for keys wave*16 .. +16 of the page, all 16 rows; operand reads
      // run two steps ahead of the MFMAs
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      u32x4 kf[3];
      kf[0] = ld_lds16(cur + kchunk_off<0>(krow, g));
      kf[1] = ld_lds16(cur + kchunk_off<1>(krow, g));
      static_for<0, 18>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        if constexpr (ks + 2 < 18) kf[(ks + 2) % 3] = ld_lds16(cur + kchunk_off<ks + 2>(krow, g));
        s = Dt<T>::mfma32(kf[ks % 3], qf[ks], s);
      });
      const int key0 = pg * kPage + wave * 16 + 4 * g;
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float t = (key0 + r < cnt) ? s[r] * p.scale_log2 : -INFINITY;
        s[r] = t;
        mx = fmaxf(mx, t);
      }
      mx = max_across_groups(mx);
      float alpha = 1.f;
      if (mx > m_run + kRescaleSlack) {
        alpha = exp2f(m_run - mx);
        m_run = mx;
      }
      const float msub = (m_run == -INFINITY) ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[r] = __builtin_amdgcn_exp2f(s[r] - msub);
        rs += s[r];
      }
      l_part = l_part * alpha + rs;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int ct = 0; ct < 32; ++ct) o[ct] *= alpha;
      }
      const u32x2 pk = {Dt<T>::pack2(s[0], s[1]), Dt<T>::pack2(s[2], s[3])};
      constexpr int kAhead = 4;
      u32x2 vf[kAhead + 1];
      auto vaddr = [&](int ct) { return cur + vbase + (ct >> 3) * 256 + ((((2 * ct) & 15) + vh) ^ vkey) * 16; };
#pragma unroll
      for (int ct = 0; ct < kAhead; ++ct) vf[ct] = ld_lds_tr(vaddr(ct));
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) {
        if (ct + kAhead < 32) vf[(ct + kAhead) % (kAhead + 1)] = ld_lds_tr(vaddr(ct + kAhead));
        o[ct] = Dt<T>::mfma16(vf[ct % (kAhead + 1)], pk, o[ct]);
      }
      if (pg + 1 < c.hi) stage_store(st[P ^ 1], nxt, wave, lane);
      lds_barrier();
    });

    // merge the four per-wave states of this range
    const float lw = sum_across_groups(l_part);
    if (g == 0) {
      m_w[wave][li] = m_run;
      l_w[wave][li] = lw;
    }
    lds_barrier();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_w[w][li]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      L += (m_w[w][li] == -INFINITY) ? 0.f : l_w[w][li] * exp2f(m_w[w][li] - M);
    const float f = (L > 0.f && m_run != -INFINITY) ? exp2f(m_run - M) / L : 0.f;
    // merge buffer: [wave][16 rows][kMergeStride] floats, waves 0-1 in the first
    // page buffer and waves 2-3 in the second
    auto mrow = [&](int w, int row) -> float* {
      return (float*)(w < 2 ? kbuf0_raw : kbuf1_raw) + ((w & 1) * 16 + row) * kMergeStride;
    };
    {
      float* dst = mrow(wave, li);
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) *(f32x4*)(dst + ct * 16 + 4 * g) = o[ct] * f;
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = tid + kThreads * k;
      const int row = idx >> 7;
      const int col = (idx & 127) * 4;
      if (row < p.rows) {
        f32x4 acc = *(f32x4*)(mrow(0, row) + col);
#pragma unroll
        for (int w = 1; w < kWaves; ++w) acc += *(f32x4*)(mrow(w, row) + col);
        if (c.nsplit == 1) {
          store_out4<T>(p, c.b, row, col, acc);
        } else {
          const int64_t slot = c.slot0 + c.split;
          *(f32x4*)(p.part_o + (slot * p.rows + row) * kDV + col) = acc;
        }
      }
    }
    if (tid < 16 && tid < p.rows) {
      float Mx = -INFINITY, Ls = 0.f;
      for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, m_w[w][tid]);
      for (int w = 0; w < kWaves; ++w)
        Ls += (m_w[w][tid] == -INFINITY) ? 0.f : l_w[w][tid] * exp2f(m_w[w][tid] - Mx);
      const float lse = lse_of(Mx, Ls);
      if (c.nsplit == 1) p.lse[(int64_t)c.b * p.rows + tid] = lse;
      else p.part_lse[(int64_t)(c.slot0 + c.split) * p.rows + tid] = lse;
    }
    lds_barrier();
    if (c.nsplit > 1 && c.nsplit <= p.fuse_max) fused_merge<T, 16, kThreads>(p, c, 0, merge_s);
  });
}

hipError_t launch_splitkv_narrow(const DecodeParams& p, int dtype, hipStream_t st) {
  if (p.kv_fp8) return launch_splitkv_fp8(p, st);   // fp8 cache: mla_splitkv_fp8.hip
  if (dtype == 0) hipLaunchKernelGGL(splitkv_narrow_kernel<__bf16>, dim3(p.num_parts, 1), dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(splitkv_narrow_kernel<_Float16>, dim3(p.num_parts, 1), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
