// Paged multi-head / grouped-query decode attention (gfx950): separate K and V
// caches [pages, 64, h_kv, d] with head size d in {64, 128, 256} and h_kv
// dividing h_q, in the style of the key/value-cache decode call of page
// "FlashAttention终极指南：如何通过动态计算图实现3倍推理加速" (section "核心代码实现解析":
// q against k_cache and v_cache with cache_seqlens and a causal flag; section
// "问题二：精度偏差处理": the LSE returned beside the output).  The work is cut
// into (request, KV head) units by the same split-KV scheduler as the MLA path
// and merged by LSE afterwards.
//
// Decode attention with a few query rows per KV head is bound by HBM bandwidth
// (rows FLOP per byte: 8 for a group of 8 heads, against a ridge of ~312), so
// the kernel is built to keep the K/V stream moving:
//   * one workgroup (4 waves) per partition; K and V of KS keys of the unit's
//     KV head stream HBM -> LDS by direct (LDS-DMA) loads into four buffers
//     named at compile time, three steps ahead of their use;
//   * every wave forms the scores of all KS keys for all of the workgroup's
//     query rows (the score MFMAs are cheap at this intensity) and so runs the
//     online softmax of every row itself: no score exchange, and after the
//     loop no merge of per-wave states;
//   * wave w accumulates output columns w * d_v/4 .. +d_v/4 of every row, the
//     V^T operand coming from transposed LDS reads, the P^T operand straight
//     from the score accumulators' registers.
// Keys past a request's length in its last page are read over a range that
// ends at its last valid row, so they arrive as zeros whatever the cache holds
// there.
//
// fp8 caches (KV8): K and V hold e4m3 codes with one fp32 scale per page and
// KV head.  The LDS image keeps the codes (half the bytes; eight buffers, seven
// steps ahead) and operands are converted to bf16 as they are read (exact:
// every e4m3 value is a bf16 value).  K operands are 16-byte reads whose 16
// codes feed two MFMAs (the Q fragments are loaded in that column order); V^T
// operands come from 8-bit transposed reads (eight keys of one column per
// lane).  The K scale multiplies the scores, the V scale the probabilities
// before their bf16 rounding (the denominator sums the unscaled ones).
#include "mla_common.hpp"
#include "mla_internal.h"
#include "mla_sched.hpp"

namespace mla {

// 16-byte chunk swizzle of an LDS row of `cpr` chunks: rows of 256 bytes or
// more key on row & 7 (two consecutive chunks of 8 rows then cover the 16
// bank groups); rows of 128 bytes, two per bank row, key on (row >> 1) & 3.
template <int CPR>
__device__ __forceinline__ int mha_swz(int row) {
  if constexpr (CPR >= 16) return (row & 7) << 1;
  else if constexpr (CPR == 8) return ((row >> 1) & 3) << 1;
  else return ((row >> 2) & 1) << 1;          // 64-byte rows, four per bank row
}

__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

__device__ __forceinline__ u32x2 mha_ld_tr8(const MLA_LDS char* p) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS v2i*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Buffer descriptor over the rows of one page and KV head (elements of ESZ
// bytes); rows at or past `valid` are out of range (their loads return
// zeros).  valid <= 0: empty.
template <int ESZ>
__device__ __forceinline__ BufRsrc mha_rows_rsrc(const void* base, int64_t elem_off, int64_t row_stride, int width,
                                                 int valid) {
  const int bytes = valid > 0 ? (int)(((int64_t)(valid - 1) * row_stride + width) * ESZ) : 0;
  return page_rsrc((const char*)base + elem_off * ESZ, bytes);
}

template <typename T, int D, int RT, bool KV8, bool RS, bool NT>
__global__ __launch_bounds__(256, 1) void mha_splitkv_kernel(MhaParams p) {
  constexpr int DV = D;
  constexpr int KS = D <= 128 ? 64 : 32;     // keys per step
  constexpr int KT = KS / 16;                // 16-key score tiles per step
  constexpr int SPP = kPage / KS;            // steps per page
  constexpr int ESZ = KV8 ? 1 : 2;           // bytes per cached element
  constexpr int NB = KV8 ? 8 : 4;            // LDS buffers (NB - 1 steps in flight)
  constexpr int ROWB = D * ESZ;              // bytes of a K (and V) row in LDS
  constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  constexpr int KBYTES = KS * ROWB;
  constexpr int BUF = 2 * KBYTES;            // K rows, then V rows
  constexpr int DC = D / 32;                 // 32-deep contraction steps of Q.K
  // RS (row split, for blocks of more than 16 rows): wave w owns rows
  // 16w .. 16w+15 of the block and all output columns, so no wave repeats
  // another's scores; else every wave takes all RT row tiles and a quarter
  // of the columns
  constexpr int RTW = RS ? 1 : RT;           // row tiles per wave
  constexpr int CW = RS ? DV : DV / 4;       // output columns per wave
  constexpr int CT = CW / 16;                // 16-column output tiles per wave
  constexpr int NDMA = 2 * KBYTES / 1024 / 4;  // LDS-DMA instructions per wave and step
  constexpr int NLD = NDMA + (KV8 ? 2 : 0);  // and with the two scale loads
  constexpr int RPI = 1024 / ROWB;           // rows per DMA instruction
  static_assert(KT % 2 == 0 && CT >= 1 && NDMA >= 1 && 2 * KBYTES % 4096 == 0, "tile shape");
  static_assert((NB - 1) * NLD <= 63, "loads in flight fit the wait counter");
  // NT: the unit's rows fit one row block, so its K/V bytes are read once
  // (non-temporal loads); otherwise the row blocks of one unit may meet in L2
  constexpr int kAux = NT ? 2 : 0;
  // one array per buffer, so that the compiler can tell the reads of one from
  // the loads in flight into another (it tells apart at most eight LDS-DMA
  // targets, so the fp8 scales live at the end of their buffer's array)
  constexpr int SCB = KV8 ? 2 * 4 * 64 * 4 : 0;   // fp8: K and V scale slots, 64 floats per wave
  constexpr int BUFA = BUF + SCB;
  constexpr int BUFX = NB > 4 ? BUFA : 16;
  __shared__ __attribute__((aligned(1024))) char b0_raw[BUFA];
  __shared__ __attribute__((aligned(1024))) char b1_raw[BUFA];
  __shared__ __attribute__((aligned(1024))) char b2_raw[BUFA];
  __shared__ __attribute__((aligned(1024))) char b3_raw[BUFA];
  __shared__ __attribute__((aligned(1024))) char b4_raw[BUFX];
  __shared__ __attribute__((aligned(1024))) char b5_raw[BUFX];
  __shared__ __attribute__((aligned(1024))) char b6_raw[BUFX];
  __shared__ __attribute__((aligned(1024))) char b7_raw[BUFX];
  auto buf = [&](auto ic) -> MLA_LDS char* {
    constexpr int i = decltype(ic)::value % NB;
    if constexpr (i == 0) return (MLA_LDS char*)b0_raw;
    else if constexpr (i == 1) return (MLA_LDS char*)b1_raw;
    else if constexpr (i == 2) return (MLA_LDS char*)b2_raw;
    else if constexpr (i == 3) return (MLA_LDS char*)b3_raw;
    else if constexpr (i == 4) return (MLA_LDS char*)b4_raw;
    else if constexpr (i == 5) return (MLA_LDS char*)b5_raw;
    else if constexpr (i == 6) return (MLA_LDS char*)b6_raw;
    else return (MLA_LDS char*)b7_raw;
  };
  // fp8: the step's K and V scales, landed by LDS-DMA (each wave fills its own
  // 64 floats, all read the first)
  auto sbuf = [&](auto ic) -> MLA_LDS float* { return (MLA_LDS float*)(buf(ic) + BUF); };

  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int mrow0 = blockIdx.y * 64 + (RS ? 16 * wave : 0);
  const int cb = RS ? 0 : wave * CW;         // first output column of this wave
  const int ksw = mha_swz<CPR>(li);          // swizzle of K rows kt*16 + li

  // row split: this lane's source offsets (within the step's first row) for
  // its DMA instructions, computed once
  int doff[RS ? NDMA : 1];
  if constexpr (RS) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int j = wave * NDMA + i;
      const bool isv = j >= KBYTES / 1024;
      const int jj = isv ? j - KBYTES / 1024 : j;
      const int r = jj * RPI + lane / CPR;
      const int c = (lane % CPR) ^ mha_swz<CPR>(r);
      const int64_t rs = isv ? p.v_s1 : p.k_s1;
      doff[i] = (int)(r * rs * ESZ) + c * 16;
    }
  }

  // the schedule row, precomputed or derived here
  const PartRow pr = part_row(p.sched, p.seqlens, p.batch * p.h_kv, p.h_kv, p.num_parts, p.sched_f, blockIdx.x);
  const int len0 = pr.len0;
  int sched_start = pr.start, sched_slot = pr.slot;
  for (int u = pr.begin; u <= pr.end; ++u) {
    const int b = u / p.h_kv;
    const int hk = u - b * p.h_kv;
    const int n = (pr.inl && u == pr.begin) ? len0 : ldu(p.seqlens + b);
    const int npages = (n + kPage - 1) / kPage;
    int slot0, nsplit;
    unit_slots(pr.inl, p.split_offsets, u, n, p.sched_f, pr.width, sched_start, sched_slot, slot0, nsplit);
    const int lo = (u == pr.begin) ? pr.begin_page : 0;
    const int hi = (u == pr.end) ? pr.end_page : npages;
    if (lo >= hi) continue;
    const int split = (u == pr.begin) ? pr.begin_split : 0;
    // steps of this chunk: its pages, less trailing steps wholly past the end
    const int ks0 = lo * SPP;
    const int nsteps = (min(n, hi * kPage) - lo * kPage + KS - 1) / KS;

    BlockWindow bw;
    bw.init(p.block_table + (int64_t)b * p.bt_s, lo, hi, lane);

    // Q fragments (B operand of S^T = K . Q^T): row rt*16 + li, columns
    // ks*32 + 8g .. +8 (fp8: fragment 2m columns 64m + 16g .. +8 and 2m + 1
    // the next 8, the order of the 16 codes one K read brings); rows past the
    // unit's rows are zero
    u32x4 qf[RTW][DC];
    int cnt[RTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int row = mrow0 + rt * 16 + li;
      if (row < p.rows) {
        const int tok = row / p.group;
        const int head = hk * p.group + (row - tok * p.group);
        const T* qp = (const T*)p.q + b * p.q_s0 + tok * p.q_s1 + head * p.q_s2 + 8 * g;
#pragma unroll
        for (int ks = 0; ks < DC; ++ks) {
          const int col = KV8 ? 64 * (ks >> 1) + 8 * g + 8 * (ks & 1) : ks * 32;   // past qp's 8g
          qf[rt][ks] = *(const u32x4*)(qp + col);
        }
        cnt[rt] = visible_count(n, p.s_q, tok, p.causal);
      } else {
#pragma unroll
        for (int ks = 0; ks < DC; ++ks) qf[rt][ks] = u32x4{0, 0, 0, 0};
        cnt[rt] = 0;
      }
    }

    // LDS-DMA loads of step s (keys (ks0 + s) * KS ..) into buffer ic: wave w
    // moves instructions w*NDMA .. +NDMA of the K rows then the V rows, 1 KiB
    // (RPI rows) each; lane l fills slot l of its instruction, i.e. row
    // j*RPI + l / CPR, chunk (l % CPR) ^ swizzle(row).  Steps past the chunk
    // use empty descriptors, so every step issues the same loads.
    auto issue = [&](auto ic, int s) {
      MLA_LDS char* bp = buf(ic);
      const bool real = s < nsteps;
      const int kstep = ks0 + s;
      const int page = kstep / SPP;
      const int sub = kstep - page * SPP;
      const int phys = real ? bw.phys(page) : 0;
      const int valid = real ? min(kPage, n - page * kPage) : 0;
      const BufRsrc kr = mha_rows_rsrc<ESZ>(p.k, (int64_t)phys * p.k_s0 + hk * p.k_s2, p.k_s1, D, valid);
      const BufRsrc vr = mha_rows_rsrc<ESZ>(p.v, (int64_t)phys * p.v_s0 + hk * p.v_s2, p.v_s1, DV, valid);
      int ln = lane;                             // opaque: offsets are rebuilt per step (keeping
      asm volatile("" : "+v"(ln));               // them in registers measured 4 % slower with the
#pragma unroll                                   // column split; the row split keeps them)
      for (int i = 0; i < NDMA; ++i) {
        const int j = wave * NDMA + i;           // instruction of this step, 0 .. 2*KBYTES/1024
        const bool isv = j >= KBYTES / 1024;
        const int jj = isv ? j - KBYTES / 1024 : j;
        const int64_t rs = isv ? p.v_s1 : p.k_s1;
        int voff;
        if constexpr (RS) {
          voff = doff[i] + (int)(sub * KS * rs * ESZ);
        } else {
          const int r = jj * RPI + ln / CPR;     // row of the step
          const int c = (ln % CPR) ^ mha_swz<CPR>(r);
          const int key = sub * KS + r;          // slot within the page
          voff = (int)(key * rs * ESZ) + c * 16;
        }
        dma16<kAux>(isv ? vr : kr, bp + (isv ? KBYTES : 0) + jj * 1024, voff, 0);
      }
      if constexpr (KV8) {
        MLA_LDS float* sp = sbuf(ic) + wave * 64;
        const int soff = (phys * p.h_kv + hk) * 4;
        const BufRsrc ks = page_rsrc((const char*)p.k_scale, p.k_scale && real ? 0x7FFFFFFF : 0);
        const BufRsrc vs = page_rsrc((const char*)p.v_scale, p.v_scale && real ? 0x7FFFFFFF : 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ks, (MLA_LDS void*)sp, 4, 0, soff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vs, (MLA_LDS void*)(sp + 4 * 64), 4, 0, soff, 0, 0);
      }
    };

    float m_run[RTW], l_part[RTW];
    f32x4 o[RTW][CT];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      m_run[rt] = -INFINITY;
      l_part[rt] = 0.f;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    static_for<0, NB - 1>([&](auto ic) { issue(ic, decltype(ic)::value); });

    auto step = [&](auto Hc, int s) {
      constexpr int H = decltype(Hc)::value;
      dma_barrier<(NB - 2) * NLD>();             // step s landed, everyone done with step s-1
      issue(std::integral_constant<int, H + NB - 1>{}, s + NB - 1);
      MLA_LDS char* kb = buf(Hc);
      MLA_LDS char* vb = kb + KBYTES;
      float kscl = 1.f, vscl = 1.f;              // fp8: this step's K and V scales
      if constexpr (KV8) {
        if (p.k_scale) kscl = sbuf(Hc)[0];
        if (p.v_scale) vscl = sbuf(Hc)[4 * 64];
      }
      // S^T tiles: keys kt*16 + 4g .. +4 of row li of tile rt
      f32x4 sc4[KT][RTW];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) sc4[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const MLA_LDS char* krow = kb + (kt * 16 + li) * ROWB;
        if constexpr (KV8) {
#pragma unroll
          for (int m = 0; m < DC / 2; ++m) {
            const u32x4 kw = ld_lds16(krow + (((m * 4 + g) ^ ksw) << 4));
            const u32x4 ka = e4m3x8_to_bf16(kw[0], kw[1]);
            const u32x4 kc = e4m3x8_to_bf16(kw[2], kw[3]);
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
              sc4[kt][rt] = Dt<T>::mfma32(ka, qf[rt][2 * m], sc4[kt][rt]);
              sc4[kt][rt] = Dt<T>::mfma32(kc, qf[rt][2 * m + 1], sc4[kt][rt]);
            }
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < DC; ++ks) {
            const u32x4 kf = ld_lds16(krow + (((ks * 4 + g) ^ ksw) << 4));
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) sc4[kt][rt] = Dt<T>::mfma32(kf, qf[rt][ks], sc4[kt][rt]);
          }
        }
      }
      // online softmax per row tile; probabilities packed as the B operand of
      // the P.V MFMA: k-slots 8g .. 8g+7 = keys 4g..4g+3 of tiles 2kp, 2kp+1
      u32x4 pf[RTW][KT / 2];
      float alpha[RTW];
      const int key0 = (ks0 + s) * KS + 4 * g;
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        float x[KT][4];
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[kt][e] = (key0 + kt * 16 + e < cnt[rt]) ? sc4[kt][rt][e] * kscl : -INFINITY;
            mx = fmaxf(mx, x[kt][e]);
          }
        mx = max_across_groups(mx) * p.scale_log2;   // scale > 0 commutes with the max
        alpha[rt] = 1.f;
        if (mx > m_run[rt] + kRescaleSlack) {
          alpha[rt] = __builtin_amdgcn_exp2f(m_run[rt] - mx);
          m_run[rt] = mx;
        }
        const float msub = (m_run[rt] == -INFINITY) ? 0.f : m_run[rt];
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[kt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[kt][e], p.scale_log2, -msub));
            rs += x[kt][e];
          }
        l_part[rt] = l_part[rt] * alpha[rt] + rs;
        if constexpr (KV8) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[kt][e] *= vscl;
        }
#pragma unroll
        for (int kp = 0; kp < KT / 2; ++kp)
          pf[rt][kp] = u32x4{Dt<T>::pack2(x[2 * kp][0], x[2 * kp][1]), Dt<T>::pack2(x[2 * kp][2], x[2 * kp][3]),
                             Dt<T>::pack2(x[2 * kp + 1][0], x[2 * kp + 1][1]),
                             Dt<T>::pack2(x[2 * kp + 1][2], x[2 * kp + 1][3])};
      }
      bool resc = false;
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) resc |= alpha[rt] != 1.f;
      if (__any(resc)) {
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) o[rt][ct] *= alpha[rt];
      }
      // O^T += V^T . P^T for this wave's columns: transposed reads of value
      // rows 32kp + 4g + li/4 (lo) and +16 (hi), columns 4(li&3) .. +4 of the
      // 16-column tile
      if constexpr (KV8) {
        // lane 2r + h of group g addresses key slot r (keys 4g..4g+3, then
        // 16+4g..16+4g+3 of the pair), column bytes 8h .. 8h+7 of the tile
        const int vs = li >> 1;
        const int vkey = vs < 4 ? 4 * g + vs : 12 + 4 * g + vs;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int chunk = (cb + ct * 16) / 16;
#pragma unroll
          for (int kp = 0; kp < KT / 2; ++kp) {
            const int r = 32 * kp + vkey;
            // the offset masked to the V half, so the compiler can see that the
            // read stays inside this buffer (else it waits for every load in flight)
            const int off = (r * ROWB + ((chunk ^ mha_swz<CPR>(r)) << 4) + (li & 1) * 8) & (KBYTES - 1);
            const u32x2 w = mha_ld_tr8(vb + off);
            const u32x4 vf = e4m3x8_to_bf16(w[0], w[1]);
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) o[rt][ct] = Dt<T>::mfma32(vf, pf[rt][kp], o[rt][ct]);
          }
        }
      } else {
        const int vr = 4 * g + (li >> 2);
        const int vsw = mha_swz<CPR>(vr);          // the same for vr + 16, vr + 32
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int chunk = (cb + ct * 16) / 8 + ((li >> 1) & 1);
          const int coff = ((chunk ^ vsw) << 4) + (li & 1) * 8;
#pragma unroll
          for (int kp = 0; kp < KT / 2; ++kp) {
            const u32x2 lo4 = ld_lds_tr(vb + (32 * kp + vr) * ROWB + coff);
            const u32x2 hi4 = ld_lds_tr(vb + (32 * kp + 16 + vr) * ROWB + coff);
            const u32x4 vf = u32x4{lo4[0], lo4[1], hi4[0], hi4[1]};
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) o[rt][ct] = Dt<T>::mfma32(vf, pf[rt][kp], o[rt][ct]);
          }
        }
      }
    };
    // whole groups of NB steps, then the tail: every step of the loop body
    // runs, so the compiler sees which buffer each load in flight targets
    int s0 = 0;
    for (; s0 + NB <= nsteps; s0 += NB) static_for<0, NB>([&](auto Hc) { step(Hc, s0 + decltype(Hc)::value); });
    static_for<0, NB - 1>([&](auto Hc) {
      const int s = s0 + decltype(Hc)::value;
      if (s < nsteps) step(Hc, s);
    });
    // drain the loads issued past the end before the buffers are reused
    dma_barrier<0>();

    // epilogue: O / l, LSE; wave w writes its columns, wave 0 the LSEs
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const float l = sum_across_groups(l_part[rt]);
      const int row = mrow0 + rt * 16 + li;
      if (row >= p.rows) continue;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const float lse = l > 0.f ? (m_run[rt] + __log2f(l)) * kLn2 : -INFINITY;
      const int tok = row / p.group;
      const int head = hk * p.group + (row - tok * p.group);
      if (nsplit == 1) {
        T* dst = (T*)p.out + b * p.o_s0 + tok * p.o_s1 + head * p.o_s2 + cb + 4 * g;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const f32x4 v = o[rt][ct] * inv;
          *(u32x2*)(dst + ct * 16) = u32x2{Dt<T>::pack2(v[0], v[1]), Dt<T>::pack2(v[2], v[3])};
        }
        if ((RS || wave == 0) && g == 0) p.lse[((int64_t)b * p.s_q + tok) * p.h_q + head] = lse;
      } else {
        const int64_t slot = slot0 + split;
        float* dst = p.part_o + (slot * p.rows + row) * DV + cb + 4 * g;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) *(f32x4*)(dst + ct * 16) = o[rt][ct] * inv;
        if ((RS || wave == 0) && g == 0) p.part_lse[slot * p.rows + row] = lse;
      }
    }
  }
}

// ----------------------------------------------------------- key split --
// Variant for few query rows per unit (row tiles RT with RT * d <= 256): the
// four waves split each step's 64 keys instead of the output columns.  Wave w
// scores keys 16w .. 16w+15 of the step for all of the block's rows, runs its
// own online softmax over them and accumulates all d output columns from its
// own keys (16x16x16 MFMAs, the P^T operand straight from the score
// registers); the four partial states merge once per chunk through LDS.  Per
// step and wave this is a quarter of the score MFMAs, operand reads, fp8
// conversions and softmax arithmetic of the column-split kernel above, which
// repeats all of them in every wave; at one wave per SIMD that instruction
// stream, not HBM, bounds the column-split kernel for small groups.
// The staging of K and V (LDS-DMA, buffers named at compile time, steps in
// flight, fp8 scales) is that of the kernel above.
template <typename T, int D, int RT, bool KV8, bool NT>
__global__ __launch_bounds__(256, 1) void mha_keysplit_kernel(MhaParams p) {
  constexpr int KS = 64;                     // keys per step (one page), 16 per wave
  constexpr int ESZ = KV8 ? 1 : 2;
  constexpr int ROWB = D * ESZ;
  constexpr int CPR = ROWB / 16;
  constexpr int KBYTES = KS * ROWB;
  constexpr int BUF = 2 * KBYTES;
  constexpr int SCB = KV8 ? 2 * 4 * 64 * 4 : 0;
  constexpr int MRG = RT * D * 64;           // one wave's partial O in the merge
  constexpr int BUFA = BUF + SCB > MRG ? BUF + SCB : MRG;
  // four buffers, three steps in flight: eight (seven in flight) measured 2 %
  // slower on an fp8 GQA workload, so the K/V stream is not what bounds it
  constexpr int NB = 4;
  constexpr int DC = D / 32;
  constexpr int NCT = D / 16;                // 16-column output tiles (all of them, per wave)
  constexpr int MCT = NCT / 4;               // tiles each wave merges
  constexpr int NDMA = 2 * KBYTES / 1024 / 4;
  constexpr int NLD = NDMA + (KV8 ? 2 : 0);
  constexpr int RPI = 1024 / ROWB;
  static_assert(RT * D <= 256 && MCT >= 1 && NDMA >= 1 && 2 * KBYTES % 4096 == 0, "tile shape");
  static_assert((NB - 1) * NLD <= 63, "loads in flight fit the wait counter");
  static_assert(NB * BUFA <= 160 * 1024 - 2 * 4 * 64 * 4, "LDS");
  // non-temporal loads when a unit's rows fit one row block (its K/V rows are
  // then read once); with several row blocks they share the pages in L2
  constexpr int kAux = NT ? 2 : 0;
  __shared__ __attribute__((aligned(1024))) char b0_raw[BUFA];
  __shared__ __attribute__((aligned(1024))) char b1_raw[BUFA];
  __shared__ __attribute__((aligned(1024))) char b2_raw[BUFA];
  __shared__ __attribute__((aligned(1024))) char b3_raw[BUFA];
  __shared__ float ml_s[2][4][64];           // merge: each wave's row maxima and sums
  auto buf = [&](auto ic) -> MLA_LDS char* {
    constexpr int i = decltype(ic)::value % NB;
    if constexpr (i == 0) return (MLA_LDS char*)b0_raw;
    else if constexpr (i == 1) return (MLA_LDS char*)b1_raw;
    else if constexpr (i == 2) return (MLA_LDS char*)b2_raw;
    else return (MLA_LDS char*)b3_raw;
  };
  auto sbuf = [&](auto ic) -> MLA_LDS float* { return (MLA_LDS float*)(buf(ic) + BUF); };

  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int mrow0 = blockIdx.y * 64;
  const int krow = 16 * wave + li;           // K row of the step this lane feeds to the score MFMAs
  const int ksw = mha_swz<CPR>(krow);

  // this lane's source offset (within the step's first page row) for each of
  // the wave's DMA instructions: instruction j moves 1 KiB, K rows then V
  // rows, lane l filling slot l, i.e. row j*RPI + l / CPR, chunk
  // (l % CPR) ^ swizzle(row).  Computed once: rebuilt per step, the 64-bit
  // stride products cost more than the loads' issue.
  int doff[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int j = wave * NDMA + i;
    const bool isv = j >= KBYTES / 1024;
    const int jj = isv ? j - KBYTES / 1024 : j;
    const int r = jj * RPI + lane / CPR;
    const int c = (lane % CPR) ^ mha_swz<CPR>(r);
    const int64_t rs = isv ? p.v_s1 : p.k_s1;
    doff[i] = (int)(r * rs * ESZ) + c * 16;
  }

  // the schedule row, precomputed or derived here
  const PartRow pr = part_row(p.sched, p.seqlens, p.batch * p.h_kv, p.h_kv, p.num_parts, p.sched_f, blockIdx.x);
  const int len0 = pr.len0;
  int sched_start = pr.start, sched_slot = pr.slot;
  for (int u = pr.begin; u <= pr.end; ++u) {
    const int b = u / p.h_kv;
    const int hk = u - b * p.h_kv;
    const int n = (pr.inl && u == pr.begin) ? len0 : ldu(p.seqlens + b);
    const int npages = (n + kPage - 1) / kPage;
    int slot0, nsplit;
    unit_slots(pr.inl, p.split_offsets, u, n, p.sched_f, pr.width, sched_start, sched_slot, slot0, nsplit);
    const int lo = (u == pr.begin) ? pr.begin_page : 0;
    const int hi = (u == pr.end) ? pr.end_page : npages;
    if (lo >= hi) continue;
    const int split = (u == pr.begin) ? pr.begin_split : 0;
    const int nsteps = hi - lo;              // one step per page

    BlockWindow bw;
    bw.init(p.block_table + (int64_t)b * p.bt_s, lo, hi, lane);

    // Q fragments: the B operand of S^T = K . Q^T, as in the kernel above
    u32x4 qf[RT][DC];
    int cnt[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = mrow0 + rt * 16 + li;
      if (row < p.rows) {
        const int tok = row / p.group;
        const int head = hk * p.group + (row - tok * p.group);
        const T* qp = (const T*)p.q + b * p.q_s0 + tok * p.q_s1 + head * p.q_s2 + 8 * g;
#pragma unroll
        for (int ks = 0; ks < DC; ++ks) {
          const int col = KV8 ? 64 * (ks >> 1) + 8 * g + 8 * (ks & 1) : ks * 32;   // past qp's 8g
          qf[rt][ks] = *(const u32x4*)(qp + col);
        }
        cnt[rt] = visible_count(n, p.s_q, tok, p.causal);
      } else {
#pragma unroll
        for (int ks = 0; ks < DC; ++ks) qf[rt][ks] = u32x4{0, 0, 0, 0};
        cnt[rt] = 0;
      }
    }

    // LDS-DMA loads of page lo + s into buffer ic (every wave moves NDMA KiB
    // of the K then V rows, at the offsets doff); steps past the chunk use
    // empty descriptors, so every step issues the same loads.
    auto issue = [&](auto ic, int s) {
      MLA_LDS char* bp = buf(ic);
      const bool real = s < nsteps;
      const int page = lo + s;
      const int phys = real ? bw.phys(page) : 0;
      const int valid = real ? min(kPage, n - page * kPage) : 0;
      const BufRsrc kr = mha_rows_rsrc<ESZ>(p.k, (int64_t)phys * p.k_s0 + hk * p.k_s2, p.k_s1, D, valid);
      const BufRsrc vr = mha_rows_rsrc<ESZ>(p.v, (int64_t)phys * p.v_s0 + hk * p.v_s2, p.v_s1, D, valid);
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int j = wave * NDMA + i;
        const bool isv = j >= KBYTES / 1024;
        const int jj = isv ? j - KBYTES / 1024 : j;
        dma16<kAux>(isv ? vr : kr, bp + (isv ? KBYTES : 0) + jj * 1024, doff[i], 0);
      }
      if constexpr (KV8) {
        MLA_LDS float* sp = sbuf(ic) + wave * 64;
        const int soff = (phys * p.h_kv + hk) * 4;
        const BufRsrc ksr = page_rsrc((const char*)p.k_scale, p.k_scale && real ? 0x7FFFFFFF : 0);
        const BufRsrc vsr = page_rsrc((const char*)p.v_scale, p.v_scale && real ? 0x7FFFFFFF : 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ksr, (MLA_LDS void*)sp, 4, 0, soff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vsr, (MLA_LDS void*)(sp + 4 * 64), 4, 0, soff, 0, 0);
      }
    };

    float m_run[RT], l_part[RT];
    f32x4 o[RT][NCT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      m_run[rt] = -INFINITY;
      l_part[rt] = 0.f;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) o[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    static_for<0, NB - 1>([&](auto ic) { issue(ic, decltype(ic)::value); });

    auto step = [&](auto Hc, int s) {
      constexpr int H = decltype(Hc)::value;
      dma_barrier<(NB - 2) * NLD>();             // step s landed, everyone done with step s-1
      issue(std::integral_constant<int, H + NB - 1>{}, s + NB - 1);
      MLA_LDS char* kb = buf(Hc);
      MLA_LDS char* vb = kb + KBYTES;
      // operand reads first (with one wave per SIMD nothing else hides their
      // latency): the K rows of this wave's keys, then the V^T tiles
      const MLA_LDS char* kp = kb + krow * ROWB;
      u32x4 kf[KV8 ? DC / 2 : DC];
#pragma unroll
      for (int m = 0; m < (KV8 ? DC / 2 : DC); ++m) kf[m] = ld_lds16(kp + (((m * 4 + g) ^ ksw) << 4));
      // V^T: bf16 - lane (li, g) addresses key 16w + 4g + li/4, columns
      // 16ct + 4(li&3) .. +4 and receives column li of keys 16w+4g .. +4;
      // fp8 - lane 2r + h addresses key 16w + 4g + (r&3), bytes 8h..8h+7 of
      // tile 2cp + r/4, and receives column li of those four keys in tiles
      // 2cp and 2cp + 1
      constexpr int NVR = KV8 ? NCT / 2 : NCT;
      u32x2 vw[NVR];
      if constexpr (KV8) {
        const int vrow = 16 * wave + 4 * g + ((li >> 1) & 3);
        const int vsw = mha_swz<CPR>(vrow);
#pragma unroll
        for (int cp = 0; cp < NVR; ++cp) {
          const int chunk = 2 * cp + (li >> 3);
          const int off = (vrow * ROWB + ((chunk ^ vsw) << 4) + (li & 1) * 8) & (KBYTES - 1);
          vw[cp] = mha_ld_tr8(vb + off);
        }
      } else {
        const int vrow = 16 * wave + 4 * g + (li >> 2);
        const int vsw = mha_swz<CPR>(vrow);
#pragma unroll
        for (int ct = 0; ct < NVR; ++ct) {
          const int chunk = 2 * ct + ((li >> 1) & 1);
          const int off = (vrow * ROWB + ((chunk ^ vsw) << 4) + (li & 1) * 8) & (KBYTES - 1);
          vw[ct] = ld_lds_tr(vb + off);
        }
      }
      float kscl = 1.f, vscl = 1.f;
      if constexpr (KV8) {
        if (p.k_scale) kscl = sbuf(Hc)[0];
        if (p.v_scale) vscl = sbuf(Hc)[4 * 64];
      }
      // S^T: keys 16w + 4g .. +4 (of the step) of row li of tile rt
      f32x4 sc4[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sc4[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (KV8) {
#pragma unroll
        for (int m = 0; m < DC / 2; ++m) {
          const u32x4 ka = e4m3x8_to_bf16(kf[m][0], kf[m][1]);
          const u32x4 kc = e4m3x8_to_bf16(kf[m][2], kf[m][3]);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            sc4[rt] = Dt<T>::mfma32(ka, qf[rt][2 * m], sc4[rt]);
            sc4[rt] = Dt<T>::mfma32(kc, qf[rt][2 * m + 1], sc4[rt]);
          }
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < DC; ++ks)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) sc4[rt] = Dt<T>::mfma32(kf[ks], qf[rt][ks], sc4[rt]);
      }
      // online softmax over this wave's keys; P^T operand = the lane's four
      // probabilities (keys 4g .. 4g+3 of the wave's 16, row li)
      u32x2 pf[RT];
      float alpha[RT];
      const int key0 = (lo + s) * KS + 16 * wave + 4 * g;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float x[4];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = (key0 + e < cnt[rt]) ? sc4[rt][e] * kscl : -INFINITY;
          mx = fmaxf(mx, x[e]);
        }
        mx = max_across_groups(mx) * p.scale_log2;
        alpha[rt] = 1.f;
        if (mx > m_run[rt] + kRescaleSlack) {
          alpha[rt] = __builtin_amdgcn_exp2f(m_run[rt] - mx);
          m_run[rt] = mx;
        }
        const float msub = (m_run[rt] == -INFINITY) ? 0.f : m_run[rt];
        float rs = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], p.scale_log2, -msub));
          rs += x[e];
        }
        l_part[rt] = l_part[rt] * alpha[rt] + rs;
        if constexpr (KV8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] *= vscl;
        }
        pf[rt] = u32x2{Dt<T>::pack2(x[0], x[1]), Dt<T>::pack2(x[2], x[3])};
      }
      bool resc = false;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) resc |= alpha[rt] != 1.f;
      if (__any(resc)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) o[rt][ct] *= alpha[rt];
      }
      // O^T += V^T . P^T over the wave's 16 keys, every column tile
      if constexpr (KV8) {
#pragma unroll
        for (int cp = 0; cp < NVR; ++cp) {
          const u32x4 vf = e4m3x8_to_bf16(vw[cp][0], vw[cp][1]);
          const u32x2 va = u32x2{vf[0], vf[1]}, vc = u32x2{vf[2], vf[3]};
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            o[rt][2 * cp] = Dt<T>::mfma16(va, pf[rt], o[rt][2 * cp]);
            o[rt][2 * cp + 1] = Dt<T>::mfma16(vc, pf[rt], o[rt][2 * cp + 1]);
          }
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) o[rt][ct] = Dt<T>::mfma16(vw[ct], pf[rt], o[rt][ct]);
      }
    };
    int s0 = 0;
    for (; s0 + NB <= nsteps; s0 += NB) static_for<0, NB>([&](auto Hc) { step(Hc, s0 + decltype(Hc)::value); });
    static_for<0, NB - 1>([&](auto Hc) {
      const int s = s0 + decltype(Hc)::value;
      if (s < nsteps) step(Hc, s);
    });
    // drain the loads issued past the end; after this barrier no wave reads
    // the buffers, which now take the partial states
    dma_barrier<0>();

    // merge of the four waves' states: wave w's O tiles go to buffer w as
    // [rt][ct][lane] (16 bytes per lane), its row maxima and sums to ml_s
    {
      MLA_LDS char* mine = wave == 0 ? buf(std::integral_constant<int, 0>{})
                         : wave == 1 ? buf(std::integral_constant<int, 1>{})
                         : wave == 2 ? buf(std::integral_constant<int, 2>{})
                                     : buf(std::integral_constant<int, 3>{});
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float l = sum_across_groups(l_part[rt]);
        if (g == 0) {
          ml_s[0][wave][rt * 16 + li] = m_run[rt];
          ml_s[1][wave][rt * 16 + li] = l;
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) *(MLA_LDS f32x4*)(mine + ((rt * NCT + ct) * 64 + lane) * 16) = o[rt][ct];
      }
    }
    lds_barrier();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = mrow0 + rt * 16 + li;
      float mw[4], M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        mw[w] = ml_s[0][w][rt * 16 + li];
        M = fmaxf(M, mw[w]);
      }
      float sw[4], L = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        sw[w] = (mw[w] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
        L += sw[w] * ml_s[1][w][rt * 16 + li];
      }
      if (row >= p.rows) continue;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      const float lse = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
      const int tok = row / p.group;
      const int head = hk * p.group + (row - tok * p.group);
      f32x4 acc[MCT];
#pragma unroll
      for (int j = 0; j < MCT; ++j) {
        const int ct = wave * MCT + j;
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        static_for<0, 4>([&](auto wc) {
          constexpr int w = decltype(wc)::value;
          const f32x4 v = *(const MLA_LDS f32x4*)(buf(wc) + ((rt * NCT + ct) * 64 + lane) * 16);
          acc[j] += v * sw[w];
        });
        acc[j] *= inv;
      }
      if (nsplit == 1) {
        T* dst = (T*)p.out + b * p.o_s0 + tok * p.o_s1 + head * p.o_s2 + 4 * g;
#pragma unroll
        for (int j = 0; j < MCT; ++j)
          *(u32x2*)(dst + (wave * MCT + j) * 16) = u32x2{Dt<T>::pack2(acc[j][0], acc[j][1]),
                                                         Dt<T>::pack2(acc[j][2], acc[j][3])};
        if (wave == 0 && g == 0) p.lse[((int64_t)b * p.s_q + tok) * p.h_q + head] = lse;
      } else {
        const int64_t slot = slot0 + split;
        float* dst = p.part_o + (slot * p.rows + row) * D + 4 * g;
#pragma unroll
        for (int j = 0; j < MCT; ++j) *(f32x4*)(dst + (wave * MCT + j) * 16) = acc[j];
        if (wave == 0 && g == 0) p.part_lse[slot * p.rows + row] = lse;
      }
    }
    // the buffers are refilled by the next chunk's loads: everyone must be
    // done reading the partial states first
    lds_barrier();
  }
}

// ------------------------------------------------------------- combine --
// Merge of the split pieces of a unit by their LSE (the same identity as the
// MLA combine): LSE = log sum_k exp(LSE_k), O = sum_k exp(LSE_k - LSE) O_k.
// One wave per row, DV / 64 (at least 2) columns per lane; lane k holds piece k's LSE for
// the reductions; eight pieces' loads in flight.  Units with no cached token
// get O = 0 and LSE = -inf; unsplit units are skipped.
template <typename T, int DV>
__global__ __launch_bounds__(256) void mha_combine_kernel(MhaParams p) {
  constexpr int CPL = DV >= 128 ? DV / 64 : 2;   // columns per lane (lanes past DV / CPL idle)
  typedef float fv __attribute__((ext_vector_type(CPL)));
  const int u = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + wave;
  if (row >= p.rows) return;
  int s0, ns;
  if (p.split_offsets) {
    s0 = ldu(p.split_offsets + u);
    ns = ldu(p.split_offsets + u + 1) - s0;
  } else {                                       // the schedule derived in place
    int before, own;
    sched_slots(p.seqlens, p.batch * p.h_kv, p.h_kv, p.num_parts, p.sched_f, u, before, own);
    s0 = __builtin_amdgcn_readfirstlane(before);   // lane 0 holds unit u
    ns = __builtin_amdgcn_readfirstlane(own);
  }
  if (ns == 1) return;
  const int b = u / p.h_kv, hk = u - b * p.h_kv;
  const int tok = row / p.group;
  const int head = hk * p.group + (row - tok * p.group);
  const int col = min(lane * CPL, DV - CPL);      // idle lanes repeat the last columns
  const bool writer = lane * CPL < DV;
  fv acc;
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
  float L = -INFINITY;
  const float* lse_k = p.part_lse + (int64_t)s0 * p.rows + row;
  const float* src = p.part_o + ((int64_t)s0 * p.rows + row) * DV + col;
  const int64_t piece = (int64_t)p.rows * DV;
  if (ns > 0) {
    float mx = -INFINITY;
    for (int k = lane; k < ns; k += 64) mx = fmaxf(mx, lse_k[(int64_t)k * p.rows]);
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sft));
    if (mx != -INFINITY) {
      float sum = 0.f;
      for (int k = lane; k < ns; k += 64) sum += __builtin_amdgcn_exp2f((lse_k[(int64_t)k * p.rows] - mx) * kLog2e);
#pragma unroll
      for (int sft = 32; sft >= 1; sft >>= 1) sum += __shfl_xor(sum, sft);
      L = mx + __logf(sum);
      for (int k0 = 0; k0 < ns; k0 += 64) {
        const int kl = k0 + lane;
        const float w = kl < ns ? __builtin_amdgcn_exp2f((lse_k[(int64_t)kl * p.rows] - L) * kLog2e) : 0.f;
        const int cnt = min(64, ns - k0);
        for (int j = 0; j < cnt; j += 8) {
          fv v[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            if (j + t < cnt) {
              v[t] = *(const fv*)(src + (k0 + j + t) * piece);
            } else {
#pragma unroll
              for (int i = 0; i < CPL; ++i) v[t][i] = 0.f;
            }
          }
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(j + t, 63)));
            if (j + t < cnt) acc += wt * v[t];
          }
        }
      }
    }
  }
  T* dst = (T*)p.out + b * p.o_s0 + tok * p.o_s1 + head * p.o_s2 + col;
  if (writer) {
#pragma unroll
    for (int i = 0; i < CPL; i += 2) *(uint32_t*)(dst + i) = Dt<T>::pack2(acc[i], acc[i + 1]);
  }
  if (lane == 0) p.lse[((int64_t)b * p.s_q + tok) * p.h_q + head] = L;
}

namespace {

// Key-split kernel for fp8 caches where its per-wave state fits
// (RT * d <= 256).  With bf16/fp16 caches the column-split kernel is HBM
// bound already and measured 4 % faster on two GQA workloads.
template <typename T, int D, bool KV8, int RT>
constexpr bool kKeySplit = KV8 && RT * D <= 256;

template <typename T, int D, bool KV8, int RT>
bool launch_keysplit(int rt, dim3 grid, const MhaParams& p, hipStream_t st) {
  if constexpr (kKeySplit<T, D, KV8, RT>) {
    if (rt == RT) {
      if (grid.y == 1) hipLaunchKernelGGL((mha_keysplit_kernel<T, D, RT, KV8, true>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((mha_keysplit_kernel<T, D, RT, KV8, false>), grid, dim3(256), 0, st, p);
      return true;
    }
  }
  return false;
}

template <typename T, int D, bool KV8>
hipError_t launch_mha_d(const MhaParams& p, hipStream_t st) {
  const int m_blocks = (p.rows + 63) / 64;
  const int rt = p.rows >= 64 ? 4 : (p.rows + 15) / 16;
  const dim3 grid(p.num_parts, m_blocks);
  if (launch_keysplit<T, D, KV8, 1>(rt, grid, p, st) || launch_keysplit<T, D, KV8, 2>(rt, grid, p, st) ||
      launch_keysplit<T, D, KV8, 3>(rt, grid, p, st) || launch_keysplit<T, D, KV8, 4>(rt, grid, p, st))
    return hipGetLastError();
  // one row tile: the column split; more: the row split (no wave repeats
  // another's scores)
  switch (rt) {
    case 1: hipLaunchKernelGGL((mha_splitkv_kernel<T, D, 1, KV8, false, true>), grid, dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL((mha_splitkv_kernel<T, D, 2, KV8, true, true>), grid, dim3(256), 0, st, p); break;
    case 3: hipLaunchKernelGGL((mha_splitkv_kernel<T, D, 3, KV8, true, true>), grid, dim3(256), 0, st, p); break;
    default:
      if (m_blocks == 1) hipLaunchKernelGGL((mha_splitkv_kernel<T, D, 4, KV8, true, true>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((mha_splitkv_kernel<T, D, 4, KV8, true, false>), grid, dim3(256), 0, st, p);
      break;
  }
  return hipGetLastError();
}

template <typename T, bool KV8>
hipError_t launch_mha_t(const MhaParams& p, int head_dim, hipStream_t st) {
  switch (head_dim) {
    case 64: return launch_mha_d<T, 64, KV8>(p, st);
    case 128: return launch_mha_d<T, 128, KV8>(p, st);
    case 256: return launch_mha_d<T, 256, KV8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_mha_combine_t(const MhaParams& p, int head_dim, hipStream_t st) {
  const dim3 grid(p.batch * p.h_kv, (p.rows + 3) / 4);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((mha_combine_kernel<T, 64>), grid, dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL((mha_combine_kernel<T, 128>), grid, dim3(256), 0, st, p); break;
    case 256: hipLaunchKernelGGL((mha_combine_kernel<T, 256>), grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mha_splitkv(const MhaParams& p, int dtype, int head_dim, hipStream_t st) {
  if (p.kv_fp8) return launch_mha_t<__bf16, true>(p, head_dim, st);
  return dtype == 0 ? launch_mha_t<__bf16, false>(p, head_dim, st) : launch_mha_t<_Float16, false>(p, head_dim, st);
}

hipError_t launch_mha_combine(const MhaParams& p, int dtype, int head_dim, hipStream_t st) {
  return dtype == 0 ? launch_mha_combine_t<__bf16>(p, head_dim, st) : launch_mha_combine_t<_Float16>(p, head_dim, st);
}

}  // namespace mla
