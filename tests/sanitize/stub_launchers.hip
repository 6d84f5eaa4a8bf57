// Stand-ins for the kernel launchers of mla_internal.h, for the host-side
// sanitizer build of the C ABI: they record what the ABI asked for and launch
// nothing, so the argument checks and the dispatch run without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../mla_decode_attention_02_amd/csrc/mla_common.hpp"
#include "../../mla_decode_attention_02_amd/csrc/mla_internal.h"

namespace {
std::atomic<int> g_calls[10];
thread_local int t_num_parts, t_rows, t_fuse_max, t_m_blocks, t_fixed, t_units, t_kv_fp8;
}  // namespace

enum { WIDE, NARROW, FP8, WIDE_FP8, COMBINE, MERGE, METADATA, MHA_SPLITKV, MHA_COMBINE, NKINDS };

namespace mla {

static void note(int kind, const DecodeParams* p, int m_blocks) {
  g_calls[kind]++;
  if (p) {
    t_num_parts = p->num_parts;
    t_rows = p->rows;
    t_fuse_max = p->fuse_max;
    t_kv_fp8 = p->kv_fp8;
  }
  if (m_blocks >= 0) t_m_blocks = m_blocks;
}

hipError_t launch_splitkv_wide(const DecodeParams& p, int, int m_blocks, hipStream_t) {
  note(WIDE, &p, m_blocks);
  return hipSuccess;
}
hipError_t launch_splitkv_narrow(const DecodeParams& p, int, hipStream_t) {
  note(p.kv_fp8 ? FP8 : NARROW, &p, 1);
  return hipSuccess;
}
hipError_t launch_splitkv_fp8(const DecodeParams& p, hipStream_t) {
  note(FP8, &p, 1);
  return hipSuccess;
}
hipError_t launch_splitkv_wide_fp8(const DecodeParams& p, int m_blocks, hipStream_t) {
  note(WIDE_FP8, &p, m_blocks);
  return hipSuccess;
}
hipError_t launch_combine(const DecodeParams& p, int, hipStream_t) {
  note(COMBINE, &p, -1);
  return hipSuccess;
}
hipError_t launch_merge(const MergeParams&, int, hipStream_t) {
  note(MERGE, nullptr, -1);
  return hipSuccess;
}
hipError_t launch_metadata(const int32_t*, int units, int, int num_parts, int fixed_overhead, int32_t*, int32_t*,
                           hipStream_t) {
  note(METADATA, nullptr, -1);
  t_units = units;
  t_num_parts = num_parts;
  t_fixed = fixed_overhead;
  return hipSuccess;
}
hipError_t launch_mha_splitkv(const MhaParams& p, int, int, hipStream_t) {
  g_calls[MHA_SPLITKV]++;
  t_num_parts = p.num_parts;
  t_rows = p.rows;
  return hipSuccess;
}
hipError_t launch_mha_combine(const MhaParams&, int, int, hipStream_t) {
  g_calls[MHA_COMBINE]++;
  return hipSuccess;
}

}  // namespace mla

extern "C" int stub_calls(int kind) { return g_calls[kind].load(); }
extern "C" int stub_last(int what) {
  switch (what) {
    case 0: return t_num_parts;
    case 1: return t_rows;
    case 2: return t_fuse_max;
    case 3: return t_m_blocks;
    case 4: return t_fixed;
    case 5: return t_units;
    default: return t_kv_fp8;
  }
}
