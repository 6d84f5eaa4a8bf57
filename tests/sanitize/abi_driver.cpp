// Host-side driver of the C ABI for the AddressSanitizer / UndefinedBehavior-
// Sanitizer build: every entry point through its rejections and, with the
// kernel launchers replaced by stubs, through its dispatch; then the same
// calls from several threads at once.  Exits non-zero on the first wrong
// status; the sanitizers abort on any memory or UB error they see.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/mha_decode.h"
#include "../../include/mla_decode.h"

extern "C" int stub_calls(int kind);
extern "C" int stub_last(int what);
enum { WIDE, NARROW, FP8, WIDE_FP8, COMBINE, MERGE, METADATA, MHA_SPLITKV, MHA_COMBINE };
enum { NUM_PARTS, ROWS, FUSE_MAX, M_BLOCKS, FIXED, UNITS, KV_FP8 };

static int g_fail = 0;
#define EXPECT(cond)                                                                 \
  do {                                                                               \
    if (!(cond)) {                                                                   \
      std::fprintf(stderr, "%s:%d: expectation failed: %s (last error: %s)\n", __FILE__, \
                   __LINE__, #cond, mla_last_error());                               \
      ++g_fail;                                                                      \
    }                                                                                \
  } while (0)

// fake, never dereferenced device addresses (aligned)
static void* addr(uintptr_t a) { return reinterpret_cast<void*>(a); }

static mla_decode_args valid_args(int h_q, int kv_fp8) {
  mla_decode_args a;
  std::memset(&a, 0, sizeof(a));
  a.dtype = MLA_DTYPE_BF16;
  a.batch = 2;
  a.s_q = 1;
  a.h_q = h_q;
  a.h_kv = 1;
  a.d_k = 576;
  a.d_v = 512;
  a.page_size = 64;
  a.num_pages = 3;
  a.max_pages_per_seq = 2;
  a.q = addr(1 << 20);
  a.q_stride[0] = (int64_t)h_q * 576;
  a.q_stride[1] = (int64_t)h_q * 576;
  a.q_stride[2] = 576;
  a.k_cache = addr(2 << 20);
  a.k_stride[0] = 64 * 576;
  a.k_stride[1] = 576;
  a.k_stride[2] = 576;
  a.block_table = static_cast<const int32_t*>(addr(3 << 20));
  a.bt_stride = 2;
  a.cache_seqlens = static_cast<const int32_t*>(addr(4 << 20));
  a.sched = static_cast<const int32_t*>(addr(5 << 20));
  a.split_offsets = static_cast<const int32_t*>(addr(6 << 20));
  a.softmax_scale = 0.0416666f;
  a.num_parts = 4;
  size_t ws = 0;
  mla_workspace_size(a.batch, a.s_q, a.h_q, a.num_parts, &ws);
  a.workspace = addr(7 << 20);
  a.workspace_bytes = ws;
  a.out = addr(64 << 20);
  a.out_stride[0] = (int64_t)h_q * 512;
  a.out_stride[1] = (int64_t)h_q * 512;
  a.out_stride[2] = 512;
  a.lse = static_cast<float*>(addr(96 << 20));
  a.kv_dtype = kv_fp8 ? MLA_KV_FP8_E4M3 : MLA_KV_SAME;
  return a;
}

static void mla_entry_points() {
  EXPECT(mla_abi_version() == MLA_ABI_VERSION);
  EXPECT(mla_last_error() != nullptr);

  int parts = 0, se = 0, so = 0;
  EXPECT(mla_get_metadata_shape(256, 2, 1, 16, 1, &parts, &se, &so) == MLA_SUCCESS);
  EXPECT(parts == 256 && se == 256 * MLA_SCHED_FIELDS && so == 3);
  EXPECT(mla_get_metadata_shape(256, 64, 1, 128, 1, &parts, &se, &so) == MLA_SUCCESS && parts == 128);
  EXPECT(mla_get_metadata_shape(256, 32, 2, 128, 1, &parts, &se, &so) == MLA_SUCCESS && parts == 64);
  EXPECT(mla_get_metadata_shape(256, 0, 1, 16, 1, &parts, &se, &so) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_get_metadata_shape(256, 2, 1, 16, 2, &parts, &se, &so) == MLA_ERROR_UNSUPPORTED);
  EXPECT(mla_get_metadata_shape(256, 2, 1, 16, 1, nullptr, &se, &so) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_get_metadata_shape(-1, 2, 1, 16, 1, &parts, &se, &so) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_get_metadata_shape(1, 0x7fffffff, 0x7fffffff, 0x7fffffff, 1, &parts, &se, &so) ==
         MLA_ERROR_INVALID_VALUE);

  const int32_t* seq = static_cast<const int32_t*>(addr(4 << 20));
  int32_t* sched = static_cast<int32_t*>(addr(5 << 20));
  int32_t* offs = static_cast<int32_t*>(addr(6 << 20));
  const int meta0 = stub_calls(METADATA);
  EXPECT(mla_get_metadata(seq, 9, 1, 16, 1, 7, sched, offs, nullptr) == MLA_SUCCESS);
  EXPECT(stub_calls(METADATA) == meta0 + 1 && stub_last(FIXED) == MLA_FIXED_OVERHEAD && stub_last(UNITS) == 9 &&
         stub_last(NUM_PARTS) == 7);
  EXPECT(mla_get_metadata_ex(seq, 9, 1, 16, 1, 7, 64, sched, offs, nullptr) == MLA_SUCCESS && stub_last(FIXED) == 64);
  EXPECT(mla_get_metadata_ex(seq, 9, 1, 16, 1, 7, 65, sched, offs, nullptr) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_get_metadata_ex(seq, 9, 1, 16, 1, 7, -1, sched, offs, nullptr) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_get_metadata(nullptr, 9, 1, 16, 1, 7, sched, offs, nullptr) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_get_metadata(seq, 9, 1, 16, 1, 0, sched, offs, nullptr) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_get_metadata(seq + 1, 9, 1, 16, 1, 7, sched, offs, nullptr) == MLA_SUCCESS);   // 4-byte aligned
  EXPECT(mla_get_metadata(reinterpret_cast<const int32_t*>(addr((4 << 20) + 2)), 9, 1, 16, 1, 7, sched, offs,
                          nullptr) == MLA_ERROR_INVALID_VALUE);
  EXPECT(stub_calls(METADATA) == meta0 + 3);

  size_t ws = 0;
  EXPECT(mla_workspace_size(64, 1, 128, 128, &ws) == MLA_SUCCESS && ws > 0 && ws % 256 == 0);
  EXPECT(mla_workspace_size(64, 1, 128, 0, &ws) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_workspace_size(64, 1, 128, 128, nullptr) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_workspace_size(268435455, 2, 2048, 1 << 30, &ws) == MLA_SUCCESS);   // large, no overflow

  // dispatch: 16 rows -> narrow, more -> wide; fp8 caches to their kernels
  struct Case {
    int h_q, fp8, kind, m_blocks;
  } cases[] = {{16, 0, NARROW, 1}, {128, 0, WIDE, 2}, {16, 1, FP8, 1}, {128, 1, WIDE_FP8, 2}, {17, 0, WIDE, 1}};
  for (const Case& c : cases) {
    mla_decode_args a = valid_args(c.h_q, c.fp8);
    const int k0 = stub_calls(c.kind), c0 = stub_calls(COMBINE);
    EXPECT(mla_decode(&a, nullptr) == MLA_SUCCESS);
    EXPECT(stub_calls(c.kind) == k0 + 1 && stub_calls(COMBINE) == c0 + 1);
    EXPECT(stub_last(ROWS) == c.h_q && stub_last(FUSE_MAX) == 0 && stub_last(KV_FP8) == c.fp8);
    if (c.kind == WIDE || c.kind == WIDE_FP8) EXPECT(stub_last(M_BLOCKS) == c.m_blocks);
    EXPECT(mla_decode_fused(&a, nullptr) == MLA_SUCCESS && stub_last(FUSE_MAX) == MLA_FUSED_MAX_PIECES);
    EXPECT(mla_decode_splitkv(&a, nullptr) == MLA_SUCCESS);
    EXPECT(mla_decode_combine(&a, nullptr) == MLA_SUCCESS);
  }

  // each broken field is rejected before anything launches
  struct Break {
    const char* name;
    void (*apply)(mla_decode_args&);
    mla_status st;
  } breaks[] = {
      {"dtype", [](mla_decode_args& a) { a.dtype = 7; }, MLA_ERROR_UNSUPPORTED},
      {"d_k", [](mla_decode_args& a) { a.d_k = 512; }, MLA_ERROR_UNSUPPORTED},
      {"page", [](mla_decode_args& a) { a.page_size = 128; }, MLA_ERROR_UNSUPPORTED},
      {"h_kv", [](mla_decode_args& a) { a.h_kv = 2; }, MLA_ERROR_UNSUPPORTED},
      {"batch", [](mla_decode_args& a) { a.batch = 0; }, MLA_ERROR_INVALID_VALUE},
      {"q null", [](mla_decode_args& a) { a.q = nullptr; }, MLA_ERROR_INVALID_VALUE},
      {"q align", [](mla_decode_args& a) { a.q = addr((1 << 20) + 8); }, MLA_ERROR_INVALID_VALUE},
      {"q stride", [](mla_decode_args& a) { a.q_stride[2] = 4; }, MLA_ERROR_INVALID_VALUE},
      {"k stride", [](mla_decode_args& a) { a.k_stride[1] = 100; }, MLA_ERROR_INVALID_VALUE},
      {"k stride huge", [](mla_decode_args& a) { a.k_stride[1] = (int64_t)1 << 40; }, MLA_ERROR_INVALID_VALUE},
      {"bt stride", [](mla_decode_args& a) { a.bt_stride = 1; }, MLA_ERROR_INVALID_VALUE},
      {"scale nan", [](mla_decode_args& a) { a.softmax_scale = __builtin_nanf(""); }, MLA_ERROR_INVALID_VALUE},
      {"scale inf", [](mla_decode_args& a) { a.softmax_scale = __builtin_inff(); }, MLA_ERROR_INVALID_VALUE},
      {"scale 0", [](mla_decode_args& a) { a.softmax_scale = 0.f; }, MLA_ERROR_INVALID_VALUE},
      {"causal", [](mla_decode_args& a) { a.causal = 2; }, MLA_ERROR_INVALID_VALUE},
      {"kv dtype", [](mla_decode_args& a) { a.kv_dtype = 3; }, MLA_ERROR_UNSUPPORTED},
      {"fp8 fp16", [](mla_decode_args& a) { a.kv_dtype = MLA_KV_FP8_E4M3; a.dtype = MLA_DTYPE_FP16; },
       MLA_ERROR_UNSUPPORTED},
      {"workspace", [](mla_decode_args& a) { a.workspace_bytes -= 1; }, MLA_ERROR_WORKSPACE_TOO_SMALL},
      {"num_parts", [](mla_decode_args& a) { a.num_parts = 0; }, MLA_ERROR_INVALID_VALUE},
      {"rows", [](mla_decode_args& a) { a.h_q = 64 * 65535 + 1; }, MLA_ERROR_INVALID_VALUE},
  };
  const int before = stub_calls(NARROW) + stub_calls(WIDE) + stub_calls(COMBINE);
  for (const Break& b : breaks) {
    mla_decode_args a = valid_args(16, 0);
    b.apply(a);
    const mla_status st = mla_decode(&a, nullptr);
    if (st != b.st) std::fprintf(stderr, "break %s: status %d, expected %d\n", b.name, (int)st, (int)b.st);
    EXPECT(st == b.st);
    EXPECT(std::strlen(mla_last_error()) > 0);
  }
  EXPECT(stub_calls(NARROW) + stub_calls(WIDE) + stub_calls(COMBINE) == before);
  EXPECT(mla_decode(nullptr, nullptr) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_decode_fused(nullptr, nullptr) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mla_decode_noalloc(nullptr, nullptr) == MLA_ERROR_INVALID_VALUE);

  // the allocation-free entry point: oversized shapes are refused on the host;
  // a fitting one reaches the device lookup (an error here, without a GPU)
  {
    mla_decode_args a = valid_args(128, 0);
    a.batch = 64;
    a.num_parts = 256;
    EXPECT(mla_decode_noalloc(&a, nullptr) == MLA_ERROR_WORKSPACE_TOO_SMALL);
    mla_decode_args b = valid_args(16, 0);
    const mla_status st = mla_decode_noalloc(&b, nullptr);
    EXPECT(st == MLA_SUCCESS || st == MLA_ERROR_HIP);
  }

  // device input check: host rejections, then (without a GPU) a HIP error
  {
    const int32_t* bt = static_cast<const int32_t*>(addr(3 << 20));
    EXPECT(mla_check_paged_inputs(nullptr, 2, seq, 2, 2, 3, nullptr) == MLA_ERROR_INVALID_VALUE);
    EXPECT(mla_check_paged_inputs(bt, 1, seq, 2, 2, 3, nullptr) == MLA_ERROR_INVALID_VALUE);
    EXPECT(mla_check_paged_inputs(bt, 2, seq, 0, 2, 3, nullptr) == MLA_ERROR_INVALID_VALUE);
    const mla_status st = mla_check_paged_inputs(bt, 2, seq, 2, 2, 3, nullptr);
    EXPECT(st == MLA_SUCCESS || st == MLA_ERROR_HIP || st == MLA_ERROR_INVALID_VALUE);
  }

  // merge of context-parallel shards
  {
    mla_merge_args m;
    std::memset(&m, 0, sizeof(m));
    m.dtype = MLA_DTYPE_BF16;
    m.num_shards = 3;
    m.batch = 2;
    m.s_q = 1;
    m.h_q = 16;
    m.part_out = addr(1 << 20);
    m.part_out_stride[0] = 2 * 16 * 512;
    m.part_out_stride[1] = 16 * 512;
    m.part_out_stride[2] = 16 * 512;
    m.part_out_stride[3] = 512;
    m.part_lse = static_cast<const float*>(addr(2 << 20));
    m.part_lse_stride = 32;
    m.out = addr(3 << 20);
    m.out_stride[0] = 16 * 512;
    m.out_stride[1] = 16 * 512;
    m.out_stride[2] = 512;
    m.lse = static_cast<float*>(addr(4 << 20));
    const int k0 = stub_calls(MERGE);
    EXPECT(mla_merge_partials(&m, nullptr) == MLA_SUCCESS && stub_calls(MERGE) == k0 + 1);
    m.part_lse_stride = 31;
    EXPECT(mla_merge_partials(&m, nullptr) == MLA_ERROR_INVALID_VALUE);
    EXPECT(mla_merge_partials(nullptr, nullptr) == MLA_ERROR_INVALID_VALUE);
  }
}

static mha_decode_args valid_mha(int h_q, int h_kv, int d, int fp8) {
  mha_decode_args a;
  std::memset(&a, 0, sizeof(a));
  a.dtype = MLA_DTYPE_BF16;
  a.batch = 2;
  a.s_q = 1;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.head_dim = d;
  a.page_size = 64;
  a.num_pages = 3;
  a.max_pages_per_seq = 2;
  a.q = addr(1 << 20);
  a.q_stride[0] = (int64_t)h_q * d;
  a.q_stride[1] = (int64_t)h_q * d;
  a.q_stride[2] = d;
  a.k_cache = addr(2 << 20);
  a.k_stride[0] = (int64_t)64 * h_kv * d;
  a.k_stride[1] = (int64_t)h_kv * d;
  a.k_stride[2] = d;
  a.v_cache = addr(3 << 20);
  for (int i = 0; i < 3; ++i) a.v_stride[i] = a.k_stride[i];
  a.block_table = static_cast<const int32_t*>(addr(4 << 20));
  a.bt_stride = 2;
  a.cache_seqlens = static_cast<const int32_t*>(addr(5 << 20));
  a.sched = static_cast<const int32_t*>(addr(6 << 20));
  a.split_offsets = static_cast<const int32_t*>(addr(7 << 20));
  a.num_parts = 5;
  a.softmax_scale = 0.088f;
  size_t ws = 0;
  mha_workspace_size(a.batch, a.s_q, a.h_q, a.h_kv, d, a.num_parts, &ws);
  a.workspace = addr(8 << 20);
  a.workspace_bytes = ws;
  a.out = addr(64 << 20);
  a.out_stride[0] = (int64_t)h_q * d;
  a.out_stride[1] = (int64_t)h_q * d;
  a.out_stride[2] = d;
  a.lse = static_cast<float*>(addr(96 << 20));
  a.kv_dtype = fp8 ? MLA_KV_FP8_E4M3 : MLA_KV_SAME;
  return a;
}

static void mha_entry_points() {
  int parts = 0, se = 0, so = 0;
  EXPECT(mha_get_metadata_shape(256, 4, 1, 64, 8, &parts, &se, &so) == MLA_SUCCESS && so == 4 * 8 + 1);
  EXPECT(mha_get_metadata_shape(256, 4, 1, 60, 8, &parts, &se, &so) == MLA_ERROR_INVALID_VALUE);
  size_t ws = 0;
  EXPECT(mha_workspace_size(4, 1, 64, 8, 128, 64, &ws) == MLA_SUCCESS && ws % 256 == 0);
  EXPECT(mha_workspace_size(4, 1, 64, 8, 128, 0, &ws) == MLA_ERROR_INVALID_VALUE);
  const int32_t* seq = static_cast<const int32_t*>(addr(5 << 20));
  EXPECT(mha_get_metadata(seq, 4, 8, 64, static_cast<int32_t*>(addr(6 << 20)), static_cast<int32_t*>(addr(7 << 20)),
                          nullptr) == MLA_SUCCESS);
  EXPECT(stub_last(UNITS) == 32);
  const int dims[] = {64, 128, 256};
  for (int d : dims)
    for (int fp8 = 0; fp8 < 2; ++fp8) {
      mha_decode_args a = valid_mha(16, 2, d, fp8);
      const int k0 = stub_calls(MHA_SPLITKV), c0 = stub_calls(MHA_COMBINE);
      EXPECT(mha_decode(&a, nullptr) == MLA_SUCCESS);
      EXPECT(stub_calls(MHA_SPLITKV) == k0 + 1 && stub_calls(MHA_COMBINE) == c0 + 1 && stub_last(ROWS) == 8);
    }
  mha_decode_args a = valid_mha(16, 2, 128, 0);
  a.head_dim = 96;
  EXPECT(mha_decode(&a, nullptr) == MLA_ERROR_UNSUPPORTED);
  a = valid_mha(16, 2, 128, 0);
  a.h_q = 15;
  EXPECT(mha_decode(&a, nullptr) != MLA_SUCCESS);
  a = valid_mha(16, 2, 128, 1);
  a.k_stride[2] = 136;
  EXPECT(mha_decode(&a, nullptr) == MLA_ERROR_INVALID_VALUE);
  EXPECT(mha_decode(nullptr, nullptr) == MLA_ERROR_INVALID_VALUE);
}

// The error text is per thread: concurrent failing and succeeding calls each
// see their own message.
static void threads() {
  std::vector<std::thread> ts;
  std::vector<int> bad(8, 0);
  for (int t = 0; t < 8; ++t)
    ts.emplace_back([t, &bad] {
      for (int i = 0; i < 2000; ++i) {
        mla_decode_args a = valid_args(t % 2 ? 16 : 128, t % 3 == 0);
        if (i % 2) {
          a.num_parts = 0;
          if (mla_decode(&a, nullptr) != MLA_ERROR_INVALID_VALUE) ++bad[t];
          if (std::strstr(mla_last_error(), "num_parts") == nullptr) ++bad[t];
        } else {
          if (mla_decode(&a, nullptr) != MLA_SUCCESS) ++bad[t];
          if (mla_last_error()[0] != '\0') ++bad[t];
        }
        size_t ws = 0;
        if (mla_workspace_size(t + 1, 1, 16, 0, &ws) != MLA_ERROR_INVALID_VALUE) ++bad[t];
      }
    });
  for (auto& th : ts) th.join();
  for (int t = 0; t < 8; ++t) EXPECT(bad[t] == 0);
}

int main() {
  unsetenv("MLA_DEBUG");
  mla_entry_points();
  mha_entry_points();
  threads();
  // with MLA_DEBUG set, the decode entry points run the device check first
  // (without a GPU: a HIP error, and nothing is launched)
  setenv("MLA_DEBUG", "1", 1);
  {
    mla_decode_args a = valid_args(16, 0);
    const int k0 = stub_calls(NARROW);
    const mla_status st = mla_decode(&a, nullptr);
    EXPECT(st == MLA_SUCCESS || st == MLA_ERROR_HIP || st == MLA_ERROR_INVALID_VALUE);
    if (st != MLA_SUCCESS) EXPECT(stub_calls(NARROW) == k0);
  }
  unsetenv("MLA_DEBUG");
  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("abi driver: all expectations met\n");
  return 0;
}
