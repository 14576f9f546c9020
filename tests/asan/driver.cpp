// Host-side sanitizer run of the C ABI layer (argument validation, planning
// arithmetic and workspace layout), built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code and linked against recording
// launchers (launch_stubs.cpp), so it runs without a GPU.  Exit status 0 when
// every check holds; a sanitizer report aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "dsa.h"
#include "../../sparse_attention_07_amd/csrc/dsa_params.h"

namespace dsa {
extern IdxParams g_idx;
extern MlaParams g_mla;
extern int g_idx_calls, g_mla_calls, g_quant_calls, g_idx_grid;
extern void* g_clear_ptr;
extern size_t g_clear_bytes;
}

static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

// fake device pointers: aligned addresses of a host buffer, never dereferenced
alignas(256) static unsigned char fake[1 << 12];
static void* P(size_t off = 0) { return fake + off; }

static dsa_indexer_args idx_args(int T, int B, int max_blocks, int64_t nb, int dtype, int mq, bool qseq) {
  dsa_indexer_args a{};
  a.T = T; a.B = B; a.H_idx = 64; a.D_idx = 128; a.idx_dtype = dtype;
  a.q_idx = P(); a.q_idx_scale = dtype == DSA_IDX_BF16 ? nullptr : P(); a.w = (const float*)P();
  a.k_idx_pool = P(); a.num_blocks = nb; a.block_table = (const int32_t*)P(); a.max_blocks = max_blocks;
  a.seq_lens = (const int32_t*)P(); a.q_seq = qseq ? (const int32_t*)P() : nullptr;
  a.q_visible = qseq ? (const int32_t*)P() : nullptr; a.max_q_per_seq = mq;
  return a;
}
static dsa_mla_args mla_args(int T, int H, int64_t nb) {
  dsa_mla_args m{};
  m.T = T; m.H = H; m.q = P(); m.kv_pool = P(); m.num_blocks = nb; m.kv_dtype = DSA_KV_BF16;
  return m;
}

// every workspace pointer of the recorded parameter blocks lies inside [ws, ws + bytes)
static bool inside(const void* p, const unsigned char* ws, size_t bytes) {
  if (!p) return true;
  const unsigned char* c = (const unsigned char*)p;
  return c >= ws && c < ws + bytes;
}
static void check_idx_layout(const unsigned char* ws, size_t bytes) {
  const dsa::IdxParams& p = dsa::g_idx;
  const void* always[] = {p.hdr, p.groups, p.qgroup, p.wg_first};
  for (const void* q : always) CHECK(inside(q, ws, bytes));
  CHECK(inside(p.groups + (int64_t)p.T * dsa::G_FIELDS - 1, ws, bytes));
  CHECK(inside(p.qgroup + p.T - 1, ws, bytes));
  CHECK(inside(p.wg_first + p.nwg - 1, ws, bytes));
  // a call of at most 64 queries plans inside the indexer
  CHECK(p.inplan == (p.T <= 64 ? 1 : 0));
  // the plan tables and the lists sit past the counter region
  CHECK((const unsigned char*)p.hdr >= ws + DSA_WS_RESERVED_BYTES);
  if (p.run_done) {  // candidate lists (queries spanning several slices): 2 MQ nwg of K entries each
    const int64_t lists = (int64_t)2 * p.MQ * p.nwg;
    // the arrival counters: at the start of the counter region, clear of everything else
    CHECK((const unsigned char*)p.run_done == ws);
    CHECK((const unsigned char*)(p.run_done + lists) <= ws + DSA_WS_RESERVED_BYTES);
    CHECK((const unsigned char*)p.list_cnt >= ws + DSA_WS_RESERVED_BYTES);
    CHECK(inside(p.list_cnt + lists - 1, ws, bytes));
    CHECK(inside(p.list_min + lists - 1, ws, bytes));
    CHECK(inside(p.list_keys + lists * p.K - 1, ws, bytes));
    CHECK(inside(p.list_pos + lists * p.K - 1, ws, bytes));
    CHECK(inside(p.run_done + lists - 1, ws, bytes));
    if (p.mlist_pos) {
      CHECK(inside(p.mlist_cnt + lists - 1, ws, bytes));
      CHECK(inside(p.mlist_min + lists - 1, ws, bytes));
      CHECK(inside(p.mlist_keys + lists * p.K - 1, ws, bytes));
      CHECK(inside(p.mlist_pos + lists * p.K - 1, ws, bytes));
      CHECK(inside(p.merge_done + p.T - 1, ws, bytes));
      // per-query counters: in the counter region for a small call, else past it
      if (p.T <= 64) {
        CHECK((const unsigned char*)p.merge_done >= (const unsigned char*)(p.run_done + lists));
        CHECK((const unsigned char*)(p.merge_done + p.T) <= ws + DSA_WS_RESERVED_BYTES);
      } else {
        CHECK((const unsigned char*)p.merge_done >= ws + DSA_WS_RESERVED_BYTES);
      }
    }
  }
}

int main() {
  // ---- valid decode / prefill / mixed shapes: validation passes and every
  // workspace address the launch would use lies in the sized workspace
  struct Case { int T, B, max_blocks; int64_t nb; int dtype, mq, H, K; bool qseq; };
  const Case cases[] = {
      {64, 64, 2048, 100000, DSA_IDX_FP8_E4M3FN, 1, 128, 2048, false},   // 128K decode batch
      {32, 32, 512, 16384, DSA_IDX_BF16, 1, 128, 2048, false},           // 32K bf16 decode
      {11, 8, 16384, 44352, DSA_IDX_FP8_E4M3FN, 4, 128, 2048, true},     // mixed 4K..1M
      {4096, 1, 256, 256, DSA_IDX_FP8_E4M3FN, 4096, 128, 2048, true},    // prefill chunk
      {4096, 1, 16384, 16384, DSA_IDX_FP8_E4M3FN, 4096, 16, 2048, true}, // last chunk of a 1M prefill
      {1, 1, 64, 64, DSA_IDX_BF16, 1, 16, 256, false},                   // tiny decode
      {5000, 1, 79, 79, DSA_IDX_MXFP8_E4M3, 5000, 16, 256, true},        // more queries than staged in LDS
  };
  for (const Case& c : cases) {
    dsa_indexer_args a = idx_args(c.T, c.B, c.max_blocks, c.nb, c.dtype, c.mq, c.qseq);
    dsa_mla_args m = mla_args(c.T, c.H, c.nb);
    const size_t need_i = dsa_workspace_bytes(&a, nullptr, c.K);
    const size_t need_l = dsa_workspace_bytes(&a, &m, c.K);
    CHECK(need_i > 0 && need_l > need_i);
    std::vector<unsigned char> ws(need_l + 512);
    unsigned char* w = (unsigned char*)(((uintptr_t)ws.data() + 255) / 256 * 256);
    const int before = dsa::g_idx_calls;
    CHECK(dsa_indexer_topk(&a, c.K, (int32_t*)P(), w, need_i, nullptr) == DSA_OK);
    CHECK(dsa::g_idx_calls == before + 1);
    check_idx_layout(w, need_i);
    CHECK(dsa_indexer_topk(&a, c.K, (int32_t*)P(), w, need_i - 1, nullptr) == DSA_ERR_WORKSPACE);
    CHECK(dsa_layer(&a, &m, c.K, 0.04f, nullptr, P(), w, need_l, nullptr) == DSA_OK);
    check_idx_layout(w, need_l);
    CHECK(inside(dsa::g_mla.indices, w, need_l));
    if (dsa::g_mla.part_o) {
      CHECK(inside(dsa::g_mla.part_o + (int64_t)c.T * dsa::g_mla.S * c.H * 512 - 1, w, need_l));
      CHECK(inside(dsa::g_mla.part_ml + (int64_t)c.T * dsa::g_mla.S * c.H * 2 - 1, w, need_l));
    }
    CHECK(dsa::g_mla.S * dsa::g_mla.rows_per_split >= c.K && dsa::g_mla.rows_per_split % 32 == 0);
    CHECK(dsa_layer(&a, &m, c.K, 0.04f, nullptr, P(), w, need_l - 256, nullptr) == DSA_ERR_WORKSPACE);
    // a standalone attention call keeps its partials out of the counter region
    const size_t need_m = dsa_workspace_bytes(nullptr, &m, c.K);
    CHECK(dsa_sparse_mla_attn(&m, (const int32_t*)P(), c.K, 0.04f, P(), w, need_m, nullptr) == DSA_OK);
    if (dsa::g_mla.part_o) {
      CHECK(need_m > DSA_WS_RESERVED_BYTES);
      CHECK((const unsigned char*)dsa::g_mla.part_o >= w + DSA_WS_RESERVED_BYTES);
      CHECK(inside(dsa::g_mla.part_ml + (int64_t)c.T * dsa::g_mla.S * c.H * 2 - 1, w, need_m));
    } else {
      CHECK(need_m == 0);
    }
    const size_t need_s = dsa_workspace_bytes(&a, nullptr, 1);
    CHECK(dsa_indexer_scores(&a, (float*)P(), (int64_t)64 * c.max_blocks, w, need_s, nullptr) == DSA_OK);
    CHECK(dsa_indexer_scores(&a, (float*)P(), (int64_t)64 * c.max_blocks - 1, w, need_s, nullptr) == DSA_ERR_SHAPE);
  }
  // ---- the key-space bound: T * (max_blocks + 72) <= 2^30 pages
  {
    const int edge = (1 << 30) / 4096 - 72;
    dsa_indexer_args a = idx_args(4096, 1, edge, edge, DSA_IDX_FP8_E4M3FN, 1, true);
    CHECK(dsa_workspace_bytes(&a, nullptr, 2048) > 0);
    a.max_blocks = edge + 1;
    a.num_blocks = edge + 1;
    CHECK(dsa_workspace_bytes(&a, nullptr, 2048) == 0);
    CHECK(dsa_indexer_topk(&a, 2048, (int32_t*)P(), P(), 1 << 20, nullptr) == DSA_ERR_SHAPE);
    dsa_indexer_args b = idx_args(INT32_MAX, 1, 1 << 24, 1 << 24, DSA_IDX_FP8_E4M3FN, 1, true);
    CHECK(dsa_indexer_topk(&b, 2048, (int32_t*)P(), P(), 1 << 20, nullptr) == DSA_ERR_SHAPE);
  }
  // ---- extreme sizes through the sizing arithmetic (no overflow, no crash)
  {
    dsa_indexer_args a = idx_args(1 << 20, 1 << 20, 1, 1 << 24, DSA_IDX_BF16, 1, false);
    CHECK(dsa_workspace_bytes(&a, nullptr, 2048) > 0);
    dsa_mla_args m = mla_args(1 << 20, 128, 1 << 24);
    CHECK(dsa_workspace_bytes(nullptr, &m, 2048) == 0);  // one split per query: no workspace
    dsa_mla_args m1 = mla_args(1, 128, 1 << 24);
    CHECK(dsa_workspace_bytes(nullptr, &m1, 2048) > 0);  // 8 splits: partials
    dsa_mla_args bad = mla_args(1, 128, (int64_t)1 << 40);
    CHECK(dsa_workspace_bytes(nullptr, &bad, 2048) == 0);
  }
  // ---- argument errors: a status, nothing launched
  {
    const int before = dsa::g_idx_calls + dsa::g_mla_calls + dsa::g_quant_calls;
    dsa_indexer_args a = idx_args(4, 4, 10, 100, DSA_IDX_FP8_E4M3FN, 1, false);
    dsa_mla_args m = mla_args(4, 128, 100);
    CHECK(dsa_indexer_topk(nullptr, 2048, (int32_t*)P(), P(), 1 << 20, nullptr) == DSA_ERR_NULL);
    CHECK(dsa_indexer_topk(&a, 0, (int32_t*)P(), P(), 1 << 20, nullptr) == DSA_ERR_K);
    CHECK(dsa_indexer_topk(&a, 2048, (int32_t*)P(2), P(), 1 << 20, nullptr) == DSA_ERR_ALIGN);
    a.idx_dtype = 9;
    CHECK(dsa_indexer_topk(&a, 2048, (int32_t*)P(), P(), 1 << 20, nullptr) == DSA_ERR_DTYPE);
    a.idx_dtype = DSA_IDX_FP8_E4M3FN;
    a.H_idx = 65;
    CHECK(dsa_indexer_topk(&a, 2048, (int32_t*)P(), P(), 1 << 20, nullptr) == DSA_ERR_SHAPE);
    a.H_idx = 64;
    m.H = 48;
    CHECK(dsa_sparse_mla_attn(&m, (const int32_t*)P(), 2048, 0.04f, P(), P(), 1 << 20, nullptr) == DSA_ERR_SHAPE);
    m.H = 128;
    CHECK(dsa_layer(&a, &m, 2048, 0.04f, nullptr, nullptr, P(), 1 << 20, nullptr) == DSA_ERR_NULL);
    CHECK(dsa_quantize_index_q(P(), 64, 96, DSA_IDX_FP8_E4M3FN, P(), P(), nullptr) == DSA_ERR_SHAPE);
    CHECK(dsa_quantize_index_q(P(), -1, 128, DSA_IDX_FP8_E4M3FN, P(), P(), nullptr) == DSA_ERR_SHAPE);
    CHECK(dsa::g_idx_calls + dsa::g_mla_calls + dsa::g_quant_calls == before);
    for (int s = 0; s <= 10; ++s) CHECK(dsa_status_str((dsa_status)s) != nullptr);
    CHECK(dsa_workspace_init(nullptr, 1 << 20, nullptr) == DSA_ERR_NULL);
    CHECK(dsa_workspace_init(P(16), 1 << 20, nullptr) == DSA_ERR_ALIGN);
    CHECK(dsa_abi_version() == DSA_ABI_VERSION);
  }
  // ---- dsa_workspace_init clears the counter region (or less, for a smaller workspace)
  {
    CHECK(dsa_workspace_init(nullptr, 0, nullptr) == DSA_OK);
    CHECK(dsa_workspace_init(P(), 1 << 20, nullptr) == DSA_OK);
    CHECK(dsa::g_clear_ptr == P() && dsa::g_clear_bytes == DSA_WS_RESERVED_BYTES);
    CHECK(dsa_workspace_init(P(), 4096, nullptr) == DSA_OK);
    CHECK(dsa::g_clear_bytes == 4096);
  }
  // ---- the static-scratch layer rejects calls larger than its array before
  // touching the device
  {
    dsa_indexer_args a = idx_args(8192, 1, 128, 128, DSA_IDX_FP8_E4M3FN, 8192, true);
    dsa_mla_args m = mla_args(8192, 128, 128);
    CHECK(dsa_layer_static(&a, &m, 2048, 0.04f, nullptr, P(), nullptr) == DSA_ERR_TOO_LARGE);
  }
  // ---- host-copy table checks: every entry of a small call, one planted error per table
  {
    dsa_indexer_args a = idx_args(4, 3, 5, 12, DSA_IDX_FP8_E4M3FN, 2, true);
    std::vector<int32_t> lens = {300, 64, 1}, bt(3 * 5, 0), qs = {0, 0, 1, 2}, qv = {299, 300, 64, 1};
    for (int i = 0; i < 15; ++i) bt[i] = i % 12;
    int32_t tab = -1;
    int64_t at = -1;
    CHECK(dsa_check_tables(&a, lens.data(), bt.data(), qs.data(), qv.data(), &tab, &at) == DSA_OK);
    bt[4] = 12;
    CHECK(dsa_check_tables(&a, lens.data(), bt.data(), qs.data(), qv.data(), &tab, &at) == DSA_ERR_TABLE);
    CHECK(tab == 1 && at == 4);
    bt[4] = 0;
    qv[1] = 301;
    CHECK(dsa_check_tables(&a, lens.data(), bt.data(), qs.data(), qv.data(), &tab, &at) == DSA_ERR_TABLE);
    CHECK(tab == 3 && at == 1);
    qv[1] = 300;
    qs[3] = 3;
    CHECK(dsa_check_tables(&a, lens.data(), bt.data(), qs.data(), qv.data(), nullptr, nullptr) == DSA_ERR_TABLE);
    qs[3] = 2;
    lens[2] = 321;
    CHECK(dsa_check_tables(&a, lens.data(), bt.data(), qs.data(), qv.data(), &tab, &at) == DSA_ERR_TABLE);
    CHECK(tab == 0 && at == 2);
    CHECK(dsa_check_tables(&a, lens.data(), bt.data(), nullptr, qv.data(), &tab, &at) == DSA_ERR_NULL);
  }
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host sanitizer run: all checks passed\n");
  return 0;
}
