// C ABI of the DSA layer: argument validation, workspace layout, launch order.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/dsa.h"
#include "dsa_device.h"
#include "dsa_params.h"

namespace dsa {
hipError_t launch_indexer(const IdxParams& p, int idx_dtype, int D, int grid, hipStream_t st);
hipError_t launch_mla(const MlaParams& p, hipStream_t st);
hipError_t launch_quantize_q(const void* q, int64_t rows, int D, int idx_dtype, void* codes, void* scales,
                             hipStream_t st);
hipError_t launch_clear_counters(void* ws, size_t bytes, hipStream_t st);

namespace {

constexpr int MLA_TARGET_WGS = 256;
constexpr int MLA_MIN_ROWS = 32;
constexpr int MLA_MAX_SPLITS = 8;
constexpr int64_t KEYSPACE_MAX_PAGES = (int64_t)1 << 30;
// The workspace's counter region (its first DSA_WS_RESERVED_BYTES): the list
// merges' arrival counters, which every call leaves clear, at fixed offsets so
// that calls of any shape sharing a workspace agree on them.  Run counters:
// one per candidate-list slot, at most 2 * MQ * nwg <= 4 * NWG_MAX; per-query
// counters of calls with at most SMALL_T queries after them.
constexpr int NWG_MAX = 1024;
constexpr int SMALL_T = 64;  // calls with at most this many queries plan inside the indexer
constexpr size_t RES_RUN = 0;
constexpr size_t RES_MDONE = (size_t)4 * NWG_MAX * 4;
static_assert(RES_MDONE + SMALL_T * 4 <= DSA_WS_RESERVED_BYTES, "counter region");

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct IdxPlan {
  int MQ = 1, nwg = 256;
  bool need_merge = false;
  int merge_runs = 1;  // runs of MERGE_FAN lists a query may need (second merge level when > 1)
  int64_t lists = 0;  // candidate lists the workspace holds
  size_t off_run = 0, off_mcnt = 0, off_mmin = 0, off_mkeys = 0, off_mpos = 0, off_mdone = 0;
  size_t off_hdr = 0, off_groups = 0, off_qgroup = 0, off_wgfirst = 0, off_lcnt = 0, off_lmin = 0, off_lkeys = 0, off_lpos = 0,
         end = 0;
};

struct MlaPlan {
  int S = 1, RPS = 0;
  size_t off_o = 0, off_ml = 0, off_ss = 0, end = 0;
};

dsa_status check_indexer(const dsa_indexer_args* a, int K) {
  if (!a) return DSA_ERR_NULL;
  if (K <= 0 || K > DSA_MAX_K) return DSA_ERR_K;
  if (a->idx_dtype != DSA_IDX_BF16 && a->idx_dtype != DSA_IDX_FP8_E4M3FN && a->idx_dtype != DSA_IDX_MXFP8_E4M3)
    return DSA_ERR_DTYPE;
  if (!a->q_idx || !a->w || !a->k_idx_pool || !a->block_table || !a->seq_lens) return DSA_ERR_NULL;
  if (a->idx_dtype != DSA_IDX_BF16 && !a->q_idx_scale) return DSA_ERR_NULL;
  if (a->idx_dtype == DSA_IDX_BF16 && a->q_idx_scale) return DSA_ERR_DTYPE;
  if (a->T < 1 || a->B < 1 || a->max_blocks < 1 || a->num_blocks < 1 || a->max_q_per_seq < 1) return DSA_ERR_SHAPE;
  if (a->H_idx < 1 || a->H_idx > DSA_MAX_INDEX_HEADS) return DSA_ERR_SHAPE;
  if (a->idx_dtype == DSA_IDX_BF16 && a->D_idx != 64 && a->D_idx != 128) return DSA_ERR_SHAPE;
  if (a->idx_dtype != DSA_IDX_BF16 && a->D_idx != 128) return DSA_ERR_UNSUPPORTED;
  if (!a->q_seq && a->T != a->B) return DSA_ERR_SHAPE;
  if ((int64_t)a->max_blocks * DSA_PAGE_TOKENS > (int64_t)INT32_MAX / 2) return DSA_ERR_SHAPE;
  if ((int64_t)a->num_blocks * DSA_PAGE_TOKENS > (int64_t)INT32_MAX) return DSA_ERR_SHAPE;
  // The stream-K key space (every query group's visible range padded to whole
  // pages, plus a fixed per-segment weight) is counted in pages in 32 bits;
  // bound its largest possible total: at most T groups of max_blocks pages.
  if ((int64_t)a->T * ((int64_t)a->max_blocks + SEG_COST_PG) > KEYSPACE_MAX_PAGES) return DSA_ERR_SHAPE;
  if (!aligned(a->q_idx, 16) || !aligned(a->k_idx_pool, 16) || !aligned(a->w, 4) || !aligned(a->block_table, 4) ||
      !aligned(a->seq_lens, 4) || !aligned(a->q_idx_scale, 4) || !aligned(a->q_seq, 4) ||
      !aligned(a->q_visible, 4))
    return DSA_ERR_ALIGN;
  return DSA_OK;
}

dsa_status check_mla(const dsa_mla_args* m, int K) {
  if (!m) return DSA_ERR_NULL;
  if (K <= 0 || K > DSA_MAX_K) return DSA_ERR_K;
  if (!m->q || !m->kv_pool) return DSA_ERR_NULL;
  if (m->T < 1 || m->num_blocks < 1) return DSA_ERR_SHAPE;
  if (m->H != 16 && m->H != 32 && m->H != 64 && m->H != 128) return DSA_ERR_SHAPE;
  if (m->kv_dtype != DSA_KV_BF16 && m->kv_dtype != DSA_KV_FP8_TILE128) return DSA_ERR_DTYPE;
  if (m->residual) {
    if (!m->norm_weight || !m->residual_out) return DSA_ERR_NULL;
    if (!(m->norm_eps >= 0.f) || std::isinf(m->norm_eps)) return DSA_ERR_SHAPE;
    if (!aligned(m->residual, 8) || !aligned(m->norm_weight, 16) || !aligned(m->residual_out, 16))
      return DSA_ERR_ALIGN;
  }
  if ((int64_t)m->num_blocks * DSA_PAGE_TOKENS > (int64_t)INT32_MAX) return DSA_ERR_SHAPE;
  if (!aligned(m->q, 16) || !aligned(m->kv_pool, 16)) return DSA_ERR_ALIGN;
  return DSA_OK;
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return std::min(n, NWG_MAX);
}

// nwg: indexer workgroups (one per CU); the workspace depends on it, so the
// same value must be used for sizing and for the call.
IdxPlan plan_indexer(const dsa_indexer_args* a, int K, int nwg) {
  IdxPlan pl;
  // Adjacent queries of one sequence are scored in pairs, sharing each key
  // load, only when there are many of them (chunked prefill).  For a handful of
  // speculative queries on long sequences the pairs cost more than the extra
  // key reads save: measured on the mixed batch (four queries on a 1M-token
  // sequence), pairs streamed the keys in 91 us instead of 128 us but the
  // call took 251 us instead of 182, the selection and the list merges of two
  // queries per workgroup outweighing the saved reads.
  pl.MQ = a->max_q_per_seq >= 8 ? 2 : 1;
  pl.nwg = nwg;
  const int64_t maxlen = (int64_t)a->max_blocks * DSA_PAGE_TOKENS;
  const int64_t T = a->T;
  // a query group is split over workgroups (and then needs candidate lists and
  // the merge) only if the whole key space exceeds one minimum slice
  // (the last group's segment-cost weight holds no keys, hence - SEG_COST)
  const int64_t max_total = T * (std::max<int64_t>(16, (maxlen + 15) & ~15) + SEG_COST);
  pl.need_merge = max_total - SEG_COST > MIN_SLICE;
  pl.lists = pl.need_merge ? (int64_t)2 * pl.MQ * nwg : 0;
  size_t off = DSA_WS_RESERVED_BYTES;
  pl.off_hdr = off;
  off = align_up(off + 64, 256);
  pl.off_groups = off;
  off = align_up(off + (size_t)T * G_FIELDS * 4, 256);
  pl.off_qgroup = off;
  off = align_up(off + (size_t)T * 4, 256);
  pl.off_wgfirst = off;
  off = align_up(off + (size_t)nwg * 4, 256);
  pl.off_lcnt = off;
  off = align_up(off + (size_t)pl.lists * 4, 256);
  pl.off_lmin = off;
  off = align_up(off + (size_t)pl.lists * 4, 256);
  pl.off_lkeys = off;
  off = align_up(off + (size_t)pl.lists * K * 4, 256);
  pl.off_lpos = off;
  off = align_up(off + (size_t)pl.lists * K * 4, 256);
  pl.off_run = RES_RUN;  // in the counter region
  // a query's lists: at most one per workgroup, and its keys cover at most
  // maxlen / MIN_SLICE + 2 slices
  const int64_t nl_max = std::min<int64_t>(nwg, maxlen / MIN_SLICE + 2);
  pl.merge_runs = pl.need_merge ? (int)((nl_max + MERGE_FAN - 1) / MERGE_FAN) : 1;
  if (pl.merge_runs > 1) {
    pl.off_mcnt = off;
    off = align_up(off + (size_t)pl.lists * 4, 256);
    pl.off_mmin = off;
    off = align_up(off + (size_t)pl.lists * 4, 256);
    pl.off_mkeys = off;
    off = align_up(off + (size_t)pl.lists * K * 4, 256);
    pl.off_mpos = off;
    off = align_up(off + (size_t)pl.lists * K * 4, 256);
    if (T <= SMALL_T) {
      pl.off_mdone = RES_MDONE;  // in the counter region
    } else {
      pl.off_mdone = off;  // cleared by the planning kernel
      off = align_up(off + (size_t)T * 4, 256);
    }
  }
  pl.end = off;
  return pl;
}

MlaPlan plan_mla(const dsa_mla_args* m, int K, size_t base) {
  MlaPlan pl;
  int S = (MLA_TARGET_WGS + m->T - 1) / m->T;
  S = std::max(1, std::min(S, std::max(1, K / MLA_MIN_ROWS)));
  S = std::min(S, MLA_MAX_SPLITS);  // the combine kernel merges at most this many
  int rps = (K + S - 1) / S;
  rps = (rps + 31) / 32 * 32;
  S = (K + rps - 1) / rps;
  pl.S = S;
  pl.RPS = rps;
  size_t off = align_up(base, 256);
  if (S > 1) {
    pl.off_o = off;
    off = align_up(off + (size_t)m->T * S * m->H * DSA_VALUE_DIM * 2, 256);
    pl.off_ml = off;
    off = align_up(off + (size_t)m->T * S * m->H * 2 * 4, 256);
    if (m->residual) {
      pl.off_ss = off;
      off = align_up(off + (size_t)m->T * m->H * 4, 256);
    }
  }
  pl.end = off;
  return pl;
}

// A standalone attention call: its partials sit past the counter region (the
// workspace may be shared with indexer calls); with one split it needs none.
MlaPlan mla_alone(const dsa_mla_args* m, int K) {
  MlaPlan pl = plan_mla(m, K, DSA_WS_RESERVED_BYTES);
  if (pl.S == 1) pl.end = 0;
  return pl;
}

IdxParams make_idx_params(const dsa_indexer_args* a, int K, int32_t* indices, unsigned char* ws, const IdxPlan& pl) {
  IdxParams p{};
  p.q_idx = (const uint8_t*)a->q_idx;
  p.q_scale = a->q_idx_scale;
  p.w = a->w;
  p.k_pool = (const uint8_t*)a->k_idx_pool;
  p.num_blocks = a->num_blocks;
  const int es = a->idx_dtype == DSA_IDX_BF16 ? 2 : 1;
  // per-row scale bytes after the codes: fp32 per token, or one E8M0 byte per 32 elements
  const int scale_bytes = a->idx_dtype == DSA_IDX_FP8_E4M3FN ? 4 : (a->idx_dtype == DSA_IDX_MXFP8_E4M3 ? a->D_idx / 32 : 0);
  p.page_bytes = (int64_t)DSA_PAGE_TOKENS * (a->D_idx * es + scale_bytes);
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.q_seq = a->q_seq;
  p.q_visible = a->q_visible;
  p.max_blocks = a->max_blocks;
  p.T = a->T;
  p.B = a->B;
  p.H_idx = a->H_idx;
  p.K = K;
  p.nwg = pl.nwg;
  p.MQ = pl.MQ;
  p.inplan = a->T <= SMALL_T ? 1 : 0;
  p.indices = indices;
  p.hdr = (int32_t*)(ws + pl.off_hdr);
  p.groups = (int32_t*)(ws + pl.off_groups);
  p.qgroup = (int32_t*)(ws + pl.off_qgroup);
  p.wg_first = (int32_t*)(ws + pl.off_wgfirst);
  p.list_cnt = (int32_t*)(ws + pl.off_lcnt);
  p.list_min = (uint32_t*)(ws + pl.off_lmin);
  p.list_keys = (uint32_t*)(ws + pl.off_lkeys);
  p.list_pos = (int32_t*)(ws + pl.off_lpos);
  p.run_done = pl.need_merge ? (int32_t*)(ws + pl.off_run) : nullptr;
  const bool two = pl.merge_runs > 1;
  p.mlist_cnt = two ? (int32_t*)(ws + pl.off_mcnt) : nullptr;
  p.mlist_min = two ? (uint32_t*)(ws + pl.off_mmin) : nullptr;
  p.mlist_keys = two ? (uint32_t*)(ws + pl.off_mkeys) : nullptr;
  p.mlist_pos = two ? (int32_t*)(ws + pl.off_mpos) : nullptr;
  p.merge_done = two ? (int32_t*)(ws + pl.off_mdone) : nullptr;
  return p;
}

MlaParams make_mla_params(const dsa_mla_args* m, const int32_t* indices, int K, float scale, void* out,
                          unsigned char* ws, const MlaPlan& pl) {
  MlaParams p{};
  p.q = (const uint16_t*)m->q;
  p.kv = (const uint16_t*)m->kv_pool;
  p.kv8 = m->kv_dtype == DSA_KV_FP8_TILE128 ? 1 : 0;
  p.num_slots = m->num_blocks * DSA_PAGE_TOKENS;
  p.indices = indices;
  p.T = m->T;
  p.H = m->H;
  p.K = K;
  p.S = pl.S;
  p.rows_per_split = pl.RPS;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.out = (uint16_t*)out;
  p.part_o = pl.S > 1 ? (uint16_t*)(ws + pl.off_o) : nullptr;
  p.part_ml = pl.S > 1 ? (float*)(ws + pl.off_ml) : nullptr;
  p.residual = (const uint16_t*)m->residual;
  p.gamma = (const uint16_t*)m->norm_weight;
  p.res_out = (uint16_t*)m->residual_out;
  p.eps = m->norm_eps;
  p.ssq = (pl.S > 1 && m->residual) ? (float*)(ws + pl.off_ss) : nullptr;
  return p;
}

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// Argument checks and layout of one layer call: the workspace bytes it needs.
dsa_status layer_check(const dsa_indexer_args* idx, const dsa_mla_args* mla, int K, const int32_t* indices_out,
                       const void* out, size_t* need) {
  dsa_status st = check_indexer(idx, K);
  if (st != DSA_OK) return st;
  st = check_mla(mla, K);
  if (st != DSA_OK) return st;
  if (idx->T != mla->T || idx->num_blocks != mla->num_blocks) return DSA_ERR_SHAPE;
  if (!out) return DSA_ERR_NULL;
  if (!aligned(out, 8) || !aligned(indices_out, 4)) return DSA_ERR_ALIGN;
  const IdxPlan ip = plan_indexer(idx, K, device_cus());
  const size_t idx_end = align_up(align_up(ip.end, 256) + (size_t)idx->T * K * 4, 256);
  *need = plan_mla(mla, K, idx_end).end;
  return DSA_OK;
}

// The layer's launch sequence on a checked call, with a workspace of at least
// layer_check's bytes.
dsa_status layer_launch(const dsa_indexer_args* idx, const dsa_mla_args* mla, int K, float scale,
                        int32_t* indices_out, void* out, unsigned char* w, hipStream_t s) {
  const IdxPlan ip = plan_indexer(idx, K, device_cus());
  const size_t off_idx = align_up(ip.end, 256);
  const size_t idx_end = align_up(off_idx + (size_t)idx->T * K * 4, 256);
  const MlaPlan mp = plan_mla(mla, K, idx_end);
  int32_t* indices = indices_out ? indices_out : (int32_t*)(w + off_idx);
  IdxParams p = make_idx_params(idx, K, indices, w, ip);
  dsa_status st = hip_status(launch_indexer(p, idx->idx_dtype, idx->D_idx, ip.nwg, s));
  if (st != DSA_OK) return st;
  MlaParams q = make_mla_params(mla, indices, K, scale, out, w, mp);
  return hip_status(launch_mla(q, s));
}

// ---- The library's own scratch for dsa_layer_static: one array per GPU,
// allocated with the code object (a host-side name only; kernels get its
// device address, looked up once per device).
__device__ __align__(256) unsigned char scratch[DSA_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The device address of the current GPU's array, looked up on the device's
// first call, which also clears the array's counter region (a kernel on the
// call's stream, ahead of the call's own kernels).
dsa_status scratch_of_current_device(unsigned char** out, hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return DSA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DSA_ERR_HIP;
    if (launch_clear_counters(ptr, DSA_WS_RESERVED_BYTES, st) != hipSuccess) return DSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = (unsigned char*)g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace
}  // namespace dsa

using namespace dsa;

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_str(dsa_status s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_DTYPE: return "bad index dtype (or scale pointer inconsistent with it)";
    case DSA_ERR_SHAPE: return "a size is out of range";
    case DSA_ERR_K: return "K must be in 1..2048";
    case DSA_ERR_ALIGN: return "a pointer is misaligned";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_UNSUPPORTED: return "unsupported combination";
    case DSA_ERR_HIP: return "HIP launch failed";
    case DSA_ERR_TOO_LARGE: return "the call needs more scratch than the library's static array holds";
    case DSA_ERR_TABLE: return "a table entry is out of range";
  }
  return "unknown status";
}

size_t dsa_workspace_bytes(const dsa_indexer_args* idx, const dsa_mla_args* mla, int K) {
  size_t end = 0;
  if (idx) {
    if (check_indexer(idx, K) != DSA_OK) return 0;
    end = plan_indexer(idx, K, device_cus()).end;
  }
  if (mla) {
    if (check_mla(mla, K) != DSA_OK) return 0;
    if (!idx) return mla_alone(mla, K).end;
    end = align_up(end + (size_t)idx->T * K * 4, 256);  // indices kept for the layer
    end = plan_mla(mla, K, end).end;
  }
  return end;
}

dsa_status dsa_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (ws_bytes == 0) return DSA_OK;
  if (!ws) return DSA_ERR_NULL;
  if (!aligned(ws, 256)) return DSA_ERR_ALIGN;
  return hip_status(launch_clear_counters(ws, std::min(ws_bytes, (size_t)DSA_WS_RESERVED_BYTES), (hipStream_t)stream));
}

dsa_status dsa_indexer_topk(const dsa_indexer_args* a, int K, int32_t* indices_out, void* ws, size_t ws_bytes,
                            void* stream) {
  dsa_status st = check_indexer(a, K);
  if (st != DSA_OK) return st;
  if (!indices_out) return DSA_ERR_NULL;
  if (!aligned(indices_out, 4)) return DSA_ERR_ALIGN;
  const IdxPlan pl = plan_indexer(a, K, device_cus());
  if (!ws || ws_bytes < pl.end || !aligned(ws, 256)) return DSA_ERR_WORKSPACE;
  IdxParams p = make_idx_params(a, K, indices_out, (unsigned char*)ws, pl);
  return hip_status(launch_indexer(p, a->idx_dtype, a->D_idx, pl.nwg, (hipStream_t)stream));
}

dsa_status dsa_indexer_scores(const dsa_indexer_args* a, float* scores, int64_t ld, void* ws, size_t ws_bytes,
                              void* stream) {
  dsa_status st = check_indexer(a, 1);
  if (st != DSA_OK) return st;
  if (!scores) return DSA_ERR_NULL;
  if (!aligned(scores, 4)) return DSA_ERR_ALIGN;
  if (ld < (int64_t)a->max_blocks * DSA_PAGE_TOKENS) return DSA_ERR_SHAPE;
  const IdxPlan pl = plan_indexer(a, 1, device_cus());
  if (!ws || ws_bytes < pl.end || !aligned(ws, 256)) return DSA_ERR_WORKSPACE;
  IdxParams p = make_idx_params(a, 1, nullptr, (unsigned char*)ws, pl);
  p.scores = scores;
  p.scores_ld = ld;
  return hip_status(launch_indexer(p, a->idx_dtype, a->D_idx, pl.nwg, (hipStream_t)stream));
}

dsa_status dsa_sparse_mla_attn(const dsa_mla_args* m, const int32_t* indices, int K, float scale, void* out, void* ws,
                               size_t ws_bytes, void* stream) {
  dsa_status st = check_mla(m, K);
  if (st != DSA_OK) return st;
  if (!indices || !out) return DSA_ERR_NULL;
  if (!aligned(indices, 4) || !aligned(out, 8)) return DSA_ERR_ALIGN;
  const MlaPlan pl = mla_alone(m, K);
  if (pl.end > 0 && (!ws || ws_bytes < pl.end || !aligned(ws, 256))) return DSA_ERR_WORKSPACE;
  MlaParams p = make_mla_params(m, indices, K, scale, out, (unsigned char*)ws, pl);
  return hip_status(launch_mla(p, (hipStream_t)stream));
}

dsa_status dsa_layer(const dsa_indexer_args* idx, const dsa_mla_args* mla, int K, float scale, int32_t* indices_out,
                     void* out, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  dsa_status st = layer_check(idx, mla, K, indices_out, out, &need);
  if (st != DSA_OK) return st;
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return DSA_ERR_WORKSPACE;
  return layer_launch(idx, mla, K, scale, indices_out, out, (unsigned char*)ws, (hipStream_t)stream);
}

dsa_status dsa_layer_static(const dsa_indexer_args* idx, const dsa_mla_args* mla, int K, float scale,
                            int32_t* indices_out, void* out, void* stream) {
  size_t need = 0;
  dsa_status st = layer_check(idx, mla, K, indices_out, out, &need);
  if (st != DSA_OK) return st;
  if (need > DSA_STATIC_SCRATCH_BYTES) return DSA_ERR_TOO_LARGE;
  unsigned char* w = nullptr;
  st = scratch_of_current_device(&w, (hipStream_t)stream);
  if (st != DSA_OK) return st;
  return layer_launch(idx, mla, K, scale, indices_out, out, w, (hipStream_t)stream);
}

dsa_status dsa_check_tables(const dsa_indexer_args* a, const int32_t* seq_lens, const int32_t* block_table,
                            const int32_t* q_seq, const int32_t* q_visible, int32_t* bad_table,
                            int64_t* bad_index) {
  dsa_status st = check_indexer(a, 1);
  if (st != DSA_OK) return st;
  if (!seq_lens || !block_table) return DSA_ERR_NULL;
  if ((a->q_seq != nullptr) != (q_seq != nullptr) || (a->q_visible != nullptr) != (q_visible != nullptr))
    return DSA_ERR_NULL;
  auto bad = [&](int table, int64_t index) {
    if (bad_table) *bad_table = table;
    if (bad_index) *bad_index = index;
    return DSA_ERR_TABLE;
  };
  const int64_t maxlen = (int64_t)a->max_blocks * DSA_PAGE_TOKENS;
  for (int64_t b = 0; b < a->B; ++b)
    if (seq_lens[b] < 0 || seq_lens[b] > maxlen) return bad(0, b);
  for (int64_t b = 0; b < a->B; ++b) {
    const int64_t pages = ((int64_t)seq_lens[b] + DSA_PAGE_TOKENS - 1) / DSA_PAGE_TOKENS;
    for (int64_t i = 0; i < pages; ++i) {
      const int32_t pg = block_table[b * a->max_blocks + i];
      if (pg < 0 || pg >= a->num_blocks) return bad(1, b * a->max_blocks + i);
    }
  }
  for (int64_t t = 0; t < a->T; ++t) {
    const int64_t b = q_seq ? q_seq[t] : t;
    if (b < 0 || b >= a->B) return bad(2, t);
    if (q_visible && (q_visible[t] < 0 || q_visible[t] > seq_lens[b])) return bad(3, t);
  }
  return DSA_OK;
}

dsa_status dsa_quantize_index_q(const void* q, int64_t rows, int32_t D, int32_t idx_dtype, void* codes,
                                void* scales, void* stream) {
  if (idx_dtype != DSA_IDX_FP8_E4M3FN && idx_dtype != DSA_IDX_MXFP8_E4M3) return DSA_ERR_DTYPE;
  if (D != 32 && D != 64 && D != 128 && D != 256 && D != 512) return DSA_ERR_SHAPE;
  if (rows < 0 || rows > (int64_t)INT32_MAX * 8 / D) return DSA_ERR_SHAPE;
  if (rows == 0) return DSA_OK;
  if (!q || !codes || !scales) return DSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(codes, 16) || (idx_dtype == DSA_IDX_FP8_E4M3FN && !aligned(scales, 4)))
    return DSA_ERR_ALIGN;
  return hip_status(launch_quantize_q(q, rows, D, idx_dtype, codes, scales, (hipStream_t)stream));
}

}  // extern "C"
