// Kernel parameter blocks shared by the host launch code and the kernels.
#pragma once

#include <stdint.h>

namespace dsa {

// Per-group record written by the planning kernel (int32 fields): first query,
// query count, sequence, visible key range, offset of the group in the
// concatenated (page-padded) key space in 64-key pages, number of indexer
// workgroups whose slice overlaps the group, first candidate-list slot, first
// workgroup.
enum GroupField { G_T0 = 0, G_NQ, G_SEQ, G_RANGE, G_OFF, G_NL, G_LIST, G_W0, G_FIELDS };

struct IdxParams {
  const uint8_t* q_idx;   // [T][H_idx][D_idx] bf16 or e4m3fn codes
  const void* q_scale;    // FP8: [T][H_idx] fp32; MXFP8: [T][H_idx][D/32] E8M0 bytes
  const float* w;         // [T][H_idx]
  const uint8_t* k_pool;  // paged index-K pool
  int64_t num_blocks;
  int64_t page_bytes;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* q_seq;      // may be null
  const int32_t* q_visible;  // may be null
  int32_t max_blocks;
  int32_t T, B, H_idx, K;
  int32_t nwg;  // indexer workgroups (each scans one equal slice of the key space)
  int32_t MQ;   // max queries per group
  int32_t inplan;  // at most 64 queries: the indexer plans itself (no planning kernel, no hdr/groups/qgroup/wg_first)
  int32_t* indices;  // [T][K] output
  float* scores;      // score dump instead of selection (null: select): [T][scores_ld] fp32
  int64_t scores_ld;
  // workspace
  int32_t* hdr;        // [0] groups, [1] pages in the padded key space, [2] pages per workgroup slice
  int32_t* groups;     // [T][G_FIELDS]
  int32_t* qgroup;     // [T] group of each query
  int32_t* wg_first;   // [nwg] first group of each indexer workgroup
  int32_t* list_cnt;   // per (query, chunk) candidate list: entry count
  uint32_t* list_min;  //   [.] smallest key of the list (read only when the list is full)
  uint32_t* list_keys; //   [.][K] order keys, ascending position
  int32_t* list_pos;   //   [.][K] logical positions
  int32_t* run_done;   //   [.] lists written of the run starting at each slot (clear at entry, cleared by the run's last arrival)
  // two-level merge of queries with many lists: intermediate lists (same
  // layout and slots as above) and a per-query count of finished runs
  int32_t* mlist_cnt;
  uint32_t* mlist_min;
  uint32_t* mlist_keys;
  int32_t* mlist_pos;
  int32_t* merge_done;  // [T], clear at entry, cleared by the query's last run
};

struct MlaParams {
  const uint16_t* q;        // [T][H][576] bf16
  const uint16_t* kv;       // [num_slots][576] bf16, or rows of 656 bytes (FP8, kv8 = 1)
  int32_t kv8;              // latent rows are FP8 (e4m3fn nope, fp32 per 128, bf16 rope)
  int64_t num_slots;
  const int32_t* indices;   // [T][K]
  int32_t T, H, K;
  int32_t S;                // splits per query
  int32_t rows_per_split;   // multiple of 32
  float scale_log2;         // softmax scale * log2(e)
  uint16_t* out;            // [T][H][512] bf16
  uint16_t* part_o;         // [T][S][H][512] bf16, unnormalised O of each split (S > 1)
  float* part_ml;           // [T][S][H][2]   fp32 (S > 1)
  // residual + RMSNorm epilogue (residual == nullptr: none)
  const uint16_t* residual; // [T][H][512] bf16
  const uint16_t* gamma;    // [H*512] bf16
  uint16_t* res_out;        // [T][H][512] bf16
  float eps;
  float* ssq;               // [T][H] fp32 sums of squares of res_out (S > 1)
};

}  // namespace dsa
