// Kernel parameter blocks shared by the host launch code and the kernels.
#pragma once

#include <stdint.h>

namespace dsa {

// Per-group record written by the planning kernel (int32 fields).
enum GroupField { G_T0 = 0, G_NQ, G_SEQ, G_RANGE, G_NCH, G_ITEM, G_LIST, G_CTR, G_FIELDS };

struct IdxParams {
  const uint8_t* q_idx;   // [T][H_idx][D_idx] bf16 or e4m3fn codes
  const float* q_scale;   // [T][H_idx] (FP8 only)
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
  int32_t CH;  // keys per chunk, multiple of ROUND
  int32_t MQ;  // max queries per group
  int32_t* indices;  // [T][K] output
  // workspace
  int32_t* hdr;      // [0] groups, [1] items
  int32_t* groups;   // [T][G_FIELDS]
  uint32_t* ctr;     // merge-tree arrival counters
  int32_t* list_cnt;
  uint32_t* list_keys;
  int32_t* list_pos;
};

struct MlaParams {
  const uint16_t* q;        // [T][H][576] bf16
  const uint16_t* kv;       // [num_slots][576] bf16
  int64_t num_slots;
  const int32_t* indices;   // [T][K]
  int32_t T, H, K;
  int32_t S;                // splits per query
  int32_t rows_per_split;   // multiple of 32
  float scale_log2;         // softmax scale * log2(e)
  uint16_t* out;            // [T][H][512] bf16
  float* part_o;            // [T][S][H][512] fp32 (S > 1)
  float* part_ml;           // [T][S][H][2]   fp32 (S > 1)
};

}  // namespace dsa
