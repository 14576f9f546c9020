/*
 * dsa.h -- C ABI of the DSA sparse-attention layer for MI355X (gfx950).
 *
 * The layer (pages: "Day 0 Inference Adaptation and Performance Optimization
 * for Hybrid Attention LLMs", section "Index-Selected Sparse Attention";
 * "Inference Acceleration for a New Domestic LLM Architecture", section 3
 * "DSA Integration", whose illustrative listing chains a fused lightning
 * indexer, a Top-K selection and a sparse flash attention):
 *
 *   1. indexer:  S[t,p] = sum_h w[t,h] * ReLU(q_idx[t,h,:] . k_idx[p,:]) for
 *                every cached position p visible to query token t, reading the
 *                paged index-K cache directly;
 *   2. Top-K:    the k_t = min(K, n_t) positions with the largest S (ties go to
 *                the lower logical position);
 *   3. sparse MLA: softmax(scale * q[t,h,:576] . C[j,:576]) over the selected
 *                latent rows C, times C[j,:512] (value = first 512 dims).
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers unless stated otherwise; the
 *     argument structs themselves live in host memory and are read during the
 *     call only.
 *   - Every buffer is owned by the caller.  The library never allocates device
 *     memory; scratch comes from the caller's workspace (`ws`, `ws_bytes`),
 *     sized by dsa_workspace_bytes().  A workspace's first
 *     DSA_WS_RESERVED_BYTES hold the Top-K merges' arrival counters: they must
 *     be zero before the workspace's first use (dsa_workspace_init, or any
 *     zero fill), and every call leaves them zero again.  The rest needs no
 *     initialisation.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream),
 *     never synchronise, and keep no mutable global state.  Two calls that share
 *     a workspace must be ordered on one stream.
 *   - Argument errors are detected on the host before anything is launched and
 *     returned as a dsa_status; nothing is enqueued then.  A failed launch
 *     returns DSA_ERR_HIP.  No exception crosses the ABI.
 *   - Device-side contents (block_table, seq_lens, q_seq, q_visible, indices)
 *     are the caller's responsibility: page ids outside [0, num_blocks) and
 *     index slots outside [0, 64*num_blocks) are treated as absent (never read),
 *     and visible counts are clamped to [0, seq_len] and to 64*max_blocks.
 *
 * Paged cache layout (64-token pages; one block table serves both caches)
 *   - index-K pool, BF16:  [num_blocks][64][D_idx] bf16.
 *   - index-K pool, FP8:   num_blocks pages of (64*D_idx + 256) bytes: 64 rows of
 *                          D_idx OCP e4m3fn codes, then 64 fp32 dequantisation
 *                          scales (one per token).  8448 B per page at D_idx=128.
 *   - index-K pool, MXFP8: num_blocks pages of (64*D_idx + 64*D_idx/32) bytes:
 *                          64 rows of D_idx e4m3fn codes, then per row D_idx/32
 *                          E8M0 scale bytes (row-major; the value of code c in
 *                          group g is e4m3(c) * 2^(scale[g] - 127)).  Group size
 *                          32 ("Optimizing Inference for Hybrid-Architecture
 *                          LLMs", section 4.2).  8448 B per page at D_idx=128.
 *   - latent pool, BF16:   [num_blocks*64][576] bf16 (512 nope + 64 rope), row
 *                          `slot` = page*64 + offset.
 *   - latent pool, FP8:    [num_blocks*64] rows of 656 bytes: the 512 nope dims
 *                          as e4m3fn codes, 4 little-endian fp32 scales (scale t
 *                          covers nope dims 128t..128t+127), the 64 rope dims in
 *                          bf16.  Nope dim d = e4m3(code[d]) * scale[d / 128]
 *                          ("Hybrid Attention LLM Inference Acceleration",
 *                          section 5: main KV in FP8 with one scale per token and
 *                          128-element tile; the rope dims' storage is not given
 *                          there and stays bf16).
 *   - block_table:         [B][max_blocks] int32, logical page -> physical page.
 *   - seq_lens:            [B] int32 cached tokens per sequence.
 *   Logical position p of sequence b lives at slot block_table[b][p/64]*64 + p%64.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 8
#define DSA_PAGE_TOKENS 64
#define DSA_LATENT_DIM 576
#define DSA_VALUE_DIM 512
#define DSA_MAX_K 2048
#define DSA_MAX_INDEX_HEADS 64
#define DSA_STATIC_SCRATCH_BYTES ((size_t)64 << 20) /* dsa_layer_static's scratch per GPU */
#define DSA_WS_RESERVED_BYTES ((size_t)32768)       /* counter region at the start of a workspace */

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  DSA_ERR_DTYPE = 2,       /* unknown index dtype enum                            */
  DSA_ERR_SHAPE = 3,       /* a size is out of range (T, B, heads, dims, blocks)  */
  DSA_ERR_K = 4,           /* K <= 0 or K > DSA_MAX_K                             */
  DSA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                    */
  DSA_ERR_WORKSPACE = 6,   /* ws_bytes < dsa_workspace_bytes(...) or ws NULL      */
  DSA_ERR_UNSUPPORTED = 7, /* a valid but unimplemented combination               */
  DSA_ERR_HIP = 8,         /* a HIP launch failed                                 */
  DSA_ERR_TOO_LARGE = 9,   /* dsa_layer_static: the call needs more scratch than  */
                           /* DSA_STATIC_SCRATCH_BYTES                            */
  DSA_ERR_TABLE = 10       /* dsa_check_tables: a table entry is out of range     */
} dsa_status;

typedef enum dsa_kv_dtype {
  DSA_KV_BF16 = 0,         /* latent rows of 576 bf16                                   */
  DSA_KV_FP8_TILE128 = 1   /* latent rows of 656 B: e4m3fn nope + fp32 per 128 + bf16 rope */
} dsa_kv_dtype;

typedef enum dsa_idx_dtype {
  DSA_IDX_BF16 = 0,        /* q_idx and the index-K pool are bf16                       */
  DSA_IDX_FP8_E4M3FN = 1,  /* OCP e4m3fn codes with fp32 per-token / per-head scales    */
  DSA_IDX_MXFP8_E4M3 = 2   /* OCP e4m3fn codes with an E8M0 scale per 32 elements      */
} dsa_idx_dtype;

/*
 * Indexer inputs ("Optimizing Inference for Hybrid-Architecture LLMs", section
 * 3.1: scoring, head-weight weighting and Top-K selection fused, reading the
 * paged K cache directly).
 *   T            query tokens in this call (>= 1)
 *   B            sequences (>= 1)
 *   H_idx        indexer heads, 1..64
 *   D_idx        indexer head dim: 64 or 128 (BF16), 128 (FP8, MXFP8)
 *   idx_dtype    dsa_idx_dtype
 *   q_idx        [T][H_idx][D_idx] bf16, or e4m3fn codes (uint8)
 *   q_idx_scale  FP8: [T][H_idx] fp32 dequantisation scale per (token, head),
 *                > 0.  MXFP8: [T][H_idx][D_idx/32] uint8 E8M0 group scales
 *                (255, the E8M0 NaN, is not allowed).  Must be NULL for BF16.
 *   w            [T][H_idx] fp32 head weights (any sign)
 *   k_idx_pool   paged index-K pool (layout above)
 *   num_blocks   pages in both pools
 *   block_table  [B][max_blocks] int32
 *   max_blocks   row length of block_table (>= 1)
 *   seq_lens     [B] int32
 *   q_seq        [T] int32 sequence of each query, or NULL (then T == B and
 *                query t belongs to sequence t).  Queries of one sequence that
 *                are adjacent in t share one pass over its keys.
 *   q_visible    [T] int32 causal horizon n_t (query t sees positions
 *                0..n_t-1), or NULL (then n_t = seq_lens[q_seq[t]])
 *   max_q_per_seq host-side upper bound on adjacent queries of one sequence
 *                (1 for plain decode); it only selects the kernel variant.
 * Size limits (DSA_ERR_SHAPE otherwise): 64 * max_blocks <= 2^30 - 1,
 * 64 * num_blocks <= 2^31 - 1, and T * (max_blocks + 72) <= 2^30 (the indexer
 * lays all query groups' key ranges end to end in one page-counted space;
 * e.g. a 4096-query chunk may see up to about 2^24 pages = 2^30 tokens).
 */
typedef struct dsa_indexer_args {
  int32_t T, B, H_idx, D_idx;
  int32_t idx_dtype;
  const void* q_idx;
  const void* q_idx_scale;
  const float* w;
  const void* k_idx_pool;
  int64_t num_blocks;
  const int32_t* block_table;
  int32_t max_blocks;
  const int32_t* seq_lens;
  const int32_t* q_seq;
  const int32_t* q_visible;
  int32_t max_q_per_seq;
} dsa_indexer_args;

/*
 * Sparse MLA inputs ("Hybrid Attention LLM Inference Acceleration", section 2:
 * read the main attention KV at the selected indices and attend over the Top-K
 * positions only).
 *   T          query tokens (>= 1)
 *   H          attention heads: 16, 32, 64 or 128
 *   q          [T][H][576] bf16 (rope part already applied)
 *   kv_pool    latent rows (layout above: bf16 [num_blocks*64][576], or FP8 rows
 *              of 656 bytes)
 *   num_blocks pages in the pool
 *   kv_dtype   dsa_kv_dtype of kv_pool.  FP8 rows are dequantized to bf16 on
 *              chip (one rounding of code * scale) and attended like bf16 rows.
 *
 * Optional epilogue: residual connection + RMSNorm fused into the attention's
 * tail ("Day-0 Inference Adaptation for LLMs", operator section 2).  When
 * `residual` is non-NULL, per query token t over its H*512 output values:
 *   residual_out[t] = bf16(attn[t] + residual[t])            (the new residual)
 *   out[t]          = bf16(r * residual_out[t] * norm_weight),
 *   r = 1 / sqrt(mean(residual_out[t]^2) + norm_eps)
 * (the norm reads the stored bf16 residual_out), and attn itself is never
 * written.  With one split per query everything happens in the attention
 * kernel; with several, the split combine adds the residual and a small
 * kernel applies the norm.
 *   residual      [T][H][512] bf16 or NULL (no epilogue; the fields below are
 *                 then ignored)
 *   norm_weight   [H*512] bf16, 16-byte aligned
 *   residual_out  [T][H][512] bf16, 16-byte aligned; may be the residual
 *                 buffer itself (residual: 8-byte aligned)
 *   norm_eps      >= 0
 */
typedef struct dsa_mla_args {
  int32_t T, H;
  const void* q;
  const void* kv_pool;
  int64_t num_blocks;
  int32_t kv_dtype;
  const void* residual;
  const void* norm_weight;
  void* residual_out;
  float norm_eps;
} dsa_mla_args;

/* Bytes of workspace the call needs.  Pass NULL for the struct a call does not
 * use (dsa_indexer_topk: mla = NULL; dsa_sparse_mla_attn: idx = NULL).  Returns
 * 0 when the arguments are invalid (the call itself reports why), and for an
 * attention call that needs no workspace.  Every non-zero size includes the
 * counter region, DSA_WS_RESERVED_BYTES. */
size_t dsa_workspace_bytes(const dsa_indexer_args* idx, const dsa_mla_args* mla, int K);

/* Prepares a new workspace: enqueues on `stream` a kernel that zeroes its first
 * min(ws_bytes, DSA_WS_RESERVED_BYTES) bytes, the counter region.  Needed once
 * per workspace, before its first call (calls leave the region zero).
 * ws: device, 256-byte aligned (DSA_ERR_ALIGN); NULL only with ws_bytes == 0
 * (DSA_ERR_NULL), which enqueues nothing. */
dsa_status dsa_workspace_init(void* ws, size_t ws_bytes, void* stream);

/*
 * Steps 1+2.  Writes indices_out[T][K] (int32 device): for each query the
 * k_t = min(K, n_t) selected PHYSICAL pool slots in ascending logical-position
 * order, then K - k_t entries of -1.  Scores never leave the chip except as
 * bounded per-chunk candidate lists in the workspace.
 */
dsa_status dsa_indexer_topk(const dsa_indexer_args* a, int K, int32_t* indices_out,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Debugging aid for step 1 (the pages' alignment checklist, "Day 0 Inference
 * Adaptation and Performance Optimization for Hybrid Attention LLMs", section
 * "Engineering Execution", item 2: align the sparse index selection results
 * module by module).  Runs the indexer kernel of dsa_indexer_topk with the
 * same arguments, but instead of selecting it writes each fused score, exactly
 * as the selection compares it, as fp32:
 *   scores[t * ld + p] = S[t,p] for every position p < n_t whose page is
 *   present; every other entry is left untouched (callers pre-fill it).
 *   scores  float device, [T][ld]; ld >= 64 * max_blocks (else DSA_ERR_SHAPE)
 *   ws      workspace of dsa_workspace_bytes(a, NULL, 1) bytes
 * Argument errors are those of dsa_indexer_topk.  Meant for tests and
 * debugging: it writes T * n_t floats, unlike the fused call.
 */
dsa_status dsa_indexer_scores(const dsa_indexer_args* a, float* scores, int64_t ld, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * Step 3.  indices [T][K] int32 device pool slots; entries < 0 (or outside the
 * pool) are skipped.  out [T][H][512] bf16 device (fp32 accumulation).  A query
 * with no valid entry gets zeros.  scale is the softmax scale (1/sqrt(576) for
 * the pages' model).
 */
dsa_status dsa_sparse_mla_attn(const dsa_mla_args* a, const int32_t* indices, int K, float scale, void* out,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * Steps 1-3 as one launch sequence on `stream`.  idx->T must equal mla->T and
 * both must use the same num_blocks.  indices_out may be NULL (the indices then
 * stay in the workspace); otherwise it receives what dsa_indexer_topk writes.
 */
dsa_status dsa_layer(const dsa_indexer_args* idx, const dsa_mla_args* mla, int K, float scale,
                     int32_t* indices_out, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_layer for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same launch sequence and results, with the scratch taken from an array the
 * library holds on each GPU (DSA_STATIC_SCRATCH_BYTES, allocated with the code
 * object when the library is first used on that GPU and held until the
 * process ends) instead of a caller workspace.  The call allocates nothing.
 *   Returns DSA_ERR_TOO_LARGE, before anything is launched, when the call
 *   needs more than that (dsa_workspace_bytes(idx, mla, K) bytes: the five
 *   workloads of the pages' model need at most about 49 MiB on a 256-CU GPU).
 *   Every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents (the first call on a GPU clears the array's counter region with a
 *   kernel on its stream; every call leaves it clear): calls that overlap on
 *   one GPU (different streams, or threads without ordering) race and must be
 *   serialised by the caller.  The device is the current one.
 */
dsa_status dsa_layer_static(const dsa_indexer_args* idx, const dsa_mla_args* mla, int K, float scale,
                            int32_t* indices_out, void* out, void* stream);

/*
 * Index-query quantization, the step before step 1 ("Inference Acceleration
 * for a New Domestic LLM Architecture", section 3: a Q-quantization launch
 * prepares the fused indexer's query; "Optimizing Inference for
 * Hybrid-Architecture LLMs", section 3.2 for its place in the input
 * preparation and section 4.2 for per-group dynamic quantization with one
 * scale per 32 elements).  Each row of D bf16 values is quantized on its own:
 *   DSA_IDX_FP8_E4M3FN  s = amax|x| / 448 rounded to fp32 (s = 1 when that is
 *                       0); code = e4m3fn(x / s) with x / s rounded to fp32,
 *                       clamped to +-448, round-to-nearest-even.
 *                       scales: fp32 [rows] (the s above).
 *   DSA_IDX_MXFP8_E4M3  per group of 32: e = floor(log2 amax|x|) - 8 clamped
 *                       to [-127, 127] (e = 0 for an all-zero group); code =
 *                       e4m3fn(clamp(x * 2^-e, +-448)), round-to-nearest-even.
 *                       scales: uint8 [rows][D/32], byte e + 127.
 *   q       [rows][D] bf16 device, finite values, 16-byte aligned
 *   rows    >= 0 (0 enqueues nothing); for an indexer query rows = T * H_idx
 *   D       32, 64, 128, 256 or 512
 *   codes   [rows][D] uint8 device (written), 16-byte aligned
 *   scales  as above (written), 4-byte aligned for FP8
 * codes and scales are exactly the q_idx and q_idx_scale dsa_indexer_topk
 * takes.  Needs no workspace.
 */
dsa_status dsa_quantize_index_q(const void* q, int64_t rows, int32_t D, int32_t idx_dtype, void* codes,
                                void* scales, void* stream);

/*
 * Debugging aid for the device-side contents the indexer reads (they are the
 * caller's responsibility; the kernels treat bad entries as absent pages or
 * clamp them, see the conventions above).  Checks HOST copies of the tables of
 * a dsa_indexer_args call, without touching the device:
 *   seq_lens[b]        in [0, 64 * max_blocks]                  (table 0)
 *   block_table[b][i]  in [0, num_blocks) for the pages that hold
 *                      positions 0 .. seq_lens[b] - 1            (table 1)
 *   q_seq[t]           in [0, B)                                (table 2)
 *   q_visible[t]       in [0, seq_lens[q_seq[t]]]                (table 3)
 * seq_lens [B] and block_table [B][max_blocks] are required; q_seq and
 * q_visible are required exactly when the call's device pointers are set.
 * Returns DSA_OK, or DSA_ERR_TABLE with *bad_table and *bad_index (flat index
 * into that table) naming the first bad entry; argument errors as for
 * dsa_indexer_topk (K is not checked).  bad_table / bad_index may be NULL.
 */
dsa_status dsa_check_tables(const dsa_indexer_args* a, const int32_t* seq_lens, const int32_t* block_table,
                            const int32_t* q_seq, const int32_t* q_visible, int32_t* bad_table,
                            int64_t* bad_index);

/* Static string for a status code ("unknown status" for anything else). */
const char* dsa_status_str(dsa_status s);

/* DSA_ABI_VERSION of the loaded library. */
int dsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
