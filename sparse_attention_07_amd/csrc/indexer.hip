// Lightning indexer + Top-K for gfx950.
//
// What is computed ("Optimizing Inference for Hybrid-Architecture LLMs",
// section 3.1, indexer three-in-one fusion; "Hybrid Attention LLM Inference
// Acceleration", section 4 (1)): for every query token t and every visible
// cached position p,
//     S[t,p] = sum_h w[t,h] * ReLU(q_idx[t,h,:] . k_idx[p,:]),
// then the min(K, n_t) largest S are kept (ties to the lower position).  The
// paged index-K cache is read directly, the per-head dot products never leave
// registers, and scores only live in LDS; what reaches memory are bounded
// per-chunk candidate lists (<= K entries each).
//
// Design for CDNA4 (not the pages' accelerator):
//  * a planning kernel turns (seq_lens, q_seq, q_visible) into query groups
//    (adjacent queries of one sequence, up to MQ) laid end to end in one key
//    space, each charged a fixed extra weight for its per-segment cost, and
//    cuts that space into one equal slice per CU (stream-K): every workgroup
//    streams the same amount, whatever the sequence lengths;
//  * each wave streams 16-key slices of 64-token pages straight into MFMA
//    operand registers (per lane 64 contiguous bytes per key per load pair)
//    through a 4-deep register prefetch ring; page offsets come from an LDS
//    copy of the segment's block-table slice, read one group ahead, so no
//    load in the ring depends on another;
//  * MFMA M = 16 indexer heads per tile, N = 16 keys, K = head dim
//    (FP8: one 16x16x128 e4m3 MFMA per head tile; BF16: 16x16x32 steps);
//    each group's MFMAs issue back to back into separate accumulators, then
//    ReLU (an integer max on the bit pattern) and the head-weighted reduction
//    run on them; one permlane butterfly then sums the four head groups of
//    four consecutive groups at once, leaving one key per lane (64 keys) for
//    the key scale, the bound test and the candidate ballots;
//  * selection streams: after each 512-key round (1024 for paired queries) the keys above the current
//    bound (a lower bound of the K-th score) are appended, in position order,
//    to an LDS candidate buffer (one barrier per round: a wave's offset is
//    the count of the waves before it); only when a round would not fit is
//    the buffer cut back by a block radix select, which raises the bound
//    (it stops at the bin holding the K-th largest key once that bin fits:
//    a bound needs no exact K; the final selection is exact);
//  * a query whose keys span several slices gets one list per slice; the
//    workgroup that writes the last of them (an arrival counter; lists are
//    written and read device-coherent) merges them in the same launch: from the
//    largest minimum key of any full list -- that list alone already holds K
//    entries at or above it -- it selects the final K from the lists held in
//    registers, while other workgroups are still streaming.
#include <algorithm>

#include "dsa_device.h"
#include "dsa_params.h"

namespace dsa {

// The file is compiled once per part (DSA_IDX_PART): part 0 holds the
// planning kernel and the launch dispatcher, parts 1-4 the indexer kernels of
// one index format each, so the instantiations build in parallel.
#ifndef DSA_IDX_PART
#define DSA_IDX_PART 0
#endif

// =============================================================================
// Planning inside the indexer, for calls of at most PLAN_SMALL_T queries (every
// decode batch): each workgroup derives the same plan as the planning kernel
// below from the call's tables at its start, one query and then one group per
// lane, so the call needs no planning launch and no round trips to read a plan
// back.  This only works because the arrival counters of the list merges need
// no clearing launch: each is cleared again by its run's last arrival, and a
// workspace's counter region starts out clear (the C ABI's contract).
// =============================================================================
constexpr int PLAN_SMALL_T = 64;

struct SmallPlan {
  int grp[PLAN_SMALL_T * G_FIELDS];  // the planning kernel's group records
  int qgroup[PLAN_SMALL_T];          // group of each query
  int vis[PLAN_SMALL_T];             // visible keys of each query
  int hdr[4];                        // groups, pages in the key space, pages per slice, this workgroup's first group
};

// One group record into registers: from the in-kernel plan (LDS reads) or
// from the planning kernel's table (global loads), by an explicit branch so
// that neither path becomes a generic (flat) access.
__device__ __forceinline__ void read_group(const IdxParams& p, const SmallPlan& sp, int g, int (&r)[G_FIELDS]) {
  if (p.inplan) {
#pragma unroll
    for (int f = 0; f < G_FIELDS; ++f) r[f] = sp.grp[g * G_FIELDS + f];
  } else {
#pragma unroll
    for (int f = 0; f < G_FIELDS; ++f) r[f] = p.groups[(int64_t)g * G_FIELDS + f];
  }
#pragma unroll
  for (int f = 0; f < G_FIELDS; ++f) r[f] = __builtin_amdgcn_readfirstlane(r[f]);
}

// Every wave computes the plan in registers; wave 0 stores it.  The caller
// synchronises the workgroup before reading `sp`.
__device__ __forceinline__ void plan_small(const IdxParams& p, SmallPlan& sp) {
  const int lane = threadIdx.x & 63;
  const int T = p.T;
  const bool act = lane < T;
  // query `lane`: its sequence (-1: none) and visible count, as in the planning kernel's first pass
  int b = -1, qv = 0;
  if (act) {
    b = p.q_seq ? p.q_seq[lane] : lane;
    qv = p.q_visible ? p.q_visible[lane] : 0;
  }
  b = (b >= 0 && b < p.B) ? b : -1;
  const int len = b >= 0 ? p.seq_lens[b] : 0;
  const int L = min(max(len, 0), p.max_blocks * PAGE);
  const int vis = b >= 0 ? min(max(p.q_visible ? qv : L, 0), L) : 0;
  // groups: runs of one sequence, cut every MQ queries
  const int bprev = __shfl(b, max(lane - 1, 0));
  const bool f = act && (lane == 0 || b != bprev);
  const int run = wave_incl_max(f ? lane : -1);
  const bool gs = act && ((lane - run) % p.MQ == 0);
  const uint64_t gmask = ballot(gs);
  const int n_groups = __builtin_popcountll(gmask);
  const int qg = lanes_below(gmask) + (gs ? 1 : 0) - 1;
  // lane g now stands for group g: its first query is the (g+1)-th set bit of
  // gmask, the smallest t with g+1 starts in [0, t] (binary search on counts)
  const bool isg = lane < n_groups;
  int t0 = 0;
#pragma unroll
  for (int step = 32; step > 0; step >>= 1)
    if (__builtin_popcountll(gmask & ((2ull << (t0 + step - 1)) - 1ull)) < lane + 1) t0 += step;
  if (!isg) t0 = T;
  const int tn = __shfl(t0, min(lane + 1, 63));
  const int t1 = lane + 1 < n_groups ? tn : T;
  int range = 0;
  for (int k = 0; k < p.MQ; ++k) {
    const int vk = __shfl(vis, min(t0 + k, 63));
    if (isg && t0 + k < t1) range = max(range, vk);
  }
  const int seq = __shfl(b, min(t0, 63));
  // key-space offsets (pages) and the slices, as in the planning kernel's second and third passes
  const int wreal = max(1, (range + PAGE - 1) / PAGE);
  const int wgt = isg ? wreal + SEG_COST_PG : 0;
  const int incl = (int)wave_incl_scan((uint32_t)wgt);
  const int off = incl - wgt;
  const int total = __builtin_amdgcn_readlane(incl, 63);
  const int slice = max(MIN_SLICE_PG, (total + p.nwg - 1) / p.nwg);
  const int w0 = off / slice, w1 = (off + wreal - 1) / slice;
  const int lists = (isg && w1 > w0) ? (t1 - t0) * (w1 - w0 + 1) : 0;
  const int lincl = (int)wave_incl_scan((uint32_t)lists);
  // this workgroup's slice starts inside the group whose weight covers it
  const int a0 = (int)blockIdx.x * slice;
  const int first = __builtin_popcountll(ballot(isg && off + wgt <= a0));
  if (threadIdx.x < 64) {
    if (isg) {
      int* gr = sp.grp + lane * G_FIELDS;
      gr[G_T0] = t0;
      gr[G_NQ] = t1 - t0;
      gr[G_SEQ] = seq;
      gr[G_RANGE] = range;
      gr[G_OFF] = off;
      gr[G_NL] = w1 - w0 + 1;
      gr[G_LIST] = lincl - lists;
      gr[G_W0] = w0;
    }
    if (act) {
      sp.qgroup[lane] = qg;
      sp.vis[lane] = vis;
    }
    if (lane == 0) {
      sp.hdr[0] = n_groups;
      sp.hdr[1] = total;
      sp.hdr[2] = slice;
      sp.hdr[3] = first;
    }
  }
}

#if DSA_IDX_PART == 0
// =============================================================================
// Planning kernel: one workgroup (1024 threads; 256 for at most 256 queries,
// one wave for at most 64).
// =============================================================================
constexpr int PLAN_NT = 1024;

__device__ __forceinline__ int block_scan_incl(int v, int* s_w, bool is_max) {
  // inclusive scan (sum or max) over the workgroup (<= PLAN_NT threads); s_w: >= 16 ints of LDS
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = is_max ? wave_incl_max(v) : (int)wave_incl_scan((uint32_t)v);
  if (lane == 63) s_w[wave] = v;
  __syncthreads();
  int add = is_max ? -1 : 0;
  for (int w = 0; w < wave; ++w) add = is_max ? max(add, s_w[w]) : add + s_w[w];
  __syncthreads();
  return is_max ? max(v, add) : v + add;
}

__device__ __forceinline__ int plan_seq(const IdxParams& p, int t) {
  int b = p.q_seq ? p.q_seq[t] : t;
  return (b >= 0 && b < p.B) ? b : -1;
}

__device__ __forceinline__ int plan_vis(const IdxParams& p, int t) {
  const int b = plan_seq(p, t);
  if (b < 0) return 0;
  const int maxlen = p.max_blocks * PAGE;
  int L = min(max(p.seq_lens[b], 0), maxlen);
  int v = p.q_visible ? p.q_visible[t] : L;
  return min(max(v, 0), L);
}

// Up to PLAN_LDS_T queries, the per-query visible counts and the per-group
// fields the later passes read are kept in LDS (dynamic, PLAN_LDS_BYTES), so
// no pass waits on a global round trip for what an earlier pass produced.
constexpr int PLAN_LDS_T = 4096;
constexpr int PLAN_LOADS = PLAN_LDS_T / PLAN_NT;  // queries per thread when staged in LDS
constexpr size_t PLAN_LDS_BYTES = (size_t)6 * PLAN_LDS_T * sizeof(int);
static_assert(PLAN_LDS_T % PLAN_NT == 0, "staged queries per thread");

__global__ __launch_bounds__(PLAN_NT) void dsa_plan_kernel(IdxParams p) {
  __shared__ int s_w[16];
  __shared__ int s_carry[4];
  extern __shared__ int plan_lds[];
  const bool in_lds = p.T <= PLAN_LDS_T;
  int* s_vis = plan_lds;                    // [T] visible count of each query
  int* s_t0 = plan_lds + PLAN_LDS_T;        // [groups] first query
  int* s_nq = plan_lds + 2 * PLAN_LDS_T;    // [groups] queries
  int* s_rng = plan_lds + 3 * PLAN_LDS_T;   // [groups] key range
  int* s_off = plan_lds + 4 * PLAN_LDS_T;   // [groups] offset in the key space
  int* s_seq = plan_lds + 5 * PLAN_LDS_T;   // [T] sequence of each query (-1: none)
  const int tid = threadIdx.x;
  const int nt = blockDim.x;  // fewer waves per barrier for a short batch
  // ---- pass 0 (queries staged in LDS): every query's sequence and horizon
  // loaded at once (one round trip), then the sequences' lengths (a second)
  if (in_lds) {
    int qs[PLAN_LOADS], qv[PLAN_LOADS];
#pragma unroll
    for (int i = 0; i < PLAN_LOADS; ++i) {
      const int t = tid + i * nt;
      qs[i] = t < p.T ? (p.q_seq ? p.q_seq[t] : t) : -1;
      qv[i] = (t < p.T && p.q_visible) ? p.q_visible[t] : 0;
    }
    int len[PLAN_LOADS];
#pragma unroll
    for (int i = 0; i < PLAN_LOADS; ++i) {
      qs[i] = (qs[i] >= 0 && qs[i] < p.B) ? qs[i] : -1;
      len[i] = qs[i] >= 0 ? p.seq_lens[qs[i]] : 0;
    }
    const int maxlen = p.max_blocks * PAGE;
#pragma unroll
    for (int i = 0; i < PLAN_LOADS; ++i) {
      const int t = tid + i * nt;
      if (t < p.T) {
        const int L = min(max(len[i], 0), maxlen);
        const int v = p.q_visible ? qv[i] : L;
        s_seq[t] = qs[i];
        s_vis[t] = qs[i] >= 0 ? min(max(v, 0), L) : 0;
      }
    }
    __syncthreads();
  }
  // ---- pass 1: group starts (runs of one sequence, cut every MQ queries)
  int carry_run = 0, carry_gid = 0;
  for (int base = 0; base < p.T; base += nt) {
    const int t = base + tid;
    const bool valid = t < p.T;
    const int b = valid ? (in_lds ? s_seq[t] : plan_seq(p, t)) : -2;
    const int bprev = (valid && t > 0) ? (in_lds ? s_seq[t - 1] : plan_seq(p, t - 1)) : -3;
    const bool f = valid && (t == 0 || b != bprev);
    int run = block_scan_incl(f ? t : -1, s_w, true);
    run = max(run, carry_run);
    const bool gs = valid && ((t - run) % p.MQ == 0);
    const int gincl = block_scan_incl(gs ? 1 : 0, s_w, false);
    const int gid = carry_gid + gincl - (gs ? 1 : 0);
    if (gs) {
      int* g = p.groups + (int64_t)gid * G_FIELDS;
      g[G_T0] = t;
      g[G_SEQ] = b;
      if (in_lds) s_t0[gid] = t;
    }
    if (tid == nt - 1) {
      s_carry[0] = run;
      s_carry[1] = carry_gid + gincl;
    }
    __syncthreads();
    carry_run = s_carry[0];
    carry_gid = s_carry[1];
    __syncthreads();
  }
  const int n_groups = carry_gid;
  // ---- pass 2: per-group key ranges and their offsets in the concatenated
  // key space, counted in 64-key pages (each group padded to whole pages, at
  // least one, so every slice and segment starts on a page: four consecutive
  // 16-key groups of the indexer are one page)
  int c_off = 0;
  for (int base = 0; base < n_groups; base += nt) {
    const int g = base + tid;
    int wgt = 0;
    int* gr = p.groups + (int64_t)g * G_FIELDS;
    if (g < n_groups) {
      const int t0 = in_lds ? s_t0[g] : gr[G_T0];
      const int t1 = (g + 1 < n_groups) ? (in_lds ? s_t0[g + 1] : p.groups[(int64_t)(g + 1) * G_FIELDS + G_T0])
                                        : p.T;
      int range = 0;
      for (int t = t0; t < t1; ++t) {
        range = max(range, in_lds ? s_vis[t] : plan_vis(p, t));
        p.qgroup[t] = g;
      }
      gr[G_NQ] = t1 - t0;
      gr[G_RANGE] = range;
      if (in_lds) {
        s_nq[g] = t1 - t0;
        s_rng[g] = range;
      }
      wgt = max(1, (range + PAGE - 1) / PAGE) + SEG_COST_PG;
    }
    const int so = block_scan_incl(wgt, s_w, false);
    if (g < n_groups) {
      gr[G_OFF] = c_off + so - wgt;
      if (in_lds) s_off[g] = c_off + so - wgt;
    }
    if (tid == nt - 1) s_carry[0] = c_off + so;
    __syncthreads();
    c_off = s_carry[0];
    __syncthreads();
  }
  const int total = c_off;  // pages (the host keeps it below 2^30)
  const int slice = max(MIN_SLICE_PG, (total + p.nwg - 1) / p.nwg);
  // ---- pass 3: workgroups overlapping each group; list slots of split groups
  int c_list = 0;
  for (int base = 0; base < n_groups; base += nt) {
    const int g = base + tid;
    int lists = 0;
    int* gr = p.groups + (int64_t)g * G_FIELDS;
    if (g < n_groups) {
      const int off = in_lds ? s_off[g] : gr[G_OFF];
      const int range = in_lds ? s_rng[g] : gr[G_RANGE];
      const int nq = in_lds ? s_nq[g] : gr[G_NQ];
      // workgroups holding the group's keys (the extra weight that stands
      // for the segment cost follows them and holds no keys)
      const int wreal = max(1, (range + PAGE - 1) / PAGE);
      const int w0 = off / slice, w1 = (off + wreal - 1) / slice;
      const int wlast = (off + wreal + SEG_COST_PG - 1) / slice;
      gr[G_W0] = w0;
      gr[G_NL] = w1 - w0 + 1;
      // workgroups whose slice starts inside this group begin with it
      for (int w = (off + slice - 1) / slice; w <= wlast && w < p.nwg; ++w) p.wg_first[w] = g;
      lists = w1 > w0 ? nq * (w1 - w0 + 1) : 0;
    }
    const int sl = block_scan_incl(lists, s_w, false);
    if (g < n_groups) gr[G_LIST] = c_list + sl - lists;
    if (tid == nt - 1) s_carry[0] = c_list + sl;
    __syncthreads();
    c_list = s_carry[0];
    __syncthreads();
  }
  if (p.run_done)
    for (int u = tid; u < c_list; u += nt) p.run_done[u] = 0;
  if (p.merge_done)
    for (int t = tid; t < p.T; t += nt) p.merge_done[t] = 0;
  if (tid == 0) {
    p.hdr[0] = n_groups;
    p.hdr[1] = total;
    p.hdr[2] = slice;
  }
}

// Clears the counter region at the start of a workspace (before its first use;
// every call leaves it clear again).
__global__ __launch_bounds__(256) void dsa_clear_kernel(uint32_t* w, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) w[i] = 0u;
}

hipError_t launch_clear_counters(void* ws, size_t bytes, hipStream_t st) {
  const int n = (int)(bytes / 4);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(dsa_clear_kernel, dim3((n + 255) / 256 < 64 ? (n + 255) / 256 : 64), dim3(256), 0, st,
                     (uint32_t*)ws, n);
  return hipGetLastError();
}

#endif  // DSA_IDX_PART == 0

// =============================================================================
// Block-wide selection primitives (shared by the indexer and the merge).
// =============================================================================

// ---- Top-K selection over register-resident candidates --------------------
//
// A workgroup of NW waves holds candidates in registers, R slots per lane:
// slot s of lane l in wave w is entry w * (64 R) + 64 s + l, so entries are in
// position order wave by wave.  Keys are >= 1 (0 marks an empty slot) and
// positions are distinct.  The Top-K under (larger key first, then earlier
// position) is found by radix select over the composite: digits come from the
// offset above the smallest candidate (key - min, then pmax - pos among equal
// keys), 8 bits at a time from the top of the range actually spanned, so float
// scores of one magnitude spread over many bins instead of piling onto the
// one or two bins their exponent bits share (which would serialise the LDS
// atomics).  Each wave counts into its own histogram and two histogram sets
// alternate, so clearing the next one needs no barrier of its own.

// Which candidates are kept: key > ka, or key == kb and pmx - pos >= lo.
struct SelRule {
  uint32_t ka, kb, lo, pmx;
  __device__ __forceinline__ bool keep(uint32_t k, int32_t ps) const {
    return (k > ka) | ((k == kb) & (pmx - (uint32_t)ps >= lo));
  }
};

// Finds the rule that keeps exactly min(K, candidates) entries (all of them
// when there are at most K).  With keep_max > K it may stop early, as soon as
// the keys at or above the bin holding the K-th largest number at most
// keep_max: the rule then keeps that whole bin (at least K entries, every one
// of the Top-K among them), which is all a bound for later keys needs.
// hist: 2 * NW * 256 words, 16-byte aligned; wtmp: 8 * NW words; sel: 4 words.
// Ends with every wave past its last LDS read of wtmp.
template <int NW, int R>
__device__ __forceinline__ SelRule select_rule(const uint32_t (&rk)[R], const int32_t (&rp)[R], int K,
                                               uint32_t* hist, int32_t* sel, uint32_t* wtmp, int keep_max = 0) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t mn = 0xffffffffu, mx = 0u, pmn = 0xffffffffu, pmx = 0u, cnt = 0u;
#pragma unroll
  for (int s = 0; s < R; ++s) {
    const bool v = rk[s] != 0u;
    mn = min(mn, v ? rk[s] : 0xffffffffu);
    mx = max(mx, rk[s]);
    pmn = min(pmn, v ? (uint32_t)rp[s] : 0xffffffffu);
    pmx = max(pmx, v ? (uint32_t)rp[s] : 0u);
    cnt += (uint32_t)__builtin_popcountll(ballot(v));
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  pmn = wave_min_u32(pmn);
  pmx = wave_max_u32(pmx);
  if (lane == 0) {
    wtmp[8 * wave + 0] = mn;
    wtmp[8 * wave + 1] = mx;
    wtmp[8 * wave + 2] = pmn;
    wtmp[8 * wave + 3] = pmx;
    wtmp[8 * wave + 4] = cnt;
  }
  for (int i = tid; i < NW * 256; i += NT) hist[i] = 0u;
  lds_barrier();
  mn = 0xffffffffu;
  mx = 0u;
  pmn = 0xffffffffu;
  pmx = 0u;
  cnt = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mn = min(mn, wtmp[8 * w + 0]);
    mx = max(mx, wtmp[8 * w + 1]);
    pmn = min(pmn, wtmp[8 * w + 2]);
    pmx = max(pmx, wtmp[8 * w + 3]);
    cnt += wtmp[8 * w + 4];
  }
  if (cnt <= (uint32_t)K) return SelRule{0u, 0xffffffffu, 0u, 0u};  // keep every candidate
  // phase 0 resolves the key, phase 1 (equal keys) the position; in each,
  // the candidates still in play lie in [lo, lo + 2^sb - 1] of the phase's value
  auto bits_of = [](uint32_t r) { return r == 0u ? 0 : 32 - __builtin_clz(r); };
  int phase = 0;
  uint32_t klo = mn, lo = mn;
  int sb = bits_of(mx - mn);
  if (sb == 0) {
    phase = 1;
    lo = 0u;
    sb = bits_of(pmx - pmn);
  }
  int need = K;
  bool done = false;
  int pass = 0;
  while (!done && pass < 10) {  // at most 4 key and 4 position passes
    const int wd = min(8, sb);
    const int shift = sb - wd;
    uint32_t* hb = hist + (pass & 1) * (NW * 256);
    uint32_t* wh = hb + wave * 256;
    // branch-free match: value in [lo, lo + span], and (phase 1) key == klo
    const uint32_t span = sb >= 32 ? 0xffffffffu : (1u << sb) - 1u;
    const bool ph1 = phase == 1;
    const uint32_t kreq = ph1 ? klo : 0u;
#pragma unroll
    for (int s = 0; s < R; ++s) {
      const uint32_t k = rk[s];
      const uint32_t off = (ph1 ? pmx - (uint32_t)rp[s] : k) - lo;
      const bool m = (k != 0u) & (off <= span) & ((k == kreq) | !ph1);
      if (m) atomicAdd(&wh[off >> shift], 1u);
    }
    // the other set is cleared for the next pass (its last reader, wave 0's
    // scan of the previous pass, finished before the previous barrier)
    uint32_t* ho = hist + ((pass + 1) & 1) * (NW * 256);
    for (int i = tid; i < NW * 256; i += NT) ho[i] = 0u;
    lds_barrier();
    if (tid < 64) {
      // lane L owns bins 255-4L .. 252-4L (descending), summed over the waves
      // (one 16-byte read per wave histogram)
      uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const v4u v = *reinterpret_cast<const v4u*>(hb + w * 256 + 252 - 4 * lane);
        c[0] += v.w;
        c[1] += v.z;
        c[2] += v.y;
        c[3] += v.x;
      }
      const uint32_t sum = c[0] + c[1] + c[2] + c[3];
      const uint32_t incl = wave_incl_scan(sum);
      const uint32_t excl = incl - sum;
      if (excl < (uint32_t)need && (uint32_t)need <= incl) {
        uint32_t acc = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (acc < (uint32_t)need && acc + c[j] >= (uint32_t)need) {
            sel[0] = 255 - 4 * lane - j;
            sel[1] = (int)acc;
            sel[2] = (int)c[j];
          }
          acc += c[j];
        }
      }
    }
    lds_barrier();
    // sel is rewritten only after the next pass's first barrier, which every
    // wave reaches after this read
    const int bin = sel[0], above = sel[1], cb = sel[2];
    need -= above;
    lo += (uint32_t)bin << shift;
    sb = shift;
    ++pass;
    if (cb == need || (phase == 1 && sb == 0)) {
      done = true;
    } else if (phase == 0 && K - need + cb <= keep_max) {
      done = true;  // keys >= lo: the Top-K and the rest of their bin
    } else if (sb == 0) {
      // phase 0 resolved the key exactly; phase 1 cannot get here (positions
      // are distinct, so a resolved bin holds one entry)
      klo = lo;
      phase = 1;
      lo = 0u;
      sb = bits_of(pmx - pmn);
    }
  }
  // phase 0 keeps keys >= lo (kb is a key no candidate has); empty slots fail both
  return phase == 0 ? SelRule{lo - 1u, 0xffffffffu, 0u, 0u} : SelRule{klo, klo, lo, pmx};
}

// Order-preserving output of the kept candidates: write(o, key, pos) for the
// o-th kept entry in position order.  Returns the kept count; kmin receives
// the smallest kept key (0xffffffff if none).  wtmp: the 8 * NW words given
// to select_rule (words 8w+5 and 8w+6, which it leaves alone, so a wave may get
// here while others still read its results).  Ends with a barrier.
template <int NW, int R, typename W>
__device__ __forceinline__ int select_output(const uint32_t (&rk)[R], const int32_t (&rp)[R], const SelRule& rule,
                                             uint32_t* wtmp, uint32_t& kmin, W&& write) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t wc = 0, km = 0xffffffffu;
#pragma unroll
  for (int s = 0; s < R; ++s) {
    const bool kp = (rk[s] != 0u) & rule.keep(rk[s], rp[s]);
    wc += (uint32_t)__builtin_popcountll(ballot(kp));
    km = min(km, kp ? rk[s] : 0xffffffffu);
  }
  km = wave_min_u32(km);
  if (lane == 0) {
    wtmp[8 * wave + 5] = wc;
    wtmp[8 * wave + 6] = km;
  }
  lds_barrier();
  int run = 0, total = 0;
  km = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    run += (w < wave) ? (int)wtmp[8 * w + 5] : 0;
    total += (int)wtmp[8 * w + 5];
    km = min(km, wtmp[8 * w + 6]);
  }
#pragma unroll
  for (int s = 0; s < R; ++s) {
    const bool kp = (rk[s] != 0u) & rule.keep(rk[s], rp[s]);
    const uint64_t m = ballot(kp);
    if (kp) write(run + lanes_below(m), rk[s], rp[s]);
    run += (int)__builtin_popcountll(m);
  }
  lds_barrier();
  kmin = km;
  return total;
}

// Top-K of keys/pos[0..n) in LDS (K < n <= R * NW * 64), in place: exactly K
// entries remain at [0..K), in their original (position) order (with
// keep_max > K, between K and keep_max entries that include the Top-K; their
// count goes to *kept).  Returns the smallest kept key: an entry at a later
// position whose key is <= it can never enter.  hist: 2 * NW * 256 words;
// wtmp: 8 * NW words.
template <int NW, int R>
__device__ __forceinline__ uint32_t block_select(uint32_t* keys, int32_t* pos, int n, int K, uint32_t* hist, int32_t* sel,
                                                 uint32_t* wtmp, int keep_max = 0, int* kept = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  lds_barrier();  // entries appended by other waves are visible
  const int chunk = (((n + NW - 1) / NW) + 63) & ~63;
  const int wbeg = wave * chunk;
  uint32_t rk[R];
  int32_t rp[R];
  // every slot is read (from a clamped index, so all reads go out at once)
  // and masked afterwards
#pragma unroll
  for (int s = 0; s < R; ++s) {
    const int i = wbeg + s * 64 + lane;
    const int ic = min(i, n - 1);
    const uint32_t k = keys[ic];
    rp[s] = pos[ic];
    rk[s] = (s * 64 < chunk && i < n) ? k : 0u;
  }
  const SelRule rule = select_rule<NW, R>(rk, rp, K, hist, sel, wtmp, keep_max);
  uint32_t kmin;
  const int total = select_output<NW, R>(rk, rp, rule, wtmp, kmin, [&](int o, uint32_t k, int32_t ps) {
    keys[o] = k;
    pos[o] = ps;
  });
  if (kept) *kept = total;
  return kmin;
}

// Order-preserving append of the entries (kk[s], pp[s]) held by this thread
// for slots s (entry index s*NT + tid) whose key exceeds thr, at keys/pos[base..].
// Returns the new count (the same in every thread).  wcnt: 2*SL*NW + 1 words of
// LDS (counts per (slot, wave), then their exclusive scan and the total).
template <int NW, int SL>
__device__ __forceinline__ int block_append(uint32_t* keys, int32_t* pos, int base, uint32_t thr, const uint32_t (&kk)[SL],
                            const int32_t (&pp)[SL], uint32_t* wcnt) {
  static_assert(SL * NW <= 64, "one wave scans the (slot, wave) counts");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t mk[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    mk[s] = ballot(kk[s] > thr);
    if (lane == 0) wcnt[s * NW + wave] = (uint32_t)__builtin_popcountll(mk[s]);
  }
  lds_barrier();
  if (wave == 0) {
    const uint32_t c = lane < SL * NW ? wcnt[lane] : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (lane < SL * NW) wcnt[SL * NW + lane] = incl - c;
    if (lane == 63) wcnt[2 * SL * NW] = incl;
  }
  lds_barrier();
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    if (kk[s] > thr) {
      const int o = base + (int)wcnt[SL * NW + s * NW + wave] + lanes_below(mk[s]);
      keys[o] = kk[s];
      pos[o] = pp[s];
    }
  }
  const int total = base + (int)wcnt[2 * SL * NW];
  lds_barrier();
  return total;
}

// Smallest key of keys[0..n) (block-wide; n >= 1).
template <int NW>
__device__ __forceinline__ uint32_t block_min(const uint32_t* keys, int n, uint32_t* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t mn = 0xffffffffu;
  for (int i = tid; i < n; i += NW * 64) mn = min(mn, keys[i]);
  mn = wave_min_u32(mn);
  if (lane == 0) red[wave] = mn;
  lds_barrier();
  mn = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < NW; ++w) mn = min(mn, red[w]);
  lds_barrier();
  return mn;
}

// =============================================================================
// Merge: the candidate lists of queries whose keys span several slices.
//
// Every full list (K entries) is itself the Top-K of its slice, so the largest
// list minimum lb bounds the final K-th key from below and keys below lb are
// out.  A run of lists (in position order; slots past a list's count hold key
// 0) is read in chunks of MRG_RS entries per lane, wide and all at once.  A
// chunk's entries above the running bound are appended in order to an LDS
// buffer; when they would not fit, the buffer is first cut to its Top-K,
// which raises the bound.  A run that fits one chunk (up to MRG_FAN lists)
// selects straight from registers.
//
// The merge runs inside the indexer kernel, in the workgroup that writes the
// last list of a run: a per-run arrival counter (cleared by the planning
// kernel), moved once the workgroup's list stores have completed; lists are
// written and read with device-coherent accesses, so no fence is needed.  A
// query with up to MRG_FAN lists is one run.  A longer query merges in two
// levels: run j (lists MRG_FAN j ... MRG_FAN j + MRG_FAN - 1) goes to an
// intermediate list of the same layout (second list area, slot unit0 + j), and
// the workgroup that finishes the query's last run (a per-query counter)
// merges the intermediate lists.  A run's Top-K keeps every entry of the
// query's Top-K that the run holds, so the two levels select what one would.
// A split group is the last group a workgroup streams or its first (whose
// other lists are written later, at the end of earlier slices), so the merge
// usually starts when its workgroup has nothing left to stream and overlaps
// the other workgroups' streaming.
// =============================================================================
constexpr int MRG_NW = 8;
constexpr int MRG_NT = MRG_NW * 64;
constexpr int MRG_RS = 32;                  // entries per lane per chunk
constexpr int MRG_CHUNK = MRG_RS * MRG_NT;  // 16384
constexpr int MRG_CAP = 16384;              // LDS candidate buffer
constexpr int MRG_FAN = MERGE_FAN;          // lists one single-chunk merge takes
constexpr int MRG_BT = 2048;                // block-table entries a final merge stages in LDS
static_assert(KMAX + MRG_BT <= MRG_CAP, "staged block table after the kept entries");
static_assert(MRG_BT == 4 * MRG_NT, "block-table staging: one 16-byte piece per lane");
static_assert(MRG_FAN * KMAX <= MRG_CHUNK, "a run of MRG_FAN lists is one chunk");

struct MergeSmem {
  uint32_t cand_key[MRG_CAP];
  int32_t cand_pos[MRG_CAP];
  uint32_t hist[2 * MRG_NW * 256];
  uint32_t red[8 * MRG_NW];
  int32_t sel[4];
};
static_assert(MRG_CAP >= 2 * KMAX, "the buffer cut to K takes a chunk cut to K");

// Block-wide maximum of one value per thread (the lower bound each list
// gives), at least 1.  Ends with a barrier.
__device__ __forceinline__ uint32_t block_lb(uint32_t lb, MergeSmem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  lb = wave_max_u32(lb);
  if (lane == 0) sm.red[wave] = lb;
  lds_barrier();
  lb = 1u;
#pragma unroll
  for (int w = 0; w < MRG_NW; ++w) lb = max(lb, sm.red[w]);
  lds_barrier();
  return lb;
}

// Top-K of the n <= MRG_NT lists at keys0/pos0 (list i at offset i K; counts
// and minima at cnt0/min0, a minimum being read only for a full list), keys
// below the largest minimum of a full list (or below lb0) excluded: the kept
// entries, in position order, go to sm.cand_key/cand_pos [0, cnt); returns cnt
// and sets kmin to the smallest kept key.  Ends with a barrier.
template <int RS>
__device__ __forceinline__ int merge_lists_rs(const uint32_t* keys0, const int32_t* pos0, const int32_t* cnt0,
                                              const uint32_t* min0, int n, uint32_t lb0, int K, MergeSmem& sm,
                                              uint32_t& kmin) {
  static_assert(RS <= MRG_RS && RS % 4 == 0, "entries per lane");
  constexpr int CH = RS * MRG_NT;  // entries per chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // list counts and minima: loaded before the first chunk, reduced after it
  // has been issued, so the two latencies overlap
  int lc = 0;
  uint32_t lm = 0u;
  if (tid < n) {
    lc = ld_dev(cnt0 + tid);
    lm = ld_dev(min0 + tid);
  }
  const int total = n * K;
  // fewer entries per lane than MRG_RS: the caller guarantees one chunk
  const int nchunks = RS < MRG_RS ? 1 : (total + CH - 1) / CH;

  // Chunk layout: wave w holds entries [w * wch, (w + 1) * wch) of the chunk,
  // 64 per slot; every load comes from a clamped index and out-of-range slots
  // are dropped afterwards (loading them too keeps all loads in one straight
  // run: a branch per slot made the compiler wait between them, 3.7 -> 6.5 us).
  uint32_t rk[RS];
  int32_t rp[RS];
  auto load_chunk = [&](int c) {
    const int cb = c * CH;
    const int cn = min(CH, total - cb);
    const int wch = (((cn + MRG_NW - 1) / MRG_NW) + 63) & ~63;
#pragma unroll
    for (int s = 0; s < RS; ++s) {
      const int e = cb + min(wave * wch + s * 64 + lane, cn - 1);
      rk[s] = ld_dev(keys0 + e);
      rp[s] = ld_dev(pos0 + e);
    }
    return wch;
  };
  int wch = load_chunk(0);
  const uint32_t lb = max(lb0, block_lb(tid < n && lc == K ? lm : 1u, sm));
  uint32_t thr = lb - 1u;  // keep keys > thr
  int cnt = 0;
  uint32_t kbuf = 0xffffffffu;  // smallest key in the buffer (several chunks)
  for (int c = 0; c < nchunks; ++c) {
    if (c > 0) wch = load_chunk(c);
    const int cn = min(CH, total - c * CH);
    auto mask = [&]() {
#pragma unroll
      for (int s = 0; s < RS; ++s) {
        const int e = wave * wch + s * 64 + lane;
        if (s * 64 >= wch || e >= cn || rk[s] <= thr) rk[s] = 0u;
      }
    };
    mask();
    if (nchunks == 1) {
      // ---- single chunk: select straight from the registers
      const SelRule rule = select_rule<MRG_NW, RS>(rk, rp, K, sm.hist, sm.sel, sm.red);
      cnt = select_output<MRG_NW, RS>(rk, rp, rule, sm.red, kmin, [&](int o, uint32_t k, int32_t ps) {
        sm.cand_key[o] = k;
        sm.cand_pos[o] = ps;
      });
      break;
    }
    // survivors of this chunk (word 8w+7 of red is used by nothing else)
    auto count_valid = [&]() {
      uint32_t wc = 0;
#pragma unroll
      for (int s = 0; s < RS; ++s) wc += (uint32_t)__builtin_popcountll(ballot(rk[s] != 0u));
      if (lane == 0) sm.red[8 * wave + 7] = wc;
      lds_barrier();
      int m = 0;
#pragma unroll
      for (int w = 0; w < MRG_NW; ++w) m += (int)sm.red[8 * w + 7];
      return m;
    };
    int tot = count_valid();
    if (cnt + tot > MRG_CAP && cnt > K) {
      // cut the buffer to its Top-K (raising the bound), then drop the chunk's
      // entries that no longer pass
      kbuf = block_select<MRG_NW, MRG_CAP / MRG_NT>(sm.cand_key, sm.cand_pos, cnt, K, sm.hist, sm.sel, sm.red);
      thr = max(thr, kbuf);
      cnt = K;
      mask();
      tot = count_valid();
    }
    // append in order: every valid entry, or only the chunk's own Top-K when
    // that does not fit (cnt <= K then, and cnt + K <= MRG_CAP)
    const SelRule rule = cnt + tot > MRG_CAP ? select_rule<MRG_NW, RS>(rk, rp, K, sm.hist, sm.sel, sm.red)
                                             : SelRule{0u, 0xffffffffu, 0u, 0u};
    uint32_t kapp;
    cnt += select_output<MRG_NW, RS>(rk, rp, rule, sm.red, kapp,
                                         [&](int o, uint32_t k, int32_t ps) {
                                           sm.cand_key[cnt + o] = k;
                                           sm.cand_pos[cnt + o] = ps;
                                         });
    kbuf = min(kbuf, kapp);
  }
  if (nchunks > 1 && cnt > K) {
    kbuf = block_select<MRG_NW, MRG_CAP / MRG_NT>(sm.cand_key, sm.cand_pos, cnt, K, sm.hist, sm.sel, sm.red);
    cnt = K;
  }
  if (nchunks > 1) kmin = kbuf;
  return cnt;
}

// Merge over the entries per lane the lists need: a chunk of 16, 24 or 28
// entries per lane holds 4, 6 or 7 full lists of K = 2048 (a selection's
// passes cost in proportion to the entries each lane holds); 32 per lane,
// in one chunk or several, otherwise.
__device__ __forceinline__ int merge_lists(const uint32_t* keys0, const int32_t* pos0, const int32_t* cnt0,
                                           const uint32_t* min0, int n, uint32_t lb0, int K, MergeSmem& sm,
                                           uint32_t& kmin) {
  const int total = n * K;
  if (total <= 16 * MRG_NT) return merge_lists_rs<16>(keys0, pos0, cnt0, min0, n, lb0, K, sm, kmin);
  if (total <= 24 * MRG_NT) return merge_lists_rs<24>(keys0, pos0, cnt0, min0, n, lb0, K, sm, kmin);
  if (total <= 28 * MRG_NT) return merge_lists_rs<28>(keys0, pos0, cnt0, min0, n, lb0, K, sm, kmin);
  return merge_lists_rs<MRG_RS>(keys0, pos0, cnt0, min0, n, lb0, K, sm, kmin);
}

// One merge step for query t, run j, in the workgroup that wrote the run's
// last list (every list of the run is complete and visible).  Block-wide;
// ends with a barrier, after which the caller may reuse the LDS.
__device__ __forceinline__ void merge_query(const IdxParams& p, const SmallPlan& spl, int t, int j, MergeSmem& sm) {
  const int tid = threadIdx.x;
  // the query's group record: the in-kernel plan's or the planning kernel's
  int gr[G_FIELDS];
  read_group(p, spl, __builtin_amdgcn_readfirstlane(p.inplan ? spl.qgroup[t] : p.qgroup[t]), gr);
  const int nl = gr[G_NL];  // lists of this query (one per overlapping indexer workgroup)
  const int nrun = nl > MRG_FAN ? (nl + MRG_FAN - 1) / MRG_FAN : 1;
  const int seq = gr[G_SEQ];
  const int64_t unit0 = (int64_t)gr[G_LIST] + (int64_t)(t - gr[G_T0]) * nl;
  const int K = p.K;
  const int32_t* bt = p.block_table + (int64_t)max(seq, 0) * p.max_blocks;
  // The final step of a single-chunk merge copies the block-table slice
  // into LDS (cand_key[KMAX ..] is unused then) with direct-to-LDS loads
  // that fly while the lists load: 16 bytes (4 pages) per lane, so the row
  // must be 16-byte aligned and a whole number of such pieces.
  const int npg = (gr[G_RANGE] + PAGE - 1) / PAGE;  // pages holding the group's keys
  const bool stage = nrun == 1 && nl * K <= MRG_CHUNK && npg <= MRG_BT && (p.max_blocks & 3) == 0 &&
                     ((uintptr_t)bt & 15) == 0;
  int32_t* sbt = reinterpret_cast<int32_t*>(sm.cand_key + KMAX);
  if (stage) {
    const int wave = tid >> 6, lane = tid & 63;
    const int c = wave * 64 + lane;      // pages 4c .. 4c + 3
    const int cc = 4 * c < npg ? c : 0;  // past the slice: a harmless valid piece (its LDS slot is unused)
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int32_t*)(sbt + 256 * wave);
    dma16_to_lds(bt + 4 * cc, uniform(lds_addr));
  }
  // this run's lists (the other runs may still be streaming)
  const int c0 = j * MRG_FAN;
  const int nj = nrun == 1 ? nl : min(MRG_FAN, nl - c0);
  uint32_t kmin;
  int cnt = merge_lists(p.list_keys + (unit0 + c0) * K, p.list_pos + (unit0 + c0) * K, p.list_cnt + unit0 + c0,
                        p.list_min + unit0 + c0, nj, 1u, K, sm, kmin);
  if (nrun > 1) {
    // ---- first level: the run's Top-K becomes intermediate list unit0 + j
    const int64_t u = unit0 + j;
    for (int i = tid; i < K; i += MRG_NT) {
      st_dev(p.mlist_keys + u * K + i, i < cnt ? sm.cand_key[i] : 0u);
      if (i < cnt) st_dev(p.mlist_pos + u * K + i, sm.cand_pos[i]);
    }
    if (tid == 0) {
      st_dev(p.mlist_cnt + u, cnt);
      st_dev(p.mlist_min + u, kmin);
    }
    // the workgroup that finishes the last run merges the intermediate lists
    wait_vm();
    __syncthreads();
    if (tid == 0) {
      // the last run's arrival clears the counter for the next call
      const int old = atomicAdd(p.merge_done + t, 1);
      if (old == nrun - 1) st_dev(p.merge_done + t, 0);
      sm.sel[3] = old;
    }
    __syncthreads();
    const bool last = uniform(sm.sel[3]) == nrun - 1;
    lds_barrier();
    if (!last) return;
    cnt = merge_lists(p.mlist_keys + unit0 * K, p.mlist_pos + unit0 * K, p.mlist_cnt + unit0, p.mlist_min + unit0,
                      nrun, 1u, K, sm, kmin);
  }
  // ---- output: kept positions (in LDS, in order) to pool slots
  if (stage) {
    wait_vm();  // this wave's block-table piece has landed
    lds_barrier();
  }
  int32_t* out = p.indices + (int64_t)t * K;
  for (int i = tid; i < K; i += MRG_NT) {
    int v = -1;
    if (i < cnt) {
      const int ps = sm.cand_pos[i];
      v = (stage ? sbt[ps >> 6] : bt[ps >> 6]) * PAGE + (ps & 63);
    }
    out[i] = v;
  }
  lds_barrier();
}

// =============================================================================
// Main indexer kernel.
// =============================================================================
// Candidate buffer entries per query (a multiple of the workgroup's threads:
// the selections hold CAP / NT entries per thread, and a selection's passes
// cost in proportion to that).  Two queries per group: 5120 measured 3 %
// faster per prefill call than 4096 (fewer in-stream cuts), 4608 and 6144 in
// between, 8192 slower.  One query per group: 5120 against 4096 / 6144 /
// 8192 / 10240 gave decode_b32_32k 0.130 against 0.135 / 0.134 / 0.139 /
// 0.140 ms per layer step, mixed_1m 0.200 against 0.200 / 0.201 / 0.202 /
// 0.205, and the 128K batch within 0.5 us of the best.
template <int MQ>
struct CapOf {
  static constexpr int value = 5120;
};
// An in-stream cut keeps the Top-K plus at most this many more: the radix
// select may stop at the pass that finds the bin of the K-th largest key once
// that bin is small enough.  A slack of CAP - ROUND (the least that frees a
// round) made most cuts one pass but left so little room that the buffer
// filled again soon; 512 measured 1 % faster on the 128K decode batch and 3 %
// per prefill call (256 and 1024 alike) with 8192-entry single-query buffers.
// With 5120 entries for every group, 1024 against 512 / 256: 128K decode step
// 0.2399 against 0.2407 / 0.2404 ms, mixed_1m 0.1946 / 0.1958 / 0.1965.
constexpr int CUT_SLACK = 1024;

template <int NW, int MQ>
struct IdxSmem {
  static constexpr int CAP = CapOf<MQ>::value;
  static constexpr int NT = NW * 64;
  static constexpr int R = CAP / NT;  // candidate entries per thread in a selection
  static_assert(CAP % NT == 0, "selection register slots");
  static_assert(CAP >= KMAX + CUT_SLACK + round_keys(MQ), "after a cut the buffer holds one more round");
  uint32_t cand_key[MQ][CAP];
  int32_t cand_pos[MQ][CAP];
  uint32_t hist[2 * NW * 256];
  uint32_t wcnt[2][MQ][NW];  // per-round candidate counts of each wave (rounds alternate)
  uint32_t red[8 * NW];
  int32_t sel[4];
  // the sub-chunk's block-table slice as byte offsets of the pages in the
  // pool, in 256-byte units (every page layout is a multiple of 256 bytes,
  // and with at most 2^25 pages of at most 16 KB the offsets fit 32 bits);
  // ~0 marks an invalid page.  +1 entry when the slice is unaligned.
  uint32_t pages[SUB / PAGE + 1];
  float wq[MQ][64];               // head weight x query scale of the group's queries
};

// Offset of the in-kernel plan in the indexer's LDS: past the streaming and
// the merge layouts, which share the start.
template <int NW, int MQ>
struct SmallPlanOff {
  static constexpr size_t value =
      ((sizeof(IdxSmem<NW, MQ>) > sizeof(MergeSmem) ? sizeof(IdxSmem<NW, MQ>) : sizeof(MergeSmem)) + 15) / 16 * 16;
};

template <int DT, int D>
struct Frag {
  // bf16: one 16-byte piece per 32-wide k step; fp8: two 16-byte pieces (k=128)
  static constexpr int NP = DT == 0 ? D / 32 : 2;
  v4i d[NP];
};

template <int DT, int D>
struct BFrag {
  Frag<DT, D> f;
  float sc;  // MXFP8: E8M0 group byte (as bits); unused otherwise
};

template <int DT, int D, int HT, int MQ, int NW>
__global__ __launch_bounds__(NW * 64, 1) void dsa_indexer_kernel(IdxParams p) {
  using Sm = IdxSmem<NW, MQ>;
  constexpr int NT = NW * 64;
  constexpr int CAP = Sm::CAP;
  constexpr int R = Sm::R;
  constexpr int ROUND = round_keys(MQ);  // keys per round
  constexpr int GPW = ROUND / 16 / NW;  // 16-key groups per wave per round
  constexpr int ES = DT == 0 ? 2 : 1;   // bytes per element
  constexpr int ROWB = D * ES;          // bytes per key row
  // register prefetch depth (16-key groups): one quad ahead, about 8.5 KB of FP8
  // loads in flight per wave (8 groups measured 0.3-0.45 % slower on the decode
  // batches once keys are scored four groups at a time)
  constexpr int PF = 4;
  static_assert(PF == 4, "quad key scales are loaded one quad ahead, with the ring");
  static_assert(GPW % PF == 0, "prefetch ring must divide the round");
  static_assert(GPW % 4 == 0, "groups are scored four at a time");
  constexpr int NQD = GPW / 4;  // quads of groups per wave per round
  static_assert(DT == 0 || D == 128, "fp8 path is 128-wide");

  static_assert(NW == MRG_NW, "the merge runs in the indexer's workgroup");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  MergeSmem& msm = *reinterpret_cast<MergeSmem*>(smem_raw);  // same LDS, between segments
  // the in-kernel plan sits past both (read until the last merge)
  SmallPlan& spl = *reinterpret_cast<SmallPlan*>(smem_raw + SmallPlanOff<NW, MQ>::value);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int g4 = lane >> 4;
  const int n16 = lane & 15;

  // the plan: computed here for a small call, else the planning kernel's
  // (the tables are picked where they are read, not held in registers)
  if (p.inplan) {
    plan_small(p, spl);
    __syncthreads();
  }

  // this workgroup's slice [a0, a1) of the key space, in pages
  const int* hdr = p.inplan ? spl.hdr : p.hdr;
  const int n_groups = uniform(hdr[0]);
  const int total = uniform(hdr[1]);
  const int slice = uniform(hdr[2]);
  const int a0 = blockIdx.x * slice;
  const int a1 = min(a0 + slice, total);
  if (a0 >= a1) return;

  // first group overlapping [a0, a1)
  int g = uniform(p.inplan ? spl.hdr[3] : p.wg_first[blockIdx.x]);
  // runs this workgroup completes, merged once its slice is streamed: at most
  // two split groups overlap a slice (the one across each end), each entry
  // (group << 8) | (run << 2) | query mask
  int pend0 = -1, pend1 = -1;

  for (; g < n_groups; ++g) {
    int gr[G_FIELDS];
    read_group(p, spl, g, gr);
    const int off = gr[G_OFF];
    if (off >= a1) break;
    const int t0 = gr[G_T0];
    const int nq = gr[G_NQ];
    const int seq = gr[G_SEQ];
    const int range = gr[G_RANGE];
    const int nl = gr[G_NL];
    const int list_base = gr[G_LIST];
    const int w0 = gr[G_W0];
    const int wreal = max(1, (range + PAGE - 1) / PAGE);  // pages
    if ((int)blockIdx.x >= w0 + nl) continue;  // only the group's cost weight lies in this slice
    // this workgroup's keys of the group: [seg_lo, seg_hi), seg_lo a multiple of 64
    const int seg_lo = (max(a0, off) - off) * PAGE;
    const int seg_hi = min((min(a1, off + wreal) - off) * PAGE, range);
    const int32_t* bt = p.block_table + (int64_t)max(seq, 0) * p.max_blocks;

    int vis[MQ];
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      int v = 0;
      if (q < nq && seq >= 0) {
        if (p.inplan) {
          v = spl.vis[t0 + q];
        } else {
          const int L = min(max(p.seq_lens[seq], 0), p.max_blocks * PAGE);
          v = p.q_visible ? p.q_visible[t0 + q] : L;
          v = min(max(v, 0), L);
        }
      }
      vis[q] = uniform(v);
    }

    // ---- query operands (identical in every wave).  Every load is issued
    // unconditionally from a clamped index and masked afterwards, so they all
    // go out back to back instead of one branch (and one wait) at a time.
    // Head weights (times the query scales) go through LDS below, together
    // with the first sub-chunk's page ids.
    Frag<DT, D> a[MQ][HT];
    float wv[MQ][HT][4];
    // MXFP8: this lane's E8M0 scale operand = group g4 of head n16 of the tile
    // (the block-scaled MFMA takes the scale of (row, k-group) from lane
    // row + 16 * group)
    int qsx[MQ][HT];
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      const int64_t tq = t0 + min(q, nq - 1);
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) {
        const int h = mt * 16 + n16;
        const bool okh = q < nq && h < p.H_idx;
        const int64_t hrow = tq * p.H_idx + min(h, p.H_idx - 1);
        const uint8_t* row = p.q_idx + hrow * ROWB;
#pragma unroll
        for (int j = 0; j < Frag<DT, D>::NP; ++j) {
          const int off_b = DT == 0 ? 2 * (32 * j + 8 * g4) : (64 * j + 16 * g4);
          const v4i v = *reinterpret_cast<const v4i*>(row + off_b);
          a[q][mt].d[j] = okh ? v : v4i{0, 0, 0, 0};
        }
        qsx[q][mt] = DT == 2 ? (int)reinterpret_cast<const uint8_t*>(p.q_scale)[hrow * (D / 32) + g4] : 0;
      }
    }

    // candidate count and filter bound of each query (identical in every thread)
    int cnt[MQ];
    uint32_t thr[MQ];
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      cnt[q] = 0;
      thr[q] = 0u;
    }
    int rpar = 0;

    // ---- stream the segment in sub-chunks (page ids of a sub-chunk staged in LDS)
    for (int kb = seg_lo; kb < seg_hi; kb += SUB) {
      const int ke = min(kb + SUB, seg_hi);
      const int pg0 = kb >> 6;
      if (kb == seg_lo) {
        for (int i = tid; i < MQ * 64; i += NT) {
          const int q = i >> 6, hh = i & 63;
          float wt = 0.f;
          if (q < nq && hh < p.H_idx) {
            const int64_t o = (int64_t)(t0 + q) * p.H_idx + hh;
            wt = p.w[o];
            if (DT == 1) wt *= reinterpret_cast<const float*>(p.q_scale)[o];
          }
          sm.wq[q][hh] = wt;
        }
      }
      for (int i = tid; i <= ((ke - 1) >> 6) - pg0; i += NT) {
        const int pg = bt[pg0 + i];
        sm.pages[i] = (pg >= 0 && (int64_t)pg < p.num_blocks) ? (uint32_t)pg * (uint32_t)(p.page_bytes >> 8) : ~0u;
      }
      lds_barrier();
      if (kb == seg_lo) {
#pragma unroll
        for (int q = 0; q < MQ; ++q)
#pragma unroll
          for (int mt = 0; mt < HT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[q][mt][i] = sm.wq[q][mt * 16 + 4 * g4 + i];
      }
      int lim[MQ];
#pragma unroll
      for (int q = 0; q < MQ; ++q) lim[q] = min(vis[q], ke);

      const int nkeys = ke - kb;
      const int nrounds = (nkeys + ROUND - 1) / ROUND;
      auto group_p0 = [&](int j) { return kb + (j / GPW) * ROUND + (wave * GPW + (j % GPW)) * 16; };

      // Page entry of the group at p0 (read one group ahead of its load, so
      // the LDS latency is spent under the current group's MFMAs).
      auto page_of = [&](int p0) { return sm.pages[(p0 >> 6) - pg0]; };
      // The group's rows: a uniform base (page and first row) plus a 32-bit
      // per-lane offset, so the loads take the scalar-base form.
      auto load_b = [&](BFrag<DT, D>& bf, int p0, uint32_t pu) {
        const bool ok = pu != ~0u;
        const uint8_t* rowp = p.k_pool + ((uint64_t)(ok ? pu : 0u) << 8) + (p0 & 63) * ROWB;
#pragma unroll
        for (int j = 0; j < Frag<DT, D>::NP; ++j) {
          const uint32_t off_b = n16 * ROWB + (DT == 0 ? 2 * (32 * j + 8 * g4) : (64 * j + 16 * g4));
          bf.f.d[j] = *reinterpret_cast<const v4i*>(rowp + off_b);
        }
        // MXFP8: the E8M0 byte of group g4 of key r (carried in sc's bits), for
        // the MFMA; the scales follow the page's 64 rows (FP8 key scales are
        // read once per quad instead)
        const uint8_t* scp = p.k_pool + ((uint64_t)(ok ? pu : 0u) << 8) + PAGE * ROWB;
        if (DT == 2) bf.sc = __int_as_float((int)scp[(D / 32) * ((p0 & 63) + n16) + g4]);
        else bf.sc = 1.f;
      };

      // One 16-key group: each lane sums w * ReLU(q . k) over its 4 rows of
      // every head tile (16 of the 64 heads) for key n16; the four lane groups
      // are summed later, four groups at once.  Every query's MFMAs go first
      // (independent accumulators), then the VALU.  Queries past the group's
      // count have zero operands and no visible keys, so they need no branch.
      auto partial_group = [&](const BFrag<DT, D>& bf, float (&part)[MQ][4], int u) {
        v4f acc[MQ][HT];
#pragma unroll
        for (int q = 0; q < MQ; ++q)
#pragma unroll
          for (int mt = 0; mt < HT; ++mt) {
            acc[q][mt] = v4f{0.f, 0.f, 0.f, 0.f};
            if constexpr (DT == 1) {
              const v8i av = __builtin_shufflevector(a[q][mt].d[0], a[q][mt].d[1], 0, 1, 2, 3, 4, 5, 6, 7);
              const v8i bv = __builtin_shufflevector(bf.f.d[0], bf.f.d[1], 0, 1, 2, 3, 4, 5, 6, 7);
              acc[q][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[q][mt], 0, 0, 0, 0, 0, 0);
            } else if constexpr (DT == 2) {
              // group scales applied by the MFMA: A = q (E8M0 in qsx), B = keys
              const v8i av = __builtin_shufflevector(a[q][mt].d[0], a[q][mt].d[1], 0, 1, 2, 3, 4, 5, 6, 7);
              const v8i bv = __builtin_shufflevector(bf.f.d[0], bf.f.d[1], 0, 1, 2, 3, 4, 5, 6, 7);
              acc[q][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[q][mt], 0, 0, 0, qsx[q][mt],
                                                                            0, __float_as_int(bf.sc));
            } else {
#pragma unroll
              for (int j = 0; j < Frag<DT, D>::NP; ++j)
                acc[q][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[q][mt].d[j]),
                                                                     __builtin_bit_cast(v8bf, bf.f.d[j]), acc[q][mt],
                                                                     0, 0, 0);
            }
          }
#pragma unroll
        for (int q = 0; q < MQ; ++q) {
          float sum = 0.f;
#pragma unroll
          for (int mt = 0; mt < HT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // ReLU as an integer max on the bit pattern: negative floats
              // (sign bit set) become +0, everything else is unchanged
              const float d = __int_as_float(max(__float_as_int(acc[q][mt][i]), 0));
              sum = fmaf(wv[q][mt][i], d, sum);
            }
          // pinned here: sinking the sum to the quad's end would keep every
          // group's accumulators alive at once
          asm volatile("" : "+v"(sum));
          part[q][u] = sum;
        }
        // the next page entry's LDS read, the group's MFMAs back to back, then
        // its VALU: interleaving MFMAs and VALU would make each MFMA wait for
        // the previous tile's ReLU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MQ * HT * (DT == 0 ? Frag<DT, D>::NP : 1), 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 1000, 0);
      };

      // Four consecutive groups: 64 keys from p0, one page (segments start on
      // pages).  After the cross-lane sum, lane l holds the score of key
      // p0 + l; ksc is that key's scale (one load per lane and quad), ok the
      // page's validity.
      auto finish_quad = [&](const float (&part)[MQ][4], float ksc, bool ok, int p0, uint32_t (&kk)[MQ]) {
        const int pos = p0 + lane;
#pragma unroll
        for (int q = 0; q < MQ; ++q) {
          float sc = sum_lane_groups4(part[q][0], part[q][1], part[q][2], part[q][3]);
          if (DT == 1) sc *= ksc;
          kk[q] = (ok && pos < lim[q]) ? order_key(sc) : 0u;
        }
      };
      // the quad's key scales (FP8): lane l reads the scale of row l of the page
      auto load_qscale = [&](uint32_t pu) {
        if (DT != 1) return 1.f;
        const uint8_t* scp = p.k_pool + ((uint64_t)(pu != ~0u ? pu : 0u) << 8) + PAGE * ROWB;
        return *reinterpret_cast<const float*>(scp + 4 * lane);
      };

      // Loads are unconditional so the prefetch queue depth stays static: slots
      // past the sub-chunk end re-read its last 16-key group (a cache hit).
      const int last_p0 = kb + ((nkeys - 1) & ~15);
      auto load_p0 = [&](int j) { return min(group_p0(j), last_p0); };
      // The prologue issues the ring in slot order (scheduling barriers keep
      // the compiler from reordering it): the wait counts at the loop head
      // are merged over the prologue and the back edge, and a slot loaded
      // last here would force a wait for every load in flight each round.
      BFrag<DT, D> buf[PF];
#pragma unroll
      for (int s = 0; s < PF; ++s) {
        load_b(buf[s], load_p0(s), page_of(load_p0(s)));
        __builtin_amdgcn_sched_barrier(0);
      }
      // Page entries of the loads.  One query per group: read one group ahead
      // (pu_next).  Two: once per quad (a quad is one page, and clamped groups
      // past the end stay on the last group's page), at the quad's start; the
      // per-quad read measured 1.8 % faster for two queries and 0.3 % slower
      // for one.
      uint32_t pu_next = MQ == 1 ? page_of(load_p0(PF)) : 0u, pu_q = 0u;
      // key scales and page validity of the current and the next quad (the
      // ring runs one quad ahead), indexed by quad parity
      float qsc[2];
      bool qok[2];
      {
        const uint32_t pu0 = page_of(load_p0(0));
        qsc[0] = load_qscale(pu0);
        qok[0] = pu0 != ~0u;
      }
      for (int r = 0; r < nrounds; ++r) {
        // score this wave's GPW groups, four at a time (one key per lane);
        // keys past the sub-chunk end fail the visibility test
        uint32_t kk[MQ][NQD];
#pragma unroll
        for (int qd = 0; qd < NQD; ++qd) {
          float part[MQ][4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int s = 4 * qd + u;
            uint32_t pu;
            if constexpr (MQ == 2) {
              if (u == 0) pu_q = page_of(load_p0(r * GPW + s + PF));
              pu = pu_q;
            } else {
              pu = pu_next;
              pu_next = page_of(load_p0(r * GPW + s + PF + 1));
            }
            partial_group(buf[s % PF], part, u);
            load_b(buf[s % PF], load_p0(r * GPW + s + PF), pu);
            if (u == 0) {  // the next quad's first group: its page is the quad's
              qsc[(qd + 1) & 1] = load_qscale(pu);
              qok[(qd + 1) & 1] = pu != ~0u;
            }
            // one group at a time: hoisting the next group's MFMAs would need
            // a second accumulator set
            __builtin_amdgcn_sched_barrier(0);
          }
          uint32_t kq[MQ];
          finish_quad(part, qsc[qd & 1], qok[qd & 1], group_p0(r * GPW + 4 * qd), kq);
#pragma unroll
          for (int q = 0; q < MQ; ++q) kk[q][qd] = kq[q];
        }
        if constexpr (NQD % 2 == 1) {
          // an odd number of quads per round: the next round's first quad is
          // in slot 1, so the slots trade places (the parity is the quad's
          // place in the whole stream, not in the round)
          const float ts = qsc[0];
          qsc[0] = qsc[1];
          qsc[1] = ts;
          const bool tk = qok[0];
          qok[0] = qok[1];
          qok[1] = tk;
        }
        if (p.scores) {
          // score dump (a debugging call): the fused scores exactly as the
          // selection sees them (their order keys mapped back to fp32) for the
          // visible positions of present pages; nothing is selected
#pragma unroll
          for (int q = 0; q < MQ; ++q)
#pragma unroll
            for (int qd = 0; qd < NQD; ++qd)
              if (q < nq && kk[q][qd] != 0u)
                p.scores[(int64_t)(t0 + q) * p.scores_ld + group_p0(r * GPW + 4 * qd) + lane] = key_float(kk[q][qd]);
          continue;
        }
        // append the keys above each query's bound: a wave's groups are
        // consecutive positions and waves follow each other, so a wave's
        // offset is the count of the waves before it (one barrier per round).
        // When the round's keys would not fit, the buffer is cut to K first
        // (raising the bound) and the round is counted again.
        auto count_round = [&](int q) {
          uint32_t wc = 0;
#pragma unroll
          for (int qd = 0; qd < NQD; ++qd) wc += (uint32_t)__builtin_popcountll(ballot(kk[q][qd] > thr[q]));
          if (lane == 0) sm.wcnt[rpar][q][wave] = wc;
        };
#pragma unroll
        for (int q = 0; q < MQ; ++q) count_round(q);
        lds_barrier();
#pragma unroll
        for (int q = 0; q < MQ; ++q) {
          if (q < nq) {
            int pre = 0, tot = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
              const int c = (int)sm.wcnt[rpar][q][w];
              pre += (w < wave) ? c : 0;
              tot += c;
            }
            if (cnt[q] + tot > CAP) {
              // cnt[q] > CAP - ROUND >= K + CUT_SLACK, so the select has work to
              // do; it leaves at most K + CUT_SLACK entries, so the round then fits
              int kept;
              thr[q] = max(thr[q], block_select<NW, R>(sm.cand_key[q], sm.cand_pos[q], cnt[q], p.K, sm.hist,
                                                       sm.sel, sm.red, p.K + CUT_SLACK, &kept));
              cnt[q] = kept;
              count_round(q);  // every wave read the old counts before the select's first barrier
              lds_barrier();
              pre = 0;
              tot = 0;
#pragma unroll
              for (int w = 0; w < NW; ++w) {
                const int c = (int)sm.wcnt[rpar][q][w];
                pre += (w < wave) ? c : 0;
                tot += c;
              }
            }
            int o = cnt[q] + pre;
#pragma unroll
            for (int qd = 0; qd < NQD; ++qd) {
              const bool t = kk[q][qd] > thr[q];
              const uint64_t m = ballot(t);
              if (t) {
                const int oo = o + lanes_below(m);
                sm.cand_key[q][oo] = kk[q][qd];
                sm.cand_pos[q][oo] = group_p0(r * GPW + 4 * qd) + lane;
              }
              o += (int)__builtin_popcountll(m);
            }
            cnt[q] += tot;
          }
        }
        rpar ^= 1;
      }
    }

    if (p.scores) continue;  // score dump: no selection, no lists

    // ---- final selection and output
    // split group: this workgroup's list is list il of each query; run jr
    // (of runs with rs lists) is the one it belongs to
    const int il = (int)blockIdx.x - w0;
    const int nrun = nl > MERGE_FAN ? (nl + MERGE_FAN - 1) / MERGE_FAN : 1;
    const int jr = nrun > 1 ? il / MERGE_FAN : 0;
    const int rs = nrun > 1 ? min(MERGE_FAN, nl - jr * MERGE_FAN) : nl;
    int pend = 0;  // queries of the group whose run this workgroup completes
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      if (q < nq) {
        int c = cnt[q];
        uint32_t kmin = 0u;  // smallest kept key, when a selection ran
        if (c > p.K) {
          // as few entries per thread as the buffer needs (a selection's
          // passes cost in proportion to them)
          if (c <= 6 * NT)
            kmin = block_select<NW, 6>(sm.cand_key[q], sm.cand_pos[q], c, p.K, sm.hist, sm.sel, sm.red);
          else if (c <= 8 * NT)
            kmin = block_select<NW, 8>(sm.cand_key[q], sm.cand_pos[q], c, p.K, sm.hist, sm.sel, sm.red);
          else
            kmin = block_select<NW, R>(sm.cand_key[q], sm.cand_pos[q], c, p.K, sm.hist, sm.sel, sm.red);
          c = p.K;
        } else {
          lds_barrier();  // other waves' appends are visible
        }
        if (nl == 1) {
          // all block-table reads go out before the first store (clamped
          // indices, masked afterwards), so their latencies overlap
          int32_t* out = p.indices + (int64_t)(t0 + q) * p.K;
          constexpr int OPT = (KMAX + NT - 1) / NT;  // output slots per thread
          int ps[OPT], pg[OPT];
#pragma unroll
          for (int u = 0; u < OPT; ++u) {
            const int i = tid + u * NT;
            ps[u] = i < c ? sm.cand_pos[q][i] : -1;
          }
#pragma unroll
          for (int u = 0; u < OPT; ++u) pg[u] = bt[max(ps[u], 0) >> 6];
#pragma unroll
          for (int u = 0; u < OPT; ++u) {
            const int i = tid + u * NT;
            if (i < p.K) out[i] = ps[u] >= 0 ? pg[u] * PAGE + (ps[u] & 63) : -1;
          }
        } else {
          const int64_t unit = (int64_t)list_base + (int64_t)q * nl + (blockIdx.x - w0);
          // slots past the count get key 0 (no candidate), so a reader may
          // take all K slots without looking at the count
          for (int i = tid; i < p.K; i += NT) {
            st_dev(p.list_keys + unit * p.K + i, i < c ? sm.cand_key[q][i] : 0u);
            if (i < c) st_dev(p.list_pos + unit * p.K + i, sm.cand_pos[q][i]);
          }
          // a list's minimum is read only when it is full (it then bounds the
          // query's K-th key from below): the selection's, or one pass when
          // exactly K candidates needed no selection
          if (c == p.K && cnt[q] == p.K) kmin = block_min<NW>(sm.cand_key[q], c, sm.red);
          if (tid == 0) {
            st_dev(p.list_cnt + unit, c);
            st_dev(p.list_min + unit, kmin);
          }
          // arrival: the list is complete before the run's counter moves
          wait_vm();
          __syncthreads();
          if (tid == 0) {
            // the run's last arrival clears the counter for the next call
            int* ctr = p.run_done + (unit - il + jr);
            const int old = atomicAdd(ctr, 1);
            if (old == rs - 1) st_dev(ctr, 0);
            sm.sel[3] = old;
          }
          __syncthreads();
          if (uniform(sm.sel[3]) == rs - 1) pend |= 1 << q;
        }
        lds_barrier();
      }
    }
    if (pend) {
      const int e = (g << 8) | (jr << 2) | pend;
      if (pend0 < 0) pend0 = e;
      else pend1 = e;
    }
  }

  // ---- merge the runs this workgroup completed (every list of them is
  // complete; they are read with device-coherent loads)
  if (pend0 < 0) return;
#pragma unroll 1
  for (int k = 0; k < 2; ++k) {
    const int e = uniform(k == 0 ? pend0 : pend1);
    if (e < 0) break;
    int ge[G_FIELDS];
    read_group(p, spl, e >> 8, ge);
    const int t0 = ge[G_T0];
#pragma unroll 1
    for (int q = 0; q < MQ; ++q)
      if ((e >> q) & 1)
        merge_query(p, spl, t0 + q, (e >> 2) & 63, msm);
  }
}

// =============================================================================
// Host-side launch helpers (called from the C ABI layer).
// =============================================================================
template <int DT, int D, int HT, int MQ, int NW>
static hipError_t launch_indexer_t(const IdxParams& p, int grid, hipStream_t st) {
  auto kfn = dsa_indexer_kernel<DT, D, HT, MQ, NW>;
  // the merge reuses the workgroup's LDS when lists exist; the in-kernel plan
  // follows both
  const size_t smem = p.inplan ? SmallPlanOff<NW, MQ>::value + sizeof(SmallPlan)
                               : (p.run_done ? std::max(sizeof(IdxSmem<NW, MQ>), sizeof(MergeSmem))
                                             : sizeof(IdxSmem<NW, MQ>));
  hipError_t e = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(grid), dim3(NW * 64), smem, st, p);
  return hipGetLastError();
}

template <int DT, int D, int HT>
static hipError_t launch_indexer_mq(const IdxParams& p, int grid, hipStream_t st) {
  return p.MQ == 1 ? launch_indexer_t<DT, D, HT, 1, 8>(p, grid, st) : launch_indexer_t<DT, D, HT, 2, 8>(p, grid, st);
}

template <int DT, int D>
static hipError_t launch_indexer_heads(const IdxParams& p, int grid, hipStream_t st) {
  return p.H_idx <= 16 ? launch_indexer_mq<DT, D, 1>(p, grid, st) : launch_indexer_mq<DT, D, 4>(p, grid, st);
}

// one launcher per index format, each defined in its own part
hipError_t launch_indexer_fp8(const IdxParams& p, int grid, hipStream_t st);
hipError_t launch_indexer_mxfp8(const IdxParams& p, int grid, hipStream_t st);
hipError_t launch_indexer_bf16_128(const IdxParams& p, int grid, hipStream_t st);
hipError_t launch_indexer_bf16_64(const IdxParams& p, int grid, hipStream_t st);

#if DSA_IDX_PART == 1
hipError_t launch_indexer_fp8(const IdxParams& p, int grid, hipStream_t st) {
  return launch_indexer_heads<1, 128>(p, grid, st);
}
#elif DSA_IDX_PART == 2
hipError_t launch_indexer_mxfp8(const IdxParams& p, int grid, hipStream_t st) {
  return launch_indexer_heads<2, 128>(p, grid, st);
}
#elif DSA_IDX_PART == 3
hipError_t launch_indexer_bf16_128(const IdxParams& p, int grid, hipStream_t st) {
  return launch_indexer_heads<0, 128>(p, grid, st);
}
#elif DSA_IDX_PART == 4
hipError_t launch_indexer_bf16_64(const IdxParams& p, int grid, hipStream_t st) {
  return launch_indexer_heads<0, 64>(p, grid, st);
}
#endif

#if DSA_IDX_PART == 0
hipError_t launch_indexer(const IdxParams& p, int idx_dtype, int D, int grid, hipStream_t st) {
  const size_t plan_smem = p.T <= PLAN_LDS_T ? PLAN_LDS_BYTES : 0;
  hipError_t e = hipSuccess;
  if (!p.inplan) {  // a small call plans inside the indexer
    e = hipFuncSetAttribute((const void*)dsa_plan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)PLAN_LDS_BYTES);
    if (e != hipSuccess) return e;
    const int plan_nt = p.T <= 64 ? 64 : (p.T <= 256 ? 256 : PLAN_NT);
    hipLaunchKernelGGL(dsa_plan_kernel, dim3(1), dim3(plan_nt), plan_smem, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (idx_dtype == 1) return launch_indexer_fp8(p, grid, st);
  if (idx_dtype == 2) return launch_indexer_mxfp8(p, grid, st);
  return D == 64 ? launch_indexer_bf16_64(p, grid, st) : launch_indexer_bf16_128(p, grid, st);
}
#endif

}  // namespace dsa
