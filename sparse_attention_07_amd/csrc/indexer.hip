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
// per-chunk candidate lists (<= K entries) that a merge tree reduces.
//
// Design for CDNA4 (not the pages' accelerator):
//  * a planning kernel turns (seq_lens, q_seq, q_visible) into query groups
//    (adjacent queries of one sequence, up to MQ) and equal-size key chunks;
//  * one persistent workgroup per CU walks chunks.  Each wave streams 16-key
//    slices of 64-token pages straight into MFMA operand registers (per lane
//    64 contiguous bytes per key per load pair), with a 4-deep register
//    prefetch ring;
//  * MFMA M = 16 indexer heads per tile, N = 16 keys, K = head dim
//    (FP8: one 16x16x128 e4m3 MFMA per head tile; BF16: 16x16x32 steps);
//    ReLU and the head-weighted reduction run on the accumulators, then a
//    2-step permlane butterfly sums the four head groups;
//  * selection streams: each 1024-key round's scores are filtered against the
//    current K-th score into an LDS candidate buffer; when the buffer fills, a
//    block-wide 8-bit radix select (ties broken by position through a 64-bit
//    composite key) cuts it back to K.  Candidates stay in position order;
//  * a chunk's K survivors go to the workspace; the last chunk of each group of
//    8 to finish merges its siblings (arrival counter, no spinning), up to the
//    root, which writes the final pool slots.
#include "dsa_device.h"
#include "dsa_params.h"

namespace dsa {

// =============================================================================
// Planning kernel: one workgroup of 1024 threads.
// =============================================================================
constexpr int PLAN_NT = 1024;

__device__ __forceinline__ int block_scan_incl(int v, int* s_w, bool is_max) {
  // inclusive scan (sum or max) over PLAN_NT threads; s_w: >= 16 ints of LDS
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v = is_max ? max(v, o) : v + o;
  }
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

__global__ __launch_bounds__(PLAN_NT) void dsa_plan_kernel(IdxParams p) {
  __shared__ int s_w[16];
  __shared__ int s_carry[4];
  const int tid = threadIdx.x;
  // ---- pass 1: group starts (runs of one sequence, cut every MQ queries)
  int carry_run = 0, carry_gid = 0;
  for (int base = 0; base < p.T; base += PLAN_NT) {
    const int t = base + tid;
    const bool valid = t < p.T;
    const int b = valid ? plan_seq(p, t) : -2;
    const int bprev = (valid && t > 0) ? plan_seq(p, t - 1) : -3;
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
    }
    if (tid == PLAN_NT - 1) {
      s_carry[0] = run;
      s_carry[1] = carry_gid + gincl;
    }
    __syncthreads();
    carry_run = s_carry[0];
    carry_gid = s_carry[1];
    __syncthreads();
  }
  const int n_groups = carry_gid;
  __threadfence_block();
  __syncthreads();
  // ---- pass 2 + 3: per-group sizes and exclusive prefix sums
  int c_item = 0, c_list = 0, c_ctr = 0;
  for (int base = 0; base < n_groups; base += PLAN_NT) {
    const int g = base + tid;
    int items = 0, lists = 0, ctrs = 0;
    int* gr = p.groups + (int64_t)g * G_FIELDS;
    if (g < n_groups) {
      const int t0 = gr[G_T0];
      const int t1 = (g + 1 < n_groups) ? p.groups[(int64_t)(g + 1) * G_FIELDS + G_T0] : p.T;
      const int nq = t1 - t0;
      int range = 0;
      for (int t = t0; t < t1; ++t) range = max(range, plan_vis(p, t));
      const int nch = max(1, (range + p.CH - 1) / p.CH);
      gr[G_NQ] = nq;
      gr[G_RANGE] = range;
      gr[G_NCH] = nch;
      items = nch;
      lists = nq * tree_lists(nch);
      ctrs = tree_counters(nch);
    }
    const int si = block_scan_incl(items, s_w, false);
    const int sl = block_scan_incl(lists, s_w, false);
    const int sc = block_scan_incl(ctrs, s_w, false);
    if (g < n_groups) {
      gr[G_ITEM] = c_item + si - items;
      gr[G_LIST] = c_list + sl - lists;
      gr[G_CTR] = c_ctr + sc - ctrs;
    }
    if (tid == PLAN_NT - 1) {
      s_carry[0] = c_item + si;
      s_carry[1] = c_list + sl;
      s_carry[2] = c_ctr + sc;
    }
    __syncthreads();
    c_item = s_carry[0];
    c_list = s_carry[1];
    c_ctr = s_carry[2];
    __syncthreads();
  }
  for (int i = tid; i < c_ctr; i += PLAN_NT) p.ctr[i] = 0u;
  if (tid == 0) {
    p.hdr[0] = n_groups;
    p.hdr[1] = c_item;
  }
}

// =============================================================================
// Main indexer kernel.
// =============================================================================
template <int MQ>
struct CapOf {
  static constexpr int value = MQ == 1 ? 8192 : (MQ == 2 ? 4096 : 3072);
};

template <int NW, int MQ>
struct IdxSmem {
  static constexpr int CAP = CapOf<MQ>::value;
  static constexpr int NT = NW * 64;
  static constexpr int SL = ROUND / NT;
  uint32_t cand_key[MQ][CAP];
  int32_t cand_pos[MQ][CAP];
  uint32_t rb[2][MQ][ROUND];
  uint32_t hist[256];
  uint32_t wcnt[MQ][SL][NW];
  int32_t cnt[MQ];
  uint32_t thr[MQ];
  int32_t sel[4];
  int32_t flag;
  int32_t grp[G_FIELDS];
  int32_t pages[CH_MAX / PAGE];  // the chunk's block-table slice (-1 = invalid page)
};

// Block-wide Top-K of keys/pos[0..n) (n > K) by 8-bit radix select over the
// 64-bit composite (key, ~pos); exactly K entries remain, in their original
// (position) order, at [0..K).  Returns a lower bound of the smallest kept key
// (a later, higher position with key <= bound can never enter the Top-K).
template <int NW>
__device__ uint32_t block_select(uint32_t* keys, int32_t* pos, int n, int K, uint32_t* hist, int32_t* sel,
                                 uint32_t* wtmp) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t kpref = 0, ppref = 0;
  int need = K;
  int d = 0;
  for (; d < 8; ++d) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0u;
    lds_barrier();
    const bool onpos = d >= 4;
    const int dd = onpos ? d - 4 : d;
    const int shift = 24 - 8 * dd;
    for (int i = tid; i < n; i += NT) {
      const uint32_t k = keys[i];
      const uint32_t pp = ~(uint32_t)pos[i];
      bool m;
      if (!onpos)
        m = (dd == 0) || ((k >> (32 - 8 * dd)) == (kpref >> (32 - 8 * dd)));
      else
        m = (k == kpref) && ((dd == 0) || ((pp >> (32 - 8 * dd)) == (ppref >> (32 - 8 * dd))));
      if (m) atomicAdd(&hist[((onpos ? pp : k) >> shift) & 255u], 1u);
    }
    lds_barrier();
    if (tid < 64) {
      // lane L owns bins 255-4L .. 252-4L (descending)
      uint32_t c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * lane - j];
        s += c[j];
      }
      const uint32_t incl = wave_incl_scan(s);
      const uint32_t excl = incl - s;
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
    const int bin = sel[0], above = sel[1], cb = sel[2];
    lds_barrier();
    need -= above;
    if (!onpos)
      kpref |= (uint32_t)bin << shift;
    else
      ppref |= (uint32_t)bin << shift;
    if (cb == need) break;
  }
  if (d > 7) d = 7;
  // ---- order-preserving compaction of the selected entries
  const bool onpos = d >= 4;
  const int kshift = onpos ? 0 : 24 - 8 * d;
  const int pshift = onpos ? 24 - 8 * (d - 4) : 0;
  int running = 0;
  for (int base = 0; base < n; base += NT) {
    const int i = base + tid;
    uint32_t k = 0;
    int32_t ps = 0;
    bool s = false;
    if (i < n) {
      k = keys[i];
      ps = pos[i];
      if (!onpos)
        s = (k >> kshift) >= (kpref >> kshift);
      else
        s = (k > kpref) || (k == kpref && ((~(uint32_t)ps) >> pshift) >= (ppref >> pshift));
    }
    const uint64_t m = ballot(s);
    if (lane == 0) wtmp[wave] = (uint32_t)__builtin_popcountll(m);
    lds_barrier();
    int pre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = (int)wtmp[w];
      pre += (w < wave) ? c : 0;
      tot += c;
    }
    if (s) {
      const int o = running + pre + lanes_below(m);
      keys[o] = k;
      pos[o] = ps;
    }
    running += tot;
    lds_barrier();
  }
  return kpref;
}

template <int DT, int D>
struct Frag {
  // bf16: one 16-byte piece per 32-wide k step; fp8: two 16-byte pieces (k=128)
  static constexpr int NP = DT == 0 ? D / 32 : 2;
  v4i d[NP];
};

template <int DT, int D>
struct BFrag {
  Frag<DT, D> f;
  float sc;
  int ok;
};

template <int DT, int D, int HT, int MQ, int NW>
__global__ __launch_bounds__(NW * 64, 1) void dsa_indexer_kernel(IdxParams p) {
  using Sm = IdxSmem<NW, MQ>;
  constexpr int NT = NW * 64;
  constexpr int CAP = Sm::CAP;
  constexpr int SL = Sm::SL;
  constexpr int GPW = ROUND / 16 / NW;  // 16-key groups per wave per round
  constexpr int PF = 4;                 // register prefetch depth (groups)
  constexpr int ES = DT == 0 ? 2 : 1;   // bytes per element
  constexpr int ROWB = D * ES;          // bytes per key row
  static_assert(GPW % PF == 0, "prefetch ring must divide the round");
  static_assert(DT == 0 || D == 128, "fp8 path is 128-wide");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int g4 = lane >> 4;
  const int n16 = lane & 15;

  const int n_items = p.hdr[1];
  const int n_groups = p.hdr[0];

  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int item = n_items - 1 - it;  // heaviest (last) groups first
    // ---- locate the group of this item (binary search on item starts)
    int lo = 0, hi = n_groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.groups[(int64_t)mid * G_FIELDS + G_ITEM] <= item)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int* gr = p.groups + (int64_t)lo * G_FIELDS;
    const int t0 = uniform(gr[G_T0]);
    const int nq = uniform(gr[G_NQ]);
    const int seq = uniform(gr[G_SEQ]);
    const int range = uniform(gr[G_RANGE]);
    const int nch = uniform(gr[G_NCH]);
    const int chunk = item - uniform(gr[G_ITEM]);
    const int list_base = uniform(gr[G_LIST]);
    const int ctr_base = uniform(gr[G_CTR]);
    const int kb = chunk * p.CH;
    const int ke = min(kb + p.CH, range);
    const int32_t* bt = p.block_table + (int64_t)max(seq, 0) * p.max_blocks;

    int lim[MQ];
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      int v = 0;
      if (q < nq) {
        const int t = t0 + q;
        const int b = seq;
        if (b >= 0) {
          const int L = min(max(p.seq_lens[b], 0), p.max_blocks * PAGE);
          v = p.q_visible ? p.q_visible[t] : L;
          v = min(max(v, 0), L);
        }
      }
      lim[q] = uniform(min(v, ke));
    }

    // ---- query operands and weights (identical in every wave)
    Frag<DT, D> a[MQ][HT];
    float wv[MQ][HT][4];
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) {
        const int h = mt * 16 + n16;
        const bool okh = q < nq && h < p.H_idx;
        const uint8_t* row = p.q_idx + ((int64_t)(t0 + q) * p.H_idx + h) * ROWB;
#pragma unroll
        for (int j = 0; j < Frag<DT, D>::NP; ++j) {
          const int off = DT == 0 ? 2 * (32 * j + 8 * g4) : (64 * j + 16 * g4);
          a[q][mt].d[j] = okh ? *reinterpret_cast<const v4i*>(row + off) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hh = mt * 16 + 4 * g4 + i;
          float wt = 0.f;
          if (q < nq && hh < p.H_idx) {
            const int64_t o = (int64_t)(t0 + q) * p.H_idx + hh;
            wt = p.w[o];
            if (DT == 1) wt *= p.q_scale[o];
          }
          wv[q][mt][i] = wt;
        }
      }
    }

    if (tid < MQ) {
      sm.cnt[tid] = 0;
      sm.thr[tid] = 0u;
    }
    for (int i = tid; i < (ke - kb + PAGE - 1) / PAGE; i += NT) {
      const int pg = bt[(kb >> 6) + i];
      sm.pages[i] = (pg >= 0 && (int64_t)pg < p.num_blocks) ? pg : -1;
    }
    lds_barrier();

    // ---- streaming rounds
    const int nkeys = max(ke - kb, 0);
    const int nrounds = (nkeys + ROUND - 1) / ROUND;
    const int total_j = nrounds * GPW;
    auto group_p0 = [&](int j) { return kb + (j / GPW) * ROUND + (wave * GPW + (j % GPW)) * 16; };

    auto load_b = [&](BFrag<DT, D>& bf, int p0) {
      int page = sm.pages[(p0 - kb) >> 6];
      const bool ok = page >= 0;
      page = ok ? page : 0;
      const int r = (p0 & 63) + n16;
      const uint8_t* pg = p.k_pool + (int64_t)page * p.page_bytes;
      const uint8_t* rowp = pg + r * ROWB;
#pragma unroll
      for (int j = 0; j < Frag<DT, D>::NP; ++j) {
        const int off = DT == 0 ? 2 * (32 * j + 8 * g4) : (64 * j + 16 * g4);
        bf.f.d[j] = *reinterpret_cast<const v4i*>(rowp + off);
      }
      bf.sc = DT == 1 ? *reinterpret_cast<const float*>(pg + PAGE * ROWB + 4 * r) : 1.f;
      bf.ok = ok;
    };

    auto score_group = [&](const BFrag<DT, D>& bf, int p0, int rs, int rbuf) {
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        if (q < nq) {
          // all head tiles' MFMAs first (independent accumulators), then the VALU
          v4f acc[HT];
#pragma unroll
          for (int mt = 0; mt < HT; ++mt) {
            acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
            if constexpr (DT == 1) {
              const v8i av = __builtin_shufflevector(a[q][mt].d[0], a[q][mt].d[1], 0, 1, 2, 3, 4, 5, 6, 7);
              const v8i bv = __builtin_shufflevector(bf.f.d[0], bf.f.d[1], 0, 1, 2, 3, 4, 5, 6, 7);
              acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mt], 0, 0, 0, 0, 0, 0);
            } else {
#pragma unroll
              for (int j = 0; j < Frag<DT, D>::NP; ++j)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[q][mt].d[j]),
                                                                  __builtin_bit_cast(v8bf, bf.f.d[j]), acc[mt], 0, 0, 0);
            }
          }
          float part = 0.f;
#pragma unroll
          for (int mt = 0; mt < HT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // ReLU as an integer max on the bit pattern: negative floats
              // (sign bit set) become +0, everything else is unchanged
              const float d = __int_as_float(max(__float_as_int(acc[mt][i]), 0));
              part = fmaf(wv[q][mt][i], d, part);
            }
          float s = sum_lane_groups(part);
          if (DT == 1) s *= bf.sc;
          const int pp = p0 + n16;
          const bool valid = bf.ok && pp < lim[q];
          if (lane < 16) sm.rb[rbuf][q][pp - rs] = valid ? order_key(s) : 0u;
        }
      }
    };

    // streaming filter of one batch of up to ROUND (key, pos) pairs into the
    // candidate buffers, keeping position order
    auto filter_append = [&](int q, int n, auto get) {
      const uint32_t thr = sm.thr[q];
      const int base = sm.cnt[q];
      uint32_t kk[SL];
      int32_t pp[SL];
      uint64_t mk[SL];
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        const int i = s * NT + tid;
        kk[s] = 0u;
        pp[s] = 0;
        if (i < n) get(i, kk[s], pp[s]);
        mk[s] = ballot(kk[s] > thr);
        if (lane == 0) sm.wcnt[q][s][wave] = (uint32_t)__builtin_popcountll(mk[s]);
      }
      lds_barrier();
      int running = base;
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        int pre = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int c = (int)sm.wcnt[q][s][w];
          pre += (w < wave) ? c : 0;
          tot += c;
        }
        if (kk[s] > thr) {
          const int o = running + pre + lanes_below(mk[s]);
          sm.cand_key[q][o] = kk[s];
          sm.cand_pos[q][o] = pp[s];
        }
        running += tot;
      }
      lds_barrier();
      if (tid == 0) sm.cnt[q] = running;
      lds_barrier();
      if (running > CAP - ROUND) {
        const uint32_t t = block_select<NW>(sm.cand_key[q], sm.cand_pos[q], running, p.K, sm.hist, sm.sel,
                                            &sm.wcnt[0][0][0]);
        if (tid == 0) {
          sm.cnt[q] = p.K;
          sm.thr[q] = t;
        }
        lds_barrier();
      }
    };

    {
      // Loads are unconditional so the prefetch queue depth stays static: slots
      // past the chunk end re-read the chunk's last 16-key group (a cache hit).
      const int last_p0 = kb + ((max(nkeys, 1) - 1) & ~15);
      auto load_p0 = [&](int j) { return min(group_p0(j), last_p0); };
      BFrag<DT, D> buf[PF];
      if (nkeys > 0) {
#pragma unroll
        for (int s = 0; s < PF; ++s) load_b(buf[s], load_p0(s));
      }
      for (int r = 0; r < nrounds; ++r) {
        const int rs = kb + r * ROUND;
        const int rbuf = r & 1;
#pragma unroll
        for (int s = 0; s < GPW; ++s) {
          const int j = r * GPW + s;
          const int p0 = group_p0(j);
          if (p0 < ke) score_group(buf[s % PF], p0, rs, rbuf);
          load_b(buf[s % PF], load_p0(j + PF));
        }
        lds_barrier();
        const int nr = min(ROUND, ke - rs);
#pragma unroll
        for (int q = 0; q < MQ; ++q)
          if (q < nq)
            filter_append(q, nr, [&](int i, uint32_t& k, int32_t& ps) {
              k = sm.rb[rbuf][q][i];
              ps = rs + i;
            });
      }
    }

    auto finish_select = [&]() {
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        if (q < nq) {
          const int c = sm.cnt[q];
          if (c > p.K) {
            block_select<NW>(sm.cand_key[q], sm.cand_pos[q], c, p.K, sm.hist, sm.sel, &sm.wcnt[0][0][0]);
            lds_barrier();
            if (tid == 0) sm.cnt[q] = p.K;
            lds_barrier();
          }
        }
      }
    };
    auto write_final = [&]() {
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        if (q < nq) {
          const int c = sm.cnt[q];
          int32_t* out = p.indices + (int64_t)(t0 + q) * p.K;
          for (int i = tid; i < p.K; i += NT) {
            int v = -1;
            if (i < c) {
              const int ps = sm.cand_pos[q][i];
              v = bt[ps >> 6] * PAGE + (ps & 63);
            }
            out[i] = v;
          }
        }
      }
    };

    finish_select();
    if (nch == 1) {
      write_final();
      lds_barrier();
      continue;
    }

    // ---- merge tree over the group's chunks (last arrival merges)
    const int U = tree_lists(nch);
    int idx = chunk, n_level = nch, off_list = 0, off_ctr = 0;
    while (true) {
      // store this node's lists
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        if (q < nq) {
          const int64_t unit = (int64_t)list_base + (int64_t)q * U + off_list + idx;
          const int c = sm.cnt[q];
          for (int i = tid; i < c; i += NT) {
            p.list_keys[unit * p.K + i] = sm.cand_key[q][i];
            p.list_pos[unit * p.K + i] = sm.cand_pos[q][i];
          }
          if (tid == 0) p.list_cnt[unit] = c;
        }
      }
      __threadfence();
      __syncthreads();
      const int parent = idx / FANIN;
      const int n_parent = (n_level + FANIN - 1) / FANIN;
      const int nchild = min(FANIN, n_level - parent * FANIN);
      if (tid == 0) {
        const uint32_t old = atomicAdd(&p.ctr[ctr_base + off_ctr + parent], 1u);
        sm.flag = (old == (uint32_t)(nchild - 1)) ? 1 : 0;
      }
      __syncthreads();
      if (!sm.flag) break;
      __threadfence();
      // merge the children of `parent`
      if (tid < MQ) {
        sm.cnt[tid] = 0;
        sm.thr[tid] = 0u;
      }
      __syncthreads();
      for (int ch = 0; ch < nchild; ++ch) {
        const int cidx = parent * FANIN + ch;
#pragma unroll
        for (int q = 0; q < MQ; ++q) {
          if (q < nq) {
            const int64_t unit = (int64_t)list_base + (int64_t)q * U + off_list + cidx;
            const int n_c = __hip_atomic_load(&p.list_cnt[unit], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t* lk = p.list_keys + unit * p.K;
            const int32_t* lp = p.list_pos + unit * p.K;
            for (int s0 = 0; s0 < n_c; s0 += ROUND) {
              filter_append(q, min(ROUND, n_c - s0), [&](int i, uint32_t& k, int32_t& ps) {
                k = lk[s0 + i];
                ps = lp[s0 + i];
              });
            }
          }
        }
      }
      finish_select();
      off_list += n_level;
      off_ctr += n_parent;
      idx = parent;
      n_level = n_parent;
      if (n_level == 1) {
        write_final();
        break;
      }
    }
    __syncthreads();
  }
}

// =============================================================================
// Host-side launch helpers (called from the C ABI layer).
// =============================================================================
template <int DT, int D, int HT, int MQ, int NW>
static hipError_t launch_indexer_t(const IdxParams& p, int grid, hipStream_t st) {
  auto kfn = dsa_indexer_kernel<DT, D, HT, MQ, NW>;
  const size_t smem = sizeof(IdxSmem<NW, MQ>);
  hipError_t e = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(grid), dim3(NW * 64), smem, st, p);
  return hipGetLastError();
}

template <int DT, int D, int HT>
static hipError_t launch_indexer_mq(const IdxParams& p, int grid, hipStream_t st) {
  switch (p.MQ) {
    case 1: return launch_indexer_t<DT, D, HT, 1, 8>(p, grid, st);
    case 2: return launch_indexer_t<DT, D, HT, 2, 8>(p, grid, st);
    default: return launch_indexer_t<DT, D, HT, 4, 4>(p, grid, st);
  }
}

hipError_t launch_indexer(const IdxParams& p, int is_fp8, int D, int grid, hipStream_t st) {
  hipLaunchKernelGGL(dsa_plan_kernel, dim3(1), dim3(PLAN_NT), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool small_heads = p.H_idx <= 16;
  if (is_fp8) return small_heads ? launch_indexer_mq<1, 128, 1>(p, grid, st) : launch_indexer_mq<1, 128, 4>(p, grid, st);
  if (D == 64) return small_heads ? launch_indexer_mq<0, 64, 1>(p, grid, st) : launch_indexer_mq<0, 64, 4>(p, grid, st);
  return small_heads ? launch_indexer_mq<0, 128, 1>(p, grid, st) : launch_indexer_mq<0, 128, 4>(p, grid, st);
}

size_t indexer_smem_bytes(int MQ) {
  switch (MQ) {
    case 1: return sizeof(IdxSmem<8, 1>);
    case 2: return sizeof(IdxSmem<8, 2>);
    default: return sizeof(IdxSmem<4, 4>);
  }
}

}  // namespace dsa
