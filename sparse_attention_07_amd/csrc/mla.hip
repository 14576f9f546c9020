// Sparse MLA over the selected latent rows, for gfx950.
//
// What is computed ("Hybrid Attention LLM Inference Acceleration", section 2,
// sparse attention computation; "Day-0 Inference Adaptation for LLMs",
// operator section 2: the filter results go straight to the compute kernel):
// for query token t and head h over the selected rows C_j (576-wide latent,
// 512 nope + 64 rope),
//     out[t,h,:] = sum_j softmax_j(scale * q[t,h,:] . C_j) * C_j[:512].
//
// Design for CDNA4:
//  * grid = (split, query); a workgroup owns a contiguous slice of the query's
//    index list and all H heads, so every gathered row leaves HBM once;
//  * rows are gathered 32 at a time with direct-to-LDS 16-byte loads
//    (global_load_lds_dwordx4) into a 3-stage ring: a row's 512 value dims
//    are one 64-lane load from a uniform (scalar) row address, its rope dims
//    a fifth of a load; rows sit in a permuted slot order at padded strides
//    that keep the operand reads of both phases free of bank conflicts (see
//    row_slot), and operand addresses stay base + immediate;
//  * H/16 waves.  Logits: wave w owns heads 16w..16w+15, keeps their q in
//    registers as the MFMA B operand and computes S^T = C q^T (bf16 16x16x32;
//    rows on M in an order that makes the probabilities come out as 8
//    consecutive rows per lane), runs the online softmax (exp2 domain) and
//    writes P^T (bf16) and the per-head rescale factor to LDS.
//    PV: wave w owns value dims [512w/NW, 512(w+1)/NW) for all heads and
//    accumulates O^T += C^T P^T, reading C^T with the gfx950 LDS transpose
//    read (ds_read_b64_tr_b16) and P^T with plain 16-byte reads;
//  * the tile loop is software-pipelined with one barrier per tile (the PV
//    of tile i-1 and the logits and softmax of tile i in one iteration); the
//    two waves of a SIMD run those phases in opposite orders, and the logits'
//    A operands are read two k-steps ahead of their MFMAs;
//  * each head's reference maximum moves only when a tile's maximum exceeds
//    it by more than 2^8 (probabilities stay below 256, exact in the end:
//    O and l carry the same offset), so the O rescale is skipped for a wave
//    unless some head's maximum jumped; on tiles whose rows are all present
//    the probabilities are taken against the reference first and the tile
//    maximum is computed only when one of them passes the bound;
//  * with several splits, each split stores its partial output O, not yet
//    divided by l, as bf16 (probabilities below 2^8 over at most 2048 rows:
//    |O| stays within 2^19 times the largest value entry, far inside bf16's
//    range), plus (m, l) in fp32, and a small kernel merges them with
//    log-sum-exp weights and divides once;
//  * optional residual + RMSNorm epilogue over the token's H x 512 values: with
//    one split the workgroup holds the whole token and finishes it; with
//    several, the combine adds the residual and stores per-head sums of
//    squares, and a small kernel applies the norm;
//  * FP8 latent rows (656 B: e4m3fn nope, one fp32 scale per 128 dims, bf16
//    rope) are gathered into a 2-stage ring of their own (41 sixteen-byte
//    units per row, each lane stepping through the ring), then all waves
//    dequantize the tile once into the bf16 tile layout above (code * scale
//    rounded to bf16), so the MFMA phases are the bf16 ones.  That saves 43 %
//    of the gathered bytes and of the cache's footprint, but the dequantization
//    and its second barrier per tile sit on every tile's critical path, so it
//    runs slower than bf16 rows.
#include "dsa_device.h"
#include "dsa_params.h"


namespace dsa {
typedef int v2i __attribute__((ext_vector_type(2)));  // 8-byte streaming stores

constexpr int TILE_ROWS = 32;
constexpr float RESCALE_SLACK = 8.f;  // log2 of the largest unnormalised probability
constexpr float RESCALE_BOUND = 256.f;  // 2^RESCALE_SLACK
constexpr int MLA_SMAX = 8;  // most splits of a query's index list (K / 256 for K <= 2048)
constexpr int A_STRIDE = 66;                          // value region: units per row slot (64 + 2 padding)
constexpr int B_UNIT0 = TILE_ROWS * A_STRIDE;         // rope region: first unit
constexpr int B_STRIDE = 10;                          // rope region: units per row slot (8 + 2 padding)
constexpr int ROPE_LOADS = (TILE_ROWS * B_STRIDE + 63) / 64;  // 5 wave-loads
constexpr int PT_STRIDE = TILE_ROWS + 16;             // P^T row (bf16): 6 sixteen-byte units
constexpr int STAGES = 3;
constexpr int OB_STRIDE = VDIM * 2 + 16;                // O row (bf16) staged in LDS for the store
constexpr int LDS_AHEAD = 2;  // logits: k-steps of A operands read ahead (3 needs more registers than a wave has)
constexpr int STAGE_BYTES = (B_UNIT0 + ROPE_LOADS * 64) * 16;  // 38,912 B

// FP8 latent rows: 512 code bytes, 4 fp32 scales, 64 bf16 rope dims
constexpr int KV8_ROW_UNITS = 41;                                   // 656 B
constexpr int KV8_SCALE_OFF = 512;
constexpr int KV8_ROPE_OFF = 528;
constexpr int KV8_TILE_LOADS = (TILE_ROWS * KV8_ROW_UNITS + 63) / 64;  // 21 wave-loads of 64 units
constexpr int KV8_STAGE_BYTES = KV8_TILE_LOADS * 64 * 16;

// LDS layout of a bf16 tile.  Tile row r is stored in row slot
// p(r) = 4*(r/8) + r%4 + 16*((r/4)%2): the logits A operand of M-tile mt
// reads tile rows 8*(n/4) + n%4 + 4*mt for lanes n = 0..15, i.e. 16
// consecutive slots, and the PV transpose reads (rows 8*g + j and 8*g + 4 + j)
// fall on consecutive slots too.  A slot's 512 value dims (64 sixteen-byte
// units) sit in the value region at a stride of 66 units, its 64 rope dims in
// the rope region at 10 units.  Bank conflicts (measured with the LDS
// counters on gfx950): a wave's 16-byte reads that put 16 lanes on 16 slots,
// the 4 lane groups one unit apart, are conflict-free when the slots lie
// 2 mod 4 units apart and take 2-4 cycles more otherwise.  The split of the
// two regions makes one row's value units one 64-lane direct-to-LDS load
// from a uniform row address.
__device__ __forceinline__ int row_slot(int r) { return 4 * (r >> 3) + (r & 3) + 16 * ((r >> 2) & 1); }
__device__ __forceinline__ int slot_row(int p) { return 8 * ((p & 15) >> 2) + (p & 3) + 4 * (p >> 4); }
// unit, inside a stage, of value unit u (0..63) and of rope unit j (0..7) of tile row r
__device__ __forceinline__ int val_unit(int r, int u) { return A_STRIDE * row_slot(r) + u; }
__device__ __forceinline__ int rope_unit(int r, int j) { return B_UNIT0 + B_STRIDE * row_slot(r) + j; }

template <int NW, bool KV8>
struct alignas(16) MlaSmem {
  static constexpr int NSTAGE = KV8 ? 2 : STAGES;
  unsigned char stage[NSTAGE][KV8 ? KV8_STAGE_BYTES : STAGE_BYTES];  // gather ring
  unsigned char tile[KV8 ? 2 : 1][KV8 ? STAGE_BYTES : 16];          // FP8 only: two dequantized bf16 tiles
  uint16_t pt[2][16 * NW][PT_STRIDE];  // P^T as [head][row] bf16, two tiles (rows padded: no bank conflicts)
  float alpha[2][16 * NW];             // per-head rescale factor, two tiles
  float mfin[16 * NW];
  float lfin[16 * NW];
  float red[NW];  // per-wave partial sums (residual + RMSNorm epilogue)
  // followed by the slice's slots (int32, 16-byte aligned)
};

// The lane index computed afresh (two VALU operations, no input), for
// per-lane addresses used once per tile: nothing derived from the lane then
// stays live across the tile loop.
__device__ __forceinline__ int lane_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// 16 e4m3fn codes times one scale -> 16 bf16 (round to nearest even)
__device__ __forceinline__ void dequant16(const v4i c, float sc, v4i& lo, v4i& hi) {
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8(c[j], false);
    const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8(c[j], true);
    __bf16 o4[4] = {(__bf16)(a[0] * sc), (__bf16)(a[1] * sc), (__bf16)(b[0] * sc), (__bf16)(b[1] * sc)};
    const uint2 u = __builtin_bit_cast(uint2, o4);
    w[2 * j] = u.x;
    w[2 * j + 1] = u.y;
  }
  lo = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  hi = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
}

template <int NW, bool KV8>
__global__ __launch_bounds__(NW * 64, 1) void dsa_mla_split_kernel(MlaParams p) {
  constexpr int NT = NW * 64;
  constexpr int H = 16 * NW;
  constexpr int VT = 32 / NW;  // 16-wide value tiles per wave in PV
  constexpr int LOADS = KV8_TILE_LOADS;                // FP8 rows: wave-loads per tile
  constexpr int RUNITS = KV8_ROW_UNITS;                // FP8 rows: units per row in the gather ring
  constexpr int LMIN = LOADS / NW;                     // FP8 rows: DMA loads of every wave per tile
  constexpr int LEXTRA = LOADS - LMIN * NW;            // FP8 rows: waves [0, LEXTRA) issue one more
  constexpr int RPW = TILE_ROWS / NW;                  // bf16 rows: value rows each wave gathers per tile
  extern __shared__ __align__(16) unsigned char smem_raw[];
  MlaSmem<NW, KV8>& sm = *reinterpret_cast<MlaSmem<NW, KV8>*>(smem_raw);
  int32_t* sidx = reinterpret_cast<int32_t*>(smem_raw + sizeof(MlaSmem<NW, KV8>));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int g4 = lane >> 4;
  const int n16 = lane & 15;
  // ---- workgroup -> (query, split).  Workgroups go to the 8 XCDs round-robin
  // by linear id; with T a multiple of 8 the splits of a query are given ids of
  // one XCD, so the query's q rows, which every split reads, come from that
  // XCD's L2 after the first read instead of from HBM once per split.
  int t, s;
  {
    const int id = blockIdx.y * gridDim.x + blockIdx.x;
    if ((p.T & 7) == 0) {
      const int k = id >> 3;
      t = (k / p.S) * 8 + (id & 7);
      s = k % p.S;
    } else {
      t = blockIdx.y;
      s = blockIdx.x;
    }
    t = uniform(t);
    s = uniform(s);
  }
  const int r_begin = s * p.rows_per_split;
  const int r_end = min(p.K, r_begin + p.rows_per_split);
  const int nrows = max(0, r_end - r_begin);
  const int ntiles = (nrows + TILE_ROWS - 1) / TILE_ROWS;

  // ---- the slice's pool slots (invalid -> -1), and q of this wave's 16 heads
  // as the logits B operand (k = latent dim).  Every slot load is issued
  // before q, unconditionally (a slice holds at most KMAX rows; indices past
  // the slice are clamped and their values masked afterwards), so no branch
  // and no wait for q sits in front of the first tile's gather: it starts
  // while q is still in flight.
  constexpr int SPT = KMAX / NT;  // slot loads per thread
  const int32_t* irow = p.indices + (int64_t)t * p.K;
  const int ncap = ntiles * TILE_ROWS;  // slot entries; entry ncap takes the writes past them
  int sv[SPT];
#pragma unroll
  for (int k = 0; k < SPT; ++k) sv[k] = irow[min(r_begin + min(tid + k * NT, max(nrows - 1, 0)), p.K - 1)];
  const int hq = wave * 16 + n16;
  v4i qb[18];
  {
    const uint16_t* qrow = p.q + ((int64_t)t * H + hq) * LATENT;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qb[ks] = *reinterpret_cast<const v4i*>(qrow + 32 * ks + 8 * g4);
  }
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int i = tid + k * NT;
    const int v = sv[k];
    sidx[i < ncap ? i : ncap] = (i < nrows && v >= 0 && (int64_t)v < p.num_slots) ? v : -1;
  }
  lds_barrier();

  constexpr int NSTAGE = MlaSmem<NW, KV8>::NSTAGE;
  // FP8 rows: load k of this wave covers ring units (first + k) * 64 + lane;
  // the lane's row and 16-byte column advance by 64 units (less than one row)
  // per load, so they are stepped, not divided.
  const int first_u = (wave * LMIN + min(wave, LEXTRA)) * 64 + lane;
  const int r_first = first_u / RUNITS;
  const int c_first = first_u - r_first * RUNITS;
  // bf16 rows: the DMA loads of tile ti into gather stage stage_i
  auto issue_tile_bf16 = [&](int stage_i, int ti) {
    const uint32_t st_lds = uniform((uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)sm.stage[stage_i]);
    // value units: one wave-load per row (lane i: unit i), from a uniform row
    // address, so the address arithmetic is scalar
#pragma unroll
    for (int i0 = 0; i0 < RPW; i0 += 4) {
      // this wave's next 4 rows (4 consecutive row slots): slots in one read
      const v4i sl = *reinterpret_cast<const v4i*>(&sidx[ti * TILE_ROWS + RPW * wave + i0]);
      const uint32_t lds0 = uniform(st_lds + 16 * A_STRIDE * row_slot(RPW * wave + i0));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = max(__builtin_amdgcn_readfirstlane(sl[i]), 0);  // absent rows: a harmless valid row
        dma16_to_lds_saddr(p.kv + (int64_t)slot * LATENT, 16 * lane, lds0 + 16 * A_STRIDE * i);
      }
    }
    // rope units: wave-load j covers rope-region units 64j + lane (the two
    // padding units of a slot get a harmless valid unit)
    for (int j = wave; j < ROPE_LOADS; j += NW) {
      const uint32_t u = 64 * j + lane_fresh();
      const uint32_t ps = u / B_STRIDE, c = u - ps * B_STRIDE;
      const int slot = max(sidx[ti * TILE_ROWS + slot_row(ps)], 0);
      dma16_to_lds(p.kv + (int64_t)slot * LATENT + 512 + 8 * (c < 8 ? c : 0), uniform(st_lds + 16 * (B_UNIT0 + 64 * j)));
    }
  };
  auto issue_tile_fp8 = [&](int ti) {  // FP8 rows: the DMA loads of tile ti
    unsigned char* st = sm.stage[ti % NSTAGE];
    const uint32_t st_lds = uniform((uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)st);
    if constexpr (KV8) {
      const int nl = LMIN + (wave < LEXTRA ? 1 : 0);
      const int first = wave * LMIN + min(wave, LEXTRA);
      int r = r_first, c = c_first;
      for (int k = 0; k < nl; ++k) {
        int rr = r, cc = c;
        if (rr >= TILE_ROWS || cc >= KV8_ROW_UNITS) {  // padding: a harmless valid unit
          rr = min(rr, TILE_ROWS - 1);
          cc = 0;
        }
        int slot = sidx[ti * TILE_ROWS + rr];
        slot = slot < 0 ? 0 : slot;
        dma16_to_lds(p.kv + (int64_t)slot * (KV8_ROW_UNITS * 8) + 8 * cc, st_lds + 16 * (first + k) * 64);
        r += 64 / RUNITS;
        c += 64 % RUNITS;
        if (c >= RUNITS) {
          c -= RUNITS;
          ++r;
        }
      }
    }
  };

  if (ntiles > 0) {
    if constexpr (!KV8)
      issue_tile_bf16(0, 0);
    else
      issue_tile_fp8(0);
  }
  // retire every plain global load here (tile 0 lands too), so no
  // compiler-inserted wait inside the tile loop can count (and drain) the row
  // DMA queue
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  lds_barrier();


  v4f o[VT][NW];  // O^T[v tile][head tile]
#pragma unroll
  for (int vt = 0; vt < VT; ++vt)
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) o[vt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // for head hq (logits role)

  // logits + online softmax of tile ti from the bf16 tile at st (writes P^T, alpha)
  auto logits_softmax = [&](int ti, const unsigned char* st) {
    // ---- logits S^T[row, head] for heads 16w..16w+15
    const uint32_t vmask = (uint32_t)ballot(lane < 32 && sidx[ti * TILE_ROWS + (lane & 31)] >= 0);
    v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    // M-tile row n16 holds tile row 8*(n16/4) + 4*mt + n16%4; k-step ks adds 64 bytes
    // (value region for k-steps 0..15, rope region for 16 and 17)
    // (per-lane offsets from a fresh lane index: nothing per lane stays live
    // across the tile loop for them)
    const int lf = lane_fresh();
    const unsigned char* la0 = st + 16 * (A_STRIDE * (lf & 15) + (lf >> 4));  // slot n16
    const unsigned char* lb0 = st + 16 * (B_UNIT0 + B_STRIDE * (lf & 15) + (lf >> 4));
    // A operands read LDS_AHEAD k-steps ahead of their MFMAs, so the LDS
    // latency is hidden behind the MFMAs of the steps in between
    v4i ar[LDS_AHEAD + 1][2];
    auto read_a = [&](int ks, v4i* a) {
      const unsigned char* a0p = ks < 16 ? la0 + 64 * ks : lb0 + 64 * (ks - 16);
      const unsigned char* a1p = a0p + 16 * 16 * (ks < 16 ? A_STRIDE : B_STRIDE);  // slot 16 + n16
      a[0] = *reinterpret_cast<const v4i*>(a0p);
      a[1] = *reinterpret_cast<const v4i*>(a1p);
    };
#pragma unroll
    for (int ks = 0; ks < LDS_AHEAD; ++ks) read_a(ks, ar[ks]);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (ks + LDS_AHEAD < 18) read_a(ks + LDS_AHEAD, ar[(ks + LDS_AHEAD) % (LDS_AHEAD + 1)]);
      const v4i* a = ar[ks % (LDS_AHEAD + 1)];
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[0]), __builtin_bit_cast(v8bf, qb[ks]),
                                                       acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[1]), __builtin_bit_cast(v8bf, qb[ks]),
                                                       acc[1], 0, 0, 0);
    }
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (ks == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2 * LDS_AHEAD, 0);
      if (ks + LDS_AHEAD < 18) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // ---- online softmax: this lane holds head hq, rows 8*g4 + 4*mt + i
    if (vmask == 0xffffffffu) {
      // every row of the tile present (almost every tile): no masking.  The
      // probabilities are first taken against the running reference maximum
      // (scale folded into the FMA that feeds the exponent); only if one of
      // the wave's exceeds 2^RESCALE_SLACK (or the reference is still -inf)
      // is the tile's maximum computed and the reference moved, so the
      // maximum and its cross-lane reduction leave the common path.
      float pr[8];
      bool big = false;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[4 * mt + i] = __builtin_amdgcn_exp2f(fmaf(acc[mt][i], p.scale_log2, -m_run));
          big |= !(pr[4 * mt + i] <= RESCALE_BOUND);
        }
      float a_ = 1.f;
      if (__builtin_amdgcn_ballot_w64(big)) {
        // the maximum (finite) is taken on the raw logits (the scale is positive)
        float tm = fmaxf(fmaxf(fmaxf(acc[0][0], acc[0][1]), fmaxf(acc[0][2], acc[0][3])),
                         fmaxf(fmaxf(acc[1][0], acc[1][1]), fmaxf(acc[1][2], acc[1][3])));
        const float tmax = max_lane_groups(tm) * p.scale_log2;
        const float m_new = (tmax > m_run + RESCALE_SLACK) ? tmax : m_run;
        a_ = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[4 * mt + i] = __builtin_amdgcn_exp2f(fmaf(acc[mt][i], p.scale_log2, -m_new));
        m_run = m_new;
      }
      float lsum = 0.f;
      __bf16 pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lsum += pr[j];
        pv[j] = (__bf16)pr[j];
      }
      l_run = l_run * a_ + lsum;
      *reinterpret_cast<v4i*>(&sm.pt[ti & 1][hq][8 * g4]) = __builtin_bit_cast(v4i, pv);
      if (g4 == 0) sm.alpha[ti & 1][wave * 16 + (lane_fresh() & 15)] = a_;
    } else {
      float x[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 8 * g4 + 4 * mt + i;
          const bool ok = (vmask >> row) & 1u;
          x[4 * mt + i] = ok ? acc[mt][i] * p.scale_log2 : -INFINITY;
          tmax = fmaxf(tmax, x[4 * mt + i]);
        }
      tmax = max_lane_groups(tmax);
      // The reference maximum moves only when the tile's exceeds it by more
      // than RESCALE_SLACK (log2 units): the probabilities then stay below
      // 2^RESCALE_SLACK, O and l carry the same offset (the normalisation and
      // the split combine remove it), and the O rescale (128 products per
      // lane) runs only on such jumps instead of on almost every tile.
      const float m_new = (tmax > m_run + RESCALE_SLACK) ? tmax : m_run;
      // the hardware exp2 (v_exp_f32): results below 2^-126 only feed sums
      // dominated by terms >= 1
      const float a_ = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      float lsum = 0.f;
      __bf16 pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pr = (m_new == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x[j] - m_new);
        lsum += pr;
        pv[j] = (__bf16)pr;
      }
      l_run = l_run * a_ + lsum;
      m_run = m_new;
      *reinterpret_cast<v4i*>(&sm.pt[ti & 1][hq][8 * g4]) = __builtin_bit_cast(v4i, pv);
      if (g4 == 0) sm.alpha[ti & 1][wave * 16 + (lane_fresh() & 15)] = a_;
    }
  };
  // O^T += C^T P^T of tile ti for this wave's value slice, from the bf16 tile at st
  // the rescale of O by the factors of tile ti (only when some head's
  // reference maximum moved)
  auto pv_rescale = [&](int ti) {
    float al[NW];
    bool any = false;
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      al[nt] = sm.alpha[ti & 1][16 * nt + n16];
      any |= (al[nt] != 1.f);
    }
    if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
      for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int nt = 0; nt < NW; ++nt) o[vt][nt] *= al[nt];
    }
  };
  auto pv = [&](int ti, const unsigned char* st) {
    // ---- PV: O^T[v, head] = alpha * O^T + C^T[v, row] P^T[row, head], v in this wave's slice
    // (the rescale by alpha is pv_rescale, run before)
    {
      // transpose-read base: row 8*g4 + n16/4, column 16*(wave*VT) + 4*(n16%4); v tile vt adds 32 bytes
      const int lf = lane_fresh();
      const unsigned char* tb = st + 16 * val_unit(8 * (lf >> 4) + ((lf & 15) >> 2), wave * VT * 2) + 8 * (lf & 3);
      v8bf av[VT];
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(tb + 32 * vt));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(tb + 16 * 16 * A_STRIDE + 32 * vt));  // row + 4: slot + 16
        av[vt] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      // P^T of head tile nt+1 is read while the MFMAs of tile nt issue
      v4i pbr[2];
      pbr[0] = *reinterpret_cast<const v4i*>(&sm.pt[ti & 1][n16][8 * g4]);
#pragma unroll
      for (int nt = 0; nt < NW; ++nt) {
        if (nt + 1 < NW) pbr[(nt + 1) & 1] = *reinterpret_cast<const v4i*>(&sm.pt[ti & 1][16 * (nt + 1) + n16][8 * g4]);
        const v4i pb = pbr[nt & 1];
#pragma unroll
        for (int vt = 0; vt < VT; ++vt)
          o[vt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[vt], __builtin_bit_cast(v8bf, pb), o[vt][nt], 0, 0, 0);
      }
#pragma unroll
      for (int nt = 0; nt < NW; ++nt) {
        if (nt == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2 * VT + 1, 0);
        if (nt + 1 < NW) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, VT, 0);
      }
    }
  };

  if constexpr (!KV8) {
    // Software pipelined, one barrier per tile: iteration ti runs the PV of
    // tile ti-1 and the logits and softmax of tile ti (P^T and the rescale
    // factors are double-buffered).  The three gather stages hold tiles ti-1
    // (PV), ti (logits) and ti+1 (in flight), so gathers run one tile ahead.
    // The two waves of a SIMD run the phases of an iteration in opposite
    // orders (PV first, or logits first), so one's MFMAs overlap the other's
    // softmax and gather issue; each order is its own loop (one loop with
    // both orders inside spills).
    if (wave < (NW + 1) / 2) {
    int stg = 0;  // stage of tile ti
    for (int ti = 0; ti <= ntiles; ++ti) {
      const int stg_prev = stg == 0 ? STAGES - 1 : stg - 1;
      const int stg_next = stg == STAGES - 1 ? 0 : stg + 1;
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // tile ti, the only one in flight, has landed
      lds_barrier_keep_dma();  // and every wave has left iteration ti-1 (stage (ti+1)%3 is free)
      if (ti > 0) {
        pv_rescale(ti - 1);
        pv(ti - 1, sm.stage[stg_prev]);
      }
      // the next tile's gather, issued after the PV (it lands during the
      // logits and the next PV)
      if (ti + 1 < ntiles) issue_tile_bf16(stg_next, ti + 1);
      if (ti < ntiles) logits_softmax(ti, sm.stage[stg]);
      stg = stg_next;
    }
    } else {
    int stg = 0;  // stage of tile ti
    for (int ti = 0; ti <= ntiles; ++ti) {
      const int stg_prev = stg == 0 ? STAGES - 1 : stg - 1;
      const int stg_next = stg == STAGES - 1 ? 0 : stg + 1;
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // tile ti, the only one in flight, has landed
      lds_barrier_keep_dma();  // and every wave has left iteration ti-1 (stage (ti+1)%3 is free)
      if (ti + 1 < ntiles) issue_tile_bf16(stg_next, ti + 1);
      if (ti < ntiles) logits_softmax(ti, sm.stage[stg]);
      if (ti > 0) {
        pv_rescale(ti - 1);
        pv(ti - 1, sm.stage[stg_prev]);
      }
      stg = stg_next;
    }
    }
  } else {
    // FP8 rows, pipelined like the bf16 loop with one more barrier: once tile
    // ti has landed, all waves dequantize it into bf16 tile ti&1; after the
    // second barrier iteration ti runs the PV of tile ti-1 (from the other
    // bf16 tile) and the logits and softmax of tile ti.  Two FP8 gather
    // stages: tile ti+1 is in flight while tile ti is dequantized.
    auto dequant = [&](int ti) {
      const unsigned char* src = sm.stage[ti % NSTAGE];
      unsigned char* dst = sm.tile[ti & 1];
      // keep the per-thread offsets out of the registers that live across the
      // tile loop: the thread index is made opaque here, so they are recomputed
      int tid_o = tid;
      asm volatile("" : "+v"(tid_o));
#pragma unroll 1
      for (int i = tid_o; i < TILE_ROWS * 32; i += NT) {  // 32 units of 16 codes per row
        const int r = i >> 5, k = i & 31;
        const unsigned char* rowp = src + 16 * KV8_ROW_UNITS * r;
        const v4i c16 = *reinterpret_cast<const v4i*>(rowp + 16 * k);
        const float sc = *reinterpret_cast<const float*>(rowp + KV8_SCALE_OFF + 4 * (k >> 3));
        v4i lo, hi;
        dequant16(c16, sc, lo, hi);
        unsigned char* d = dst + 16 * val_unit(r, 2 * k);
        *reinterpret_cast<v4i*>(d) = lo;
        *reinterpret_cast<v4i*>(d + 16) = hi;
      }
#pragma unroll 1
      for (int i = tid_o; i < TILE_ROWS * 8; i += NT) {  // rope: 8 units per row, copied
        const int r = i >> 3, j = i & 7;
        *reinterpret_cast<v4i*>(dst + 16 * rope_unit(r, j)) =
            *reinterpret_cast<const v4i*>(src + 16 * KV8_ROW_UNITS * r + KV8_ROPE_OFF + 16 * j);
      }
    };
    for (int ti = 0; ti <= ntiles; ++ti) {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // tile ti, the only one in flight, has landed
      lds_barrier_keep_dma();  // every wave has left iteration ti-1: bf16 tile ti&1 and stage (ti+1)%2 are free
      if (ti + 1 < ntiles) issue_tile_fp8(ti + 1);
      if (ti < ntiles) dequant(ti);
      lds_barrier_keep_dma();  // bf16 tile ti is complete
      if (ti > 0) {
        pv_rescale(ti - 1);
        pv(ti - 1, sm.tile[(ti - 1) & 1]);
      }
      if (ti < ntiles) logits_softmax(ti, sm.tile[ti & 1]);
    }
  }

  // ---- epilogue: per-head (m, l) from the logits role, then normalise/store
  {
    const float l_tot = sum_lane_groups(l_run);
    if (g4 == 0) {
      sm.mfin[hq] = m_run;
      sm.lfin[hq] = l_tot;
    }
  }
  lds_barrier();
  if (p.S == 1 && p.residual) {
    // y = attn + residual (stored as bf16), then RMSNorm over the token with the
    // stored values; this workgroup holds all H x 512 values of token t
    float ssl = 0.f;
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      const int h = 16 * nt + n16;
      const float l_tot = sm.lfin[h];
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const int64_t rbase = ((int64_t)t * H + h) * VDIM;
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        const int v = (wave * VT + vt) * 16 + 4 * g4;
        const uint2 rr = *reinterpret_cast<const uint2*>(p.residual + rbase + v);
        const float res[4] = {__uint_as_float(rr.x << 16), __uint_as_float(rr.x & 0xffff0000u),
                              __uint_as_float(rr.y << 16), __uint_as_float(rr.y & 0xffff0000u)};
        __bf16 b4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b4[i] = (__bf16)(o[vt][nt][i] * inv + res[i]);
          const float yb = (float)b4[i];
          o[vt][nt][i] = yb;
          ssl += yb * yb;
        }
        *reinterpret_cast<uint2*>(p.res_out + rbase + v) = __builtin_bit_cast(uint2, b4);
      }
    }
    ssl = wave_sum_f32(ssl);
    if (lane == 0) sm.red[wave] = ssl;
    lds_barrier();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += sm.red[w];
    const float r = 1.f / sqrtf(tot / (float)(H * VDIM) + p.eps);
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      const int h = 16 * nt + n16;
      uint16_t* orow = p.out + ((int64_t)t * H + h) * VDIM;
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        const int v = (wave * VT + vt) * 16 + 4 * g4;
        const uint2 gg = *reinterpret_cast<const uint2*>(p.gamma + h * VDIM + v);
        const float gm[4] = {__uint_as_float(gg.x << 16), __uint_as_float(gg.x & 0xffff0000u),
                             __uint_as_float(gg.y << 16), __uint_as_float(gg.y & 0xffff0000u)};
        __bf16 b4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) b4[i] = (__bf16)(o[vt][nt][i] * r * gm[i]);
        *reinterpret_cast<uint2*>(orow + v) = __builtin_bit_cast(uint2, b4);
      }
    }
    return;
  }
  // O / l as bf16 rows [head][512] in LDS, over the gather ring and P^T (every
  // wave is past its last read of them: the barrier above), then written out
  // one 1 KB row per wave instruction (16 bytes per lane, whole lines), where
  // the accumulator layout would give each store 32-byte pieces of 16 rows.
  // The stores stream (nontemporal): the rows are read once, by the combine
  // or the caller, and do not stay in the L2 as dirty lines that the next
  // kernels (the next layer step's indexer) would have to write back.
  using SmT = MlaSmem<NW, KV8>;
  static_assert(__builtin_offsetof(SmT, mfin) >= (size_t)H * OB_STRIDE, "O rows fit below mfin");
  // (a split's partial is O itself, unnormalised: the combine weighs it by
  // exp2(m - M) and divides by the weighted sum of the l)
#pragma unroll
  for (int nt = 0; nt < NW; ++nt) {
    const int h = 16 * nt + n16;
    const float l_tot = sm.lfin[h];
    const float inv = p.S > 1 ? 1.f : (l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f);
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      __bf16 b4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b4[i] = (__bf16)(o[vt][nt][i] * inv);
      *reinterpret_cast<uint2*>(smem_raw + h * OB_STRIDE + 2 * ((wave * VT + vt) * 16 + 4 * g4)) =
          __builtin_bit_cast(uint2, b4);
    }
  }
  lds_barrier();
  {
    uint16_t* dst = p.S == 1 ? p.out + (int64_t)t * H * VDIM : p.part_o + ((int64_t)t * p.S + s) * H * VDIM;
    for (int h = wave; h < H; h += NW)
      __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(smem_raw + h * OB_STRIDE + 16 * lane),
                                  reinterpret_cast<v4i*>(dst + (int64_t)h * VDIM + 8 * lane));
  }
  if (p.S > 1 && tid < H) {
    const int64_t rowi = ((int64_t)t * p.S + s) * H + tid;
    p.part_ml[rowi * 2 + 0] = sm.mfin[tid];
    p.part_ml[rowi * 2 + 1] = sm.lfin[tid];
  }
}

// Merge S partial results per (query, head), each split's unnormalised O_s
// with its (m_s, l_s): out = sum_s e^(m_s-M) O_s / sum_s e^(m_s-M) l_s.
// A workgroup covers 4 (query, head) rows (one wave each, 8 values per lane);
// H is a multiple of 4.  SM >= S: the splits loaded per row (4 when S <= 4,
// so no load repeats a split).
template <int SM>
__global__ __launch_bounds__(256) void dsa_mla_combine_kernel(MlaParams p) {
  const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // t * H + h
  const int t = (int)(th / p.H), h = (int)(th % p.H);
  const int v = (threadIdx.x & 63) * 8;
  // every split's (m, l) and partial row in one round of loads (splits past S
  // repeat the last one and get weight 0), then the weights.  Partial rows are
  // read once and the output rows written once: both stream (nontemporal).
  float ms[SM], ls[SM];
  uint4 raw[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    const int64_t rowi = ((int64_t)t * p.S + min(s, p.S - 1)) * p.H + h;
    ms[s] = p.part_ml[rowi * 2];
    ls[s] = p.part_ml[rowi * 2 + 1];
    raw[s] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p.part_o + rowi * VDIM + v)));
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < SM; ++s) M = s < p.S ? fmaxf(M, ms[s]) : M;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < SM; ++s) {
      const float wgt = (s < p.S && ms[s] != -INFINITY) ? exp2f(ms[s] - M) : 0.f;
      L += wgt * ls[s];
      const uint32_t rw[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};  // 8 bf16
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += wgt * __uint_as_float(rw[j] << 16);
        acc[2 * j + 1] += wgt * __uint_as_float(rw[j] & 0xffff0000u);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  __bf16 b8[8];
  if (!p.residual) {
#pragma unroll
    for (int i = 0; i < 8; ++i) b8[i] = (__bf16)(acc[i] * inv);
    uint2* o2 = reinterpret_cast<uint2*>(p.out + th * VDIM + v);  // the output is 8-byte aligned
    const uint4 u = __builtin_bit_cast(uint4, b8);
    __builtin_nontemporal_store(v2i{(int)u.x, (int)u.y}, reinterpret_cast<v2i*>(o2));
    __builtin_nontemporal_store(v2i{(int)u.z, (int)u.w}, reinterpret_cast<v2i*>(o2 + 1));
    return;
  }
  // residual epilogue: store y = attn + residual (bf16) and this head's sum of
  // squares of the stored values; the norm itself needs every head of the token
  const uint2* r2 = reinterpret_cast<const uint2*>(p.residual + th * VDIM + v);  // 8-byte aligned
  const uint2 ra = r2[0], rb = r2[1];
  const uint32_t rw[4] = {ra.x, ra.y, rb.x, rb.y};
  float ssl = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    b8[2 * j] = (__bf16)(acc[2 * j] * inv + __uint_as_float(rw[j] << 16));
    b8[2 * j + 1] = (__bf16)(acc[2 * j + 1] * inv + __uint_as_float(rw[j] & 0xffff0000u));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float yb = (float)b8[i];
    ssl += yb * yb;
  }
  *reinterpret_cast<uint4*>(p.res_out + th * VDIM + v) = __builtin_bit_cast(uint4, b8);
  ssl = wave_sum_f32(ssl);
  if ((threadIdx.x & 63) == 0) p.ssq[th] = ssl;
}

// RMSNorm of the stored residual stream: a workgroup covers 4 (query, head)
// rows of one query (H is a multiple of 4), 8 values per thread;
// out = y / sqrt(mean over the token's H x 512 values of y^2 + eps) * gamma
__global__ __launch_bounds__(256) void dsa_mla_norm_kernel(MlaParams p) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // t * H + h
  const int t = (int)(row / p.H), h = (int)(row % p.H);
  const int v = (threadIdx.x & 63) * 8;
  float part = 0.f;
  for (int i = threadIdx.x & 63; i < p.H; i += 64) part += p.ssq[(int64_t)t * p.H + i];
  const float tot = wave_sum_f32(part);
  const float r = 1.f / sqrtf(tot / (float)(p.H * VDIM) + p.eps);
  const uint4 yy = *reinterpret_cast<const uint4*>(p.res_out + row * VDIM + v);
  const uint4 gg = *reinterpret_cast<const uint4*>(p.gamma + h * VDIM + v);
  const uint32_t yw[4] = {yy.x, yy.y, yy.z, yy.w}, gw[4] = {gg.x, gg.y, gg.z, gg.w};
  __bf16 b8[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    b8[2 * j] = (__bf16)(__uint_as_float(yw[j] << 16) * r * __uint_as_float(gw[j] << 16));
    b8[2 * j + 1] = (__bf16)(__uint_as_float(yw[j] & 0xffff0000u) * r * __uint_as_float(gw[j] & 0xffff0000u));
  }
  *reinterpret_cast<uint4*>(p.out + row * VDIM + v) = __builtin_bit_cast(uint4, b8);
}

template <int NW, bool KV8>
static size_t mla_smem_t(int rows_per_split) {
  const int tiles = (rows_per_split + TILE_ROWS - 1) / TILE_ROWS;
  return sizeof(MlaSmem<NW, KV8>) + (size_t)(tiles * TILE_ROWS + 4) * 4;  // + the spare entry
}


template <int NW, bool KV8>
static hipError_t launch_mla_t(const MlaParams& p, hipStream_t st) {
  auto kfn = dsa_mla_split_kernel<NW, KV8>;
  const size_t smem = mla_smem_t<NW, KV8>(p.rows_per_split);
  hipError_t e = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(p.S, p.T), dim3(NW * 64), smem, st, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  if (p.S <= 4)
    hipLaunchKernelGGL(dsa_mla_combine_kernel<4>, dim3(p.T * p.H / 4), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(dsa_mla_combine_kernel<MLA_SMAX>, dim3(p.T * p.H / 4), dim3(256), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess || !p.residual) return e;
  hipLaunchKernelGGL(dsa_mla_norm_kernel, dim3(p.T * p.H / 4), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <bool KV8>
static hipError_t launch_mla_kv(const MlaParams& p, hipStream_t st) {
  switch (p.H) {
    case 16: return launch_mla_t<1, KV8>(p, st);
    case 32: return launch_mla_t<2, KV8>(p, st);
    case 64: return launch_mla_t<4, KV8>(p, st);
    default: return launch_mla_t<8, KV8>(p, st);
  }
}

hipError_t launch_mla(const MlaParams& p, hipStream_t st) {
  return p.kv8 ? launch_mla_kv<true>(p, st) : launch_mla_kv<false>(p, st);
}

}  // namespace dsa
