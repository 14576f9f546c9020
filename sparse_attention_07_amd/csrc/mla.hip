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
//    (global_load_lds_dwordx4) into a 3-stage ring; rows sit at a padded
//    stride of 74 sixteen-byte units in a permuted slot order that makes the
//    operand reads of both phases free of bank conflicts (see row_slot), and
//    operand addresses stay base + immediate;
//  * H/16 waves.  Logits: wave w owns heads 16w..16w+15, keeps their q in
//    registers as the MFMA B operand and computes S^T = C q^T (bf16 16x16x32;
//    rows on M in an order that makes the probabilities come out as 8
//    consecutive rows per lane), runs the online softmax (exp2 domain) and
//    writes P^T (bf16) and the per-head rescale factor to LDS.
//    PV: wave w owns value dims [512w/NW, 512(w+1)/NW) for all heads and
//    accumulates O^T += C^T P^T, reading C^T with the gfx950 LDS transpose
//    read (ds_read_b64_tr_b16) and P^T with plain 16-byte reads;
//  * the O rescale is skipped for a wave when no head's running max moved;
//  * with several splits, each split stores its normalised partial output
//    O/l as fp16 (|O/l| is bounded by the largest value entry) plus (m, l) in
//    fp32, and a small kernel merges them with log-sum-exp weights;
//  * optional residual + RMSNorm epilogue over the token's H x 512 values: with
//    one split the workgroup holds the whole token and finishes it; with
//    several, the combine adds the residual and stores per-head sums of
//    squares, and a small kernel applies the norm;
//  * FP8 latent rows (656 B: e4m3fn nope, one fp32 scale per 128 dims, bf16
//    rope) are gathered the same way into their own 3-stage ring (41 units per
//    row instead of 72), then all waves dequantize the tile once into the bf16
//    tile layout above (code * scale rounded to bf16), so the MFMA phases are
//    the bf16 ones.  That saves 43 % of the gathered bytes and of the cache's
//    footprint, but adds LDS traffic and a barrier per tile to a kernel whose
//    logits phase is bound by LDS reads, so it runs slightly slower than bf16.
#include "dsa_device.h"
#include "dsa_params.h"

namespace dsa {

constexpr int TILE_ROWS = 32;
constexpr int MLA_SMAX = 8;  // most splits of a query's index list (K / 256 for K <= 2048)
constexpr int ROW_UNITS = LATENT * 2 / 16;                         // 72 sixteen-byte units per row
constexpr int ROW_STRIDE = ROW_UNITS + 2;                          // padded row stride (units)
constexpr int TILE_LOADS = (TILE_ROWS * ROW_STRIDE + 63) / 64;     // 37 wave-loads of 64 units
constexpr int PT_STRIDE = TILE_ROWS + 16;                          // P^T row (bf16): 6 sixteen-byte units
constexpr int STAGES = 3;
constexpr int STAGE_BYTES = TILE_LOADS * 64 * 16;

// FP8 latent rows: 512 code bytes, 4 fp32 scales, 64 bf16 rope dims
constexpr int KV8_ROW_UNITS = 41;                                   // 656 B
constexpr int KV8_SCALE_OFF = 512;
constexpr int KV8_ROPE_OFF = 528;
constexpr int KV8_TILE_LOADS = (TILE_ROWS * KV8_ROW_UNITS + 63) / 64;  // 21 wave-loads of 64 units
constexpr int KV8_STAGE_BYTES = KV8_TILE_LOADS * 64 * 16;

// byte offset, inside a stage, of bf16 element (row r, column col)
// LDS layout of a tile (bank conflicts measured with the LDS counters on
// gfx950): a wave's 16-byte reads that put 16 lanes on 16 rows, the 4 lane
// groups one unit apart, are conflict-free when the rows lie 2 mod 4 units
// apart (74 here) and take 2-4 cycles more otherwise.  The logits A operand
// of M-tile mt reads tile rows 8*(n/4) + n%4 + 4*mt for lanes n = 0..15, so
// tile row r is stored in slot p(r) = 4*(r/8) + r%4 + 16*((r/4)%2): each
// M-tile reads 16 consecutive slots.  The PV transpose reads (rows 8*g + j
// and 8*g + 4 + j) then also fall on consecutive slots.
__device__ __forceinline__ int row_slot(int r) { return 4 * (r >> 3) + (r & 3) + 16 * ((r >> 2) & 1); }
__device__ __forceinline__ int slot_row(int p) { return 8 * ((p & 15) >> 2) + (p & 3) + 4 * (p >> 4); }
__device__ __forceinline__ int row_unit(int r) { return ROW_STRIDE * row_slot(r); }

// byte offset, inside a stage, of bf16 element (row r, column col)
__device__ __forceinline__ int stage_off(int r, int col) { return 16 * (row_unit(r) + (col >> 3)) + 2 * (col & 7); }

template <int NW, bool KV8>
struct MlaSmem {
  static constexpr int NSTAGE = KV8 ? 2 : STAGES;
  unsigned char stage[NSTAGE][KV8 ? KV8_STAGE_BYTES : STAGE_BYTES];  // gather ring
  unsigned char tile[KV8 ? 2 : 1][KV8 ? STAGE_BYTES : 16];          // FP8 only: two dequantized bf16 tiles
  uint16_t pt[2][16 * NW][PT_STRIDE];  // P^T as [head][row] bf16, two tiles (rows padded: no bank conflicts)
  float alpha[2][16 * NW];             // per-head rescale factor, two tiles
  float mfin[16 * NW];
  float lfin[16 * NW];
  float red[NW];  // per-wave partial sums (residual + RMSNorm epilogue)
  // followed by the slice's slots (int32)
};

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
  constexpr int LOADS = KV8 ? KV8_TILE_LOADS : TILE_LOADS;
  constexpr int RUNITS = KV8 ? KV8_ROW_UNITS : ROW_STRIDE;  // units per row in the gather ring
  constexpr int LMIN = LOADS / NW;                     // DMA loads of every wave per tile
  constexpr int LEXTRA = LOADS - LMIN * NW;            // waves [0, LEXTRA) issue one more
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
  // as the logits B operand (k = latent dim).  The first NT slots are loaded
  // before q, so the first tile's gather can start while q is in flight.
  auto slot_of = [&](int i) {
    int v = -1;
    if (i < nrows) {
      v = p.indices[(int64_t)t * p.K + r_begin + i];
      if (v < 0 || (int64_t)v >= p.num_slots) v = -1;
    }
    return v;
  };
  const int v0 = slot_of(tid);
  const int hq = wave * 16 + n16;
  v4i qb[18];
  {
    const uint16_t* qrow = p.q + ((int64_t)t * H + hq) * LATENT;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qb[ks] = *reinterpret_cast<const v4i*>(qrow + 32 * ks + 8 * g4);
  }
  if (tid < ntiles * TILE_ROWS) sidx[tid] = v0;
  for (int i = tid + NT; i < ntiles * TILE_ROWS; i += NT) sidx[i] = slot_of(i);
  lds_barrier();

  constexpr int NSTAGE = MlaSmem<NW, KV8>::NSTAGE;
  auto issue_tile = [&](int ti) {
    unsigned char* st = sm.stage[ti % NSTAGE];
    const int nl = LMIN + (wave < LEXTRA ? 1 : 0);
    const int first = wave * LMIN + min(wave, LEXTRA);
    for (int k = 0; k < nl; ++k) {
      const int u0 = (first + k) * 64;
      const int u = u0 + lane;
      int r = u / RUNITS;  // FP8: row; bf16: slot
      int c = u - r * RUNITS;
      if (r >= TILE_ROWS || c >= (KV8 ? KV8_ROW_UNITS : ROW_UNITS)) {  // padding slot: a harmless valid unit
        r = min(r, TILE_ROWS - 1);
        c = 0;
      }
      if constexpr (!KV8) r = slot_row(r);
      int slot = sidx[ti * TILE_ROWS + r];
      slot = slot < 0 ? 0 : slot;
      const uint16_t* g = KV8 ? p.kv + (int64_t)slot * (KV8_ROW_UNITS * 8) + 8 * c
                              : p.kv + (int64_t)slot * LATENT + 8 * c;
      const uint32_t lds_addr =
          (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(st + 16 * u0);
      dma16_to_lds(g, uniform(lds_addr));
    }
  };

  if (ntiles > 0) issue_tile(0);
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
    const unsigned char* la0 = st + 16 * (row_unit(8 * (n16 >> 2) + (n16 & 3)) + g4);  // slot n16
    const unsigned char* la1 = la0 + 16 * 16 * ROW_STRIDE;                              // slot 16 + n16
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const v4i a0 = *reinterpret_cast<const v4i*>(la0 + 64 * ks);
      const v4i a1 = *reinterpret_cast<const v4i*>(la1 + 64 * ks);
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a0), __builtin_bit_cast(v8bf, qb[ks]),
                                                       acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a1), __builtin_bit_cast(v8bf, qb[ks]),
                                                       acc[1], 0, 0, 0);
    }
    // ---- online softmax: this lane holds head hq, rows 8*g4 + 4*mt + i
    {
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
      const float m_new = fmaxf(m_run, tmax);
      const float a_ = (m_new > m_run) ? exp2f(m_run - m_new) : 1.f;
      float lsum = 0.f;
      __bf16 pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pr = (m_new == -INFINITY) ? 0.f : exp2f(x[j] - m_new);
        lsum += pr;
        pv[j] = (__bf16)pr;
      }
      l_run = l_run * a_ + lsum;
      m_run = m_new;
      *reinterpret_cast<v4i*>(&sm.pt[ti & 1][hq][8 * g4]) = __builtin_bit_cast(v4i, pv);
      if (g4 == 0) sm.alpha[ti & 1][hq] = a_;
    }
  };
  // O^T += C^T P^T of tile ti for this wave's value slice, from the bf16 tile at st
  auto pv = [&](int ti, const unsigned char* st) {
    // ---- PV: O^T[v, head] = alpha * O^T + C^T[v, row] P^T[row, head], v in this wave's slice
    {
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
      // transpose-read base: row 8*g4 + n16/4, column 16*(wave*VT) + 4*(n16%4); v tile vt adds 32 bytes
      const unsigned char* tb = st + stage_off(8 * g4 + (n16 >> 2), wave * VT * 16 + 4 * (n16 & 3));
      v8bf av[VT];
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(tb + 32 * vt));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(tb + 16 * 16 * ROW_STRIDE + 32 * vt));  // row + 4: slot + 16
        av[vt] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int nt = 0; nt < NW; ++nt) {
        const v4i pb = *reinterpret_cast<const v4i*>(&sm.pt[ti & 1][16 * nt + n16][8 * g4]);
#pragma unroll
        for (int vt = 0; vt < VT; ++vt)
          o[vt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[vt], __builtin_bit_cast(v8bf, pb), o[vt][nt], 0, 0, 0);
      }
    }
  };

  if constexpr (!KV8) {
    // Software pipelined, one barrier per tile: iteration ti runs the PV of
    // tile ti-1 and the logits and softmax of tile ti (P^T and the rescale
    // factors are double-buffered).  The three gather stages hold tiles ti-1
    // (PV), ti (logits) and ti+1 (in flight), so gathers run one tile ahead.
    for (int ti = 0; ti <= ntiles; ++ti) {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // tile ti, the only one in flight, has landed
      lds_barrier_keep_dma();  // and every wave has left iteration ti-1 (stage (ti+1)%3 is free)
      if (ti + 1 < ntiles) issue_tile(ti + 1);
      if (ti > 0) pv(ti - 1, sm.stage[(ti - 1) % STAGES]);
      if (ti < ntiles) logits_softmax(ti, sm.stage[ti % STAGES]);
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
        unsigned char* d = dst + 16 * (row_unit(r) + 2 * k);
        *reinterpret_cast<v4i*>(d) = lo;
        *reinterpret_cast<v4i*>(d + 16) = hi;
      }
#pragma unroll 1
      for (int i = tid_o; i < TILE_ROWS * 8; i += NT) {  // rope: 8 units per row, copied
        const int r = i >> 3, j = i & 7;
        *reinterpret_cast<v4i*>(dst + 16 * (row_unit(r) + 64 + j)) =
            *reinterpret_cast<const v4i*>(src + 16 * KV8_ROW_UNITS * r + KV8_ROPE_OFF + 16 * j);
      }
    };
    for (int ti = 0; ti <= ntiles; ++ti) {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // tile ti, the only one in flight, has landed
      lds_barrier_keep_dma();  // every wave has left iteration ti-1: bf16 tile ti&1 and stage (ti+1)%2 are free
      if (ti + 1 < ntiles) issue_tile(ti + 1);
      if (ti < ntiles) dequant(ti);
      lds_barrier_keep_dma();  // bf16 tile ti is complete
      if (ti > 0) pv(ti - 1, sm.tile[(ti - 1) & 1]);
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
#pragma unroll
  for (int nt = 0; nt < NW; ++nt) {
    const int h = 16 * nt + n16;
    const float l_tot = sm.lfin[h];
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (p.S == 1) {
      uint16_t* orow = p.out + ((int64_t)t * H + h) * VDIM;
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        __bf16 b4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) b4[i] = (__bf16)(o[vt][nt][i] * inv);
        *reinterpret_cast<uint2*>(orow + (wave * VT + vt) * 16 + 4 * g4) = __builtin_bit_cast(uint2, b4);
      }
    } else {
      const int64_t rowi = ((int64_t)t * p.S + s) * H + h;
      _Float16* prow = p.part_o + rowi * VDIM;
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        _Float16 h4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h4[i] = (_Float16)(o[vt][nt][i] * inv);
        *reinterpret_cast<uint2*>(prow + (wave * VT + vt) * 16 + 4 * g4) = __builtin_bit_cast(uint2, h4);
      }
    }
  }
  if (p.S > 1 && tid < H) {
    const int64_t rowi = ((int64_t)t * p.S + s) * H + tid;
    p.part_ml[rowi * 2 + 0] = sm.mfin[tid];
    p.part_ml[rowi * 2 + 1] = sm.lfin[tid];
  }
}

// Merge S partial results per (query, head), with O_s = l_s * (O/l)_s:
// out = sum_s e^(m_s-M) l_s (O/l)_s / sum_s e^(m_s-M) l_s.
// A workgroup covers 4 (query, head) rows (one wave each, 8 values per lane);
// H is a multiple of 4.  SM >= S: the splits loaded per row (4 when S <= 4,
// so no load repeats a split).
template <int SM>
__global__ __launch_bounds__(256) void dsa_mla_combine_kernel(MlaParams p) {
  const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // t * H + h
  const int t = (int)(th / p.H), h = (int)(th % p.H);
  const int v = (threadIdx.x & 63) * 8;
  // every split's (m, l) and partial row in one round of loads (splits past S
  // repeat the last one and get weight 0), then the weights
  float ms[SM], ls[SM];
  uint4 raw[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    const int64_t rowi = ((int64_t)t * p.S + min(s, p.S - 1)) * p.H + h;
    ms[s] = p.part_ml[rowi * 2];
    ls[s] = p.part_ml[rowi * 2 + 1];
    raw[s] = *reinterpret_cast<const uint4*>(p.part_o + rowi * VDIM + v);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < SM; ++s) M = s < p.S ? fmaxf(M, ms[s]) : M;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < SM; ++s) {
      const float wgt = (s < p.S && ms[s] != -INFINITY) ? exp2f(ms[s] - M) * ls[s] : 0.f;
      L += wgt;
      _Float16 h8[8];
      __builtin_memcpy(h8, &raw[s], 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += wgt * (float)h8[i];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  __bf16 b8[8];
  if (!p.residual) {
#pragma unroll
    for (int i = 0; i < 8; ++i) b8[i] = (__bf16)(acc[i] * inv);
    uint2* o2 = reinterpret_cast<uint2*>(p.out + th * VDIM + v);  // the output is 8-byte aligned
    const uint4 u = __builtin_bit_cast(uint4, b8);
    o2[0] = make_uint2(u.x, u.y);
    o2[1] = make_uint2(u.z, u.w);
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
  return sizeof(MlaSmem<NW, KV8>) + (size_t)tiles * TILE_ROWS * 4;
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
