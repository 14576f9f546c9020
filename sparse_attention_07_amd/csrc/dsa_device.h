// Device-side helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int PAGE = 64;
constexpr int LATENT = 576;
constexpr int VDIM = 512;
constexpr int KMAX = 2048;
// Keys scored per streaming round of the indexer (one candidate count and
// barrier per round): 512 for one query per group, 1024 for two.  Measured
// (same box): 512 against 1024 keys, mixed_1m 0.1920 against 0.1943 ms per
// layer step and the 128K decode batch 0.2370 against 0.2375, but the
// paired-query prefill indexer 4 % slower; 2048 slower everywhere.  512 is
// the least the four-group prefetch ring allows.
constexpr int round_keys(int mq) { return mq == 1 ? 512 : 1024; }
constexpr int MIN_SLICE = 4096;       // smallest key slice an indexer workgroup is given
constexpr int MERGE_FAN = 8;          // candidate lists one merge workgroup takes at once
// Fixed cost of one indexer segment (a group's keys inside one workgroup's
// slice: query setup, final selection, output), in keys streamed at full
// bandwidth.  Each group is charged this many extra keys of weight in the
// key-space partition, so slices that hold more segments get fewer keys.
// (Measured: 2560, 3584, 4608 and 5632 gave 208, 205, 202 and 203 us for the
// 128K-token decode batch; 4608 is also the best or near it for the others.)
constexpr int SEG_COST = 4608;
// The concatenated key space of the stream-K partition is counted in 64-key
// pages (every group's range is padded to whole pages), so offsets of calls
// with billions of keys in total still fit 32 bits; the host bounds the total.
constexpr int MIN_SLICE_PG = MIN_SLICE / PAGE;
constexpr int SEG_COST_PG = SEG_COST / PAGE;
static_assert(MIN_SLICE % PAGE == 0 && SEG_COST % PAGE == 0, "page-unit key space");
constexpr int SUB = 65536;            // keys whose page ids the indexer stages in LDS at once

// Order-preserving map fp32 -> uint32 (a < b  <=>  key(a) < key(b)); -0 maps
// like +0.  Key 0 is below every finite value and marks "no candidate".
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key for keys of finite values (key 0 is no value).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Sum over the four lanes l, l^16, l^32, l^48 (the four k-groups of a 16x16
// MFMA tile); every one of the four lanes receives the same value.
__device__ __forceinline__ float sum_lane_groups(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  float s = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Four such sums at once: x[r] holds one 16-wide column set in each of the
// four lane groups; afterwards lane group r holds the column sums of x[r]
// (column = lane & 15).  x0 and x2 are folded across the two halves of the
// wave, x1 and x3 likewise, then the two results across odd and even rows:
// three swaps and three adds instead of eight of each.
__device__ __forceinline__ float sum_lane_groups4(float x0, float x1, float x2, float x3) {
  // permlane32_swap(a, b) -> {[a lanes 0-31, b lanes 0-31], [a lanes 32-63, b lanes 32-63]}
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x2), false, false);
  const float u = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // rows: x0 (r0+r2, r1+r3), x2 (r0+r2, r1+r3)
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x1), __float_as_uint(x3), false, false);
  const float v = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // rows: x1 (..), x1 (..), x3 (..), x3 (..)
  // permlane16_swap(a, b) -> {[a r0, b r0, a r2, b r2], [a r1, b r1, a r3, b r3]}
  auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);  // rows: x0, x1, x2, x3
}

// Sum over all 64 lanes of a wave, returned to every lane (epilogue use only).
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v += __shfl_xor(v, m);
  return sum_lane_groups(v);
}

__device__ __forceinline__ float max_lane_groups(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  float s = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Workgroup barrier that orders LDS only.  __syncthreads() also drains every
// outstanding global load (vmcnt(0)), which would empty the prefetch queues.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier for code that also has direct-to-LDS loads in flight: waits for this
// wave's LDS instructions only (an LDS-scoped fence would also wait for every
// outstanding direct-to-LDS load).  Callers wait for the loads they need with
// an explicit vmcnt before calling it.
__device__ __forceinline__ void lds_barrier_keep_dma() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16-byte global -> LDS copy per lane: lane i writes LDS[lds_base + 16 i].
// Issued as asm so the compiler does not add its own (drain-everything) wait
// before later LDS reads; callers wait with an explicit vmcnt.  The load has no
// output register (it writes LDS).  m0 is reserved to the compiler, so the asm
// saves it in a scratch SGPR and restores it after the load has been issued.
__device__ __forceinline__ void dma16_to_lds(const void* gaddr, uint32_t lds_base) {
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "v"(gaddr), "s"(lds_base)
      : "memory");
}

// The same copy from a wave-uniform base address (SGPR pair) plus a 32-bit
// per-lane byte offset: the address arithmetic of a whole wave-load stays
// scalar.
__device__ __forceinline__ void dma16_to_lds_saddr(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}

// Device-coherent (agent-scope) loads and stores for data that one workgroup
// hands to another inside a launch.  They bypass the per-XCD cache levels a
// plain access may find stale, so no device-scope fence (a writeback and an
// invalidation of the whole L2 of the XCD) is needed: the writer waits for its
// stores to complete before it moves the arrival counter, and the reader
// issues its loads after it has read the counter.
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's global loads and stores have completed.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// Cross-lane steps through DPP (a VALU operand modifier): unlike __shfl_*,
// which go through LDS (ds_bpermute plus a wait each), these cost a few cycles.
// Controls: row_shr:n = 0x110 + n within 16-lane rows; row_bcast:15 / :31
// feed lane 15 / 31 of a row into the next row(s) selected by row_mask.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t identity, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_u32<0x111, 0xf>(0u, v);
  v += dpp_u32<0x112, 0xf>(0u, v);
  v += dpp_u32<0x114, 0xf>(0u, v);
  v += dpp_u32<0x118, 0xf>(0u, v);
  v += dpp_u32<0x142, 0xa>(0u, v);
  v += dpp_u32<0x143, 0xc>(0u, v);
  return v;
}

// Inclusive prefix maximum (signed) over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_max(int v) {
  const uint32_t id = 0x80000000u;
  v = max(v, (int)dpp_u32<0x111, 0xf>(id, (uint32_t)v));
  v = max(v, (int)dpp_u32<0x112, 0xf>(id, (uint32_t)v));
  v = max(v, (int)dpp_u32<0x114, 0xf>(id, (uint32_t)v));
  v = max(v, (int)dpp_u32<0x118, 0xf>(id, (uint32_t)v));
  v = max(v, (int)dpp_u32<0x142, 0xa>(id, (uint32_t)v));
  v = max(v, (int)dpp_u32<0x143, 0xc>(id, (uint32_t)v));
  return v;
}

// Wave-wide minimum / maximum (unsigned), returned to every lane (uniform).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0x111, 0xf>(0xffffffffu, v));
  v = min(v, dpp_u32<0x112, 0xf>(0xffffffffu, v));
  v = min(v, dpp_u32<0x114, 0xf>(0xffffffffu, v));
  v = min(v, dpp_u32<0x118, 0xf>(0xffffffffu, v));
  v = min(v, dpp_u32<0x142, 0xa>(0xffffffffu, v));
  v = min(v, dpp_u32<0x143, 0xc>(0xffffffffu, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111, 0xf>(0u, v));
  v = max(v, dpp_u32<0x112, 0xf>(0u, v));
  v = max(v, dpp_u32<0x114, 0xf>(0u, v));
  v = max(v, dpp_u32<0x118, 0xf>(0u, v));
  v = max(v, dpp_u32<0x142, 0xa>(0u, v));
  v = max(v, dpp_u32<0x143, 0xc>(0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

}  // namespace dsa
