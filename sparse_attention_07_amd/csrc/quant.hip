// Index-query quantization: bf16 rows -> OCP e4m3fn codes + scales, the step
// that prepares the fused indexer's query ("Inference Acceleration for a New
// Domestic LLM Architecture", section 3; "Optimizing Inference for
// Hybrid-Architecture LLMs", sections 3.2 and 4.2).
//
// HBM-bound streaming: 2 B read and 1 B (+ scale bytes) written per element.
// Each lane owns 16 contiguous bytes of input (8 bf16).  A row of D elements
// spans L = D/8 consecutive lanes of one wave (64 % L == 0, and a wave's first
// chunk index is a multiple of 64), so the row's amax is a DPP butterfly over L
// lanes and a 32-element group's amax one over 4 lanes.  Each lane keeps U
// independent 16-byte loads in flight before it computes (U = 2 for large
// inputs, 1 when that would leave the chip under-filled).  Loads and code
// stores are non-temporal: every byte is touched once, so caching them only
// evicts data the neighbouring kernels reuse (measured: 21 -> 18 us on a
// 4096-token chunk's query, 67 MB in, 34 MB out).
//
// x / s must be the correctly rounded fp32 quotient (the codes are decided on
// it).  Instead of eight IEEE divisions per lane, each lane forms r = 1/s once
// (correctly rounded) and refines q = x * r with two FMA residual steps: the
// first makes q faithful, the second is Markstein's correction, which turns a
// faithful quotient into the correctly rounded one given r = RN(1/s) and an
// exact residual.  The residual is exact unless it underflows, so rows with
// s < 2^-90 (amax below about 2^-81) take the plain division.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace dsa {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int QZ_NT = 256;  // threads per workgroup
constexpr int QZ_U = 2;     // 16-byte chunks per thread at large sizes
constexpr float E4M3_MAX = 448.0f;

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

// max of non-negative floats over aligned groups of W lanes (W = 4..64), as
// unsigned bit patterns (same order for non-negative floats)
template <int W>
__device__ __forceinline__ float group_max(float f) {
  uint32_t v = __float_as_uint(f);
  v = max(v, dpp<0xB1>(v));                 // quad_perm [1,0,3,2]: lane ^ 1
  v = max(v, dpp<0x4E>(v));                 // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (W >= 8) v = max(v, dpp<0x141>(v));   // row_half_mirror: the other quad of 8
  if constexpr (W >= 16) v = max(v, dpp<0x140>(v));  // row_mirror: the other half of 16
  if constexpr (W >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  if constexpr (W >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return __uint_as_float(v);
}

// correctly rounded x / s from r = RN(1/s) (see the header); sign kept for zeros
__device__ __forceinline__ float div_rn(float x, float s, float r) {
  float q = x * r;
  float e = fmaf(-q, s, x);
  q = fmaf(e, r, q);
  e = fmaf(-q, s, x);
  q = fmaf(e, r, q);
  return copysignf(q, x);
}

__device__ __forceinline__ float clamp448(float y) { return fminf(fmaxf(y, -E4M3_MAX), E4M3_MAX); }

// four values already within +-448 -> four e4m3fn codes (round to nearest even)
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// DT 1: one fp32 scale per row; DT 2: one E8M0 byte per 32 elements.  L = D/8;
// U chunks per thread.
template <int DT, int L, int U>
__global__ __launch_bounds__(QZ_NT) void quantize_q_kernel(const u32x4* __restrict__ q, int64_t chunks,
                                                           u32x2* __restrict__ codes, void* __restrict__ scales) {
  const int64_t base = (int64_t)blockIdx.x * (QZ_NT * U) + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = base + (int64_t)u * QZ_NT;
    v[u] = c < chunks ? __builtin_nontemporal_load(q + c) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = base + (int64_t)u * QZ_NT;
    float x[8] = {bf_lo(v[u].x), bf_hi(v[u].x), bf_lo(v[u].y), bf_hi(v[u].y),
                  bf_lo(v[u].z), bf_hi(v[u].z), bf_lo(v[u].w), bf_hi(v[u].w)};
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
    // chunks past the end are zero and belong to rows past the end, so the
    // butterflies never mix them into a valid row; every lane takes part
    float y[8];
    if constexpr (DT == 1) {
      am = group_max<L>(am);
      float s = am / E4M3_MAX;  // correctly rounded fp32 division
      if (s == 0.f) s = 1.f;
      if (s >= 0x1p-90f) {
        const float r = 1.0f / s;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = clamp448(div_rn(x[i], s, r));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = clamp448(x[i] / s);
      }
      if (c < chunks && (c % L) == 0) ((float*)scales)[c / L] = s;
    } else {
      am = group_max<4>(am);
      // e = floor(log2 am) - 8 from the exponent field, clamped below at -127
      // (a subnormal am lands there too); e = 0 for an all-zero group
      const int ef = (int)(__float_as_uint(am) >> 23);
      const int e = am == 0.f ? 0 : max(ef - 135, -127);
      const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-127, 120]
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = clamp448(x[i] * inv);  // exact: power-of-two factor
      if (c < chunks && (c & 3) == 0) ((uint8_t*)scales)[c >> 2] = (uint8_t)(e + 127);
    }
    if (c < chunks)
      __builtin_nontemporal_store(u32x2{pack4(y[0], y[1], y[2], y[3]), pack4(y[4], y[5], y[6], y[7])}, codes + c);
  }
}

template <int DT, int U>
hipError_t launch_u(const void* q, int64_t chunks, int L, void* codes, void* scales, hipStream_t st) {
  const int64_t grid = (chunks + QZ_NT * U - 1) / (QZ_NT * U);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(QZ_NT), 0, st, (const u32x4*)q, chunks, (u32x2*)codes,
                       scales);
    return hipGetLastError();
  };
  switch (L) {
    case 4: return go(quantize_q_kernel<DT, 4, U>);
    case 8: return go(quantize_q_kernel<DT, 8, U>);
    case 16: return go(quantize_q_kernel<DT, 16, U>);
    case 32: return go(quantize_q_kernel<DT, 32, U>);
    case 64: return go(quantize_q_kernel<DT, 64, U>);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_dt(const void* q, int64_t rows, int D, void* codes, void* scales, hipStream_t st) {
  const int L = D / 8;
  const int64_t chunks = rows * L;
  // two loads in flight per lane once that still gives >= 1024 workgroups
  if (chunks >= (int64_t)1024 * QZ_NT * QZ_U) return launch_u<DT, QZ_U>(q, chunks, L, codes, scales, st);
  return launch_u<DT, 1>(q, chunks, L, codes, scales, st);
}

}  // namespace

// D must be 32, 64, 128, 256 or 512 here (checked by the caller); rows >= 1.
hipError_t launch_quantize_q(const void* q, int64_t rows, int D, int idx_dtype, void* codes, void* scales,
                             hipStream_t st) {
  return idx_dtype == 1 ? launch_dt<1>(q, rows, D, codes, scales, st) : launch_dt<2>(q, rows, D, codes, scales, st);
}

}  // namespace dsa
