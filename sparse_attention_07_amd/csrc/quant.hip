// Index-query quantization: bf16 rows -> OCP e4m3fn codes + scales, the step
// that prepares the fused indexer's query ("Inference Acceleration for a New
// Domestic LLM Architecture", section 3; "Optimizing Inference for
// Hybrid-Architecture LLMs", sections 3.2 and 4.2).
//
// HBM-bound streaming: 2 B read and 1 B (+ scale bytes) written per element.
// Each lane owns 16 contiguous bytes of input (8 bf16).  A row of D elements
// spans L = D/8 consecutive lanes of one wave (64 % L == 0, and a wave's first
// chunk index is a multiple of 64), so the row's amax is a butterfly over L
// lanes and a 32-element group's amax a butterfly over 4 lanes.  Each lane keeps
// QZ_U independent 16-byte loads in flight before it computes.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace dsa {
namespace {

constexpr int QZ_NT = 256;  // threads per workgroup
constexpr int QZ_U = 4;     // 16-byte chunks per thread
constexpr float E4M3_MAX = 448.0f;

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float clamp448(float y) { return fminf(fmaxf(y, -E4M3_MAX), E4M3_MAX); }

// four values already within +-448 -> four e4m3fn codes (round to nearest even)
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// DT 1: one fp32 scale per row; DT 2: one E8M0 byte per 32 elements.  L = D/8.
template <int DT, int L>
__global__ __launch_bounds__(QZ_NT) void quantize_q_kernel(const uint4* __restrict__ q, int64_t chunks,
                                                           uint2* __restrict__ codes, void* __restrict__ scales) {
  const int64_t base = (int64_t)blockIdx.x * (QZ_NT * QZ_U) + threadIdx.x;
  uint4 v[QZ_U];
#pragma unroll
  for (int u = 0; u < QZ_U; ++u) {
    const int64_t c = base + (int64_t)u * QZ_NT;
    v[u] = c < chunks ? q[c] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < QZ_U; ++u) {
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
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = clamp448(x[i] / s);
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
    if (c < chunks) codes[c] = make_uint2(pack4(y[0], y[1], y[2], y[3]), pack4(y[4], y[5], y[6], y[7]));
  }
}

template <int DT>
hipError_t launch_dt(const void* q, int64_t rows, int D, void* codes, void* scales, hipStream_t st) {
  const int L = D / 8;
  const int64_t chunks = rows * L;
  const int64_t grid = (chunks + QZ_NT * QZ_U - 1) / (QZ_NT * QZ_U);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(QZ_NT), 0, st, (const uint4*)q, chunks, (uint2*)codes,
                       scales);
    return hipGetLastError();
  };
  switch (L) {
    case 4: return go(quantize_q_kernel<DT, 4>);
    case 8: return go(quantize_q_kernel<DT, 8>);
    case 16: return go(quantize_q_kernel<DT, 16>);
    case 32: return go(quantize_q_kernel<DT, 32>);
    case 64: return go(quantize_q_kernel<DT, 64>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// D must be 32, 64, 128, 256 or 512 here (checked by the caller); rows >= 1.
hipError_t launch_quantize_q(const void* q, int64_t rows, int D, int idx_dtype, void* codes, void* scales,
                             hipStream_t st) {
  return idx_dtype == 1 ? launch_dt<1>(q, rows, D, codes, scales, st) : launch_dt<2>(q, rows, D, codes, scales, st);
}

}  // namespace dsa
