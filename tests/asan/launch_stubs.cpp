// Host-only stand-ins for the kernel launchers of the DSA library, linked
// instead of the kernels when the C ABI layer (api.hip) is built with host
// sanitizers: they record the parameter blocks the ABI layer built, so the
// driver can check every workspace address against the workspace it passed.
#include <hip/hip_runtime.h>

#include "../../sparse_attention_07_amd/csrc/dsa_params.h"

namespace dsa {
IdxParams g_idx;
MlaParams g_mla;
int g_idx_calls = 0, g_mla_calls = 0, g_quant_calls = 0, g_idx_grid = 0;

hipError_t launch_indexer(const IdxParams& p, int, int, int grid, hipStream_t) {
  g_idx = p;
  g_idx_grid = grid;
  ++g_idx_calls;
  return hipSuccess;
}
hipError_t launch_mla(const MlaParams& p, hipStream_t) {
  g_mla = p;
  ++g_mla_calls;
  return hipSuccess;
}
hipError_t launch_quantize_q(const void*, int64_t, int, int, void*, void*, hipStream_t) {
  ++g_quant_calls;
  return hipSuccess;
}
void* g_clear_ptr = nullptr;
size_t g_clear_bytes = 0;
hipError_t launch_clear_counters(void* ws, size_t bytes, hipStream_t) {
  g_clear_ptr = ws;
  g_clear_bytes = bytes;
  return hipSuccess;
}
}  // namespace dsa
