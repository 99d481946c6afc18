// Machine ceilings, measured with the instruction forms the attention
// kernels use: a gather of whole 2 KiB cache rows through an index list (the
// decode kernel's access) and back-to-back F16 matrix-core products (the
// prefill kernel's instruction).  Benchmarks report them beside the
// published peaks; nothing on the attention path calls them.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.hpp"
#include "kvattn.h"

namespace kvattn {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kRowHalves = 1024;     // one 2 KiB row: 64 lanes x 16 F16

// Wavefront w of W reads rows index[w], index[w + W], ...: U rows in flight,
// each one 2 KiB wavefront access (lane l: 32 B at 32 l).  Each thread adds
// up the numbers it read (fp32), so no load is dead.
template <int U>
__global__ __launch_bounds__(kProbeThreads) void k_probe_gather(const _Float16* __restrict__ rows, int64_t n_rows,
                                                                const int32_t* __restrict__ index, int64_t n_index,
                                                                float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x) >> 6;
  const int64_t nw = (static_cast<int64_t>(gridDim.x) * kProbeThreads) >> 6;
  float acc = 0.f;
  for (int64_t i = wave; i < n_index; i += nw * U) {
    half8 v[U][2];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = i + u * nw;
      ok[u] = k < n_index;
      int64_t r = ok[u] ? index[k] : 0;
      r = r < 0 ? 0 : (r >= n_rows ? n_rows - 1 : r);
      const half8* p = reinterpret_cast<const half8*>(rows + r * kRowHalves) + lane * 2;
      v[u][0] = p[0];
      v[u][1] = p[1];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += static_cast<float>(v[u][0][e]) + static_cast<float>(v[u][1][e]);
      acc += ok[u] ? s : 0.f;
    }
  }
  out[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = acc;
}

// Four independent accumulators per wavefront, so no product waits for the
// one before it; the operands come from memory so nothing is folded.
__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma(const _Float16* __restrict__ ab, float* __restrict__ out,
                                                              int iters) {
  half8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = ab[e];
    b[e] = ab[8 + e];
  }
  floatx16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace kvattn

extern "C" int kvattn_probe_gather(const void* rows, int64_t n_rows, const int32_t* index, int64_t n_index, float* out,
                                   int32_t n_wg, void* hip_stream) {
  if (!rows || n_rows <= 0 || (n_index > 0 && !index) || n_index < 0 || !out || n_wg <= 0) return KVATTN_EINVAL;
  hipLaunchKernelGGL(kvattn::k_probe_gather<4>, dim3(n_wg), dim3(kvattn::kProbeThreads), 0,
                     static_cast<hipStream_t>(hip_stream), static_cast<const _Float16*>(rows), n_rows, index, n_index,
                     out);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_EHIP;
}

extern "C" int kvattn_probe_mfma(const void* ab, float* out, int32_t n_wg, int32_t iters, void* hip_stream) {
  if (!ab || !out || n_wg <= 0 || iters < 0) return KVATTN_EINVAL;
  hipLaunchKernelGGL(kvattn::k_probe_mfma, dim3(n_wg), dim3(kvattn::kProbeThreads), 0,
                     static_cast<hipStream_t>(hip_stream), static_cast<const _Float16*>(ab), out, iters);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_EHIP;
}
