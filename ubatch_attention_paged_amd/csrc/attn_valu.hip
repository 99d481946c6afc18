// Decode-class attention on the vector ALUs (gfx950): the kernel (its body
// is in attn_valu_body.hpp) and its launchers, plus the split-K merge.
#include <algorithm>

#include <hip/hip_ext.h>

#include "attn_valu_body.hpp"

namespace kvattn {

template <int D, int G, int E>
__global__ __launch_bounds__(256) void k_attn_valu(AttnArgs a) {
  __shared__ float red[3][64][G * 18];
  valu_body<D, G, E, 3>(a, a.items, blockIdx.x, gridDim.x / a.n_items, red);
}

template <int D, int G, int E>
static void valu_launch(const AttnArgs& a, int n_il, hipStream_t s, const KernelEvents& ev) {
  if (ev.any())
    hipExtLaunchKernelGGL((k_attn_valu<D, G, E>), dim3(a.n_items * n_il), dim3(256), 0, s, ev.start, ev.stop, 0, a);
  else
    hipLaunchKernelGGL((k_attn_valu<D, G, E>), dim3(a.n_items * n_il), dim3(256), 0, s, a);
}

template <int D, int G>
static hipError_t valu_by_row(const AttnArgs& a, int n_il, int E, hipStream_t s, const KernelEvents& ev) {
  switch (E) {
    case 512: valu_launch<D, G, 512>(a, n_il, s, ev); break;
    case 1024: valu_launch<D, G, 1024>(a, n_il, s, ev); break;
    case 2048: valu_launch<D, G, 2048>(a, n_il, s, ev); break;
    case 4096: valu_launch<D, G, 4096>(a, n_il, s, ev); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_valu(const AttnArgs& a, int n_il, int D, int G, hipStream_t s, const KernelEvents& ev) {
  if (a.n_items == 0 || n_il == 0) return hipSuccess;
  const int E = a.n_head_kv * D;
  if (D == 128 && G == 1) return valu_by_row<128, 1>(a, n_il, E, s, ev);
  if (D == 128 && G == 2) return valu_by_row<128, 2>(a, n_il, E, s, ev);
  if (D == 128 && G == 4) return valu_by_row<128, 4>(a, n_il, E, s, ev);
  if (D == 64 && G == 1) return valu_by_row<64, 1>(a, n_il, E, s, ev);
  if (D == 64 && G == 2) return valu_by_row<64, 2>(a, n_il, E, s, ev);
  if (D == 64 && G == 4) return valu_by_row<64, 4>(a, n_il, E, s, ev);
  return hipErrorInvalidValue;
}

// split-K merge.  Record k of a query holds (m_k, l_k, acc_k) for each head;
// the merged row is sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k with
// M = max_k m_k.  Two passes over the records (the maximum, then the sums),
// each with independent loads, so a query's records are fetched in parallel
// rather than as a chain.  One thread per 4 consecutive output numbers.
__global__ __launch_bounds__(1024) void k_attn_reduce(AttnArgs a, int D) {
  const int rr = blockIdx.x, il = blockIdx.y;
  const int H = a.n_head;
  const SlotInfo si = a.slots[a.red_slot[rr]];
  const int b = a.red_off[rr], e = a.red_off[rr + 1];
  const int64_t lbase = static_cast<int64_t>(il) * a.rows_per_layer;
  for (int x = threadIdx.x * 4; x < H * D; x += blockDim.x * 4) {
    const int h = x / D;
    float M = -INFINITY;
#pragma unroll 4
    for (int k = b; k < e; ++k) M = fmaxf(M, a.part_ml[((lbase + a.red_rows[k]) * H + h) * 2]);
    float L = 0.f;
    float4 o = make_float4(0, 0, 0, 0);
    if (M != -INFINITY) {
#pragma unroll 4
      for (int k = b; k < e; ++k) {
        const int64_t row = lbase + a.red_rows[k];
        const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (row * H + h) * 2);
        const float4 v = *reinterpret_cast<const float4*>(a.part_acc + row * H * D + x);
        const float w = __builtin_amdgcn_exp2f(ml.x - M);     // 0 for an empty record (m = -inf)
        L += ml.y * w;
        o.x += v.x * w; o.y += v.y * w; o.z += v.z * w; o.w += v.w * w;
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *reinterpret_cast<float4*>(a.o[il] + static_cast<int64_t>(si.out_row) * H * D + x) =
        make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

hipError_t launch_reduce(const AttnArgs& a, int n_reduced, int n_il, int D, hipStream_t s, const KernelEvents& ev) {
  if (n_reduced == 0 || n_il == 0) return hipSuccess;
  const int quads = a.n_head * D / 4;
  const int threads = std::min(1024, (quads + 63) / 64 * 64);
  if (ev.any())
    hipExtLaunchKernelGGL(k_attn_reduce, dim3(n_reduced, n_il), dim3(threads), 0, s, ev.start, ev.stop, 0, a, D);
  else
    hipLaunchKernelGGL(k_attn_reduce, dim3(n_reduced, n_il), dim3(threads), 0, s, a, D);
  return hipGetLastError();
}

}  // namespace kvattn
