// Prefill-class attention on the gfx950 matrix cores: the kernel (its body
// is in attn_mfma_body.hpp) and its launchers.
#include <hip/hip_ext.h>

#include "attn_mfma_body.hpp"

namespace kvattn {

template <int D, int G, bool SWA, int RB>
__global__ __launch_bounds__(256 / RB, 2 / RB) void k_attn_mfma(AttnArgs a) {
  mfma_body<D, G, SWA, RB>(a, a.items, blockIdx.x, blockIdx.y);
}

template <int D, int G, bool SWA>
static void mfma_launch_swa(const AttnArgs& a, int n_il, hipStream_t s, const KernelEvents& ev) {
  constexpr int RB = kMfmaRowBlocks;
  const dim3 grid(a.n_items * a.n_head_kv, n_il), block(256 / RB);
  if (ev.any())
    hipExtLaunchKernelGGL((k_attn_mfma<D, G, SWA, RB>), grid, block, 0, s, ev.start, ev.stop, 0, a);
  else
    hipLaunchKernelGGL((k_attn_mfma<D, G, SWA, RB>), grid, block, 0, s, a);
}

template <int D, int G>
static void mfma_launch(const AttnArgs& a, int n_il, hipStream_t s, const KernelEvents& ev) {
  if (a.swa > 0)
    mfma_launch_swa<D, G, true>(a, n_il, s, ev);
  else
    mfma_launch_swa<D, G, false>(a, n_il, s, ev);
}

template <int D>
static hipError_t mfma_by_group(const AttnArgs& a, int n_il, int G, hipStream_t s, const KernelEvents& ev) {
  switch (G) {
    case 1: mfma_launch<D, 1>(a, n_il, s, ev); break;
    case 2: mfma_launch<D, 2>(a, n_il, s, ev); break;
    case 4: mfma_launch<D, 4>(a, n_il, s, ev); break;
    case 8: mfma_launch<D, 8>(a, n_il, s, ev); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_mfma(const AttnArgs& a, int n_il, int D, int G, hipStream_t s, const KernelEvents& ev) {
  if (a.n_items == 0 || n_il == 0) return hipSuccess;
  switch (D) {
    case 16: return mfma_by_group<16>(a, n_il, G, s, ev);
    case 32: return mfma_by_group<32>(a, n_il, G, s, ev);
    case 64: return mfma_by_group<64>(a, n_il, G, s, ev);
    case 128: return mfma_by_group<128>(a, n_il, G, s, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvattn
