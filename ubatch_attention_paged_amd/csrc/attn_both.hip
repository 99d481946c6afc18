// Matrix-core and vector-ALU work items of one attend call in one launch.
//
// A decode step over a shared prefix plans both kinds: the prefix is one
// class read by all its queries on the matrix cores, each sequence's own
// cells are vector-ALU items.  Both halves are bandwidth-bound, and as two
// launches in order each pays its own ramp-up and drain; in one launch the
// vector-ALU workgroups fill the slots the matrix-core ones leave.  The
// first n_items * n_head_kv * n_il workgroups run the matrix-core body (in
// the order and on the XCDs the matrix-core kernel's own grid gives them),
// the rest the vector-ALU body over items2.  The workgroup holds the
// matrix-core body's LDS plus one vector-ALU merge slot per row slice (the
// merge then takes a round per wavefront), which must stay within half a
// CU's LDS so that two workgroups share a CU.
#include <hip/hip_ext.h>

#include "attn_mfma_body.hpp"
#include "attn_valu_body.hpp"

namespace kvattn {

namespace {

template <int D, int G, int E>
struct BothShape {
  static constexpr int SL = E >= 1024 ? E / 1024 : 1;            // row slices
  static constexpr int NS = 4 / SL - 1;                          // merged states per slice
  static constexpr int NSLOT = NS > 0 ? SL : 1;
  static constexpr int DP = D < 32 ? 32 : D;
  static constexpr int mfma_lds = 2 * kTileCells * (D + DP) * 2 + 2 * kTileCells * 4 + 2 * kSeqWords * kTileCells * 8;
  static constexpr int valu_lds = NSLOT * 64 * G * 18 * 4;
  static constexpr bool ok = mfma_lds + valu_lds <= 80 * 1024;
};

}  // namespace

template <int D, int G, int E>
__global__ __launch_bounds__(256, 2) void k_attn_both(AttnArgs a) {
  using S = BothShape<D, G, E>;
  const int row = a.n_items * a.n_head_kv;
  const int nm = row * a.n_il;
  const int b = blockIdx.x;
  if (b < nm) {
    mfma_body<D, G, false, 1>(a, a.items, b % row, b / row);
  } else {
    __shared__ float red[S::NSLOT][64][G * 18];
    valu_body<D, G, E, S::NSLOT>(a, a.items2, b - nm, a.n_il, red);
  }
}

namespace {

template <int D, int G, int E>
hipError_t both_launch(const AttnArgs& a0, int n_il, hipStream_t s, const KernelEvents& ev) {
  if constexpr (!BothShape<D, G, E>::ok) {
    return hipErrorInvalidValue;
  } else {
    AttnArgs a = a0;
    a.n_il = n_il;
    const dim3 grid((a.n_items * a.n_head_kv + a.n_items2) * n_il), block(256);
    if (ev.any())
      hipExtLaunchKernelGGL((k_attn_both<D, G, E>), grid, block, 0, s, ev.start, ev.stop, 0, a);
    else
      hipLaunchKernelGGL((k_attn_both<D, G, E>), grid, block, 0, s, a);
    return hipGetLastError();
  }
}

template <int D, int G>
hipError_t both_by_row(const AttnArgs& a, int n_il, int E, hipStream_t s, const KernelEvents& ev) {
  switch (E) {
    case 512: return both_launch<D, G, 512>(a, n_il, s, ev);
    case 1024: return both_launch<D, G, 1024>(a, n_il, s, ev);
    case 2048: return both_launch<D, G, 2048>(a, n_il, s, ev);
    case 4096: return both_launch<D, G, 4096>(a, n_il, s, ev);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int G>
bool both_ok_row(int E) {
  switch (E) {
    case 512: return BothShape<D, G, 512>::ok;
    case 1024: return BothShape<D, G, 1024>::ok;
    case 2048: return BothShape<D, G, 2048>::ok;
    case 4096: return BothShape<D, G, 4096>::ok;
    default: return false;
  }
}

}  // namespace

bool attn_both_supported(int D, int G, int E) {
  if (D == 128 && G == 1) return both_ok_row<128, 1>(E);
  if (D == 128 && G == 2) return both_ok_row<128, 2>(E);
  if (D == 128 && G == 4) return both_ok_row<128, 4>(E);
  if (D == 64 && G == 1) return both_ok_row<64, 1>(E);
  if (D == 64 && G == 2) return both_ok_row<64, 2>(E);
  if (D == 64 && G == 4) return both_ok_row<64, 4>(E);
  return false;
}

hipError_t launch_attn_both(const AttnArgs& a, int n_il, int D, int G, hipStream_t s, const KernelEvents& ev) {
  if (n_il == 0 || (a.n_items == 0 && a.n_items2 == 0)) return hipSuccess;
  const int E = a.n_head_kv * D;
  if (D == 128 && G == 1) return both_by_row<128, 1>(a, n_il, E, s, ev);
  if (D == 128 && G == 2) return both_by_row<128, 2>(a, n_il, E, s, ev);
  if (D == 128 && G == 4) return both_by_row<128, 4>(a, n_il, E, s, ev);
  if (D == 64 && G == 1) return both_by_row<64, 1>(a, n_il, E, s, ev);
  if (D == 64 && G == 2) return both_by_row<64, 2>(a, n_il, E, s, ev);
  if (D == 64 && G == 4) return both_by_row<64, 4>(a, n_il, E, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace kvattn
