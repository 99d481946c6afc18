// Decode-class attention on the vector ALUs (gfx950), plus the split-K merge.
//
// One workgroup = one (query, chunk of a class's cell list); its 4
// wavefronts take interleaved groups of U cells.  A cell row of one layer is
// n_head_kv * head_dim = 1024 F16 (2 KiB): lane l holds 16 consecutive
// numbers of it (two 16 B loads) -- KV head l / LPH, dims 16 * (l % LPH) ..
// +16 -- so each K or V row is one fully coalesced 2 KiB wavefront access
// wherever the cell sits in the cache.  Scores are reduced over the LPH lanes
// of a head with DPP lane moves; the softmax runs online in base 2 with the
// scale folded into q (fp32 throughout; the F16 rows are widened inside
// v_fma_mix).  The cell indices, positions and sequence sets of the next
// group of cells are fetched while the current group computes, and the
// running maximum moves (rescaling O) only when it grows by more than 2^8.
#include "device_common.hpp"
#include "launch.hpp"

namespace kvattn {

namespace {

constexpr float kSlack = 8.f;      // log2 units the running max may lag

template <int CTRL>
KVATTN_DEV float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPH lanes (LPH = 4 or 8): two quad permutes
// (xor 1, xor 2) and, for 8, the half-row mirror (lane i <-> 7 - i).
template <int LPH>
KVATTN_DEV float group_sum(float s) {
  s += dpp<0xB1>(s);                  // quad_perm [1,0,3,2]
  s += dpp<0x4E>(s);                  // quad_perm [2,3,0,1]
  if (LPH == 8) s += dpp<0x141>(s);   // row_half_mirror
  return s;
}

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(256) void k_attn_valu(AttnArgs a) {
  constexpr int LPH = D / 16;          // lanes per KV head
  constexpr int HK = 64 / LPH;         // KV heads per row (row = 1024 numbers)
  constexpr int E = HK * D;
  constexpr int H = HK * G;
  constexpr int U = 4;                 // cells in flight per wavefront step
  static_assert(LPH == 4 || LPH == 8, "head_dim 64 or 128");
  __shared__ float red[3][64][G * 18];

  const WorkItem it = a.items[blockIdx.x];
  const int il = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int kvh = lane / LPH, part = lane % LPH;
  const int qslot = a.qlist[it.q_off];
  const SlotInfo si = a.slots[qslot];
  const bool check_mask = !a.classes[it.cls].pure;
  const _Float16* __restrict__ Kl = a.k[il];
  const _Float16* __restrict__ Vl = a.v[il];

  float q[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* qp = a.q[il] + static_cast<int64_t>(si.q_row) * H * D + (kvh * G + g) * D + part * 16;
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(qp + e);
      q[g][e] = x.x * a.scale_log2e; q[g][e + 1] = x.y * a.scale_log2e;
      q[g][e + 2] = x.z * a.scale_log2e; q[g][e + 3] = x.w * a.scale_log2e;
    }
  }
  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[g][e] = 0.f;
  }
  const int64_t sbase = static_cast<int64_t>(si.stream) * a.kv_size;
  const int last = it.c1 - 1;

  // list entries of the first step
  int ncell[U], npos[U];
  uint64_t nmask[U];
  const int c_first = it.c0 + w * U;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int idx = min(c_first + u, last);
    ncell[u] = a.csr_cell[idx];
    npos[u] = a.csr_pos[idx];
    nmask[u] = check_mask ? a.csr_mask[idx] : ~0ULL;
  }

  for (int c = c_first; c < it.c1; c += 4 * U) {
    half8 kr[U][2], vr[U][2];
    bool vis[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = (sbase + ncell[u]) * E + kvh * D + part * 16;
      const half8* kp = reinterpret_cast<const half8*>(Kl + off);
      const half8* vp = reinterpret_cast<const half8*>(Vl + off);
      kr[u][0] = kp[0]; kr[u][1] = kp[1];
      vr[u][0] = vp[0]; vr[u][1] = vp[1];
      vis[u] = c + u < it.c1 && (!a.causal || npos[u] <= si.pos) && ((nmask[u] >> si.seq0) & 1ULL);
    }
    // list entries of the next step fly while this one computes
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = min(c + 4 * U + u, last);
      ncell[u] = a.csr_cell[idx];
      npos[u] = a.csr_pos[idx];
      nmask[u] = check_mask ? a.csr_mask[idx] : ~0ULL;
    }
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += q[g][e] * static_cast<float>(kr[u][0][e]);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += q[g][8 + e] * static_cast<float>(kr[u][1][e]);
        s = group_sum<LPH>(s);
        sc[u][g] = vis[u] ? s : -INFINITY;
      }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][g]);
      const bool grow = mx > m[g] + kSlack;
      if (ballot(grow)) {
        const float m_new = grow ? mx : m[g];
        const float alpha = m[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[g] - m_new);
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[g][e] *= alpha;
        m[g] = m_new;
      }
      const float m_use = m[g] == -INFINITY ? 0.f : m[g];
      float p[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = __builtin_amdgcn_exp2f(sc[u][g] - m_use);
        l[g] += p[u];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = acc[g][e];
#pragma unroll
        for (int u = 0; u < U; ++u) v += p[u] * static_cast<float>(vr[u][e >> 3][e & 7]);
        acc[g][e] = v;
      }
    }
  }

  // merge the four wavefronts' states
  if (w > 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      red[w - 1][lane][g * 18] = m[g];
      red[w - 1][lane][g * 18 + 1] = l[g];
#pragma unroll
      for (int e = 0; e < 16; ++e) red[w - 1][lane][g * 18 + 2 + e] = acc[g][e];
    }
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = m[g];
#pragma unroll
    for (int k = 0; k < 3; ++k) M = fmaxf(M, red[k][lane][g * 18]);
    const float s0 = (M == -INFINITY || m[g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[g] - M);
    float L = l[g] * s0;
    float o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = acc[g][e] * s0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const float mk = red[k][lane][g * 18];
      const float sk = (M == -INFINITY || mk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - M);
      L += red[k][lane][g * 18 + 1] * sk;
#pragma unroll
      for (int e = 0; e < 16; ++e) o[e] += red[k][lane][g * 18 + 2 + e] * sk;
    }
    const int h = kvh * G + g;
    if (it.prow < 0) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float* op = a.o[il] + static_cast<int64_t>(si.out_row) * H * D + h * D + part * 16;
#pragma unroll
      for (int e = 0; e < 16; e += 4)
        *reinterpret_cast<float4*>(op + e) = make_float4(o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv);
    } else {
      const int64_t row = static_cast<int64_t>(il) * a.rows_per_layer + it.prow;
      float* pp = a.part_acc + row * H * D + h * D + part * 16;
#pragma unroll
      for (int e = 0; e < 16; e += 4) *reinterpret_cast<float4*>(pp + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
      if (part == 0) {
        a.part_ml[(row * H + h) * 2] = M;
        a.part_ml[(row * H + h) * 2 + 1] = L;
      }
    }
  }
}

template <int D, int G>
static void valu_launch(const AttnArgs& a, int n_il, hipStream_t s) {
  hipLaunchKernelGGL((k_attn_valu<D, G>), dim3(a.n_items, n_il), dim3(256), 0, s, a);
}

hipError_t launch_attn_valu(const AttnArgs& a, int n_il, int D, int G, hipStream_t s) {
  if (a.n_items == 0 || n_il == 0) return hipSuccess;
  if (D == 128 && G == 1) valu_launch<128, 1>(a, n_il, s);
  else if (D == 128 && G == 2) valu_launch<128, 2>(a, n_il, s);
  else if (D == 128 && G == 4) valu_launch<128, 4>(a, n_il, s);
  else if (D == 64 && G == 1) valu_launch<64, 1>(a, n_il, s);
  else if (D == 64 && G == 2) valu_launch<64, 2>(a, n_il, s);
  else if (D == 64 && G == 4) valu_launch<64, 4>(a, n_il, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// split-K merge, one pass: the running (M, L, O) absorbs record k as
// M' = max(M, m_k), O' = 2^(M-M') O + 2^(m_k-M') acc_k, L' likewise.
__global__ __launch_bounds__(256) void k_attn_reduce(AttnArgs a, int D) {
  const int rr = blockIdx.x, il = blockIdx.y;
  const int H = a.n_head;
  const SlotInfo si = a.slots[a.red_slot[rr]];
  const int b = a.red_off[rr], e = a.red_off[rr + 1];
  const int64_t lbase = static_cast<int64_t>(il) * a.rows_per_layer;
  for (int x = threadIdx.x * 4; x < H * D; x += blockDim.x * 4) {
    const int h = x / D;
    float M = -INFINITY, L = 0.f;
    float4 o = make_float4(0, 0, 0, 0);
    for (int k = b; k < e; ++k) {
      const int64_t row = lbase + a.red_rows[k];
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (row * H + h) * 2);
      const float4 v = *reinterpret_cast<const float4*>(a.part_acc + row * H * D + x);
      if (ml.x == -INFINITY) continue;
      const float Mn = fmaxf(M, ml.x);
      const float so = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      const float sk = __builtin_amdgcn_exp2f(ml.x - Mn);
      L = L * so + ml.y * sk;
      o.x = o.x * so + v.x * sk; o.y = o.y * so + v.y * sk;
      o.z = o.z * so + v.z * sk; o.w = o.w * so + v.w * sk;
      M = Mn;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *reinterpret_cast<float4*>(a.o[il] + static_cast<int64_t>(si.out_row) * H * D + x) =
        make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

hipError_t launch_reduce(const AttnArgs& a, int n_reduced, int n_il, int D, hipStream_t s) {
  if (n_reduced == 0 || n_il == 0) return hipSuccess;
  hipLaunchKernelGGL(k_attn_reduce, dim3(n_reduced, n_il), dim3(256), 0, s, a, D);
  return hipGetLastError();
}

}  // namespace kvattn
