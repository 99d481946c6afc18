// Decode-class attention on the vector ALUs (gfx950): the kernel body, a
// device function, so that the combined launch of attn_both.hip can run it
// beside the matrix-core body.
//
// One workgroup = one (query, chunk of a class's cell list); its 4
// wavefronts take interleaved groups of U cells.  A cell row of one layer is
// E = n_head_kv * head_dim F16.  A wavefront reads 1024 numbers of a row per
// load: lane l holds 16 consecutive numbers (two 16 B loads) -- KV head
// l / LPH of the slice, dims 16 * (l % LPH) .. +16 -- so each access is one
// fully coalesced 2 KiB wavefront access wherever the cell sits in the
// cache.  Rows of 2048 or 4096 numbers are cut into 1024-number slices, each
// owned by 4 / slices wavefronts that split the cells between them; a
// 512-number row fills half a wavefront, so each wavefront takes two cells
// per load (one per lane half) and merges the halves' states at the end.  Scores are reduced over the LPH lanes
// of a head with DPP lane moves; the softmax runs online in base 2 with the
// scale folded into q (fp32 throughout; the F16 rows are widened inside
// v_fma_mix).  Each wavefront keeps the K/V rows of its next group of cells
// and the list entries of the group after that in flight while it computes
// the current group, and the running maximum moves (rescaling O) only when
// it grows by more than 2^8.
#pragma once

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

// The kernel body for work item items[bid / n_il], layer slot bid % n_il of
// the launch (item-major, layer-minor: the items are sorted longest first,
// so the shortest (item, layer) pairs of a launch are dispatched last).  red
// holds NSLOT wavefront states for the cross-wavefront merge: with at least
// one per wavefront beyond the first of each slice the merge takes one
// round, with one it takes a round per such wavefront (less LDS, for the
// combined launch beside the matrix-core body).
template <int D, int G, int E, int NSLOT>
KVATTN_DEV void valu_body(const AttnArgs& a, const WorkItem* items, int bid, int n_il, float (*red)[64][G * 18]) {
  constexpr int LPH = D / 16;          // lanes per KV head
  constexpr int HK = E / D;            // KV heads per row
  constexpr int H = HK * G;
  constexpr int U = 4;                 // cells in flight per lane per wavefront step
  constexpr int SL = E >= 1024 ? E / 1024 : 1;    // 1024-number slices of a row
  constexpr int CPW = E >= 1024 ? 1 : 1024 / E;   // cells per wavefront load (lane halves)
  constexpr int WPS = 4 / SL;          // wavefronts per slice
  constexpr int LPR = E / 16 / SL;     // lanes per (slice of a) row
  static_assert(LPH == 4 || LPH == 8, "head_dim 64 or 128");
  static_assert(E == 512 || E == 1024 || E == 2048 || E == 4096, "row of 512 .. 4096 numbers");
  static_assert(CPW * LPR == 64 && SL * WPS == 4, "lane and wavefront mapping");
  static_assert(NSLOT >= 1, "at least one merge slot");
  const WorkItem it = items[bid / n_il];
  const int il = bid % n_il;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int slice = w / WPS, wi = w % WPS;      // wave-uniform
  const int half = lane / LPR;                  // lane half (two cells per load), else 0
  const int rl = lane % LPR;
  const int kvh = slice * (LPR / LPH) + rl / LPH, part = rl % LPH;
  const SlotInfo si = a.qslots[it.q_off];
  const bool check_mask = !it.pure;
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
  constexpr int WSTEP = CPW * U;       // cells one wavefront covers per step
  constexpr int STEP = WPS * WSTEP;    // cells the wavefronts of a slice cover per step

  // Software pipeline over this wavefront's steps (U cells each): while
  // step s computes, the K/V rows of step s+1 and the list entries (cell,
  // position, and the word of its sequence set that holds the row's
  // sequence) of step s+2 are in flight.  Two register sets
  // A/B alternate; visibility is decided when a step's rows are issued, so
  // its list entries are dead by then.
  int lc[U], lp[U];
  uint64_t lm[U];
  auto fetch_list = [&](int c) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = min(c + half * U + u, last);
      lc[u] = a.csr_cell[idx];
      lp[u] = a.csr_pos[idx];
      lm[u] = check_mask ? a.csr_mask[idx].w[si.seq0 >> 6] : ~0ULL;
    }
  };
  auto issue = [&](int c, half8 (&kr)[U][2], half8 (&vr)[U][2], bool (&vis)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = (sbase + lc[u]) * E + kvh * D + part * 16;
      const half8* kp = reinterpret_cast<const half8*>(Kl + off);
      const half8* vp = reinterpret_cast<const half8*>(Vl + off);
      kr[u][0] = kp[0]; kr[u][1] = kp[1];
      vr[u][0] = vp[0]; vr[u][1] = vp[1];
      vis[u] = c + half * U + u < it.c1 && (!a.causal || lp[u] <= si.pos) && ((lm[u] >> (si.seq0 & 63)) & 1ULL) &&
               (a.swa == 0 || si.pos - lp[u] < a.swa);
    }
  };
  auto compute = [&](const half8 (&kr)[U][2], const half8 (&vr)[U][2], const bool (&vis)[U]) {
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
  };

  half8 kA[U][2], vA[U][2], kB[U][2], vB[U][2];
  bool visA[U], visB[U];
  const int c_first = it.c0 + wi * WSTEP;   // wave-uniform, as is every step bound below
  if (c_first < it.c1) {
    fetch_list(c_first);
    issue(c_first, kA, vA, visA);
    fetch_list(c_first + STEP);
    for (int c = c_first;; c += 2 * STEP) {
      const bool more1 = c + STEP < it.c1;
      if (more1) {
        issue(c + STEP, kB, vB, visB);
        fetch_list(c + 2 * STEP);
      }
      compute(kA, vA, visA);
      if (!more1) break;
      const bool more2 = c + 2 * STEP < it.c1;
      if (more2) {
        issue(c + 2 * STEP, kA, vA, visA);
        fetch_list(c + 3 * STEP);
      }
      compute(kB, vB, visB);
      if (!more2) break;
    }
  }

  // two cells per load: merge the lane halves' states (both halves end up
  // holding the merged state)
  if constexpr (CPW == 2) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], 32, 64), lo = __shfl_xor(l[g], 32, 64);
      const float M = fmaxf(m[g], mo);
      const float s0 = (M == -INFINITY || m[g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[g] - M);
      const float s1 = (M == -INFINITY || mo == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mo - M);
      l[g] = l[g] * s0 + lo * s1;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[g][e] = acc[g][e] * s0 + __shfl_xor(acc[g][e], 32, 64) * s1;
      m[g] = M;
    }
  }
  // merge the states of each slice's wavefronts into its first one
  constexpr int NS = WPS - 1;          // states per slice beyond the first
  constexpr bool ONE_ROUND = NSLOT >= SL * NS;
  static_assert(ONE_ROUND || NSLOT >= SL, "one merge slot per slice at least");
  // the merged row of query head kvh * G + g: output, or split-K partial
  auto emit = [&](int g, float M, float L, const float (&o)[16]) {
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
  };
  if constexpr (ONE_ROUND) {
    if (wi > 0) {
      const int k0 = slice * NS + wi - 1;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        red[k0][lane][g * 18] = m[g];
        red[k0][lane][g * 18 + 1] = l[g];
#pragma unroll
        for (int e = 0; e < 16; ++e) red[k0][lane][g * 18 + 2 + e] = acc[g][e];
      }
    }
    if constexpr (NS > 0) __syncthreads();
    if (wi != 0) return;
    if (half != 0) return;               // the other lane half holds the same state
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float M = m[g];
#pragma unroll
      for (int k = 0; k < NS; ++k) M = fmaxf(M, red[slice * NS + k][lane][g * 18]);
      const float s0 = (M == -INFINITY || m[g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[g] - M);
      float L = l[g] * s0;
      float o[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) o[e] = acc[g][e] * s0;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const float mk = red[slice * NS + k][lane][g * 18];
        const float sk = (M == -INFINITY || mk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - M);
        L = __builtin_fmaf(red[slice * NS + k][lane][g * 18 + 1], sk, L);
#pragma unroll
        for (int e = 0; e < 16; ++e) o[e] = __builtin_fmaf(red[slice * NS + k][lane][g * 18 + 2 + e], sk, o[e]);
      }
      emit(g, M, L, o);
    }
  } else {
    // One slot per slice: the same arithmetic in the same order, in rounds
    // (the fused multiply-adds are explicit in both forms, so that operand
    // contraction cannot differ between them).
    // First every wavefront's running maxima (NS * G numbers per lane), from
    // which the slice's first wavefront takes the merged maximum; then a
    // round per wavefront for its sum and accumulators.
    if (wi > 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) red[slice][lane][(wi - 1) * G + g] = m[g];
    }
    __syncthreads();
    float mk[NS > 0 ? NS : 1][G], M[G], L[G], o[G][16];
    if (wi == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        M[g] = m[g];
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          mk[k][g] = red[slice][lane][k * G + g];
          M[g] = fmaxf(M[g], mk[k][g]);
        }
        const float s0 = (M[g] == -INFINITY || m[g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[g] - M[g]);
        L[g] = l[g] * s0;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[g][e] = acc[g][e] * s0;
      }
    }
    __syncthreads();
    for (int k = 0; k < NS; ++k) {
      if (wi == k + 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          red[slice][lane][g * 18 + 1] = l[g];
#pragma unroll
          for (int e = 0; e < 16; ++e) red[slice][lane][g * 18 + 2 + e] = acc[g][e];
        }
      }
      __syncthreads();
      if (wi == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float sk = (M[g] == -INFINITY || mk[k][g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk[k][g] - M[g]);
          L[g] = __builtin_fmaf(red[slice][lane][g * 18 + 1], sk, L[g]);
#pragma unroll
          for (int e = 0; e < 16; ++e) o[g][e] = __builtin_fmaf(red[slice][lane][g * 18 + 2 + e], sk, o[g][e]);
        }
      }
      __syncthreads();
    }
    if (wi != 0) return;
    if (half != 0) return;
#pragma unroll
    for (int g = 0; g < G; ++g) emit(g, M[g], L[g], o[g]);
  }
}

}  // namespace kvattn
