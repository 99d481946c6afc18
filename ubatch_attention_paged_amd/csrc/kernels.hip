// gfx950 (MI355X, CDNA4) kernels for per-ubatch attention over a
// cell-granular F16 KV cache.  64-wide wavefronts throughout.
//
//   k_store          K/V rows of a ubatch -> F16 (nearest-even) into their cells
//   k_apply_updates  cell-table changes -> device mirror (pos, sequence set)
//   k_csr_*          per-class lists of visible cells, ascending cell index
//   k_mask_dense     dense F16 KQ mask (diagnostic form of the same predicate)
//   k_attn_valu      decode-class items: one query, all heads, a chunk of
//                    cells; 2 KiB cell rows streamed with 16 B loads per lane,
//                    fp32 math, online softmax, split-K partials
//   k_attn_mfma      prefill-class items: 128 query rows (queries x heads of
//                    one KV head) against 64-cell tiles staged in LDS;
//                    S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_f16
//   k_attn_reduce    log-sum-exp merge of split-K partials
//
// The visibility rule is the one of "llama.cpp and the ubatch", "The mask is
// doing the work": a cell is seen by a query when it is occupied, its
// sequence set holds the query's first sequence id and, under causal
// attention, its position is not later than the query's.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>

#include "launch.hpp"

namespace kvattn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

#define DEV __device__ __forceinline__

// ---------------------------------------------------------------------------
// helpers

DEV uint64_t ballot(bool p) { return __ballot(p); }
DEV int lane_id() { return threadIdx.x & 63; }
DEV uint64_t lanemask_lt() { return (1ULL << lane_id()) - 1ULL; }
DEV int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

DEV float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
DEV int wave_min_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
DEV int wave_max_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// ---------------------------------------------------------------------------
// K/V store: fp32 rows -> F16 rows of the cache.  Each thread converts 8
// consecutive values (two 16 B loads, one 16 B store).

__global__ __launch_bounds__(256) void k_store(StoreArgs a) {
  const int il = blockIdx.y;
  const int which = blockIdx.z;             // 0 = K, 1 = V
  const int vec_per_row = a.E >> 3;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= static_cast<int64_t>(a.n_rows) * vec_per_row) return;
  const int r = static_cast<int>(t / vec_per_row);
  const int c = static_cast<int>(t % vec_per_row);
  const float* src = (which ? a.v_cur[il] : a.k_cur[il]) + static_cast<int64_t>(r) * a.E + c * 8;
  _Float16* dst = (which ? a.v[il] : a.k[il]) + static_cast<int64_t>(a.dst_rows[r]) * a.E + c * 8;
  const float4 x0 = *reinterpret_cast<const float4*>(src);
  const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
  half8 h;
  h[0] = static_cast<_Float16>(x0.x); h[1] = static_cast<_Float16>(x0.y);
  h[2] = static_cast<_Float16>(x0.z); h[3] = static_cast<_Float16>(x0.w);
  h[4] = static_cast<_Float16>(x1.x); h[5] = static_cast<_Float16>(x1.y);
  h[6] = static_cast<_Float16>(x1.z); h[7] = static_cast<_Float16>(x1.w);
  *reinterpret_cast<half8*>(dst) = h;
}

hipError_t launch_store(const StoreArgs& a, int n_il, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(a.n_rows) * (a.E / 8);
  if (n == 0 || n_il == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((n + 255) / 256), n_il, 2);
  hipLaunchKernelGGL(k_store, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// commit: mirror updates, then the per-class cell lists

__global__ __launch_bounds__(256) void k_apply_updates(CsrArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.n_updates) return;
  const CellUpdate u = a.updates[i];
  a.cpos[u.idx] = u.pos;
  a.cmask[u.idx] = u.mask;
}

__global__ __launch_bounds__(256) void k_fill_zero(int32_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Class of each cell j < n_kv of stream blockIdx.y, by binary search of its
// sequence set among the ubatch's classes; per 64-cell segment counts.
__global__ __launch_bounds__(256) void k_csr_classify(CsrArgs a) {
  const int s = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  int cls = -1;
  if (j < a.n_kv) {
    const int64_t idx = static_cast<int64_t>(s) * a.kv_size + j;
    if (a.cpos[idx] >= 0) {
      const uint64_t m = a.cmask[idx];
      int lo = a.lookup_off[s], hi = a.lookup_off[s + 1] - 1;
      while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const uint64_t mm = a.lookup[mid].mask;
        if (mm == m) { cls = a.lookup[mid].cls; break; }
        if (mm < m) lo = mid + 1; else hi = mid - 1;
      }
    }
    a.cellcls[idx] = cls;
  }
  const int seg = j >> 6;
  uint64_t active = ballot(cls >= 0);
  while (active) {
    const int leader = __builtin_ctzll(active);
    const int c = readlane_i(cls, leader);
    const uint64_t same = ballot(cls == c);
    if (lane_id() == leader) a.counts[static_cast<int64_t>(c) * a.n_seg + seg] = __popcll(same);
    active &= ~same;
  }
}

// Per class: segment counts -> absolute start offsets in the csr arrays.
__global__ __launch_bounds__(64) void k_csr_scan(CsrArgs a) {
  const int c = blockIdx.x;
  const int lane = threadIdx.x;
  int32_t running = a.classes[c].cell_off;
  int32_t* row = a.counts + static_cast<int64_t>(c) * a.n_seg;
  for (int base = 0; base < a.n_seg; base += 64) {
    const int k = base + lane;
    const int v = k < a.n_seg ? row[k] : 0;
    int incl = v;
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (k < a.n_seg) row[k] = running + incl - v;
    running += __shfl(incl, 63);
  }
}

// Write every classified cell at its class offset + rank among the earlier
// cells of its class in the segment: ascending cell index within a class.
__global__ __launch_bounds__(256) void k_csr_scatter(CsrArgs a) {
  const int s = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int64_t idx = static_cast<int64_t>(s) * a.kv_size + j;
  const int cls = j < a.n_kv ? a.cellcls[idx] : -1;
  const int seg = j >> 6;
  uint64_t active = ballot(cls >= 0);
  while (active) {
    const int leader = __builtin_ctzll(active);
    const int c = readlane_i(cls, leader);
    const uint64_t same = ballot(cls == c);
    if (cls == c) {
      const int dst = a.counts[static_cast<int64_t>(c) * a.n_seg + seg] + __popcll(same & lanemask_lt());
      if (dst < a.csr_cap) {
        a.csr_cell[dst] = j;
        a.csr_pos[dst] = a.cpos[idx];
        a.csr_mask[dst] = a.cmask[idx];
      }
    }
    active &= ~same;
  }
}

hipError_t launch_commit(const CsrArgs& a, hipStream_t s) {
  if (a.n_updates > 0)
    hipLaunchKernelGGL(k_apply_updates, dim3((a.n_updates + 255) / 256), dim3(256), 0, s, a);
  if (a.n_classes == 0) return hipGetLastError();
  const int64_t nc = static_cast<int64_t>(a.n_classes) * a.n_seg;
  hipLaunchKernelGGL(k_fill_zero, dim3(static_cast<unsigned>((nc + 255) / 256)), dim3(256), 0, s, a.counts, nc);
  const dim3 grid((a.n_kv + 255) / 256, a.n_stream);
  hipLaunchKernelGGL(k_csr_classify, grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_csr_scan, dim3(a.n_classes), dim3(64), 0, s, a);
  hipLaunchKernelGGL(k_csr_scatter, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dense mask (diagnostic): 0x0000 visible, 0xFC00 (-inf) hidden

__global__ __launch_bounds__(256) void k_mask_dense(MaskArgs a) {
  const int i = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.n_kv) return;
  const SlotInfo q = a.slots[i];
  const int64_t idx = static_cast<int64_t>(q.stream) * a.kv_size + j;
  const int32_t p = a.cpos[idx];
  const bool vis = p >= 0 && ((a.cmask[idx] >> q.seq0) & 1ULL) && (!a.causal || p <= q.pos);
  a.mask[static_cast<int64_t>(i) * a.n_kv + j] = vis ? 0x0000 : 0xFC00;
}

hipError_t launch_mask(const MaskArgs& a, hipStream_t s) {
  if (a.n_rows == 0 || a.n_kv == 0) return hipSuccess;
  hipLaunchKernelGGL(k_mask_dense, dim3((a.n_kv + 255) / 256, a.n_rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode-class attention on the vector ALUs.
//
// One workgroup = one (query, chunk of a class's cell list); 4 wavefronts
// take interleaved groups of U cells.  A cell row of one layer is
// n_head_kv * head_dim = 1024 F16 (2 KiB): lane l holds 16 consecutive
// numbers of it (two 16 B loads), i.e. KV head l / LPH, dims
// 16 * (l % LPH) .. +16, so each K or V row is one fully coalesced 2 KiB
// wavefront access wherever the cell lives.  Scores are reduced over the LPH
// lanes of a head with xor shuffles.  Softmax runs in base 2 with the scale
// folded into q.

template <int D, int G>
__global__ __launch_bounds__(256) void k_attn_valu(AttnArgs a) {
  constexpr int LPH = D / 16;          // lanes per KV head
  constexpr int HK = 64 / LPH;         // KV heads per row (row = 1024 numbers)
  constexpr int E = HK * D;
  constexpr int H = HK * G;
  constexpr int U = 4;                 // cells in flight per wavefront step
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

  for (int c = it.c0 + w * U; c < it.c1; c += 4 * U) {
    half8 kr[U][2], vr[U][2];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = c + u;
      ok[u] = idx < it.c1;
      const int cell = a.csr_cell[ok[u] ? idx : it.c0];
      const int64_t off = (sbase + cell) * E + kvh * D + part * 16;
      const half8* kp = reinterpret_cast<const half8*>(Kl + off);
      const half8* vp = reinterpret_cast<const half8*>(Vl + off);
      kr[u][0] = kp[0]; kr[u][1] = kp[1];
      vr[u][0] = vp[0]; vr[u][1] = vp[1];
    }
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = ok[u] ? c + u : it.c0;
      const int cp = a.csr_pos[idx];
      bool vis = ok[u] && (!a.causal || cp <= si.pos);
      if (check_mask) vis = vis && ((a.csr_mask[idx] >> si.seq0) & 1ULL);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += q[g][e] * static_cast<float>(kr[u][0][e]);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += q[g][8 + e] * static_cast<float>(kr[u][1][e]);
#pragma unroll
        for (int o = 1; o < LPH; o <<= 1) s += __shfl_xor(s, o);
        sc[u][g] = vis ? s : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][g]);
      if (mx == -INFINITY) continue;
      const float alpha = exp2f(m[g] - mx);
      float p[U], ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) { p[u] = exp2f(sc[u][g] - mx); ps += p[u]; }
      l[g] = l[g] * alpha + ps;
      m[g] = mx;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = acc[g][e] * alpha;
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
    const float s0 = M == -INFINITY ? 0.f : exp2f(m[g] - M);
    float L = l[g] * s0;
    float o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = acc[g][e] * s0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const float mk = red[k][lane][g * 18];
      const float sk = (M == -INFINITY || mk == -INFINITY) ? 0.f : exp2f(mk - M);
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

// ---------------------------------------------------------------------------
// Prefill-class attention on the matrix cores.
//
// One workgroup = (item, KV head): 128 query rows = QT = 128 / G queries x
// the G query heads of that KV head, 4 wavefronts of 32 rows.  Per 64-cell
// tile the K rows (head slice, 256 B each) are gathered through the cell
// list into LDS as [cell][d] and the V rows transposed into LDS as [d][cell].
// Wavefront w computes S^T[64 cells][32 rows] = K Q^T (A = K from LDS,
// B = its queries held in registers as F16), applies the mask, updates the
// online softmax per row (each lane owns one row: column lane % 32 of the
// 32x32 accumulators), converts P to F16 and accumulates O^T[d][32 rows] =
// V^T P^T (A = V^T from LDS, B = P straight from the S^T accumulators: a
// lane's 16 scores of a 32-cell block are exactly the 8+8 k-values it
// supplies to the two 32x32x16 steps of that block, and V^T is read in the
// same cell order).

// accumulator register r of lane l in a 32x32 block sits at row
// 8*(r/4) + 4*(l/32) + r%4, column l%32
DEV int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int D, int G>
__global__ __launch_bounds__(256) void k_attn_mfma(AttnArgs a) {
  constexpr int QT = 128 / G;          // queries per item
  constexpr int KT = 64;               // cells per tile
  constexpr int DP = D < 32 ? 32 : D;  // O^T rows, padded to a 32-row block
  constexpr int KS = D + 8;            // LDS row stride of the K tile (halfs)
  constexpr int VS = KT + 4;           // LDS row stride of the V^T tile (halfs)
  __shared__ __attribute__((aligned(16))) _Float16 Ks[KT * KS];
  __shared__ __attribute__((aligned(16))) _Float16 Vt[DP * VS];
  __shared__ int32_t kcell[KT];
  __shared__ int32_t kpos[KT];
  __shared__ uint64_t kmask[KT];

  const int HK = a.n_head_kv;
  const int H = a.n_head;
  const int E = HK * D;
  const int kvh = blockIdx.x % HK;
  const WorkItem it = a.items[blockIdx.x / HK];
  const int il = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half_id = lane >> 5;
  const bool pure = a.classes[it.cls].pure;
  const _Float16* __restrict__ Kl = a.k[il];
  const _Float16* __restrict__ Vl = a.v[il];

  // this lane's query row
  const int r = 32 * w + (lane & 31);
  const int hg = r / QT, t = r % QT;
  const bool qvalid = t < it.n_q;
  const SlotInfo si = a.slots[a.qlist[it.q_off + (qvalid ? t : 0)]];
  const int h = kvh * G + hg;
  const int64_t sbase = static_cast<int64_t>(si.stream) * a.kv_size;

  // B operand of S^T = K Q^T: q[row][16*ks + 8*half + 0..7], scaled, F16
  half8 qb[D / 16];
  {
    const float* qp = a.q[il] + static_cast<int64_t>(si.q_row) * H * D + h * D + 8 * half_id;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const float4 x0 = qvalid ? *reinterpret_cast<const float4*>(qp + 16 * ks) : make_float4(0, 0, 0, 0);
      const float4 x1 = qvalid ? *reinterpret_cast<const float4*>(qp + 16 * ks + 4) : make_float4(0, 0, 0, 0);
      qb[ks][0] = static_cast<_Float16>(x0.x * a.scale_log2e);
      qb[ks][1] = static_cast<_Float16>(x0.y * a.scale_log2e);
      qb[ks][2] = static_cast<_Float16>(x0.z * a.scale_log2e);
      qb[ks][3] = static_cast<_Float16>(x0.w * a.scale_log2e);
      qb[ks][4] = static_cast<_Float16>(x1.x * a.scale_log2e);
      qb[ks][5] = static_cast<_Float16>(x1.y * a.scale_log2e);
      qb[ks][6] = static_cast<_Float16>(x1.z * a.scale_log2e);
      qb[ks][7] = static_cast<_Float16>(x1.w * a.scale_log2e);
    }
  }
  if (D < DP) {   // padded rows of V^T stay zero
    for (int i = tid; i < (DP - D) * VS; i += 256) Vt[D * VS + i] = static_cast<_Float16>(0.f);
  }

  floatx16 oacc[DP / 32];
#pragma unroll
  for (int db = 0; db < DP / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int c0 = it.c0; c0 < it.c1; c0 += KT) {
    const int nk = min(KT, it.c1 - c0);
    if (tid < KT) {
      const bool in = tid < nk;
      kcell[tid] = in ? a.csr_cell[c0 + tid] : 0;
      kpos[tid] = in ? a.csr_pos[c0 + tid] : INT32_MAX;
      kmask[tid] = in ? a.csr_mask[c0 + tid] : 0ULL;
    }
    __syncthreads();
    // tile-level causal test, identical in every wavefront
    const int pl = kpos[lane];
    const int kmin = wave_min_i(pl);
    const int kmax = wave_max_i(lane < nk ? pl : INT32_MIN);
    if (a.causal && kmin > it.qpos_max) {
      __syncthreads();
      continue;
    }
    const bool full = nk == KT && pure && (!a.causal || kmax <= it.qpos_min);

    // gather the tile: K as [cell][d], V transposed as [d][cell]
    for (int i = tid; i < KT * (D / 8); i += 256) {
      const int kr = i / (D / 8), seg = i % (D / 8);
      half8 kv, vv;
      if (kr < nk) {
        const int64_t off = (sbase + kcell[kr]) * E + kvh * D + seg * 8;
        kv = *reinterpret_cast<const half8*>(Kl + off);
        vv = *reinterpret_cast<const half8*>(Vl + off);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { kv[e] = static_cast<_Float16>(0.f); vv[e] = static_cast<_Float16>(0.f); }
      }
      *reinterpret_cast<half8*>(&Ks[kr * KS + seg * 8]) = kv;
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(seg * 8 + e) * VS + kr] = vv[e];
    }
    __syncthreads();

    // S^T for the two 32-cell blocks
    floatx16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const half8 ka = *reinterpret_cast<const half8*>(&Ks[(kb * 32 + (lane & 31)) * KS + 16 * ks + 8 * half_id]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qb[ks], sacc[kb], 0, 0, 0);
      }
    }
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + acc_row(i, lane);
          const int kp = kpos[key];
          bool vis = key < nk && (!a.causal || kp <= si.pos);
          if (!pure) vis = vis && ((kmask[key] >> si.seq0) & 1ULL);
          if (!vis) sacc[kb][i] = -INFINITY;
        }
    }
    // online softmax over this lane's row (the other half-wave holds the rest)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float rs = 0.f;
    half8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // the row sum uses the same F16-rounded weights the PV product sees
        const _Float16 ph = static_cast<_Float16>(exp2f(sacc[kb][i] - m_use));
        rs += static_cast<float>(ph);
        pb[kb][i >> 3][i & 7] = ph;
      }
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int key0 = kb * 32 + 16 * st + 4 * half_id;
#pragma unroll
        for (int db = 0; db < DP / 32; ++db) {
          const _Float16* vrow = &Vt[(db * 32 + (lane & 31)) * VS];
          const half4 lo = *reinterpret_cast<const half4*>(vrow + key0);
          const half4 hi = *reinterpret_cast<const half4*>(vrow + key0 + 8);
          half8 va;
          va[0] = lo[0]; va[1] = lo[1]; va[2] = lo[2]; va[3] = lo[3];
          va[4] = hi[0]; va[5] = hi[1]; va[6] = hi[2]; va[7] = hi[3];
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[kb][st], oacc[db], 0, 0, 0);
        }
      }
    __syncthreads();
  }

  if (!qvalid) return;
  if (it.prow < 0) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* op = a.o[il] + static_cast<int64_t>(si.out_row) * H * D + h * D;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + acc_row(4 * g4, lane);
        if (d < D)
          *reinterpret_cast<float4*>(op + d) =
              make_float4(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv, oacc[db][4 * g4 + 2] * inv,
                          oacc[db][4 * g4 + 3] * inv);
      }
  } else {
    const int64_t row = static_cast<int64_t>(il) * a.rows_per_layer + it.prow + t;
    float* pp = a.part_acc + row * H * D + h * D;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + acc_row(4 * g4, lane);
        if (d < D)
          *reinterpret_cast<float4*>(pp + d) =
              make_float4(oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3]);
      }
    if (half_id == 0) {
      a.part_ml[(row * H + h) * 2] = m_run;
      a.part_ml[(row * H + h) * 2 + 1] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// split-K merge: M = max_k m_k, O = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k

__global__ __launch_bounds__(256) void k_attn_reduce(AttnArgs a, int D) {
  const int rr = blockIdx.x, il = blockIdx.y;
  const int H = a.n_head;
  const SlotInfo si = a.slots[a.red_slot[rr]];
  const int b = a.red_off[rr], e = a.red_off[rr + 1];
  const int64_t lbase = static_cast<int64_t>(il) * a.rows_per_layer;
  for (int x = threadIdx.x * 4; x < H * D; x += blockDim.x * 4) {
    const int h = x / D;
    float M = -INFINITY;
    for (int k = b; k < e; ++k) M = fmaxf(M, a.part_ml[((lbase + a.red_rows[k]) * H + h) * 2]);
    float L = 0.f;
    float4 o = make_float4(0, 0, 0, 0);
    if (M != -INFINITY) {
      for (int k = b; k < e; ++k) {
        const int64_t row = lbase + a.red_rows[k];
        const float mk = a.part_ml[(row * H + h) * 2];
        if (mk == -INFINITY) continue;
        const float s = exp2f(mk - M);
        L += s * a.part_ml[(row * H + h) * 2 + 1];
        const float4 v = *reinterpret_cast<const float4*>(a.part_acc + row * H * D + x);
        o.x += s * v.x; o.y += s * v.y; o.z += s * v.z; o.w += s * v.w;
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *reinterpret_cast<float4*>(a.o[il] + static_cast<int64_t>(si.out_row) * H * D + x) =
        make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

// ---------------------------------------------------------------------------
// dispatch

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

template <int D, int G>
static void mfma_launch(const AttnArgs& a, int n_il, hipStream_t s) {
  hipLaunchKernelGGL((k_attn_mfma<D, G>), dim3(a.n_items * a.n_head_kv, n_il), dim3(256), 0, s, a);
}

template <int D>
static hipError_t mfma_by_group(const AttnArgs& a, int n_il, int G, hipStream_t s) {
  switch (G) {
    case 1: mfma_launch<D, 1>(a, n_il, s); break;
    case 2: mfma_launch<D, 2>(a, n_il, s); break;
    case 4: mfma_launch<D, 4>(a, n_il, s); break;
    case 8: mfma_launch<D, 8>(a, n_il, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_mfma(const AttnArgs& a, int n_il, int D, int G, hipStream_t s) {
  if (a.n_items == 0 || n_il == 0) return hipSuccess;
  switch (D) {
    case 16: return mfma_by_group<16>(a, n_il, G, s);
    case 32: return mfma_by_group<32>(a, n_il, G, s);
    case 64: return mfma_by_group<64>(a, n_il, G, s);
    case 128: return mfma_by_group<128>(a, n_il, G, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_reduce(const AttnArgs& a, int n_reduced, int n_il, int D, hipStream_t s) {
  if (n_reduced == 0 || n_il == 0) return hipSuccess;
  hipLaunchKernelGGL(k_attn_reduce, dim3(n_reduced, n_il), dim3(256), 0, s, a, D);
  return hipGetLastError();
}

}  // namespace kvattn
