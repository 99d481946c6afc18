// gfx950 kernels of the store/commit half of the path:
//
//   k_store          K/V rows of a ubatch -> F16 (nearest-even) into their cells
//   k_store_commit   the same, with one extra workgroup doing the whole commit
//                    below for a small cache (overlapped with the stores)
//   k_apply_updates  cell-table changes -> device mirror (pos, sequence set)
//   k_csr_*          per-class lists of visible cells, ascending cell index
//   k_tile_minmax    smallest / largest position of every 64-cell tile of a list
//   k_mask_dense     dense F16 KQ mask (diagnostic form of the same predicate)
//
// Visibility ("llama.cpp and the ubatch", "The mask is doing the work"): a
// cell is seen by a query when it is occupied, its sequence set holds the
// query's first sequence id and, under causal attention, its position is
// not later than the query's.  The class lists group cells by sequence set;
// the attention kernels apply the position test per (query, cell).
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace kvattn {

// fp32 rows -> F16 rows of the cache; each thread converts 8 consecutive
// values (two 16 B loads, one 16 B store).
KVATTN_DEV void store_rows(const StoreArgs& a) {
  const int il = blockIdx.y;
  const int which = blockIdx.z;             // 0 = K, 1 = V
  const int vec_per_row = a.E >> 3;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= static_cast<int64_t>(a.n_rows) * vec_per_row) return;
  const int r = static_cast<int>(t / vec_per_row);
  const int c = static_cast<int>(t % vec_per_row);
  const int sr = r < a.n_src ? r : a.dst_rows[a.n_rows + r - a.n_src];   // a copy stores its slot's row
  const float* src = (which ? a.v_cur[il] : a.k_cur[il]) + static_cast<int64_t>(sr) * a.E + c * 8;
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

__global__ __launch_bounds__(256) void k_store(StoreArgs a) { store_rows(a); }

hipError_t launch_store(const StoreArgs& a, int n_il, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(a.n_rows) * (a.E / 8);
  if (n == 0 || n_il == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((n + 255) / 256), n_il, 2);
  hipLaunchKernelGGL(k_store, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Mirror updates (read from the pinned staging buffer), the per-(class,
// segment) counts cleared and the plan copied from the staging buffer into
// the device arena, in one launch; the later commit kernels and the
// attention read the arena.
__global__ __launch_bounds__(256) void k_apply_updates(CsrArgs a, int64_t n_counts) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < a.plan_n16) static_cast<u32x4*>(a.plan_dst)[i] = static_cast<const u32x4*>(a.plan_src)[i];
  if (i < a.n_updates) {
    const int32_t idx = a.updates[i].idx;
    a.cpos[idx] = a.updates[i].pos;
    copy_set(&a.cmask[idx], &a.updates[i].mask);
  }
  if (i < n_counts) a.counts[i] = 0;
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
      const SeqSet m = a.cmask[idx];
      int lo = a.lookup_off[s], hi = a.lookup_off[s + 1] - 1;
      while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const SeqSet mm = a.lookup[mid].mask;
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
// Thread t owns a contiguous run of segments: one round of independent loads
// for its run's total, a workgroup scan of the totals, then its run's
// offsets.
constexpr int kScanThreads = 256;
__global__ __launch_bounds__(kScanThreads) void k_csr_scan(CsrArgs a) {
  __shared__ int32_t wsum[kScanThreads / 64];
  const int c = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int32_t* row = a.counts + static_cast<int64_t>(c) * a.n_seg;
  const int per = (a.n_seg + kScanThreads - 1) / kScanThreads;
  const int k0 = min(a.n_seg, t * per), k1 = min(a.n_seg, k0 + per);
  int total = 0;
  for (int k = k0; k < k1; ++k) total += row[k];
  int incl = total;                                  // inclusive scan over the wavefront
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = a.classes[c].cell_off;
  for (int j = 0; j < w; ++j) before += wsum[j];
  int running = before + incl - total;               // exclusive start of this thread's run
  for (int k = k0; k < k1; ++k) {
    const int v = row[k];
    row[k] = running;
    running += v;
  }
}

// Every classified cell goes to its class offset + its rank among the earlier
// cells of its class in the segment: ascending cell index within a class.
__global__ __launch_bounds__(256) void k_csr_scatter(CsrArgs a) {
  const int s = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int64_t idx = static_cast<int64_t>(s) * a.kv_size + j;
  const int cls = j < a.n_kv ? a.cellcls[idx] : -1;
  const int seg = j >> 6;
  // rank among the earlier cells of the same class in this segment; the
  // class offsets are then read once, all lanes at a time
  int rank = 0;
  uint64_t active = ballot(cls >= 0);
  while (active) {
    const int leader = __builtin_ctzll(active);
    const int c = readlane_i(cls, leader);
    const uint64_t same = ballot(cls == c);
    if (cls == c) rank = __popcll(same & lanemask_lt());
    active &= ~same;
  }
  if (cls >= 0) {
    const int dst = a.counts[static_cast<int64_t>(cls) * a.n_seg + seg] + rank;
    if (dst < a.csr_cap) {
      a.csr_cell[dst] = j;
      a.csr_pos[dst] = a.cpos[idx];
      a.csr_mask[dst] = a.cmask[idx];
    }
  }
}

// One wavefront per 64-cell tile of a class list: its position range.
__global__ __launch_bounds__(256) void k_tile_minmax(CsrArgs a) {
  const ClassInfo ci = a.classes[blockIdx.x];
  const int nt = (ci.n_cells + kTileCells - 1) / kTileCells;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int k_end = min(nt, static_cast<int>(blockIdx.y) * 16 + 16);
  for (int k = blockIdx.y * 16 + w; k < k_end; k += 4) {
    const int j = k * kTileCells + lane;
    const bool in = j < ci.n_cells;
    const int p = in ? a.csr_pos[ci.cell_off + j] : INT32_MAX;
    const int mn = wave_min_i(p);
    const int mx = wave_max_i(in ? p : INT32_MIN);
    if (lane == 0) {
      a.tile_min[ci.tile_base + k] = mn;
      a.tile_max[ci.tile_base + k] = mx;
    }
  }
}

// The whole commit in one workgroup of kCommitThreads threads, for caches of
// at most kSmallCommitCells (stream, cell) pairs below n_kv,
// kSmallCommitClasses classes and lookup entries and kSmallCommitStreams
// streams: mirror updates, classification (kept in LDS), the ordered
// per-class lists (kCommitThreads cells at a time in (stream, cell) order: a
// cell's slot is its class's running offset + the same-class cells of
// earlier wavefronts of the chunk + its rank in its wavefront), then the
// per-tile position ranges.  Produces exactly what the multi-kernel path
// produces.  The class and lookup tables are read once into LDS (they may
// sit in host memory); each thread reads its (at most four) cells' mirror
// entries -- position and 32-byte sequence set -- once, up front, and keeps
// them in registers, so the whole commit waits on global memory about once.
constexpr int kCommitThreads = 1024;
KVATTN_DEV void commit_small(const CsrArgs& a) {
  constexpr int NT = kCommitThreads, NWV = NT / 64;
  constexpr int KMAX = kSmallCommitCells / NT;      // cells per thread at most
  __shared__ int32_t wc[NWV][kSmallCommitClasses];
  __shared__ int32_t base[kSmallCommitClasses];
  __shared__ LookupEntry lk[kSmallCommitClasses];
  __shared__ ClassInfo cl[kSmallCommitClasses];
  __shared__ int32_t lko[kSmallCommitStreams + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nc = a.n_classes;
  if (tid < a.n_lookup) lk[tid] = a.lookup[tid];
  if (tid < nc) cl[tid] = a.classes[tid];
  if (tid <= a.n_stream && nc > 0) lko[tid] = a.lookup_off[tid];
  for (int i = tid; i < a.n_updates; i += NT) {
    const int32_t idx = a.updates[i].idx;
    a.cpos[idx] = a.updates[i].pos;
    copy_set(&a.cmask[idx], &a.updates[i].mask);
  }
  __syncthreads();
  if (nc == 0) return;
  const int total = a.n_stream * a.n_kv;
  // every cell this thread will place (cell tid + NT k), read once: its
  // position, sequence set and class stay in registers
  int pos_r[KMAX], cls_r[KMAX];
  SeqSet msk_r[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int i = tid + NT * k;
    pos_r[k] = -1;
    msk_r[k] = SeqSet::none();
    if (i < total) {
      const int64_t idx = static_cast<int64_t>(i / a.n_kv) * a.kv_size + i % a.n_kv;
      pos_r[k] = a.cpos[idx];
      msk_r[k] = load_set(&a.cmask[idx]);
    }
  }
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    int cls = -1;
    const int i = tid + NT * k;
    if (i < total && pos_r[k] >= 0) {
      const int s = i / a.n_kv;
      int lo = lko[s], hi = lko[s + 1] - 1;
      while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const SeqSet mm = lk[mid].mask;
        if (mm == msk_r[k]) { cls = lk[mid].cls; break; }
        if (mm < msk_r[k]) lo = mid + 1; else hi = mid - 1;
      }
    }
    cls_r[k] = cls;
  }
  if (tid < nc) base[tid] = cl[tid].cell_off;
  for (int z = tid; z < NWV * kSmallCommitClasses; z += NT) wc[z / kSmallCommitClasses][z % kSmallCommitClasses] = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (NT * k >= total) break;
    const int cls = cls_r[k];
    int rank = 0;
    uint64_t active = ballot(cls >= 0);
    while (active) {
      const int leader = __builtin_ctzll(active);
      const int c = readlane_i(cls, leader);
      const uint64_t same = ballot(cls == c);
      if (cls == c) rank = __popcll(same & lanemask_lt());
      if (lane == leader) wc[w][c] = __popcll(same);
      active &= ~same;
    }
    __syncthreads();
    if (cls >= 0) {
      int dst = base[cls] + rank;
      for (int w2 = 0; w2 < w; ++w2) dst += wc[w2][cls];
      if (dst < a.csr_cap) {
        a.csr_cell[dst] = (tid + NT * k) % a.n_kv;
        a.csr_pos[dst] = pos_r[k];
        store_set(&a.csr_mask[dst], msk_r[k]);
      }
    }
    __syncthreads();
    // the thread that folds class tid's counts into its offset also clears
    // them (only classes < nc are ever counted)
    if (tid < nc) {
      int add = 0;
#pragma unroll
      for (int w2 = 0; w2 < NWV; ++w2) {
        add += wc[w2][tid];
        wc[w2][tid] = 0;
      }
      base[tid] += add;
    }
    __syncthreads();
  }
  for (int c = 0; c < nc; ++c) {
    const ClassInfo ci = cl[c];
    const int nt = (ci.n_cells + kTileCells - 1) / kTileCells;
    for (int k = w; k < nt; k += NWV) {
      const int j = k * kTileCells + lane;
      const bool in = j < ci.n_cells;
      const int p = in ? a.csr_pos[ci.cell_off + j] : INT32_MAX;
      const int mn = wave_min_i(p);
      const int mx = wave_max_i(in ? p : INT32_MIN);
      if (lane == 0) {
        a.tile_min[ci.tile_base + k] = mn;
        a.tile_max[ci.tile_base + k] = mx;
      }
    }
  }
}

bool commit_is_small(const CsrArgs& a) {
  return static_cast<int64_t>(a.n_stream) * a.n_kv <= kSmallCommitCells && a.n_classes <= kSmallCommitClasses &&
         a.n_lookup <= kSmallCommitClasses && a.n_stream <= kSmallCommitStreams;
}

// The store grid plus one trailing x-block; that block's (y, z) = (0, 0)
// instance runs the small commit.  The other (y, z) = (0, 0) blocks also copy
// the plan from pinned host memory into the device plan arena, which the
// attention launches read after this kernel.
__global__ __launch_bounds__(kCommitThreads) void k_store_commit(StoreArgs a, CsrArgs c) {
  if (blockIdx.x == gridDim.x - 1) {
    if (blockIdx.y == 0 && blockIdx.z == 0) commit_small(c);
    return;
  }
  if (blockIdx.y == 0 && blockIdx.z == 0 && c.plan_n16 > 0) {
    const u32x4* src = static_cast<const u32x4*>(c.plan_src);
    u32x4* dst = static_cast<u32x4*>(c.plan_dst);
    const int stride = (gridDim.x - 1) * blockDim.x;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < c.plan_n16; i += stride) dst[i] = src[i];
  }
  store_rows(a);
}

hipError_t launch_store_commit(const StoreArgs& a, int n_il, const CsrArgs& c, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(a.n_rows) * (a.E / 8);
  dim3 grid(static_cast<unsigned>((n + kCommitThreads - 1) / kCommitThreads) + 1, n_il, 2);
  hipLaunchKernelGGL(k_store_commit, grid, dim3(kCommitThreads), 0, s, a, c);
  return hipGetLastError();
}

hipError_t launch_commit(const CsrArgs& a, hipStream_t s) {
  const int64_t nc = static_cast<int64_t>(a.n_classes) * a.n_seg;
  const int64_t n_apply = std::max<int64_t>(std::max<int64_t>(a.n_updates, nc), a.plan_n16);
  if (n_apply > 0)
    hipLaunchKernelGGL(k_apply_updates, dim3(static_cast<unsigned>((n_apply + 255) / 256)), dim3(256), 0, s, a, nc);
  if (a.n_classes == 0) return hipGetLastError();
  const dim3 grid((a.n_kv + 255) / 256, a.n_stream);
  hipLaunchKernelGGL(k_csr_classify, grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_csr_scan, dim3(a.n_classes), dim3(kScanThreads), 0, s, a);
  hipLaunchKernelGGL(k_csr_scatter, grid, dim3(256), 0, s, a);
  if (a.max_class_tiles > 0)
    hipLaunchKernelGGL(k_tile_minmax, dim3(a.n_classes, (a.max_class_tiles + 15) / 16), dim3(256), 0, s, a);
  return hipGetLastError();
}

// 0x0000 visible, 0xFC00 (-inf) hidden
__global__ __launch_bounds__(256) void k_mask_dense(MaskArgs a) {
  const int i = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.n_kv) return;
  const SlotInfo q = a.slots[i];
  const int64_t idx = static_cast<int64_t>(q.stream) * a.kv_size + j;
  const int32_t p = a.cpos[idx];
  const bool vis = p >= 0 && a.cmask[idx].test(q.seq0) && (!a.causal || p <= q.pos) &&
                   (a.swa == 0 || q.pos - p < a.swa);
  a.mask[static_cast<int64_t>(i) * a.n_kv + j] = vis ? 0x0000 : 0xFC00;
}

hipError_t launch_mask(const MaskArgs& a, hipStream_t s) {
  if (a.n_rows == 0 || a.n_kv == 0) return hipSuccess;
  hipLaunchKernelGGL(k_mask_dense, dim3((a.n_kv + 255) / 256, a.n_rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvattn
