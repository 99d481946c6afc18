// Sequence-state save / restore: copies between a sequence's cache rows and
// the records of a serialized blob ("What does llama.cpp's KV cache actually
// look like in memory?", "Opening the .bin dump": leading metadata, K
// records of every layer, then V records, each a 12-byte header and the
// sequence's rows).
//
// A record's rows are contiguous in the blob but start at a 4-byte aligned
// offset (12-byte headers, 4 bytes per saved position), while cache rows
// are 16-byte aligned and scattered over the cells.
#include "device_common.hpp"
#include "launch.hpp"

namespace kvattn {

constexpr int kStateThreads = 256;
constexpr int kStateUnroll = 4;
// a thread moves groups of 4 words: one 16-byte access on the cache side
// (rows are 16-byte aligned and a multiple of 16 bytes long, so a group
// never straddles two rows), four 4-byte accesses on the blob side
constexpr int kStateGroupsPerBlock = kStateThreads * kStateUnroll;

template <bool SAVE>
__global__ __launch_bounds__(kStateThreads) void k_state_copy(StateArgs a) {
  const int li = blockIdx.y;                 // layer il0 + li
  const int kind = blockIdx.z;               // 0 = K, 1 = V
  const int layer = a.il0 + li;
  const int64_t rec = static_cast<int64_t>(kind) * a.n_layer + layer;
  const int64_t rec_word = (static_cast<int64_t>(a.rec0) + rec * static_cast<int64_t>(a.rec_stride)) / 4;
  u32x4* cache = reinterpret_cast<u32x4*>(kind == 0 ? a.k[li] : a.v[li]);
  const int row_groups = a.row_words / 4;
  const int64_t total = static_cast<int64_t>(a.n) * row_groups;
  if (SAVE) {
    if (blockIdx.x == 0 && threadIdx.x < 3) {
      // record header: type, then the row size as a little-endian u64
      const uint32_t hw[3] = {kStateTypeF16, static_cast<uint32_t>(a.row_words * 4u), 0u};
      a.blob_w[rec_word + threadIdx.x] = hw[threadIdx.x];
    }
    if (blockIdx.x == 0 && li == 0 && kind == 0 && a.il0 == 0)
      for (int i = threadIdx.x; i < a.prefix_words; i += kStateThreads) a.blob_w[i] = a.prefix[i];
  }
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kStateGroupsPerBlock;
  u32x4 v[kStateUnroll];
  int64_t src[kStateUnroll];
#pragma unroll
  for (int u = 0; u < kStateUnroll; ++u) {
    const int64_t t = base + u * kStateThreads + threadIdx.x;
    src[u] = -1;
    if (t < total) {
      const int64_t i = t / row_groups, gq = t % row_groups;
      src[u] = static_cast<int64_t>(a.cells[i]) * row_groups + gq;   // 16-byte group within the layer tensor
    }
  }
#pragma unroll
  for (int u = 0; u < kStateUnroll; ++u) {
    const int64_t t = base + u * kStateThreads + threadIdx.x;
    if (src[u] >= 0) {
      if (SAVE) {
        v[u] = cache[src[u]];
      } else {
        const uint32_t* b = a.blob_r + rec_word + 3 + 4 * t;
        v[u] = u32x4{b[0], b[1], b[2], b[3]};
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kStateUnroll; ++u) {
    const int64_t t = base + u * kStateThreads + threadIdx.x;
    if (src[u] >= 0) {
      if (SAVE) {
        uint32_t* b = a.blob_w + rec_word + 3 + 4 * t;
        b[0] = v[u][0];
        b[1] = v[u][1];
        b[2] = v[u][2];
        b[3] = v[u][3];
      } else {
        cache[src[u]] = v[u];
      }
    }
  }
}

// Gather the 3-word header of each of n_rec records into out (restore
// validates them on the host).
__global__ void k_state_peek(const uint32_t* blob, uint32_t* out, int32_t n_rec, uint64_t rec0, uint64_t rec_stride) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n_rec) return;
  const int64_t w = (static_cast<int64_t>(rec0) + r * static_cast<int64_t>(rec_stride)) / 4;
  out[3 * r] = blob[w];
  out[3 * r + 1] = blob[w + 1];
  out[3 * r + 2] = blob[w + 2];
}

hipError_t launch_state_copy(const StateArgs& a, bool save, hipStream_t s) {
  if (a.n_il <= 0) return hipSuccess;
  const int64_t total = static_cast<int64_t>(a.n) * (a.row_words / 4);
  const int64_t gx = (total + kStateGroupsPerBlock - 1) / kStateGroupsPerBlock;
  // a save with no cells still writes the prefix and the record headers
  const dim3 grid(static_cast<unsigned>(gx > 0 ? gx : (save ? 1 : 0)), a.n_il, 2);
  if (grid.x == 0) return hipSuccess;
  if (save)
    hipLaunchKernelGGL(k_state_copy<true>, grid, dim3(kStateThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_state_copy<false>, grid, dim3(kStateThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_state_peek(const uint32_t* blob, uint32_t* out, int32_t n_rec, uint64_t rec0, uint64_t rec_stride,
                             hipStream_t s) {
  if (n_rec <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_state_peek, dim3((n_rec + 63) / 64), dim3(64), 0, s, blob, out, n_rec, rec0, rec_stride);
  return hipGetLastError();
}

}  // namespace kvattn
