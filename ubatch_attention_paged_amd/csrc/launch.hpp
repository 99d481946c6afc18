// Launch wrappers for the gfx950 kernels (kernels.hip).  Argument records
// are plain structs passed by value as kernel arguments.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

namespace kvattn {

struct StoreArgs {
  const float* k_cur[kMaxLayersPerLaunch];
  const float* v_cur[kMaxLayersPerLaunch];
  _Float16* k[kMaxLayersPerLaunch];
  _Float16* v[kMaxLayersPerLaunch];
  const int32_t* dst_rows;    // [n_rows] stream * kv_size + cell, then [n_rows - n_src] source slots:
                              // rows >= n_src are separate copies of slot dst_rows[n_rows + r - n_src]
  int32_t n_rows;
  int32_t n_src;              // slots of the ubatch (rows of k_cur / v_cur)
  int32_t E;
};

struct CsrArgs {
  int32_t* cpos;              // [S * C] device mirror: position, -1 empty
  SeqSet* cmask;              // [S * C] sequence set of each cell
  int32_t* cellcls;           // [S * C] class of each cell (-1 none), scratch
  int32_t* counts;            // [n_classes * n_seg] per segment counts, then offsets
  int32_t* csr_cell;          // [total] cells, class-major, ascending within a class
  int32_t* csr_pos;
  SeqSet* csr_mask;
  const ClassInfo* classes;
  const LookupEntry* lookup;
  const int32_t* lookup_off;  // [S + 1]
  const CellUpdate* updates;
  int32_t n_updates, n_classes, n_seg, kv_size, n_kv, n_stream;
  int32_t csr_cap;            // entries of csr_*: n_stream * kv_size
  int32_t* tile_min;          // per 64-cell tile of each class: smallest / largest position
  int32_t* tile_max;
  int32_t max_class_tiles;
  int32_t n_lookup;           // lookup entries (lookup_off[n_stream])
  // fused path only: the plan still sits in pinned host memory (classes,
  // lookup, lookup_off, updates point into it); the store workgroups copy
  // its plan_n16 16-byte units to the device plan arena
  const void* plan_src;
  void* plan_dst;
  int32_t plan_n16;
};

struct AttnArgs {
  const float* q[kMaxLayersPerLaunch];
  float* o[kMaxLayersPerLaunch];
  const _Float16* k[kMaxLayersPerLaunch];
  const _Float16* v[kMaxLayersPerLaunch];
  const SlotInfo* slots;
  const ClassInfo* classes;
  const SlotInfo* qslots;     // the query slots of each class, in class order (WorkItem::q_off)
  const WorkItem* items;
  const int32_t* csr_cell;
  const int32_t* csr_pos;
  const SeqSet* csr_mask;
  const int32_t* tile_min;
  const int32_t* tile_max;
  float* part_acc;            // [n_il][rows][n_head * head_dim]
  float* part_ml;             // [n_il][rows][n_head][2]  (max in log2 units, sum)
  const int32_t* red_slot;
  const int32_t* red_off;
  const int32_t* red_rows;
  int32_t rows_per_layer;
  int32_t n_items;
  int32_t kv_size;
  int32_t n_head;
  int32_t n_head_kv;
  int32_t causal;
  int32_t swa;                // sliding window in positions, 0 = none
  float scale_log2e;          // kq_scale * log2(e)
  uint32_t layer_bytes;       // bytes of one layer's K (= V) tensor, < 2 GiB
  // combined launch (attn_both.hip): the vector-ALU items beside the
  // matrix-core ones in `items`, and the layers of the launch
  const WorkItem* items2;
  int32_t n_items2;
  int32_t n_il;
};

struct MaskArgs {
  const int32_t* cpos;
  const SeqSet* cmask;
  const SlotInfo* slots;      // ubatch order
  uint16_t* mask;             // [n_rows][n_kv]
  int32_t n_rows, n_kv, kv_size, causal, swa;
};

// Sequence-state records (kernels_state.hip).  Word offsets: the blob is
// 4-byte aligned; record r = kind * n_layer + layer starts at byte
// rec0 + r * rec_stride with a 3-word header, then n rows of row_words.
constexpr uint32_t kStateTypeF16 = 1;
struct StateArgs {
  _Float16* k[kMaxLayersPerLaunch];   // layers il0 .. il0 + n_il - 1
  _Float16* v[kMaxLayersPerLaunch];
  const int32_t* cells;               // [n] stream * kv_size + cell, in record row order
  uint32_t* blob_w;                   // save: destination
  const uint32_t* blob_r;             // restore: source
  const uint32_t* prefix;             // save: the leading metadata words
  int32_t prefix_words;
  int32_t n;                          // saved cells
  int32_t n_layer;                    // every layer (record numbering)
  int32_t il0, n_il;
  int32_t row_words;
  uint64_t rec0;                      // bytes before the first record
  uint64_t rec_stride;                // bytes per record
};

hipError_t launch_store(const StoreArgs& a, int n_il, hipStream_t s);
hipError_t launch_state_copy(const StateArgs& a, bool save, hipStream_t s);
hipError_t launch_state_peek(const uint32_t* blob, uint32_t* out, int32_t n_rec, uint64_t rec0, uint64_t rec_stride,
                             hipStream_t s);
hipError_t launch_commit(const CsrArgs& a, hipStream_t s);
// a commit small enough for one workgroup (launch_store_commit can carry it)
bool commit_is_small(const CsrArgs& a);
// the stores of n_il >= 1 layers and, in one extra workgroup, a small commit
hipError_t launch_store_commit(const StoreArgs& a, int n_il, const CsrArgs& c, hipStream_t s);
hipError_t launch_mask(const MaskArgs& a, hipStream_t s);
// Optional kernel timing: a launch given either event goes through
// hipExtLaunchKernel, which stamps `start` with the kernel's own start time
// and `stop` with its end time (not the time the stream reached them).
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool any() const { return start || stop; }
};

// head_dim / group size are dispatched at run time
hipError_t launch_attn_valu(const AttnArgs& a, int n_il, int head_dim, int group, hipStream_t s,
                            const KernelEvents& ev = {});
hipError_t launch_attn_mfma(const AttnArgs& a, int n_il, int head_dim, int group, hipStream_t s,
                            const KernelEvents& ev = {});
// matrix-core items (items, n_items) and vector-ALU items (items2,
// n_items2) in one launch, for the shapes attn_both_supported accepts (no
// sliding window)
bool attn_both_supported(int head_dim, int group, int row);
hipError_t launch_attn_both(const AttnArgs& a, int n_il, int head_dim, int group, hipStream_t s,
                            const KernelEvents& ev = {});
hipError_t launch_reduce(const AttnArgs& a, int n_reduced, int n_il, int head_dim, hipStream_t s,
                         const KernelEvents& ev = {});

}  // namespace kvattn
