// Library-internal entry points: the sequence-state path for the native
// iteration loop (sched.cpp), and attention with caller-placed split-K
// partials for the allocation-free entry point (attend_static.hip).  Not
// part of the C ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "kvattn.h"

namespace kvattn {

// True when the context has device buffers (save / restore copy rows).
bool ctx_has_device(const kvattn_ctx* c);

// Restore a blob whose metadata the caller already knows -- n cells at
// positions pos[0..n) -- as sequence seq: the placement of
// kvattn_seq_state_load without reading the metadata back, so nothing
// synchronises.  On a host-only context only the placement happens.
int state_restore_known(kvattn_ctx* c, int32_t seq, const void* src, const int32_t* pos, int32_t n,
                        void* hip_stream);

// kvattn_attend with the split-K partials in part_acc ([rows][n_head *
// head_dim] fp32) and part_ml ([rows][n_head][2] fp32) instead of the
// workspace: part_rows rows, at least one layer's.  part_acc == NULL means
// the workspace's own region.  Rejects (KVATTN_ENOMEM) a plan whose partial
// rows per layer exceed part_rows; allocates nothing.
int attend_with_partials(kvattn_ctx* c, const kvattn_ubatch* ub, int32_t il0, int32_t n_il, const void* const* q,
                         void* const* out, int32_t only_outputs, void* hip_stream, float* part_acc, float* part_ml,
                         int64_t part_rows);

// Locate this library's static scratch array on the current device (once
// per device); called by the context's device set-up.
int static_scratch_init(int device);

}  // namespace kvattn
