// Library-internal entry points of the sequence-state path, for the native
// iteration loop (sched.cpp).  Not part of the C ABI.
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

}  // namespace kvattn
