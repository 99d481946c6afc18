// Allocation-free attention: kvattn_attend with its split-K partials in a
// static device array of this library instead of the caller's workspace.
//
// The array lives in the code object (one copy per GPU, held until the
// process ends).  Host code never uses its name as an address: the device
// address of each GPU's copy is looked up once per device, with that device
// current, at the context's device set-up, and only that address reaches the
// kernels.  Every call on one GPU shares its copy: nothing in it has to start
// at zero (every partial row a merge reads is written by its work item
// earlier in the same call), and calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kvattn.h"
#include "state_internal.hpp"

namespace {

constexpr size_t kScratchBytes = KVATTN_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
constexpr size_t kAlign = 256;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` on each GPU

}  // namespace

int kvattn::static_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return KVATTN_EINVAL;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch[device]) return KVATTN_OK;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != device) return KVATTN_EHIP;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVATTN_EHIP;
  g_scratch[device] = p;
  return KVATTN_OK;
}

extern "C" int kvattn_attend_noalloc(kvattn_ctx* c, const kvattn_ubatch* ub, int32_t il0, int32_t n_il,
                                     const void* const* q, void* const* out, int32_t only_outputs,
                                     void* hip_stream) {
  if (!c) return KVATTN_EINVAL;
  kvattn_params p;
  if (kvattn_get_params(c, &p) != KVATTN_OK) return KVATTN_EINVAL;
  if (p.device < 0 || p.device >= kMaxDevices) return KVATTN_EINVAL;
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    base = g_scratch[p.device];
  }
  if (!base) {
    // the context's device set-up (its first store) looks the array up;
    // without it there is no committed ubatch to attend to
    if (hipSetDevice(p.device) != hipSuccess) return KVATTN_EHIP;
    if (int rc = kvattn::static_scratch_init(p.device)) return rc;
    std::lock_guard<std::mutex> lk(g_mu);
    base = g_scratch[p.device];
  }
  // [rows][n_head * head_dim] accumulators, then [rows][n_head][2] (max, sum)
  const size_t acc_row = static_cast<size_t>(p.n_head) * p.head_dim * 4;
  const size_t ml_row = static_cast<size_t>(p.n_head) * 2 * 4;
  int64_t rows = static_cast<int64_t>(kScratchBytes / (acc_row + ml_row));
  size_t ml_off = 0;
  while (rows > 0) {
    ml_off = (static_cast<size_t>(rows) * acc_row + kAlign - 1) / kAlign * kAlign;
    if (ml_off + static_cast<size_t>(rows) * ml_row <= kScratchBytes) break;
    --rows;
  }
  float* acc = static_cast<float*>(base);
  float* ml = reinterpret_cast<float*>(static_cast<char*>(base) + ml_off);
  return kvattn::attend_with_partials(c, ub, il0, n_il, q, out, only_outputs, hip_stream, acc, ml, rows);
}
