// Small device helpers shared by the gfx950 kernels (64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "seqset.hpp"

namespace kvattn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

#define KVATTN_DEV __device__ __forceinline__

KVATTN_DEV uint64_t ballot(bool p) { return __ballot(p); }
KVATTN_DEV int lane_id() { return threadIdx.x & 63; }
KVATTN_DEV uint64_t lanemask_lt() { return (1ULL << lane_id()) - 1ULL; }
KVATTN_DEV int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

KVATTN_DEV int wave_min_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
KVATTN_DEV int wave_max_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane l receives element l % 4 of the 8-byte rows addressed by lanes
// l / 4, 4 + l / 4, 8 + l / 4 and 12 + l / 4 of its group.  So when source
// lane s points at row (r0 + s / 4), column (c0 + 4 * (s % 4)) of a
// row-major 16-bit tile, lane l gets rows r0 .. r0+3 of column c0 + l.
KVATTN_DEV half4 lds_read_tr16(const _Float16* p) {
  const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
  return __builtin_bit_cast(half4, v);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOobOffset = 0x80000000u;   // past any buffer (buffers stay below 2 GiB)

// 16 B per lane from a raw buffer straight into LDS: lane l's bytes land at
// LDS byte address lds + 16 * l (wavefront-uniform, passed through M0); an
// out-of-range offset writes zeros.  Issued as inline asm on purpose: the
// compiler then inserts no waits for it (it would otherwise drain every
// such load before any later LDS read, whatever the address), so the caller
// owns the ordering -- an s_waitcnt vmcnt(0) before the barrier that hands
// the data to other waves.
//
// buffer_rsrc_words: the four words of a raw buffer descriptor over
// [p, p + bytes) (gfx9-family word 3, stride 0).  Loads through it are
// range-checked by the hardware: an offset at or past `bytes` reads (or
// writes into LDS) zeros without touching memory.
KVATTN_DEV u32x4 buffer_rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  u32x4 r;
  r[0] = static_cast<uint32_t>(a);
  r[1] = static_cast<uint32_t>(a >> 32) & 0xffffu;   // stride 0
  r[2] = bytes;
  r[3] = 0x00020000u;
  return r;
}
KVATTN_DEV uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)(p)));
}
// M0 is a register the compiler reserves, so the asm saves and restores it
// itself instead of declaring it clobbered.
KVATTN_DEV void buffer_load16_lds(u32x4 rsrc, uint32_t lds, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(rsrc)
      : "memory");
}

// 32-byte sequence sets moved as two 16-byte vector accesses.  Copying the
// struct as a whole makes the compiler stage it through a private slot,
// which it then promotes to LDS (32 B per thread of every workgroup).
KVATTN_DEV SeqSet load_set(const SeqSet* p) {
  const u32x4* s = reinterpret_cast<const u32x4*>(p);
  const u32x4 lo = s[0], hi = s[1];
  SeqSet r;
  r.w[0] = lo[0] | (static_cast<uint64_t>(lo[1]) << 32);
  r.w[1] = lo[2] | (static_cast<uint64_t>(lo[3]) << 32);
  r.w[2] = hi[0] | (static_cast<uint64_t>(hi[1]) << 32);
  r.w[3] = hi[2] | (static_cast<uint64_t>(hi[3]) << 32);
  return r;
}
KVATTN_DEV void store_set(SeqSet* p, const SeqSet& v) {
  u32x4* d = reinterpret_cast<u32x4*>(p);
  u32x4 lo, hi;
  lo[0] = static_cast<uint32_t>(v.w[0]); lo[1] = static_cast<uint32_t>(v.w[0] >> 32);
  lo[2] = static_cast<uint32_t>(v.w[1]); lo[3] = static_cast<uint32_t>(v.w[1] >> 32);
  hi[0] = static_cast<uint32_t>(v.w[2]); hi[1] = static_cast<uint32_t>(v.w[2] >> 32);
  hi[2] = static_cast<uint32_t>(v.w[3]); hi[3] = static_cast<uint32_t>(v.w[3] >> 32);
  d[0] = lo;
  d[1] = hi;
}
KVATTN_DEV void copy_set(SeqSet* dst, const SeqSet* src) {
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  const u32x4 lo = s[0], hi = s[1];
  d[0] = lo;
  d[1] = hi;
}

// Accumulator register r of lane l in a 32x32 MFMA block holds row
// 8*(r/4) + 4*(l/32) + r%4, column l%32.
KVATTN_DEV int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

}  // namespace kvattn
