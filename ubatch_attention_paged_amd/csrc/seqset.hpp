// A set of sequence ids, one bit each (ids 0 .. kMaxSeq-1): the per-cell
// metadata the mask tests ("llama.cpp and the ubatch", "The mask is doing the
// work": a cell is visible to a query whose first sequence id is in the
// cell's set).  Plain data shared by the host core, the plan uploaded to the
// device and the kernels; the order (operator<) is that of the set read as
// one kMaxSeq-bit number, the same on both sides.
#pragma once

#include <cstddef>
#include <cstdint>

#if defined(__HIPCC__) || defined(__HIP__)
#define KVATTN_HD __host__ __device__
#else
#define KVATTN_HD
#endif

namespace kvattn {

constexpr int kSeqWords = 4;
constexpr int kMaxSeq = 64 * kSeqWords;   // sequence ids are bits of a 256-bit set

// 16-byte aligned so that a set moves in two 16-byte loads or stores
struct alignas(16) SeqSet {
  uint64_t w[kSeqWords];

  static KVATTN_HD SeqSet none() {
    SeqSet s{};
    return s;
  }
  static KVATTN_HD SeqSet one(int q) {
    SeqSet s{};
    s.w[q >> 6] = 1ULL << (q & 63);
    return s;
  }
  KVATTN_HD bool test(int q) const { return (w[q >> 6] >> (q & 63)) & 1ULL; }
  KVATTN_HD void set(int q) { w[q >> 6] |= 1ULL << (q & 63); }
  KVATTN_HD void reset(int q) { w[q >> 6] &= ~(1ULL << (q & 63)); }
  KVATTN_HD bool any() const {
    uint64_t a = 0;
    for (int i = 0; i < kSeqWords; ++i) a |= w[i];
    return a != 0;
  }
  // smallest member after `q` (-1: none); next(-1) is the smallest member
  KVATTN_HD int next(int q) const {
    for (int i = (q + 1) >> 6; i < kSeqWords; ++i) {
      uint64_t m = w[i];
      if (i == (q + 1) >> 6 && ((q + 1) & 63)) m &= ~0ULL << ((q + 1) & 63);
      if (m) return 64 * i + __builtin_ctzll(m);
    }
    return -1;
  }
  KVATTN_HD int lowest() const { return next(-1); }
  KVATTN_HD SeqSet operator|(const SeqSet& o) const {
    SeqSet r;
    for (int i = 0; i < kSeqWords; ++i) r.w[i] = w[i] | o.w[i];
    return r;
  }
  KVATTN_HD SeqSet operator&(const SeqSet& o) const {
    SeqSet r;
    for (int i = 0; i < kSeqWords; ++i) r.w[i] = w[i] & o.w[i];
    return r;
  }
  KVATTN_HD SeqSet& operator|=(const SeqSet& o) {
    for (int i = 0; i < kSeqWords; ++i) w[i] |= o.w[i];
    return *this;
  }
  KVATTN_HD bool operator==(const SeqSet& o) const {
    bool e = true;
    for (int i = 0; i < kSeqWords; ++i) e &= w[i] == o.w[i];
    return e;
  }
  KVATTN_HD bool operator!=(const SeqSet& o) const { return !(*this == o); }
  KVATTN_HD bool operator<(const SeqSet& o) const {
    for (int i = kSeqWords - 1; i >= 0; --i)
      if (w[i] != o.w[i]) return w[i] < o.w[i];
    return false;
  }
};

struct SeqSetHash {
  size_t operator()(const SeqSet& s) const {
    uint64_t h = 0x9E3779B97F4A7C15ull;
    for (int i = 0; i < kSeqWords; ++i) h = (h ^ s.w[i]) * 0xBF58476D1CE4E5B9ull;
    return static_cast<size_t>(h ^ (h >> 31));
  }
};
static_assert(sizeof(SeqSet) == 32, "a sequence set is 32 bytes");

}  // namespace kvattn
