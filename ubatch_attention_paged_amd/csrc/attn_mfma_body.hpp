// Prefill-class attention on the gfx950 matrix cores: the kernel body, a
// device function, so that the combined launch of attn_both.hip can run it
// beside the vector-ALU body.
//
// One workgroup = (work item, KV head): 128 query rows = QT = 128 / G
// queries x the G query heads that share that KV head, 4 wavefronts of 32
// rows.  The item's cells are walked in 64-cell tiles:
//
//  * K and V rows of a tile (that head's 2*D bytes of each cell row) are
//    gathered through the cell list by buffer loads that write LDS directly
//    (16 B per lane, 1 KB per wavefront instruction), one tile ahead, into a
//    double-buffered ring; the cell indices are fetched two tiles ahead.  The
//    rows sit unpadded in LDS: each lane picks which 16 B segment of its row
//    it fetches so that the segment order inside a row is XOR-swizzled by the
//    row index, which keeps the fragment reads free of bank conflicts.  One
//    barrier per tile.
//  * Wavefront w computes S^T[64 cells][its 32 rows] = K Q^T with
//    v_mfma_f32_32x32x16_f16 (A = K rows from LDS, B = its queries, held in
//    registers as F16 and pre-scaled by scale*log2(e)).  The q rows are read
//    once, coalesced (1 KB of contiguous q per wavefront instruction), and
//    reach the operand layout through a swizzled staging pass in the second
//    ring buffer, which the tile loop only fills after its first barrier.
//    The loads that depend on the work item alone (tile ranges, the first
//    cell indices, the query slots) go out together, then q, then the first
//    tile's gather.
//  * Each lane owns one query row (column lane % 32 of the accumulators):
//    mask, online base-2 softmax, then P^T goes straight from the S^T
//    accumulators into the B operand of O^T = V^T P^T -- a lane's 16 scores
//    of a 32-cell block are exactly the 8 + 8 k-values it supplies to the two
//    32x32x16 steps of that block.  The matching A operand (V^T, 8 cells of
//    one d per lane) comes from the row-major V tile through the LDS
//    transpose read, in the same cell order.
//  * The running maximum is only moved (and O rescaled) when a row's tile
//    maximum exceeds it by more than 2^8, so most tiles skip the rescale; the
//    F16 weights then stay below 256.  Row sums use v_dot2 on the same F16
//    weights the PV product consumes; each lane keeps its own share and the
//    two halves of a row are added once at the end.  The row maximum crosses
//    lane halves through v_permlane32_swap, not LDS.
//  * Tiles entirely in the future of every query of the item are never
//    loaded and tiles entirely visible skip the per-element mask, both from
//    per-tile position ranges built at commit.  The tile loop is instanced
//    per class purity: a class with one sequence set that every row belongs
//    to needs the position test only.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace kvattn {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));

KVATTN_DEV float dot2_sum(half2v h, float acc) {
  const half2v one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2, h), __builtin_bit_cast(fp16x2, one), acc, false);
}

// x[l] and x[l ^ 32] side by side in every lane through the VALU lane-half
// swap (no LDS round trip, no wait on LDS reads in flight); lanes l and
// l ^ 32 receive the same pair
KVATTN_DEV float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
KVATTN_DEV float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr float kRescaleSlack = 8.f;   // log2 units the running max may lag the true max

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};
template <int V>
struct IntTag {
  static constexpr int value = V;
};

// The kernel body for work item `items[bx / n_head_kv]`, KV head
// bx % n_head_kv, layer slot il of the launch.  Its LDS (the K / V ring and
// per ring buffer the tile cells' positions and sequence sets) is declared
// here, one static array per role.
// SWA: the sliding-window variant (a.swa > 0); the other compiles without any
// of its tests
template <int D, int G, bool SWA, int RB>
KVATTN_DEV void mfma_body(const AttnArgs& a, const WorkItem* items, int bx, int il) {
  // RB 32-row blocks per wavefront, NW wavefronts of 32 * RB rows
  constexpr int NW = 4 / RB;
  constexpr int QT = kMfmaRowsPerItem / G;        // queries per item
  static_assert(kMfmaRowsPerItem == 128 && NW * RB == 4, "NW wavefronts x RB x 32 rows = 128");
  constexpr int KT = kTileCells;                  // cells per tile (64)
  constexpr int DP = D < 32 ? 32 : D;             // O^T rows, padded to a 32-row block
  // LDS tiles: K rows of D halfs, V rows of DP halfs (columns D.. of a V
  // row are zeros), both unpadded.  One wavefront instruction of the
  // LDS-direct load fills 1 KB = 64 segments of 16 B.
  constexpr int SK = D / 8;                       // 16 B segments per K row
  constexpr int SV = DP / 8;                      // per V row; segments >= SK are zero padding
  constexpr int RK = 64 / SK, RV = 64 / SV;       // rows per instruction
  constexpr int NK = KT / RK, NV = KT / RV;       // instructions per tile
  constexpr int JK = (NK + NW - 1) / NW, JV = (NV + NW - 1) / NW;   // per wavefront
  constexpr bool SAME_ROWS = SK == SV;            // K and V instructions cover the same rows
  // Swizzles, for LDS serving 256 B (64 banks of 4 B) per cycle.  K: a
  // 16 B fragment read serves 16 lanes per cycle, 16 consecutive rows at one
  // segment -> the segment index is XORed with (row / rows-per-256-B), so the
  // 16 rows land in 16 different 16 B bank groups.  V: a transpose read
  // serves 32 lanes per cycle, 4 consecutive rows x two adjacent 32 B pairs
  // -> the segment index is XORed with a multiple of 4 (pairs stay whole)
  // chosen so the 8 (row, pair) reads fill the 8 32 B slots of 256 B; with
  // two pairs per row the row stride alone does that.
  constexpr int RBK = 16 / SK, MK = SK - 1;
  constexpr int VSH = SV >= 16 ? 0 : SV == 8 ? 1 : 2;
  __shared__ __attribute__((aligned(16))) _Float16 Ks[2][KT * D];
  __shared__ __attribute__((aligned(16))) _Float16 Vs[2][KT * DP];
  __shared__ int32_t kpos_s[2][KT];
  __shared__ uint64_t kmask_s[2][kSeqWords][KT];   // word-major: a row reads one word

  const int HK = a.n_head_kv;
  const int H = a.n_head;
  const int E = HK * D;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half_id = lane >> 5;
  const int kvh = bx % HK;
  const WorkItem it = items[bx / HK];
  const bool pure = it.pure;
  // K / V rows are gathered with range-checked buffer loads: 32-bit byte
  // offsets, and an empty slot reads zeros from an out-of-range offset
  const u32x4 krw = buffer_rsrc_words(a.k[il], a.layer_bytes);
  const u32x4 vrw = buffer_rsrc_words(a.v[il], a.layer_bytes);
  const uint32_t row_bytes = static_cast<uint32_t>(E) * 2;
  const uint32_t sbase_bytes = static_cast<uint32_t>(it.stream) * static_cast<uint32_t>(a.kv_size) * row_bytes;

  // The first loads depend on the work item alone and go out together: the
  // per-tile position ranges (trimming), the cell indices of the first two
  // tiles (without a sliding window the walk starts at tile 0) and the slot
  // records of this lane's query rows.  Then the first tile's gather and
  // the q rows.
  const int tb = it.tile_base;
  int ntile = (it.c1 - it.c0 + KT - 1) / KT;
  int last = -1;
  if (a.causal) {
    for (int k = lane; k < ntile; k += 64)
      if (a.tile_min[tb + k] <= it.qpos_max) last = k;
  }

  // loader geometry: instruction j of wavefront wv fills LDS kilobyte
  // t = wv + NW j of the tile; lane -> row t * R + lane / S, stored segment
  // lane % S, which holds the row's segment (lane % S) ^ swizzle(row)
  const int wv = __builtin_amdgcn_readfirstlane(w);
  int rowk[JK], rowv[JV];
  uint32_t colk[JK], colv[JV];     // byte column in the cache row; kOobOffset = zero padding
#pragma unroll
  for (int j = 0; j < JK; ++j) {
    rowk[j] = (wv + NW * j) * RK + lane / SK;
    const int sg = (lane % SK) ^ ((rowk[j] / RBK) & MK);
    colk[j] = static_cast<uint32_t>(kvh * D + sg * 8) * 2;
  }
#pragma unroll
  for (int j = 0; j < JV; ++j) {
    rowv[j] = (wv + NW * j) * RV + lane / SV;
    const int sg = (lane % SV) ^ (((rowv[j] & 3) >> VSH) << 2);
    colv[j] = sg < SK ? static_cast<uint32_t>(kvh * D + sg * 8) * 2 : kOobOffset;
  }
  constexpr int JC = SAME_ROWS ? JK : JK + JV;     // cell indices a lane needs per tile
  int cfirst[JC], cnext[JC];                       // raw list entries; validity is decided at use
  auto has_k = [&](int j) { return NK % NW == 0 || wv + NW * j < NK; };   // wave-uniform
  auto has_v = [&](int j) { return NV % NW == 0 || wv + NW * j < NV; };
  // list entries through a range-checked buffer over [0, c1): an entry past
  // the item's end reads as cell 0, and its row is never gathered (see
  // issue); 32-bit offsets, no clamp, no branch
  const __amdgpu_buffer_rsrc_t cellr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.csr_cell), 0, it.c1 * 4, 0x00020000);
  auto cells_of = [&](int tile, int* cells) {
    const int base = it.c0 + tile * KT;
#pragma unroll
    for (int j = 0; j < JK; ++j)
      cells[j] = has_k(j) ? __builtin_amdgcn_raw_buffer_load_b32(cellr, (base + rowk[j]) * 4, 0, 0) : 0;
    if constexpr (!SAME_ROWS) {
#pragma unroll
      for (int j = 0; j < JV; ++j)
        cells[JK + j] = has_v(j) ? __builtin_amdgcn_raw_buffer_load_b32(cellr, (base + rowv[j]) * 4, 0, 0) : 0;
    }
  };
  if constexpr (!SWA) {
    cells_of(0, cfirst);
    cells_of(1, cnext);
  }

  // this lane's query rows: row block b of wavefront w is rows
  // 32 * (w * RB + b) .. +31, the lane owning row lane % 32 of it
  int t_r[RB], h_r[RB], pos_lim[RB], pos_lo[RB], qword[RB], qbit[RB];
  bool qvalid[RB];
  SlotInfo si[RB];
  bool any_row = false;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int r = 32 * (w * RB + b) + (lane & 31);
    const int hg = r / QT;
    t_r[b] = r % QT;
    qvalid[b] = t_r[b] < it.n_q;
    si[b] = a.qslots[it.q_off + (qvalid[b] ? t_r[b] : 0)];
    h_r[b] = kvh * G + hg;
  }

  // tiles of this item; trailing tiles in the future of every query are
  // dropped, and with a sliding window leading tiles behind every query's
  // window (tiles are walked from t0)
  if (a.causal) ntile = wave_max_i(last) + 1;
  const int win_lo = SWA ? it.qpos_min - a.swa + 1 : INT32_MIN;   // no query sees below this
  int t0 = 0;
  if constexpr (SWA) {
    int first = ntile;
    for (int k = lane; k < ntile; k += 64)
      if (a.tile_max[tb + k] >= win_lo) first = min(first, k);
    t0 = wave_min_i(first);
    cells_of(t0, cfirst);
    cells_of(t0 + 1, cnext);
  }

  // Everything a tile needs from memory is requested one tile (cell
  // indices: two tiles) ahead and first read after the vmcnt(0) that opens
  // that tile, so no wait inside a tile's compute covers the loads in flight
  // (vmcnt retires in order: any wait would also wait for the next tile).
  int pk = INT32_MAX, nmin = 0, nmax = 0;
  SeqSet mk = SeqSet::none();
  auto issue = [&](int tile, int bsel, const int* cells) {
    const int lim = it.c1 - (it.c0 + tile * KT);     // rows of this tile inside the list
    // a whole tile inside the list (wave-uniform) needs no per-row test;
    // V rows need the padding test only below head size 32
    const bool whole = lim >= KT;
#pragma unroll
    for (int j = 0; j < JK; ++j)
      if (has_k(j)) {
        const uint32_t at = sbase_bytes + static_cast<uint32_t>(cells[j]) * row_bytes + colk[j];
        buffer_load16_lds(krw, lds_addr(&Ks[bsel][(wv + NW * j) * 512]), whole || rowk[j] < lim ? at : kOobOffset);
      }
#pragma unroll
    for (int j = 0; j < JV; ++j)
      if (has_v(j)) {
        const int cl = SAME_ROWS ? cells[j] : cells[JK + j];
        const uint32_t at = sbase_bytes + static_cast<uint32_t>(cl) * row_bytes + colv[j];
        const bool pad = SV != SK && colv[j] == kOobOffset;
        buffer_load16_lds(vrw, lds_addr(&Vs[bsel][(wv + NW * j) * 512]),
                          !pad && (whole || rowv[j] < lim) ? at : kOobOffset);
      }
    if (tid < KT) {
      const int idx = it.c0 + tile * KT + tid;
      const bool in = idx < it.c1;
      pk = in ? a.csr_pos[idx] : INT32_MAX;
      mk = in ? a.csr_mask[idx] : SeqSet::none();
    }
    nmin = a.tile_min[tb + tile];
    nmax = a.tile_max[tb + tile];
  };
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    pos_lim[b] = a.causal ? si[b].pos : INT32_MAX - 1;     // largest visible cell position
    pos_lo[b] = SWA ? si[b].pos - a.swa + 1 : INT32_MIN;   // smallest, with a sliding window
    qword[b] = si[b].seq0 >> 6;
    qbit[b] = si[b].seq0 & 63;
    any_row |= qvalid[b];
  }
  const bool wave_rows = ballot(any_row) != 0ULL;   // wave-uniform: padding-only waves skip the math

  // B operand of S^T = K Q^T: q[row][16*ks + 8*half + 0..7], scaled, F16.
  // Loaded coalesced -- each wavefront instruction reads 1 KB of contiguous
  // q (whole rows of D numbers: LPR lanes per row) -- converted, written to
  // this wavefront's 32 rows of a staging area, and read back in the
  // operand layout.  The staging area is ring buffer 1 (K half for waves 0
  // and 1, V half for waves 2 and 3), unused until the tile loop's first
  // barrier; each wavefront reads only the rows it wrote, so no barrier is
  // needed here.  16 B segments are XOR-swizzled by row for the reads.
  static_assert(RB == 1, "q staging assumes one 32-row block per wavefront");
  half8 qb[RB][D / 16];
  {
    constexpr int LPR = D / 4;                     // lanes per row (16 B each)
    constexpr int RPI = 64 / LPR;                  // rows per instruction
    constexpr int SEG = D / 8;                     // 16 B segments per F16 row
    _Float16* stg = (w < 2 ? &Ks[1][0] : &Vs[1][0]) + (w & 1) * 32 * D;
    constexpr int NJ = 32 / RPI;                   // instructions per wavefront
    const int p = lane % LPR;                      // this lane's 4 numbers: d = 4p .. 4p+3
    // every load is issued before any is used: addresses first (a row past
    // the item's queries reads its first row instead and is zeroed after)
    const float* src[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int rr = j * RPI + lane / LPR;         // row of the wavefront's 32
      const int r = 32 * w + rr;
      int qrow = 0;                                // lane rr holds row rr's slot
#pragma unroll
      for (int k = 0; k < RPI; ++k) {
        const int v = __builtin_amdgcn_readlane(si[0].q_row, j * RPI + k);
        qrow = lane / LPR == k ? v : qrow;
      }
      src[j] = a.q[il] + static_cast<int64_t>(qrow) * H * D + (kvh * G + r / QT) * D + 4 * p;
    }
    // q rows are read once per launch: non-temporal loads keep them from
    // displacing K/V tiles that the other items of this KV head re-read from
    // L2 (measured +1-2% on prompts; non-temporal O stores, by contrast,
    // lose 9%: the partial-line writes then miss the L2's write merging)
    typedef float f4v __attribute__((ext_vector_type(4)));
    float4 xs[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(src[j]));
      xs[j] = make_float4(t[0], t[1], t[2], t[3]);
    }
    // the first tile's gather goes out behind the q loads: waiting for q
    // (in-order completion) then leaves the gather in flight
    if (ntile > t0) issue(t0, 0, cfirst);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int rr = j * RPI + lane / LPR;
      const bool ok = (32 * w + rr) % QT < it.n_q;
      const float4 x = ok ? xs[j] : make_float4(0, 0, 0, 0);
      half4 h4;
      h4[0] = static_cast<_Float16>(x.x * a.scale_log2e);
      h4[1] = static_cast<_Float16>(x.y * a.scale_log2e);
      h4[2] = static_cast<_Float16>(x.z * a.scale_log2e);
      h4[3] = static_cast<_Float16>(x.w * a.scale_log2e);
      const int sgw = (p >> 1) ^ (rr & (SEG - 1));
      *reinterpret_cast<half4*>(stg + rr * D + sgw * 8 + (p & 1) * 4) = h4;
    }
    const int rl = lane & 31;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int sgr = (2 * ks + half_id) ^ (rl & (SEG - 1));
      qb[0][ks] = *reinterpret_cast<const half8*>(stg + rl * D + sgr * 8);
    }
  }

  floatx16 oacc[RB][DP / 32];
  // l_run: this lane's share of each row's sum (its 16 cells of every
  // 32-cell block); lanes l and l ^ 32 always hold the same running maximum,
  // so the two shares are rescaled alike and added once at the end
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    m_run[b] = -INFINITY;
    l_run[b] = 0.f;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[b][db][i] = 0.f;
  }

  const int s16 = lane & 15;
  const int dsub = 16 * ((lane >> 4) & 1);
  // read-side swizzles: row bits below the 32-row block (K) or 4-row group (V)
  const int kswz = ((lane & 31) / RBK) & MK;
  const int vswz = (((s16 >> 2) & 3) >> VSH) << 2;
  // The tile loop exists twice: for a pure class (one sequence set that
  // every row belongs to) visibility is the position test alone, otherwise
  // each cell's set membership is tested too.  Purity is per work item, so
  // the branch is taken once, outside the loop.
  // The walk is unrolled by two tiles so that the ring buffer of each tile
  // is a compile-time constant: every LDS address is then a loop-invariant
  // per-lane offset plus an immediate, with no address arithmetic per tile.
  auto tile_loop = [&](auto pure_tag) {
  constexpr bool PURE = decltype(pure_tag)::value;
  auto tile = [&](const int i, auto buf_tag) {
    constexpr int buf = decltype(buf_tag)::value;
    // stage tile i: its rows arrived by the LDS-direct loads this thread
    // issued (vmcnt), positions and masks go through registers
    if (tid < KT) {
      kpos_s[buf][tid] = pk;
      if constexpr (!PURE) {
#pragma unroll
        for (int wd = 0; wd < kSeqWords; ++wd) kmask_s[buf][wd][tid] = mk.w[wd];
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    __syncthreads();
    const int tmin = __builtin_amdgcn_readfirstlane(nmin), tmax = __builtin_amdgcn_readfirstlane(nmax);
    // tile i+1 loads and tile i+2 cell indices fly while tile i computes;
    // buffer buf ^ 1 was last read in tile i-1, which every wave has left
    if (i + 1 < ntile) {
      issue(i + 1, buf ^ 1, cnext);
      if (i + 2 < ntile) cells_of(i + 2, cnext);
    }
    if (!wave_rows) return;

    const int nk = min(KT, it.c1 - (it.c0 + i * KT));
    if (a.causal && tmin > it.qpos_max) return;
    if (SWA && tmax < win_lo) return;
    const bool full = nk == KT && PURE && (!a.causal || tmax <= it.qpos_min) &&
                      (!SWA || tmin >= it.qpos_max - a.swa + 1);

    // The tile is two 32-cell blocks, each with its own online-softmax step
    // per row block.  Every K or V fragment read from LDS feeds the RB row
    // blocks' MFMAs.  Source order interleaves matrix and vector work: S(1)
    // is issued beside the exponentials of block 0, PV(0) beside the mask
    // and maximum of block 1.  PV(0) is accumulated before block 1's step may
    // rescale O: its weights are relative to the maximum in force before.
    auto s_block = [&](int kb, floatx16 (&acc)[RB]) {
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const half8 ka = *reinterpret_cast<const half8*>(
            &Ks[buf][(kb * 32 + (lane & 31)) * D + 8 * ((2 * ks + half_id) ^ kswz)]);
#pragma unroll
        for (int b = 0; b < RB; ++b) acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qb[b][ks], acc[b], 0, 0, 0);
      }
    };
    // mask + running-max update of one block of row block b; returns the
    // offset to subtract
    auto max_block = [&](int b, int kb, floatx16& sb) {
      if (!full) {
        // branch-free: cells past the list end hold position INT32_MAX and an
        // empty sequence set, so either test removes them
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb * 32 + acc_row(e, lane);
          const int kp = kpos_s[buf][key];
          bool vis = kp <= pos_lim[b];
          if constexpr (!PURE) vis &= static_cast<bool>((kmask_s[buf][qword[b]][key] >> qbit[b]) & 1ULL);
          if constexpr (SWA) vis &= kp >= pos_lo[b];
          sb[e] = vis ? sb[e] : -INFINITY;
        }
      }
      // lane l ^ 32 holds the other 16 cells of the block for the same row
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sb[e]);
      mx = max_halves(mx);
      const bool grow = mx > m_run[b] + kRescaleSlack;     // false while the row sees nothing
      if (ballot(grow)) {
        const float m_new = grow ? mx : m_run[b];
        const float alpha = m_run[b] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[b] - m_new);
        l_run[b] *= alpha;
#pragma unroll
        for (int db = 0; db < DP / 32; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[b][db][e] *= alpha;
        m_run[b] = m_new;
      }
      return m_run[b] == -INFINITY ? 0.f : m_run[b];
    };
    // F16 weights of one block (B operand of the PV product) and their sum
    auto weights = [&](int b, const floatx16& sb, float m_use, half8 (&pb)[2]) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        half2v ph;
        ph[0] = static_cast<_Float16>(__builtin_amdgcn_exp2f(sb[e] - m_use));
        ph[1] = static_cast<_Float16>(__builtin_amdgcn_exp2f(sb[e + 1] - m_use));
        l_run[b] = dot2_sum(ph, l_run[b]);     // the row sum sees the F16 weights the PV product sees
        pb[e >> 3][e & 7] = ph[0];
        pb[e >> 3][(e & 7) + 1] = ph[1];
      }
    };
    // O^T += V^T P^T: source lane s of each 16-lane group points at cell row
    // key0 + s/4, column dsub + 4*(s%4); lane gets cells key0..key0+3 of
    // column db*32 + lane%32 (and key0+8.. for the upper four k-values).
    // That column sits in segment (dsub + 32 db) / 8 + (s%4) / 2 of the row,
    // stored at that index XOR the row's pair swizzle.
    auto pv_block = [&](int kb, const half8 (&pb)[RB][2]) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int key0 = kb * 32 + 16 * st + 4 * half_id;
        const _Float16* vb = &Vs[buf][(key0 + (s16 >> 2)) * DP + 4 * (s16 & 1)];
#pragma unroll
        for (int db = 0; db < DP / 32; ++db) {
          const int sg = (((dsub + 32 * db) >> 3) + ((s16 & 3) >> 1)) ^ vswz;
          const half4 lo = lds_read_tr16(vb + 8 * sg);
          const half4 hi = lds_read_tr16(vb + 8 * sg + 8 * DP);
          const half8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int b = 0; b < RB; ++b)
            oacc[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[b][st], oacc[b][db], 0, 0, 0);
        }
      }
    };
    floatx16 s0[RB], s1[RB];
    float mu[RB];
    half8 p0[RB][2], p1[RB][2];
    s_block(0, s0);
#pragma unroll
    for (int b = 0; b < RB; ++b) mu[b] = max_block(b, 0, s0[b]);
    s_block(1, s1);
#pragma unroll
    for (int b = 0; b < RB; ++b) weights(b, s0[b], mu[b], p0[b]);
    pv_block(0, p0);
#pragma unroll
    for (int b = 0; b < RB; ++b) mu[b] = max_block(b, 1, s1[b]);
#pragma unroll
    for (int b = 0; b < RB; ++b) weights(b, s1[b], mu[b], p1[b]);
    pv_block(1, p1);
  };
  // tile t0 + 2k sits in buffer 0, t0 + 2k + 1 in buffer 1
  for (int i = t0; i < ntile; i += 2) {
    tile(i, IntTag<0>{});
    if (i + 1 < ntile) tile(i + 1, IntTag<1>{});
  }
  };
  if (pure)
    tile_loop(BoolTag<true>{});
  else
    tile_loop(BoolTag<false>{});

#pragma unroll
  for (int b = 0; b < RB; ++b) l_run[b] = sum_halves(l_run[b]);
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if (!qvalid[b]) continue;
    if (it.prow < 0) {
      const float inv = l_run[b] > 0.f ? 1.f / l_run[b] : 0.f;
      float* op = a.o[il] + static_cast<int64_t>(si[b].out_row) * H * D + h_r[b] * D;
#pragma unroll
      for (int db = 0; db < DP / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + acc_row(4 * g4, lane);
          if (d < D)
            *reinterpret_cast<float4*>(op + d) =
                make_float4(oacc[b][db][4 * g4] * inv, oacc[b][db][4 * g4 + 1] * inv, oacc[b][db][4 * g4 + 2] * inv,
                            oacc[b][db][4 * g4 + 3] * inv);
        }
    } else {
      const int64_t row = static_cast<int64_t>(il) * a.rows_per_layer + it.prow + t_r[b];
      float* pp = a.part_acc + row * H * D + h_r[b] * D;
#pragma unroll
      for (int db = 0; db < DP / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + acc_row(4 * g4, lane);
          if (d < D)
            *reinterpret_cast<float4*>(pp + d) = make_float4(oacc[b][db][4 * g4], oacc[b][db][4 * g4 + 1],
                                                             oacc[b][db][4 * g4 + 2], oacc[b][db][4 * g4 + 3]);
        }
      if (half_id == 0) {
        a.part_ml[(row * H + h_r[b]) * 2] = m_run[b];
        a.part_ml[(row * H + h_r[b]) * 2 + 1] = l_run[b];
      }
    }
  }
}

}  // namespace kvattn
