// Plain-old-data records shared by the host planner and the gfx950 kernels.
//
// A committed ubatch is turned into a "plan": its query slots, the classes of
// cells its queries may see, and the work items the attention kernels run.
// A class is a set of committed cells of one stream whose sequence sets are
// equal (or, past a cap, a merged group of such sets); every query whose
// first sequence id lies in the class's set attends over the class's cells,
// subject to the causal test -- the mask of "llama.cpp and the ubatch", "The
// mask is doing the work", kept in sparse form.  Cells of one class are
// listed in ascending cell index by the GPU (csr_* kernels).
#pragma once

#include <cstdint>

#include "seqset.hpp"

namespace kvattn {

constexpr int kMaxLayersPerLaunch = 32;
constexpr int kMaxClasses = 1024;      // per ubatch; extra sequence sets are merged
constexpr int kSegCells = 64;          // cells per counting segment (one wavefront)
constexpr int kTileCells = 64;         // cells per attention tile; chunk starts are multiples of it
constexpr int kSmallCommitCells = 4096;   // commits of at most this many (stream, cell) pairs below n_kv
constexpr int kSmallCommitClasses = 64;   // and this many classes (and lookup entries)
constexpr int kSmallCommitStreams = 64;   // and streams run in one workgroup beside the stores
constexpr int kValuMaxQueries = 2;     // classes with more queries go to the MFMA kernel
constexpr int kMfmaRowBlocks = 1;      // 32-row blocks per wavefront of the matrix-core kernel
constexpr int kMfmaRowsPerItem = 128;  // query rows (queries x heads of one KV head) per item
// Workgroups a split-K launch should reach before its items are cut finer
// (256 CUs; the vector-ALU kernel keeps 5 workgroups per CU, the
// matrix-core kernel 2).  Measured on decode steps: long items win over a
// short tail -- each cut adds a partial row, merge work and per-item fixed
// costs (query load, pipeline ramp) -- so the targets sit near one round of
// resident workgroups or below.
constexpr int kValuTargetWorkgroups = 1024;
constexpr int kMfmaTargetWorkgroups = 320;
// Prompt-sized matrix-core classes (more than 64 query rows per KV head) are
// cut only below this many workgroups per launch -- in practice when a
// launch covers one layer, or a few short prompt chunks -- and never into
// pieces under 256 cells.  Measured: 256 beats 512 and 1024 (one-layer
// prefill calls 1-2% faster, mixed prompt-chunk ubatches 3-4% faster: fewer
// partial rows to merge), while 128 leaves one-layer calls 25% slower.
constexpr int kMfmaHighTargetWorkgroups = 256;
// Decode chunks never shrink below 256 cells: measured on one-layer decode
// launches, 64-cell chunks (4x the workgroups) ran slower than 256 (more
// partial rows to merge, more per-item ramp).
constexpr int kValuMinChunk = 256;

struct SlotInfo {        // one query slot
  int32_t stream;
  int32_t pos;
  int32_t seq0;          // first sequence id: the one the query masks with
  int32_t q_row;         // row of q (ubatch order)
  int32_t out_row;       // row of the output (ubatch row, or rank among outputs)
  int32_t pad[3];
};

struct CellUpdate {      // one cell of the device mirror to overwrite
  SeqSet mask;           // sequence set
  int32_t idx;           // stream * kv_size + cell
  int32_t pos;           // -1 = empty
  int32_t pad[2];
};

struct LookupEntry {     // sorted by (stream, mask); maps a cell's set to its class
  SeqSet mask;
  int32_t cls;
  int32_t pad[3];
};

struct ClassInfo {
  SeqSet mask;           // OR of the member sets
  int32_t stream;
  int32_t n_cells;
  int32_t cell_off;      // first entry in the csr arrays
  int32_t q_off;         // first entry in qlist
  int32_t n_q;
  int32_t pure;          // 1: one sequence set, which every listed query belongs to
  int32_t tile_base;     // first entry of this class in the per-64-cell tile tables
  int32_t pad;
};

struct WorkItem {        // one workgroup (per KV head for the MFMA kernel)
  int32_t cls;
  int32_t q_off;         // queries qslots[q_off .. q_off + n_q)
  int32_t n_q;
  int32_t c0, c1;        // csr range [c0, c1)
  int32_t prow;          // first partial row, -1 = write the output directly
  int32_t qpos_min, qpos_max;
  // copies of the class's fields, so a workgroup's first loads depend on
  // the item alone
  int32_t tile_base;     // the class's first entry in the per-tile tables
  int32_t stream;
  int32_t pure;
  int32_t pad;
};

// Byte offsets of each plan array inside the device plan arena.
struct PlanLayout {
  int64_t slots, classes, lookup, lookup_off, qslots, items_valu, items_mfma;
  int64_t red_slot, red_off, red_rows, updates;
  int64_t total;
};

}  // namespace kvattn
