// Host half of the library: batch intake, the batch -> ubatch split, cell
// placement, the committed cell table and the per-ubatch work plan.  No HIP
// here -- this compiles with any C++17 compiler and runs without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "kvattn.h"
#include "plan.hpp"

namespace kvattn {

struct Geometry {
  int32_t n_layer = 0, n_head = 0, n_head_kv = 0, head_dim = 0;
  int32_t kv_size = 0, n_stream = 1, n_seq_max = 1;
  int32_t n_batch = 0, n_ubatch = 0;    // clamped
  int32_t causal = 1;
  float kq_scale = 0.f;
  int32_t attend_layers = 1;            // layers per attend call (work-item sizing hint)
  int32_t split_mode = 0;               // KVATTN_SPLIT_SIMPLE / _EQUAL / _SEQ (AUTO resolved)
  int32_t swa = 0;                      // sliding window in positions, 0 = none
  int32_t E() const { return n_head_kv * head_dim; }
  int32_t G() const { return n_head / n_head_kv; }
};

// Validate params and fill Geometry (clamps of "llama.cpp and the ubatch",
// "Three things called batch").  Returns KVATTN_OK or KVATTN_EINVAL + err.
int make_geometry(const kvattn_params& p, Geometry& g, std::string& err);

struct UbatchRec {
  int32_t id = 0;
  int32_t n_seq_tokens = 0, n_seqs = 0;
  std::vector<int32_t> src, pos, n_seq_id, stream, cells, seq_unq;
  std::vector<SeqSet> setmask;        // ids of the slot that live in its own stream (its cell's set)
  // separate copies: a slot whose ids span several streams also gets a cell
  // in each other stream, holding the ids that live there
  std::vector<int32_t> copy_src, copy_stream, copy_cell;   // copy_src = slot index in this ubatch
  std::vector<SeqSet> copy_mask;
  std::vector<const int32_t*> seq_ptr;
  std::vector<int8_t> output;
  int32_t n_outputs = 0;
  bool committed = false;
};

struct Plan {
  int32_t n_kv = 0;
  int32_t n_seg = 0;                  // counting segments per stream (n_kv / 64, rounded up)
  int32_t total_cells = 0;            // csr entries
  int32_t total_tiles = 0;            // 64-cell tiles over all classes
  int32_t max_class_tiles = 0;
  int32_t n_partial_rows = 0;
  int32_t class_cap = 0;              // the class cap the plan was built with
  std::vector<SlotInfo> slots;
  std::vector<ClassInfo> classes;
  std::vector<LookupEntry> lookup;
  std::vector<int32_t> lookup_off;    // [n_stream + 1]
  std::vector<int32_t> qlist;
  std::vector<WorkItem> items_valu, items_mfma;
  std::vector<int32_t> red_slot, red_off, red_rows;
};

class HostCore {
 public:
  int init(const kvattn_params& p, std::string& err);
  const Geometry& geo() const { return g_; }

  // Split + reserve.  On success the ubatches are in ubatches().
  int split(const kvattn_batch& b, int32_t* output_ids, std::string& err);
  std::vector<UbatchRec>& ubatches() { return ubs_; }
  int32_t split_serial() const { return serial_; }

  // Resolve a public ubatch handle to an index of the current split (-1 = stale).
  int find(int32_t id) const;

  // Commit ubatch k: cells become visible.  Appends the device-mirror
  // updates (this ubatch's cells plus anything seq_rm changed) to *upd.
  int commit(int k, std::vector<CellUpdate>* upd, std::string& err);
  int latest_committed() const { return latest_; }

  // Work plan of ubatch k over the current table, with at most max_classes
  // classes; with shrink, fewer when the split-K partial rows would not fit
  // otherwise (plan.class_cap records the cap used).
  int build_plan(int k, bool only_outputs, int32_t max_classes, bool shrink, Plan& plan, std::string& err) const;

  int seq_rm(int32_t seq, int32_t p0, int32_t p1);
  // Committed cells holding seq (all in stream seq % n_stream), ordered by
  // (position, cell).  Returns the stream, or -1 for a bad id.
  int seq_cells(int32_t seq, std::vector<int32_t>& cells, std::vector<int32_t>& pos) const;
  // Replace seq's cells by n new ones at positions pos[], lowest free rank
  // first, committed at once.  KVATTN_NO_SLOT (nothing changed) when the
  // stream's free cells plus the cells only seq holds are fewer than n.
  int seq_restore(int32_t seq, const int32_t* pos, int32_t n, std::vector<int32_t>& cells, std::string& err);
  int32_t seq_pos_max(int32_t seq) const;
  int32_t n_kv() const;
  // mask: kSeqWords words per cell (the set's bits, id q in word q / 64, bit q % 64)
  void get_cells(int32_t s, int32_t* pos, uint64_t* mask) const;

  // limits used by the planner (bounded by the workspace)
  int32_t prow_max = 4096;            // split-K partial rows

 private:
  struct Stream {
    std::vector<int32_t> pos;         // -1 empty
    std::vector<SeqSet> mask;
    std::vector<int32_t> rank_of, cell_at;
    std::vector<uint8_t> avail;       // by rank: free and not reserved
    int32_t hint = 0, n_avail = 0, umax = 0;   // umax = used_max_p1
    std::unordered_map<SeqSet, int32_t, SeqSetHash> count;   // committed cells per set
    // per sequence: which cells hold it (bit j of the bitmap = cell j; the
    // bitmap is allocated on the sequence's first cell in this stream) and
    // how many, so that per-sequence queries visit that sequence's cells only
    std::vector<std::vector<uint64_t>> seq_bits;
    std::vector<int32_t> seq_n;
  };
  // calls f(cell) for each cell of stream s that holds seq, ascending; f may
  // change the cell table
  template <class F>
  void for_seq_cells(int s, int32_t seq, F&& f) const;
  int32_t pop_cell(int s);
  void push_cell(int s, int32_t cell);
  void release_uncommitted();
  void set_cell(int s, int32_t cell, int32_t pos, const SeqSet& mask);

  Geometry g_;
  std::vector<Stream> st_;
  std::vector<UbatchRec> ubs_;
  std::vector<int32_t> seq_flat_;
  std::vector<int32_t> pending_;      // cells (stream * kv_size + cell) changed since the last upload
  int32_t serial_ = 0, next_id_ = 1;
  int latest_ = -1;
};

}  // namespace kvattn
