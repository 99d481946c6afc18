// Host half of the library (see host_core.hpp).
#include "host_core.hpp"

#include <algorithm>
#include <cmath>
#include <numeric>

namespace kvattn {

namespace {

inline int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }
inline int32_t round_up(int64_t a, int64_t b) { return static_cast<int32_t>(ceil_div(a, b) * b); }
constexpr int32_t kNkvQuantum = 256;   // n_pad floor of get_n_kv

}  // namespace

int make_geometry(const kvattn_params& p, Geometry& g, std::string& err) {
  if (p.n_layer <= 0 || p.n_head <= 0 || p.n_head_kv <= 0 || p.head_dim <= 0) {
    err = "n_layer, n_head, n_head_kv and head_dim must be positive";
    return KVATTN_EINVAL;
  }
  if (p.n_head % p.n_head_kv != 0) {
    err = "n_head must be a multiple of n_head_kv";
    return KVATTN_EINVAL;
  }
  const int G = p.n_head / p.n_head_kv;
  if (!(p.head_dim == 16 || p.head_dim == 32 || p.head_dim == 64 || p.head_dim == 128)) {
    err = "head_dim must be 16, 32, 64 or 128";
    return KVATTN_EINVAL;
  }
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) {
    err = "n_head / n_head_kv must be 1, 2, 4 or 8";
    return KVATTN_EINVAL;
  }
  if (p.kv_size <= 0 || p.n_stream <= 0 || p.n_seq_max <= 0 || p.n_seq_max > kMaxSeq) {
    err = "kv_size and n_stream must be positive and 0 < n_seq_max <= " + std::to_string(kMaxSeq);
    return KVATTN_EINVAL;
  }
  if (static_cast<int64_t>(p.kv_size) * p.n_stream > (1LL << 30)) {
    err = "kv_size * n_stream too large";
    return KVATTN_EINVAL;
  }
  // the kernels address a layer's K or V tensor with 32-bit byte offsets
  if (static_cast<int64_t>(p.kv_size) * p.n_stream * p.n_head_kv * p.head_dim * 2 >= (1LL << 31)) {
    err = "one layer's K (or V) tensor must stay below 2 GiB";
    return KVATTN_EINVAL;
  }
  if (p.n_ubatch < 0) {
    err = "n_ubatch must be >= 0";
    return KVATTN_EINVAL;
  }
  g.n_layer = p.n_layer; g.n_head = p.n_head; g.n_head_kv = p.n_head_kv; g.head_dim = p.head_dim;
  g.kv_size = p.kv_size; g.n_stream = p.n_stream; g.n_seq_max = p.n_seq_max;
  g.causal = p.causal ? 1 : 0;
  // "llama.cpp and the ubatch", "Three things called batch": under causal
  // attention n_batch is capped at the context size; n_ubatch defaults to
  // n_batch and never exceeds it.
  const int32_t n_ctx = p.kv_size * p.n_stream;
  const int32_t nb_in = p.n_batch <= 0 ? 2048 : p.n_batch;
  g.n_batch = g.causal ? std::min(n_ctx, nb_in) : nb_in;
  g.n_ubatch = std::min(g.n_batch, p.n_ubatch == 0 ? nb_in : p.n_ubatch);
  g.kq_scale = p.kq_scale != 0.f ? p.kq_scale : 1.0f / std::sqrt(static_cast<float>(p.head_dim));
  g.attend_layers = std::max(1, std::min(p.attend_layers, p.n_layer));
  if (p.swa_window < 0) {
    err = "swa_window must be >= 0";
    return KVATTN_EINVAL;
  }
  g.swa = p.swa_window;
  if (p.split_mode < KVATTN_SPLIT_AUTO || p.split_mode > KVATTN_SPLIT_SEQ) {
    err = "split_mode must be one of KVATTN_SPLIT_AUTO, _SIMPLE, _EQUAL, _SEQ";
    return KVATTN_EINVAL;
  }
  // AUTO: the init_batch choice ("Batch、Ubatch 与解码主循环", Part C)
  g.split_mode = p.split_mode != KVATTN_SPLIT_AUTO ? p.split_mode
                 : (p.n_stream == 1 ? KVATTN_SPLIT_SIMPLE : KVATTN_SPLIT_EQUAL);
  return KVATTN_OK;
}

int HostCore::init(const kvattn_params& p, std::string& err) {
  int rc = make_geometry(p, g_, err);
  if (rc) return rc;
  st_.assign(g_.n_stream, Stream());
  for (int s = 0; s < g_.n_stream; ++s) {
    Stream& S = st_[s];
    S.pos.assign(g_.kv_size, -1);
    S.mask.assign(g_.kv_size, SeqSet::none());
    S.rank_of.assign(g_.kv_size, -1);
    S.cell_at.assign(g_.kv_size, 0);
    S.avail.assign(g_.kv_size, 1);
    S.seq_bits.assign(g_.n_seq_max, {});
    S.seq_n.assign(g_.n_seq_max, 0);
    for (int32_t r = 0; r < g_.kv_size; ++r) {
      const int32_t c = p.cell_order ? p.cell_order[static_cast<int64_t>(s) * g_.kv_size + r] : r;
      if (c < 0 || c >= g_.kv_size || S.rank_of[c] != -1) {
        err = "cell_order row " + std::to_string(s) + " is not a permutation of 0..kv_size-1";
        return KVATTN_EINVAL;
      }
      S.rank_of[c] = r;
      S.cell_at[r] = c;
    }
    S.n_avail = g_.kv_size;
  }
  return KVATTN_OK;
}

int32_t HostCore::pop_cell(int s) {
  Stream& S = st_[s];
  while (!S.avail[S.hint]) ++S.hint;
  S.avail[S.hint] = 0;
  --S.n_avail;
  return S.cell_at[S.hint];
}

void HostCore::push_cell(int s, int32_t cell) {
  Stream& S = st_[s];
  const int32_t r = S.rank_of[cell];
  if (!S.avail[r]) {
    S.avail[r] = 1;
    ++S.n_avail;
    S.hint = std::min(S.hint, r);
  }
}

void HostCore::release_uncommitted() {
  for (auto& u : ubs_)
    if (!u.committed) {
      for (size_t i = 0; i < u.cells.size(); ++i) push_cell(u.stream[i], u.cells[i]);
      for (size_t i = 0; i < u.copy_cell.size(); ++i) push_cell(u.copy_stream[i], u.copy_cell[i]);
    }
}

int HostCore::find(int32_t id) const {
  for (size_t k = 0; k < ubs_.size(); ++k)
    if (ubs_[k].id == id) return static_cast<int>(k);
  return -1;
}

// ---- batch intake and split ---------------------------------------------

int HostCore::split(const kvattn_batch& b, int32_t* output_ids, std::string& err) {
  release_uncommitted();
  ubs_.clear();
  latest_ = -1;
  ++serial_;
  const int32_t n = b.n_tokens;
  if (n < 0 || n > g_.n_batch) {
    // "llama.cpp and the ubatch", "Three things called batch": more slots than
    // n_batch is refused.
    err = "n_tokens " + std::to_string(n) + " outside [0, n_batch=" + std::to_string(g_.n_batch) + "]";
    return KVATTN_EINVAL;
  }
  // -- sequence ids: first listed id first, the rest ascending, duplicates dropped
  std::vector<int32_t> beg(n + 1, 0);
  std::vector<SeqSet> setmask(n, SeqSet::none());
  seq_flat_.clear();
  for (int32_t i = 0; i < n; ++i) {
    beg[i] = static_cast<int32_t>(seq_flat_.size());
    if (!b.seq_id) {
      seq_flat_.push_back(0);
      setmask[i] = SeqSet::one(0);
    } else {
      const int32_t k = b.n_seq_id ? b.n_seq_id[i] : 1;
      if (k < 1 || !b.seq_id[i]) {
        err = "slot " + std::to_string(i) + ": needs at least one sequence id";
        return KVATTN_EINVAL;
      }
      SeqSet m = SeqSet::none();
      for (int32_t t = 0; t < k; ++t) {
        const int32_t s = b.seq_id[i][t];
        if (s < 0 || s >= g_.n_seq_max) {
          err = "slot " + std::to_string(i) + ": sequence id " + std::to_string(s) + " outside [0, n_seq_max)";
          return KVATTN_EINVAL;
        }
        m.set(s);
      }
      const int32_t first = b.seq_id[i][0];
      seq_flat_.push_back(first);
      for (int q = m.lowest(); q >= 0; q = m.next(q))
        if (q != first) seq_flat_.push_back(q);
      setmask[i] = m;
    }
  }
  beg[n] = static_cast<int32_t>(seq_flat_.size());
  auto seq0 = [&](int32_t i) { return seq_flat_[beg[i]]; };

  // -- positions: given, or continued per first sequence id
  std::vector<int32_t> pos(n);
  if (b.pos) {
    for (int32_t i = 0; i < n; ++i) {
      if (b.pos[i] < 0) {
        err = "slot " + std::to_string(i) + ": negative position";
        return KVATTN_EINVAL;
      }
      pos[i] = b.pos[i];
    }
  } else if (n > 0) {
    std::vector<int32_t> next(g_.n_seq_max, -1);   // -1: not looked up yet
    for (int32_t i = 0; i < n; ++i) {
      int32_t& nx = next[seq0(i)];
      if (nx < 0) nx = seq_pos_max(seq0(i)) + 1;
      pos[i] = nx++;
    }
  }
  std::vector<int8_t> out(n, 0);
  if (b.output) {
    for (int32_t i = 0; i < n; ++i) out[i] = b.output[i] ? 1 : 0;
  } else if (n > 0) {
    out[n - 1] = 1;
  }

  // -- split ("Batch、Ubatch 与解码主循环", Part C): the strategy resolved at
  // create (by default split_simple for one stream, split_equal(n_ubatch,
  // true) for several)
  struct Part { std::vector<int32_t> slots; int32_t nst, ns; };
  std::vector<Part> parts;
  const int32_t U = g_.n_ubatch;
  if (g_.split_mode == KVATTN_SPLIT_SEQ) {
    // split_seq: the set of the first unused slot; its unused slots in
    // submission order, at most U of them; sets are never mixed
    std::vector<uint8_t> used(n, 0);
    int32_t first = 0;
    while (true) {
      while (first < n && used[first]) ++first;
      if (first == n) break;
      const SeqSet set = setmask[first];
      Part p;
      for (int32_t i = first; i < n && static_cast<int32_t>(p.slots.size()) < U; ++i)
        if (!used[i] && setmask[i] == set) {
          used[i] = 1;
          p.slots.push_back(i);
        }
      p.nst = static_cast<int32_t>(p.slots.size());
      p.ns = 1;
      parts.push_back(std::move(p));
    }
  } else if (g_.split_mode == KVATTN_SPLIT_SIMPLE) {
    // split_simple: next U slots in submission order, sequence ids ignored
    for (int32_t a = 0; a < n; a += U) {
      Part p;
      for (int32_t i = a; i < std::min(n, a + U); ++i) p.slots.push_back(i);
      p.nst = static_cast<int32_t>(p.slots.size());
      p.ns = 1;
      parts.push_back(std::move(p));
    }
  } else {
    // split_equal: adopt pairwise-disjoint sequence sets in submission order
    // (a set overlapping an adopted one waits), at most U sets; take the same
    // number of slots from each -- the fewest any set has left, and at most
    // U / sets -- and lay them out set by set, ascending smallest id.
    std::vector<uint8_t> used(n, 0);
    int32_t left = n;
    while (left > 0) {
      std::vector<SeqSet> sets;
      SeqSet uni = SeqSet::none();
      for (int32_t i = 0; i < n && static_cast<int32_t>(sets.size()) < U; ++i) {
        if (used[i] || (setmask[i] & uni).any()) continue;
        sets.push_back(setmask[i]);
        uni |= setmask[i];
      }
      std::vector<std::vector<int32_t>> members(sets.size());
      for (int32_t i = 0; i < n; ++i) {
        if (used[i]) continue;
        for (size_t k = 0; k < sets.size(); ++k)
          if (setmask[i] == sets[k]) { members[k].push_back(i); break; }
      }
      int32_t nst = U / static_cast<int32_t>(sets.size());
      for (auto& m : members) nst = std::min(nst, static_cast<int32_t>(m.size()));
      std::vector<size_t> order(sets.size());
      std::iota(order.begin(), order.end(), 0);
      std::sort(order.begin(), order.end(),
                [&](size_t a, size_t c) { return sets[a].lowest() < sets[c].lowest(); });
      Part p;
      for (size_t k : order)
        for (int32_t t = 0; t < nst; ++t) {
          const int32_t i = members[k][t];
          used[i] = 1;
          p.slots.push_back(i);
        }
      p.nst = nst;
      p.ns = static_cast<int32_t>(sets.size());
      left -= static_cast<int32_t>(p.slots.size());
      parts.push_back(std::move(p));
    }
  }

  // -- placement: every slot of every ubatch, all-or-nothing ("Batch、Ubatch
  // 与解码主循环", Part C: prepare reserves slots for all ubatches; Part F:
  // return 1 when the cache is full)
  // A slot's cell lives in the stream of its first id; with several streams
  // ("What does llama.cpp's KV cache ...", "Unified versus non-unified":
  // common prefixes need separate copies) a slot whose ids span streams also
  // gets one cell in each other stream, holding the ids that live there.
  std::vector<SeqSet> smask(g_.n_stream, SeqSet::none());   // ids of each stream
  for (int32_t q = 0; q < g_.n_seq_max; ++q) smask[q % g_.n_stream].set(q);
  std::vector<int32_t> need(g_.n_stream, 0);
  for (int32_t i = 0; i < n; ++i)
    for (int s = 0; s < g_.n_stream; ++s)
      if ((setmask[i] & smask[s]).any()) ++need[s];
  for (int s = 0; s < g_.n_stream; ++s)
    if (need[s] > st_[s].n_avail) {
      err = "no free cells: stream " + std::to_string(s) + " needs " + std::to_string(need[s]) +
            ", has " + std::to_string(st_[s].n_avail);
      return KVATTN_NO_SLOT;
    }
  for (auto& p : parts) {
    UbatchRec u;
    u.id = next_id_++;
    u.n_seq_tokens = p.nst;
    u.n_seqs = p.ns;
    SeqSet unq = SeqSet::none();
    for (int32_t i : p.slots) {
      const int s = seq0(i) % g_.n_stream;
      u.src.push_back(i);
      u.pos.push_back(pos[i]);
      u.n_seq_id.push_back(beg[i + 1] - beg[i]);
      u.seq_ptr.push_back(&seq_flat_[beg[i]]);
      u.setmask.push_back(setmask[i] & smask[s]);
      u.output.push_back(out[i]);
      u.n_outputs += out[i];
      u.stream.push_back(s);
      u.cells.push_back(pop_cell(s));
      for (int s2 = 0; s2 < g_.n_stream; ++s2) {
        if (s2 == s || !(setmask[i] & smask[s2]).any()) continue;
        u.copy_src.push_back(static_cast<int32_t>(u.src.size()) - 1);
        u.copy_stream.push_back(s2);
        u.copy_cell.push_back(pop_cell(s2));
        u.copy_mask.push_back(setmask[i] & smask[s2]);
      }
      unq |= setmask[i];
    }
    for (int q = unq.lowest(); q >= 0; q = unq.next(q)) u.seq_unq.push_back(q);
    ubs_.push_back(std::move(u));
  }
  if (output_ids) {
    int32_t r = 0;
    for (int32_t i = 0; i < g_.n_batch; ++i) output_ids[i] = (i < n && out[i]) ? r++ : -1;
  }
  return KVATTN_OK;
}

// ---- cell table ------------------------------------------------------------

template <class F>
void HostCore::for_seq_cells(int s, int32_t seq, F&& f) const {
  const Stream& S = st_[s];
  if (S.seq_n[seq] == 0) return;
  const std::vector<uint64_t>& bits = S.seq_bits[seq];
  const int32_t nw = (S.umax + 63) / 64;   // no cell at or past umax is occupied
  for (int32_t wi = 0; wi < nw; ++wi)
    for (uint64_t m = bits[wi]; m; m &= m - 1) f(64 * wi + __builtin_ctzll(m));
}

void HostCore::set_cell(int s, int32_t cell, int32_t pos, const SeqSet& mask) {
  Stream& S = st_[s];
  // an empty cell holds the empty set, so the old set is always S.mask[cell]
  const SeqSet& old = S.mask[cell];
  const uint64_t bit = 1ULL << (cell & 63);
  for (int wd = 0; wd < kSeqWords; ++wd) {
    for (uint64_t gone = old.w[wd] & ~mask.w[wd]; gone; gone &= gone - 1) {
      const int q = 64 * wd + __builtin_ctzll(gone);
      S.seq_bits[q][cell >> 6] &= ~bit;
      --S.seq_n[q];
    }
    for (uint64_t came = mask.w[wd] & ~old.w[wd]; came; came &= came - 1) {
      const int q = 64 * wd + __builtin_ctzll(came);
      if (S.seq_bits[q].empty()) S.seq_bits[q].assign((g_.kv_size + 63) / 64, 0);
      S.seq_bits[q][cell >> 6] |= bit;
      ++S.seq_n[q];
    }
  }
  if (S.pos[cell] >= 0) {
    auto it = S.count.find(S.mask[cell]);
    if (it != S.count.end() && --it->second == 0) S.count.erase(it);
  }
  const bool occupied = mask.any();
  S.pos[cell] = occupied ? pos : -1;
  S.mask[cell] = mask;
  if (occupied) {
    ++S.count[mask];
    S.umax = std::max(S.umax, cell + 1);
  } else {
    while (S.umax > 0 && S.pos[S.umax - 1] < 0) --S.umax;
  }
  pending_.push_back(static_cast<int32_t>(s * static_cast<int64_t>(g_.kv_size) + cell));
}

int HostCore::commit(int k, std::vector<CellUpdate>* upd, std::string& err) {
  UbatchRec& u = ubs_[k];
  if (u.committed) return KVATTN_OK;
  if (k > 0 && !ubs_[k - 1].committed) {
    err = "ubatches of one split are stored in order";
    return KVATTN_ESTATE;
  }
  for (size_t i = 0; i < u.cells.size(); ++i) set_cell(u.stream[i], u.cells[i], u.pos[i], u.setmask[i]);
  for (size_t i = 0; i < u.copy_cell.size(); ++i)
    set_cell(u.copy_stream[i], u.copy_cell[i], u.pos[u.copy_src[i]], u.copy_mask[i]);
  u.committed = true;
  latest_ = k;
  if (upd) {
    // one update per touched cell, carrying its final state: a cell freed by
    // seq_rm and placed again before this commit must not appear twice (the
    // device applies the list in parallel)
    std::sort(pending_.begin(), pending_.end());
    pending_.erase(std::unique(pending_.begin(), pending_.end()), pending_.end());
    for (int32_t idx : pending_) {
      const Stream& S = st_[idx / g_.kv_size];
      const int32_t j = idx % g_.kv_size;
      upd->push_back(CellUpdate{S.mask[j], idx, S.pos[j], {0, 0}});
    }
  }
  pending_.clear();
  return KVATTN_OK;
}

int HostCore::seq_rm(int32_t seq, int32_t p0, int32_t p1) {
  if (seq >= g_.n_seq_max) return KVATTN_EINVAL;
  const int32_t lo = p0 < 0 ? 0 : p0;
  auto in_range = [&](int32_t p) { return p >= lo && (p1 < 0 || p < p1); };
  for (int s = 0; s < g_.n_stream; ++s) {
    Stream& S = st_[s];
    if (seq < 0) {
      const int32_t end = S.umax;         // every cell at or past umax is empty
      for (int32_t j = 0; j < end; ++j) {
        const int32_t p = S.pos[j];
        if (p < 0 || !in_range(p)) continue;
        set_cell(s, j, p, SeqSet::none());
        push_cell(s, j);
      }
      continue;
    }
    for_seq_cells(s, seq, [&](int32_t j) {
      const int32_t p = S.pos[j];
      if (!in_range(p)) return;
      SeqSet m = S.mask[j];
      m.reset(seq);
      set_cell(s, j, p, m);
      if (!m.any()) push_cell(s, j);
    });
  }
  latest_ = -1;                       // the device mirror is stale until the next commit
  return KVATTN_OK;
}

int HostCore::seq_cells(int32_t seq, std::vector<int32_t>& cells, std::vector<int32_t>& pos) const {
  cells.clear();
  pos.clear();
  if (seq < 0 || seq >= g_.n_seq_max) return -1;
  const int s = seq % g_.n_stream;
  const Stream& S = st_[s];
  std::vector<std::pair<int32_t, int32_t>> v;
  for_seq_cells(s, seq, [&](int32_t j) { v.push_back({S.pos[j], j}); });
  std::sort(v.begin(), v.end());
  for (const auto& pc : v) {
    pos.push_back(pc.first);
    cells.push_back(pc.second);
  }
  return s;
}

int HostCore::seq_restore(int32_t seq, const int32_t* pos, int32_t n, std::vector<int32_t>& cells,
                          std::string& err) {
  if (seq < 0 || seq >= g_.n_seq_max || n < 0) {
    err = "sequence id out of range";
    return KVATTN_EINVAL;
  }
  for (int32_t i = 0; i < n; ++i)
    if (pos[i] < 0) {
      err = "negative position";
      return KVATTN_EINVAL;
    }
  const int s = seq % g_.n_stream;
  Stream& S = st_[s];
  const SeqSet bit = SeqSet::one(seq);
  int32_t own = 0;
  for_seq_cells(s, seq, [&](int32_t j) { own += S.mask[j] == bit; });
  if (S.n_avail + own < n) {
    err = "no room in the stream for the saved cells";
    return KVATTN_NO_SLOT;
  }
  seq_rm(seq, -1, -1);
  cells.resize(n);
  for (int32_t i = 0; i < n; ++i) {
    cells[i] = pop_cell(s);
    set_cell(s, cells[i], pos[i], bit);
  }
  latest_ = -1;                       // the device mirror follows at the next commit
  return KVATTN_OK;
}

int32_t HostCore::seq_pos_max(int32_t seq) const {
  if (seq < 0 || seq >= g_.n_seq_max) return -1;
  int32_t best = -1;
  for (int s = 0; s < g_.n_stream; ++s)
    for_seq_cells(s, seq, [&](int32_t j) { best = std::max(best, st_[s].pos[j]); });
  return best;
}

int32_t HostCore::n_kv() const {
  // get_n_kv ("llama.cpp and the ubatch", "Prefill and decode are not the
  // same shape"): occupied extent rounded up to 256, at least 256, at most
  // the stream size; largest over the streams.
  int32_t r = 0;
  for (const auto& S : st_)
    r = std::max(r, std::min(g_.kv_size, std::max(kNkvQuantum, round_up(S.umax, kNkvQuantum))));
  return r;
}

void HostCore::get_cells(int32_t s, int32_t* pos, uint64_t* mask) const {
  const Stream& S = st_[s];
  if (pos) std::copy(S.pos.begin(), S.pos.end(), pos);
  if (mask)
    for (size_t j = 0; j < S.mask.size(); ++j)
      for (int i = 0; i < kSeqWords; ++i) mask[j * kSeqWords + i] = S.mask[j].w[i];
}

// ---- work plan -------------------------------------------------------------

int HostCore::build_plan(int k, bool only_outputs, int32_t max_classes, bool shrink, Plan& P,
                         std::string& err) const {
  const UbatchRec& u = ubs_[k];
  P = Plan();
  P.n_kv = n_kv();
  P.n_seg = ceil_div(P.n_kv, kSegCells);
  const int S = g_.n_stream;
  const int32_t T = static_cast<int32_t>(u.pos.size());

  // query slots
  std::vector<int32_t> slot_of;      // plan slot -> ubatch row
  int32_t r_out = 0;
  for (int32_t i = 0; i < T; ++i) {
    if (only_outputs && !u.output[i]) continue;
    const int32_t row = only_outputs ? r_out++ : i;
    P.slots.push_back(SlotInfo{u.stream[i], u.pos[i], u.seq_ptr[i][0], i, row, {0, 0, 0}});
    slot_of.push_back(i);
  }
  const int32_t NQ = static_cast<int32_t>(P.slots.size());
  // classes come from every slot of the ubatch, so both plan variants (all
  // rows / output rows only) share one class table and one set of lists
  std::vector<SeqSet> qseqs(S, SeqSet::none());
  for (int32_t i = 0; i < T; ++i) qseqs[u.stream[i]].set(u.seq_ptr[i][0]);

  // classes: the committed sequence sets of each stream that some query can see
  std::vector<std::vector<std::pair<SeqSet, int32_t>>> rel(S);
  size_t n_rel = 0;
  for (int s = 0; s < S; ++s) {
    for (const auto& kv : st_[s].count)
      if (kv.second > 0 && (kv.first & qseqs[s]).any()) rel[s].push_back(kv);
    std::sort(rel[s].begin(), rel[s].end());
    n_rel += rel[s].size();
  }
  int32_t n_streams_rel = 0;
  for (int s = 0; s < S; ++s) n_streams_rel += rel[s].empty() ? 0 : 1;
  // queries of each class, grouped by sequence then position
  std::vector<int32_t> qorder(NQ);
  std::iota(qorder.begin(), qorder.end(), 0);
  std::sort(qorder.begin(), qorder.end(), [&](int32_t a, int32_t b) {
    const SlotInfo &x = P.slots[a], &y = P.slots[b];
    if (x.seq0 != y.seq0) return x.seq0 < y.seq0;
    if (x.pos != y.pos) return x.pos < y.pos;
    return a < b;
  });
  // Past the class cap, the tail of each stream's list is merged into one
  // class (its set: the union; its cells walked with the per-cell membership
  // test).  The cap starts at max_classes.  A query gets one partial row per
  // class it reads, so when even whole classes need more split-K partial
  // rows than the workspace holds (queries that each see many sets), the
  // cap is halved and the plan built again, when the caller allows it.
  auto plan_with_cap = [&](int32_t cap) -> int {
    P.classes.clear();
    P.lookup.clear();
    P.qlist.clear();
    P.items_valu.clear();
    P.items_mfma.clear();
    P.red_slot.clear();
    P.red_off.clear();
    P.red_rows.clear();
    P.max_class_tiles = 0;
    P.n_partial_rows = 0;
    int32_t budget = n_rel <= static_cast<size_t>(cap) ? cap : std::max(0, cap - n_streams_rel);
    P.lookup_off.assign(S + 1, 0);
    for (int s = 0; s < S; ++s) {
      P.lookup_off[s] = static_cast<int32_t>(P.lookup.size());
      int32_t merged = -1;
      for (const auto& kv : rel[s]) {
        int32_t c;
        if (budget > 0) {
          c = static_cast<int32_t>(P.classes.size());
          P.classes.push_back(ClassInfo{kv.first, s, kv.second, 0, 0, 0, 1, 0, 0});
          --budget;
        } else {
          if (merged < 0) {
            merged = static_cast<int32_t>(P.classes.size());
            P.classes.push_back(ClassInfo{SeqSet::none(), s, 0, 0, 0, 0, 0, 0, 0});
          }
          c = merged;
          P.classes[c].mask |= kv.first;
          P.classes[c].n_cells += kv.second;
        }
        P.lookup.push_back(LookupEntry{kv.first, c, {0, 0, 0}});
      }
    }
    P.lookup_off[S] = static_cast<int32_t>(P.lookup.size());
    int32_t off = 0, tiles = 0;
    for (auto& c : P.classes) {
      c.cell_off = off;
      c.tile_base = tiles;
      off += c.n_cells;
      tiles += ceil_div(c.n_cells, kTileCells);
      P.max_class_tiles = std::max(P.max_class_tiles, ceil_div(c.n_cells, kTileCells));
    }
    P.total_cells = off;
    P.total_tiles = tiles;

    for (auto& c : P.classes) {
      c.q_off = static_cast<int32_t>(P.qlist.size());
      for (int32_t q : qorder)
        if (P.slots[q].stream == c.stream && c.mask.test(P.slots[q].seq0)) P.qlist.push_back(q);
      c.n_q = static_cast<int32_t>(P.qlist.size()) - c.q_off;
    }

    // work items
    const int D = g_.head_dim, G = g_.G();
    const int32_t E = g_.E();
    const bool valu_ok = (E == 512 || E == 1024 || E == 2048 || E == 4096) && (D == 64 || D == 128) &&
                         (G == 1 || G == 2 || G == 4);
    const int32_t QT = kMfmaRowsPerItem / G;   // query rows of one matrix-core workgroup
    // Item sizing.  One attend call launches (items x layers per call)
    // workgroups.  Each bandwidth-bound class is cut into chunks of at most
    // `ch` cells; ch is the largest power of two (256 .. 8192 cells) for which
    // the launch still reaches its workgroup target, so a long context is
    // split only when there are too few queries to fill the GPU.
    const int64_t L = std::max(1, g_.attend_layers);
    std::vector<std::pair<int32_t, int32_t>> valu_lists, low_lists, high_lists;   // (cells, copies)
    for (const auto& c : P.classes) {
      if (c.n_q == 0 || c.n_cells == 0) continue;
      if (valu_ok && c.n_q <= kValuMaxQueries) valu_lists.push_back({c.n_cells, c.n_q});
      else if (c.n_q * G <= 64) low_lists.push_back({c.n_cells, ceil_div(c.n_q, QT) * g_.n_head_kv});
      else high_lists.push_back({c.n_cells, ceil_div(c.n_q, QT) * g_.n_head_kv});
    }
    auto pick_chunk = [&](const std::vector<std::pair<int32_t, int32_t>>& lists, int64_t target, int32_t lo,
                          int32_t hi) {
      int32_t ch = hi;
      while (ch > lo) {
        int64_t wg = 0;
        for (const auto& x : lists) wg += static_cast<int64_t>(ceil_div(x.first, ch)) * x.second;
        if (wg * L >= target) break;
        ch /= 2;
      }
      return ch;
    };
    int32_t chv = pick_chunk(valu_lists, kValuTargetWorkgroups, kValuMinChunk, 8192);
    // matrix-core items with few query rows are bandwidth-bound too: their
    // cells (multiples of the 64-cell tile) are cut the same way
    int32_t chm_lowreuse = pick_chunk(low_lists, kMfmaTargetWorkgroups, 256, 4096);
    // prompt-sized classes are cut only when the launch would not fill the
    // GPU otherwise (one layer per call): every cut costs a partial row per
    // query and merge work, so a layer range keeps whole cell lists
    int32_t chm_high = pick_chunk(high_lists, kMfmaHighTargetWorkgroups, 256, 1 << 30);

    for (int attempt = 0; attempt < 16; ++attempt) {
      P.items_valu.clear();
      P.items_mfma.clear();
      std::vector<int32_t> coverage(NQ, 0);
      // VALU items: (query, chunk)
      struct Pending { WorkItem it; bool valu; };
      std::vector<Pending> pend;
      for (int32_t ci = 0; ci < static_cast<int32_t>(P.classes.size()); ++ci) {
        const ClassInfo& c = P.classes[ci];
        if (c.n_q == 0 || c.n_cells == 0) continue;
        const bool valu = valu_ok && c.n_q <= kValuMaxQueries;
        if (valu) {
          const int32_t parts = ceil_div(c.n_cells, chv);
          const int32_t len = ceil_div(c.n_cells, parts);
          for (int32_t t = 0; t < c.n_q; ++t) {
            const int32_t q = P.qlist[c.q_off + t];
            for (int32_t a = 0; a < c.n_cells; a += len) {
              WorkItem it{ci, c.q_off + t, 1, c.cell_off + a, c.cell_off + std::min(c.n_cells, a + len), -1,
                          P.slots[q].pos, P.slots[q].pos, c.tile_base + a / kTileCells, c.stream, c.pure, 0};
              pend.push_back({it, true});
              ++coverage[q];
            }
          }
        } else {
          // few query rows per KV head -> bandwidth-bound -> split the cells
          const int32_t ch = (c.n_q * G <= 64) ? chm_lowreuse : chm_high;
          for (int32_t t0 = 0; t0 < c.n_q; t0 += QT) {
            const int32_t nq = std::min(QT, c.n_q - t0);
            int32_t pmin = INT32_MAX, pmax = INT32_MIN;
            for (int32_t t = 0; t < nq; ++t) {
              const int32_t p = P.slots[P.qlist[c.q_off + t0 + t]].pos;
              pmin = std::min(pmin, p);
              pmax = std::max(pmax, p);
            }
            for (int32_t a = 0; a < c.n_cells; a += ch) {
              WorkItem it{ci, c.q_off + t0, nq, c.cell_off + a, c.cell_off + std::min(c.n_cells, a + ch), -1,
                          pmin, pmax, c.tile_base + a / kTileCells, c.stream, c.pure, 0};
              pend.push_back({it, false});
              for (int32_t t = 0; t < nq; ++t) ++coverage[P.qlist[c.q_off + t0 + t]];
            }
          }
        }
      }
      // direct output when every query of the item is covered once
      int32_t rows = 0;
      std::vector<std::vector<int32_t>> qrows(NQ);
      for (auto& pd : pend) {
        bool direct = true;
        for (int32_t t = 0; t < pd.it.n_q; ++t) direct &= coverage[P.qlist[pd.it.q_off + t]] == 1;
        if (!direct) {
          pd.it.prow = rows;
          for (int32_t t = 0; t < pd.it.n_q; ++t) qrows[P.qlist[pd.it.q_off + t]].push_back(rows + t);
          rows += pd.it.n_q;
        }
        (pd.valu ? P.items_valu : P.items_mfma).push_back(pd.it);
      }
      if (rows > prow_max) {
        chv *= 2;
        chm_lowreuse *= 2;
        chm_high = std::min(chm_high, 1 << 29) * 2;
        continue;
      }
      P.n_partial_rows = rows;
      P.red_off.push_back(0);
      for (int32_t q = 0; q < NQ; ++q) {
        if (qrows[q].empty()) continue;
        P.red_slot.push_back(q);
        P.red_rows.insert(P.red_rows.end(), qrows[q].begin(), qrows[q].end());
        P.red_off.push_back(static_cast<int32_t>(P.red_rows.size()));
      }
      // longest first in both sets (the kernels dispatch items in this order):
      // the last workgroups of a launch are then the shortest ones
      std::stable_sort(P.items_valu.begin(), P.items_valu.end(),
                       [](const WorkItem& a, const WorkItem& b) { return a.c1 - a.c0 > b.c1 - b.c0; });
      // MFMA items: causal tiles late in a prompt see the most cells
      std::stable_sort(P.items_mfma.begin(), P.items_mfma.end(), [](const WorkItem& a, const WorkItem& b) {
        return std::min(a.c1 - a.c0, a.qpos_max) > std::min(b.c1 - b.c0, b.qpos_max);
      });
      return KVATTN_OK;
    }

    return KVATTN_ENOMEM;
  };
  for (int32_t cap = max_classes;; cap /= 2) {
    if (plan_with_cap(cap) == KVATTN_OK) {
      P.class_cap = cap;
      return KVATTN_OK;
    }
    if (!shrink || cap <= n_streams_rel) break;   // one class per stream already
  }
  err = "split-K partial rows exceed the workspace";
  return KVATTN_ENOMEM;
}

}  // namespace kvattn
