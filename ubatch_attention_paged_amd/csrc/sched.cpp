// The iteration-level batching loop ("Iteration-Level Batching: Reforming
// the Batch at Every Token", "The loop that replaces the batch", "The budget
// that actually binds", "Where it breaks") as a native client of the kvattn
// C ABI.  The behaviour of each step is documented in kvsched.h.
//
// The pages ask the per-iteration host work to stay well inside one forward
// pass and to keep memory allocation off that path ("What the loop costs
// elsewhere"): every table of the scheduler is sized at create, and one
// step touches only the running sequences (at most n_seq_max <= 256) and the
// waiting requests it admits, plus one kvattn_seq_rm per retired or
// preempted sequence, which visits only that sequence's cells.
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kvattn.h"
#include "kvsched.h"
#include "state_internal.hpp"

namespace {

struct Req {
  int32_t n_prompt = 0, n_generate = 0;
  int32_t seq = -1;
  int32_t n_ctx = 0;        // positions cached
  int32_t sampled = 0;      // tokens sampled
  int32_t blocks = 0;       // RESERVE: blocks held
  int32_t state = KVATTN_REQ_WAITING;
  int64_t swap_off = -1;    // SWAP: extent of its saved state while swapped out
  int64_t swap_len = 0;
  int32_t known() const { return n_prompt + sampled; }
  int32_t pending() const { return known() - n_ctx; }
  bool finished() const { return sampled >= n_generate; }
};

int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

constexpr int64_t kSwapAlign = 256;

struct Extent {
  int64_t off, len;
  int32_t req;
};

}  // namespace

struct kvattn_sched {
  kvattn_ctx* ctx = nullptr;
  int32_t kv_size = 0, n_stream = 1, n_seq_max = 1;
  int32_t budget = 0, max_running = 0, policy = KVATTN_ADMIT_PAGED, block_size = 1, chunked = 1;
  std::string err;

  std::vector<Req> reqs;                 // capacity max_requests, size = submitted
  std::vector<int32_t> wq;               // waiting queue: ring buffer of request ids
  int32_t w_head = 0, w_count = 0;
  std::vector<int32_t> run;              // running request ids in admission order
  std::vector<int32_t> chunk;            // positions of run[i] in the assembled batch
  std::vector<int32_t> seq_owner;        // request running under each sequence id, -1 free
  std::vector<int32_t> free_blocks;      // RESERVE, per stream
  std::vector<int32_t> held, need;       // PAGED, per stream: cells held or promised; single-pending count
  int32_t preempt = KVATTN_PREEMPT_RECOMPUTE;
  char* swap_space = nullptr;
  int64_t swap_bytes = 0;
  void* stream = nullptr;
  bool device = false;
  int32_t n_layer = 0, row_bytes = 0;
  std::vector<Extent> swapped;           // live extents of the swap arena, by offset
  std::vector<int32_t> iota;             // positions 0, 1, 2, ... of a restored sequence

  // the assembled iteration
  std::vector<int32_t> b_pos, b_nsid, b_req, seq_val;
  std::vector<const int32_t*> b_seq;
  std::vector<int8_t> b_out;
  std::vector<int32_t> retired, preempted, admitted, admitted_seq, swapped_out, swapped_in;
  bool assembled = false;

  int fail(int code, const char* msg) {
    err = msg;
    return code;
  }

  int32_t stream_of(int32_t seq) const { return seq % n_stream; }
  int32_t w_at(int32_t i) const { return wq[(w_head + i) % wq.size()]; }
  void w_push_back(int32_t r) {
    wq[(w_head + w_count) % wq.size()] = r;
    ++w_count;
  }
  void w_push_front(int32_t r) {
    w_head = (w_head + static_cast<int32_t>(wq.size()) - 1) % static_cast<int32_t>(wq.size());
    wq[w_head] = r;
    ++w_count;
  }
  void w_pop_front() {
    w_head = (w_head + 1) % static_cast<int32_t>(wq.size());
    --w_count;
  }

  // Cells a running sequence holds or was promised (PAGED): its cached
  // positions plus, while more than one is pending, the pending ones.
  static int32_t claim(const Req& r) { return r.n_ctx + (r.pending() > 1 ? r.pending() : 0); }

  void account() {
    std::fill(held.begin(), held.end(), 0);
    std::fill(need.begin(), need.end(), 0);
    for (int32_t id : run) {
      const Req& r = reqs[id];
      const int32_t s = stream_of(r.seq);
      held[s] += claim(r);
      need[s] += r.pending() == 1 ? 1 : 0;
    }
  }

  // Release a running request's cells and sequence id; keeps run order.
  int drop(int32_t idx) {
    Req& r = reqs[run[idx]];
    const int rc = kvattn_seq_rm(ctx, r.seq, -1, -1);
    if (rc != KVATTN_OK) return fail(rc, "kvattn_seq_rm failed on the context");
    seq_owner[r.seq] = -1;
    if (policy == KVATTN_ADMIT_RESERVE) {
      free_blocks[stream_of(r.seq)] += r.blocks;
      r.blocks = 0;
    }
    r.seq = -1;
    run.erase(run.begin() + idx);
    return KVATTN_OK;
  }

  // Lowest offset of the swap arena with `len` free bytes (first fit), -1 if none.
  int64_t swap_place(int64_t len) const {
    int64_t at = 0;
    for (const Extent& e : swapped) {
      if (e.off - at >= len) return at;
      at = e.off + e.len;
    }
    return swap_bytes - at >= len ? at : -1;
  }

  // Save a victim's cells into the arena before they are released; false
  // (recompute instead) when its blob does not fit.
  int swap_out(Req& r, int32_t id, bool* saved) {
    *saved = false;
    if (preempt != KVATTN_PREEMPT_SWAP || r.n_ctx == 0) return KVATTN_OK;
    size_t bytes = 0;
    if (kvattn_seq_state_size(ctx, r.seq, &bytes) != KVATTN_OK) return fail(KVATTN_EINVAL, "kvattn_seq_state_size failed");
    const int64_t n = r.n_ctx;
    if (static_cast<int64_t>(bytes) != 80 + 4 * n + 2 * static_cast<int64_t>(n_layer) * (12 + n * row_bytes))
      return fail(KVATTN_ESTATE, "the context's cells of a running sequence differ from its cached positions");
    const int64_t len = (static_cast<int64_t>(bytes) + kSwapAlign - 1) / kSwapAlign * kSwapAlign;
    const int64_t off = swap_place(len);
    if (off < 0) return KVATTN_OK;
    if (device) {
      const int rc = kvattn_seq_state_save(ctx, r.seq, swap_space + off, static_cast<size_t>(len), nullptr, stream);
      if (rc != KVATTN_OK) return fail(rc, "kvattn_seq_state_save failed");
    }
    auto it = std::lower_bound(swapped.begin(), swapped.end(), off,
                               [](const Extent& e, int64_t o) { return e.off < o; });
    swapped.insert(it, Extent{off, len, id});
    r.swap_off = off;
    r.swap_len = len;
    *saved = true;
    return KVATTN_OK;
  }

  int swap_in(Req& r) {
    const int rc = kvattn::state_restore_known(ctx, r.seq, device ? swap_space + r.swap_off : nullptr, iota.data(),
                                               r.n_ctx, stream);
    if (rc != KVATTN_OK) return fail(rc, "restoring a swapped-out sequence failed");
    for (size_t i = 0; i < swapped.size(); ++i)
      if (swapped[i].off == r.swap_off) {
        swapped.erase(swapped.begin() + static_cast<std::ptrdiff_t>(i));
        break;
      }
    r.swap_off = -1;
    r.swap_len = 0;
    return KVATTN_OK;
  }

  // Positions a sequence with `want` pending gets from `left`.
  int32_t take(int32_t want, int32_t left) const {
    if (chunked) return std::min(want, left);
    return want <= left ? want : 0;
  }
};

extern "C" {

int kvattn_sched_create(kvattn_ctx* ctx, const kvattn_sched_params* p, kvattn_sched** out) {
  if (!ctx || !p || !out) return KVATTN_EINVAL;
  *out = nullptr;
  kvattn_params cp;
  if (kvattn_get_params(ctx, &cp) != KVATTN_OK) return KVATTN_EINVAL;
  const int32_t max_running = p->max_running > 0 ? p->max_running : cp.n_seq_max;
  const int32_t budget = p->token_budget > 0 ? p->token_budget : cp.n_batch;
  if (max_running > cp.n_seq_max || budget < max_running || budget > cp.n_batch) return KVATTN_EINVAL;
  if (p->policy != KVATTN_ADMIT_RESERVE && p->policy != KVATTN_ADMIT_PAGED) return KVATTN_EINVAL;
  if (p->policy == KVATTN_ADMIT_RESERVE && (p->block_size < 1 || p->block_size > cp.kv_size)) return KVATTN_EINVAL;
  if (p->max_requests < 1) return KVATTN_EINVAL;
  if (p->preempt != KVATTN_PREEMPT_RECOMPUTE && p->preempt != KVATTN_PREEMPT_SWAP) return KVATTN_EINVAL;
  const bool device = kvattn::ctx_has_device(ctx);
  if (p->preempt == KVATTN_PREEMPT_SWAP && device && p->swap_bytes > 0 &&
      (!p->swap_space || (reinterpret_cast<uintptr_t>(p->swap_space) & (kSwapAlign - 1))))
    return KVATTN_EINVAL;

  kvattn_sched* s = new (std::nothrow) kvattn_sched();
  if (!s) return KVATTN_ENOMEM;
  try {
    s->ctx = ctx;
    s->kv_size = cp.kv_size;
    s->n_stream = cp.n_stream;
    s->n_seq_max = cp.n_seq_max;
    s->budget = budget;
    s->max_running = max_running;
    s->policy = p->policy;
    s->block_size = p->policy == KVATTN_ADMIT_RESERVE ? p->block_size : 1;
    s->chunked = p->chunked ? 1 : 0;
    s->preempt = p->preempt;
    s->swap_space = static_cast<char*>(p->swap_space);
    s->swap_bytes = p->preempt == KVATTN_PREEMPT_SWAP ? static_cast<int64_t>(p->swap_bytes) : 0;
    s->stream = p->hip_stream;
    s->device = device;
    s->n_layer = cp.n_layer;
    s->row_bytes = cp.n_head_kv * cp.head_dim * 2;
    s->swapped.reserve(p->max_requests);
    s->iota.resize(cp.kv_size);
    for (int32_t q = 0; q < cp.kv_size; ++q) s->iota[q] = q;
    s->swapped_out.reserve(cp.n_seq_max);
    s->swapped_in.reserve(cp.n_seq_max);
    s->reqs.reserve(p->max_requests);
    s->wq.assign(p->max_requests, -1);
    s->run.reserve(cp.n_seq_max);
    s->chunk.assign(cp.n_seq_max, 0);
    s->seq_owner.assign(cp.n_seq_max, -1);
    s->free_blocks.assign(cp.n_stream, cp.kv_size / s->block_size);
    s->held.assign(cp.n_stream, 0);
    s->need.assign(cp.n_stream, 0);
    s->b_pos.assign(budget, 0);
    s->b_nsid.assign(budget, 1);
    s->b_req.assign(budget, 0);
    s->b_seq.assign(budget, nullptr);
    s->b_out.assign(budget, 0);
    s->seq_val.resize(cp.n_seq_max);
    for (int32_t q = 0; q < cp.n_seq_max; ++q) s->seq_val[q] = q;
    s->retired.reserve(cp.n_seq_max);
    s->preempted.reserve(cp.n_seq_max);
    s->admitted.reserve(cp.n_seq_max);
    s->admitted_seq.reserve(cp.n_seq_max);
  } catch (const std::bad_alloc&) {
    delete s;
    return KVATTN_ENOMEM;
  }
  *out = s;
  return KVATTN_OK;
}

void kvattn_sched_destroy(kvattn_sched* s) { delete s; }

int kvattn_sched_submit(kvattn_sched* s, int32_t n_prompt, int32_t n_generate, int32_t* req_id) {
  if (!s) return KVATTN_EINVAL;
  if (n_prompt < 1 || n_generate < 1) return s->fail(KVATTN_EINVAL, "n_prompt and n_generate must be >= 1");
  const int64_t cached = int64_t(n_prompt) + n_generate - 1;
  if (cached > s->kv_size) return s->fail(KVATTN_EINVAL, "request holds more positions than a stream has cells");
  if (s->policy == KVATTN_ADMIT_RESERVE &&
      (int64_t(n_prompt) + n_generate + s->block_size - 1) / s->block_size > s->kv_size / s->block_size)
    return s->fail(KVATTN_EINVAL, "request needs more blocks than a stream has");
  if (!s->chunked) {
    const int64_t worst = s->policy == KVATTN_ADMIT_PAGED ? cached : n_prompt;
    if (worst > s->budget) return s->fail(KVATTN_EINVAL, "prompt longer than the token budget and chunking is off");
  }
  if (s->reqs.size() >= s->reqs.capacity()) return s->fail(KVATTN_ENOMEM, "request table full");
  Req r;
  r.n_prompt = n_prompt;
  r.n_generate = n_generate;
  s->reqs.push_back(r);
  const int32_t id = static_cast<int32_t>(s->reqs.size()) - 1;
  s->w_push_back(id);
  if (req_id) *req_id = id;
  return KVATTN_OK;
}

int kvattn_sched_step(kvattn_sched* s, kvattn_sched_iter* it) {
  if (!s || !it) return KVATTN_EINVAL;
  if (s->assembled) return s->fail(KVATTN_ESTATE, "advance the previous iteration first");
  s->retired.clear();
  s->preempted.clear();
  s->admitted.clear();
  s->admitted_seq.clear();
  s->swapped_out.clear();
  s->swapped_in.clear();

  // 1. retire finished sequences
  for (int32_t i = 0; i < static_cast<int32_t>(s->run.size());) {
    const int32_t id = s->run[i];
    if (s->reqs[id].finished()) {
      if (int rc = s->drop(i)) return rc;
      s->reqs[id].state = KVATTN_REQ_DONE;
      s->retired.push_back(id);
    } else {
      ++i;
    }
  }

  // 2. paged cache pressure: newest sequence of a short stream goes back
  if (s->policy == KVATTN_ADMIT_PAGED) {
    s->account();
    for (int32_t st = 0; st < s->n_stream; ++st) {
      while (s->kv_size - s->held[st] < s->need[st]) {
        int32_t idx = static_cast<int32_t>(s->run.size()) - 1;
        while (s->stream_of(s->reqs[s->run[idx]].seq) != st) --idx;
        const int32_t id = s->run[idx];
        Req& r = s->reqs[id];
        s->held[st] -= kvattn_sched::claim(r);
        s->need[st] -= r.pending() == 1 ? 1 : 0;
        bool saved = false;
        if (int rc = s->swap_out(r, id, &saved)) return rc;
        if (saved) s->swapped_out.push_back(id);
        if (int rc = s->drop(idx)) return rc;
        if (!saved) r.n_ctx = 0;
        r.state = KVATTN_REQ_WAITING;
        s->w_push_front(id);
        s->preempted.push_back(id);
      }
    }
  }

  // budget already promised to running sequences: single pending positions
  // first, then pending prompt positions in admission order
  int32_t left = s->budget;
  const int32_t n_run0 = static_cast<int32_t>(s->run.size());
  for (int32_t i = 0; i < n_run0; ++i) {
    const bool one = s->reqs[s->run[i]].pending() == 1;
    s->chunk[i] = one ? 1 : 0;
    left -= one ? 1 : 0;
  }
  for (int32_t i = 0; i < n_run0; ++i) {
    const int32_t pd = s->reqs[s->run[i]].pending();
    if (pd > 1) {
      s->chunk[i] = s->take(pd, left);
      left -= s->chunk[i];
    }
  }

  // 3. admission, first come first served
  while (s->w_count > 0 && static_cast<int32_t>(s->run.size()) < s->max_running) {
    const int32_t id = s->w_at(0);
    Req& r = s->reqs[id];
    const int32_t c = s->take(r.pending(), left);
    if (c == 0) break;
    int32_t seq = 0;
    while (s->seq_owner[seq] >= 0) ++seq;   // run.size() < max_running <= n_seq_max: one is free
    const int32_t st = s->stream_of(seq);
    int32_t blocks = 0;
    if (s->policy == KVATTN_ADMIT_RESERVE) {
      blocks = ceil_div(r.n_prompt + r.n_generate, s->block_size);
      if (blocks > s->free_blocks[st]) break;
    } else if (r.n_ctx + r.pending() > s->kv_size - s->held[st] - s->need[st]) {
      break;
    }
    s->w_pop_front();
    r.seq = seq;
    r.state = KVATTN_REQ_RUNNING;
    s->seq_owner[seq] = id;
    if (s->policy == KVATTN_ADMIT_RESERVE) {
      r.blocks = blocks;
      s->free_blocks[st] -= blocks;
    } else {
      s->held[st] += kvattn_sched::claim(r);
      s->need[st] += r.pending() == 1 ? 1 : 0;
    }
    if (r.swap_off >= 0) {
      if (int rc = s->swap_in(r)) return rc;
      s->swapped_in.push_back(id);
    }
    s->chunk[s->run.size()] = c;
    s->run.push_back(id);
    s->admitted.push_back(id);
    s->admitted_seq.push_back(seq);
    left -= c;
  }

  // 4. assemble in running order
  int32_t n = 0, n_decode = 0;
  for (size_t i = 0; i < s->run.size(); ++i) {
    const int32_t id = s->run[i];
    const Req& r = s->reqs[id];
    const int32_t c = s->chunk[i];
    if (r.pending() == 1) n_decode += c;
    for (int32_t p = r.n_ctx; p < r.n_ctx + c; ++p, ++n) {
      s->b_pos[n] = p;
      s->b_seq[n] = &s->seq_val[r.seq];
      s->b_req[n] = id;
      s->b_out[n] = p == r.known() - 1 ? 1 : 0;
    }
  }

  std::memset(it, 0, sizeof(*it));
  it->batch.n_tokens = n;
  it->batch.pos = s->b_pos.data();
  it->batch.n_seq_id = s->b_nsid.data();
  it->batch.seq_id = s->b_seq.data();
  it->batch.output = s->b_out.data();
  it->req = s->b_req.data();
  it->n_retired = static_cast<int32_t>(s->retired.size());
  it->retired = s->retired.data();
  it->n_preempted = static_cast<int32_t>(s->preempted.size());
  it->preempted = s->preempted.data();
  it->n_admitted = static_cast<int32_t>(s->admitted.size());
  it->admitted = s->admitted.data();
  it->admitted_seq = s->admitted_seq.data();
  it->n_swapped_out = static_cast<int32_t>(s->swapped_out.size());
  it->swapped_out = s->swapped_out.data();
  it->n_swapped_in = static_cast<int32_t>(s->swapped_in.size());
  it->swapped_in = s->swapped_in.data();
  it->n_running = static_cast<int32_t>(s->run.size());
  it->n_waiting = s->w_count;
  it->n_decode = n_decode;
  s->assembled = true;
  s->err.clear();
  return KVATTN_OK;
}

int kvattn_sched_advance(kvattn_sched* s) {
  if (!s) return KVATTN_EINVAL;
  if (!s->assembled) return s->fail(KVATTN_ESTATE, "no iteration assembled");
  for (size_t i = 0; i < s->run.size(); ++i) {
    Req& r = s->reqs[s->run[i]];
    const int32_t c = s->chunk[i];
    if (c == 0) continue;
    const bool completes = r.n_ctx + c == r.known();
    r.n_ctx += c;
    if (completes) r.sampled += 1;
  }
  s->assembled = false;
  return KVATTN_OK;
}

int kvattn_sched_request(const kvattn_sched* s, int32_t req_id, int32_t* state, int32_t* seq_id,
                         int32_t* n_cached, int32_t* n_sampled) {
  if (!s || req_id < 0 || req_id >= static_cast<int32_t>(s->reqs.size())) return KVATTN_EINVAL;
  const Req& r = s->reqs[req_id];
  if (state) *state = r.state;
  if (seq_id) *seq_id = r.seq;
  if (n_cached) *n_cached = r.n_ctx;
  if (n_sampled) *n_sampled = r.sampled;
  return KVATTN_OK;
}

const char* kvattn_sched_last_error(const kvattn_sched* s) { return s ? s->err.c_str() : ""; }

}  // extern "C"
