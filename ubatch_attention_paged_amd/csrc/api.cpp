// C ABI of the library (include/kvattn.h): context, workspace carve-up,
// pinned staging of the per-ubatch plan, and the store / attend sequences.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "host_core.hpp"
#include "kvattn.h"
#include "launch.hpp"
#include "state_internal.hpp"

using namespace kvattn;

namespace {

constexpr int kStages = 16;                // pinned staging buffers in flight
constexpr int kStagesPerEvent = 8;         // uses of the ring covered by one recorded event
static_assert(kStages >= 2 * kStagesPerEvent, "a cover event outlives the stages it covers");
constexpr int64_t kPartialRowsCap = 16384; // split-K partial rows x layers per launch
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct WsLayout {
  size_t cpos, cmask, cellcls, counts, csr_cell, csr_pos, csr_mask, tile_min, tile_max, arena, arena_bytes,
      part_acc, part_ml;
  size_t total;
};

WsLayout ws_layout(const Geometry& g) {
  WsLayout L{};
  const size_t sc = static_cast<size_t>(g.n_stream) * g.kv_size;
  const size_t nseg = (g.kv_size + kSegCells - 1) / kSegCells;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
  L.cpos = take(sc * 4);
  L.cmask = take(sc * sizeof(SeqSet));
  L.cellcls = take(sc * 4);
  L.counts = take(static_cast<size_t>(kMaxClasses) * nseg * 4);
  L.csr_cell = take(sc * 4);
  L.csr_pos = take(sc * 4);
  L.csr_mask = take(sc * sizeof(SeqSet));
  const size_t ntile = sc / kTileCells + kMaxClasses + 1;   // each class adds at most one partial tile
  L.tile_min = take(ntile * 4);
  L.tile_max = take(ntile * 4);
  L.arena_bytes = (16u << 20) + (32 + sizeof(CellUpdate)) * sc + 64 * static_cast<size_t>(g.n_ubatch);
  L.arena = take(L.arena_bytes);
  const size_t hd = static_cast<size_t>(g.n_head) * g.head_dim;
  L.part_acc = take(kPartialRowsCap * hd * 4);
  L.part_ml = take(kPartialRowsCap * g.n_head * 2 * 4);
  L.total = o;
  return L;
}

// Device offsets of one plan inside the arena.
struct VariantLayout {
  size_t slots, qslots, items_valu, items_mfma, red_slot, red_off, red_rows;
};
struct ArenaLayout {
  size_t classes, lookup, lookup_off, dst_rows, updates;
  VariantLayout v[2];
  size_t total;
};

}  // namespace

struct kvattn_ctx {
  HostCore core;
  std::string err;
  int32_t device = 0;
  bool has_dev = false;
  std::vector<void*> K, V;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  WsLayout wl{};
  bool dev_ready = false;
  bool broken = false;        // a commit could not reach the device mirror
  void* stage[kStages] = {};
  size_t stage_cap[kStages] = {};
  char* stage_dev[kStages] = {};     // device view of each pinned staging buffer
  hipEvent_t ev[kStages] = {};
  bool ev_used[kStages] = {};
  // Staging reuse: an event recorded after the GPU work of a use shows that
  // use done.  Recording one per use put a marker in the stream every
  // ubatch, and each marker held the next kernel back ~6 us; so one event
  // covers up to kStagesPerEvent consecutive uses on one stream.
  int cover[kStages];                // stage whose event covers this stage's last use, -1 = none
  kvattn_ctx() { std::fill(cover, cover + kStages, -1); }
  int uncovered[kStagesPerEvent];    // uses since the last recorded event, in order
  int n_uncovered = 0;
  hipStream_t uncovered_stream = nullptr;
  int stage_next = 0;
  Plan plan[2];
  ArenaLayout al{};
  bool plan_ok = false;
  int plan_ubatch = -1;       // index in the split of the ubatch whose plan is on the device
  int32_t plan_serial = -1;
  std::vector<CellUpdate> upd;
  std::vector<char> blob;
  CsrArgs pending{};          // commit kernels' arguments, built by upload_commit
  bool commit_pending = false;
  // fused: the commit rides in the first store launch and reads the plan
  // from staging buffer fused_stage (as the first commit kernel does when
  // the commit runs on its own)
  bool pending_fused = false;
  int fused_stage = 0;
  const int32_t* fused_dst_rows = nullptr;
  // sequence-state restore reads the blob's metadata back through this
  void* peek = nullptr;
  size_t peek_cap = 0;
  char* peek_dev = nullptr;
  // kernel timing armed for the next attend call (kind -1: none)
  int32_t time_kind = -1;
  hipEvent_t time_ev[2] = {};
  hipEvent_t time_spare = nullptr;
  char* arena() { return ws + wl.arena; }

  int fail(int code, const std::string& msg) {
    err = msg;
    return code;
  }
  int hip_fail(hipError_t e, const char* where) {
    err = std::string(where) + ": " + hipGetErrorString(e);
    return KVATTN_EHIP;
  }
  template <class T>
  T* dptr(size_t off) { return reinterpret_cast<T*>(ws + off); }
};

#define HIP_TRY(ctx, expr)                              \
  do {                                                  \
    hipError_t e_ = (expr);                             \
    if (e_ != hipSuccess) return (ctx)->hip_fail(e_, #expr); \
  } while (0)

namespace {

int ensure_device(kvattn_ctx* c) {
  if (!c->has_dev) return c->fail(KVATTN_ENODEV, "context was created without device buffers");
  if (c->broken) return c->fail(KVATTN_ESTATE, "the device cell mirror is out of date (an earlier commit failed)");
  HIP_TRY(c, hipSetDevice(c->device));
  if (c->dev_ready) return KVATTN_OK;
  for (int i = 0; i < kStages; ++i) HIP_TRY(c, hipEventCreateWithFlags(&c->ev[i], hipEventDisableTiming));
  HIP_TRY(c, hipEventCreateWithFlags(&c->time_spare, hipEventDisableSystemFence));
  // the allocation-free entry point's static array, located once per device
  if (int rc = static_scratch_init(c->device))
    return c->fail(rc, "hipGetSymbolAddress of the static scratch array failed");
  // empty device mirror: every cell free
  const size_t sc = static_cast<size_t>(c->core.geo().n_stream) * c->core.geo().kv_size;
  HIP_TRY(c, hipMemset(c->ws + c->wl.cpos, 0xFF, sc * 4));
  HIP_TRY(c, hipMemset(c->ws + c->wl.cmask, 0, sc * sizeof(SeqSet)));
  HIP_TRY(c, hipDeviceSynchronize());
  c->dev_ready = true;
  return KVATTN_OK;
}

// Record one event after the uses not yet covered by one (on the stream
// they ran on); it covers all of them.
int cover_stages(kvattn_ctx* c) {
  if (c->n_uncovered == 0) return KVATTN_OK;
  const int last = c->uncovered[c->n_uncovered - 1];
  HIP_TRY(c, hipEventRecord(c->ev[last], c->uncovered_stream));
  c->ev_used[last] = true;
  for (int i = 0; i < c->n_uncovered; ++i) c->cover[c->uncovered[i]] = last;
  c->n_uncovered = 0;
  return KVATTN_OK;
}

// Stage st is read by GPU work just enqueued on stream s.
int release_stage(kvattn_ctx* c, int st, hipStream_t s) {
  if (c->n_uncovered > 0 && s != c->uncovered_stream)
    if (int rc = cover_stages(c)) return rc;
  c->cover[st] = -1;
  c->uncovered[c->n_uncovered++] = st;
  c->uncovered_stream = s;
  return c->n_uncovered == kStagesPerEvent ? cover_stages(c) : KVATTN_OK;
}

// The next pinned staging buffer of the ring, at least `bytes` large, once
// the GPU work that last read it has finished; release_stage must follow
// the enqueuing of the work that reads it now.  A cover event is never
// recorded again before the stages it covers come round (a stage comes
// round after kStages uses, the event's own stage no sooner), so waiting on
// it is waiting on the right point of the stream.
int acquire_stage(kvattn_ctx* c, size_t bytes, int* out) {
  const int st = c->stage_next;
  c->stage_next = (st + 1) % kStages;
  // (with kStages >= 2 kStagesPerEvent the last use is always covered by now)
  for (int i = 0; i < c->n_uncovered; ++i)
    if (c->uncovered[i] == st)
      if (int rc = cover_stages(c)) return rc;
  if (c->cover[st] >= 0) HIP_TRY(c, hipEventSynchronize(c->ev[c->cover[st]]));
  c->cover[st] = -1;
  if (c->stage_cap[st] < bytes) {
    if (c->stage[st]) HIP_TRY(c, hipHostFree(c->stage[st]));
    c->stage[st] = nullptr;
    c->stage_cap[st] = 0;
    const size_t cap = std::max<size_t>(bytes, 1 << 20);
    HIP_TRY(c, hipHostMalloc(&c->stage[st], cap, hipHostMallocDefault));
    c->stage_cap[st] = cap;
    void* dv = nullptr;
    HIP_TRY(c, hipHostGetDevicePointer(&dv, c->stage[st], 0));
    c->stage_dev[st] = static_cast<char*>(dv);
  }
  *out = st;
  return KVATTN_OK;
}

template <class T>
size_t put(std::vector<char>& blob, size_t at, const std::vector<T>& v) {
  if (!v.empty()) std::memcpy(blob.data() + at, v.data(), v.size() * sizeof(T));
  return at;
}

// Plan of the committed ubatch k -> pinned staging -> device arena, then the
// mirror update and the cell-list build, all on stream s.
int upload_commit(kvattn_ctx* c, int k, hipStream_t s, bool may_fuse) {
  const Geometry& g = c->core.geo();
  UbatchRec& u = c->core.ubatches()[k];
  std::string e0, e1;
  // both variants share one class table: the output-only plan takes the
  // class cap the full plan settled on
  int rc0 = c->core.build_plan(k, false, kMaxClasses, true, c->plan[0], e0);
  int rc1 = rc0 ? rc0 : c->core.build_plan(k, true, c->plan[0].class_cap, false, c->plan[1], e1);
  c->plan_ok = rc0 == KVATTN_OK && rc1 == KVATTN_OK;
  if (!c->plan_ok) {
    c->plan[0] = Plan();
    c->plan[1] = Plan();
  }
  // destination rows of the store: the slots' cells, then the separate
  // copies; after them the source slot of each copy
  const size_t n_slot = u.cells.size(), n_copy = u.copy_cell.size();
  std::vector<int32_t> dst(n_slot + 2 * n_copy);
  for (size_t i = 0; i < n_slot; ++i)
    dst[i] = static_cast<int32_t>(static_cast<int64_t>(u.stream[i]) * g.kv_size + u.cells[i]);
  for (size_t i = 0; i < n_copy; ++i) {
    dst[n_slot + i] = static_cast<int32_t>(static_cast<int64_t>(u.copy_stream[i]) * g.kv_size + u.copy_cell[i]);
    dst[n_slot + n_copy + i] = u.copy_src[i];
  }

  // arena layout.  A plan too large for the arena is dropped like one
  // build_plan refused: the mirror update and the stores still run, attend
  // reports the missing plan.  The arena is sized (16 MiB + 48 B per cell)
  // so that the store rows and mirror updates alone always fit; if they did
  // not, nothing is launched and the context's previous layout stays.
  auto layout = [&](ArenaLayout& A) {
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
    const Plan& P0 = c->plan[0];
    A.classes = take(P0.classes.size() * sizeof(ClassInfo));
    A.lookup = take(P0.lookup.size() * sizeof(LookupEntry));
    A.lookup_off = take(P0.lookup_off.size() * 4);
    A.dst_rows = take(dst.size() * 4);
    for (int v = 0; v < 2; ++v) {
      const Plan& P = c->plan[v];
      A.v[v].slots = take(P.slots.size() * sizeof(SlotInfo));
      A.v[v].qslots = take(P.qlist.size() * sizeof(SlotInfo));
      A.v[v].items_valu = take(P.items_valu.size() * sizeof(WorkItem));
      A.v[v].items_mfma = take(P.items_mfma.size() * sizeof(WorkItem));
      A.v[v].red_slot = take(P.red_slot.size() * 4);
      A.v[v].red_off = take(P.red_off.size() * 4);
      A.v[v].red_rows = take(P.red_rows.size() * 4);
    }
    A.updates = take(c->upd.size() * sizeof(CellUpdate));
    A.total = o;
  };
  ArenaLayout A{};
  layout(A);
  if (A.total > c->wl.arena_bytes && c->plan_ok) {
    c->plan_ok = false;
    c->plan[0] = Plan();
    c->plan[1] = Plan();
    rc0 = KVATTN_ENOMEM;
    e0 = "ubatch plan exceeds the workspace plan arena";
    layout(A);
  }
  if (A.total > c->wl.arena_bytes) {
    c->plan_ok = false;
    return c->fail(KVATTN_ENOMEM, "store rows and cell updates exceed the workspace plan arena");
  }
  c->al = A;
  const Plan& P0 = c->plan[0];
  // stage
  int st = 0;
  if (int rc = acquire_stage(c, A.total, &st)) return rc;
  char* b = static_cast<char*>(c->stage[st]);
  auto copy = [&](size_t at, const void* src, size_t bytes) { if (bytes) std::memcpy(b + at, src, bytes); };
  copy(A.classes, P0.classes.data(), P0.classes.size() * sizeof(ClassInfo));
  copy(A.lookup, P0.lookup.data(), P0.lookup.size() * sizeof(LookupEntry));
  copy(A.lookup_off, P0.lookup_off.data(), P0.lookup_off.size() * 4);
  copy(A.dst_rows, dst.data(), dst.size() * 4);
  for (int v = 0; v < 2; ++v) {
    const Plan& P = c->plan[v];
    copy(A.v[v].slots, P.slots.data(), P.slots.size() * sizeof(SlotInfo));
    // each class's queries as slot records in class order (one load per
    // query row in the kernels instead of a list entry, then its slot)
    SlotInfo* qs = reinterpret_cast<SlotInfo*>(b + A.v[v].qslots);
    for (size_t i = 0; i < P.qlist.size(); ++i) qs[i] = P.slots[P.qlist[i]];
    copy(A.v[v].items_valu, P.items_valu.data(), P.items_valu.size() * sizeof(WorkItem));
    copy(A.v[v].items_mfma, P.items_mfma.data(), P.items_mfma.size() * sizeof(WorkItem));
    copy(A.v[v].red_slot, P.red_slot.data(), P.red_slot.size() * 4);
    copy(A.v[v].red_off, P.red_off.data(), P.red_off.size() * 4);
    copy(A.v[v].red_rows, P.red_rows.data(), P.red_rows.size() * 4);
  }
  copy(A.updates, c->upd.data(), c->upd.size() * sizeof(CellUpdate));
  char* arena = c->arena();
  CsrArgs ca{};
  ca.cpos = c->dptr<int32_t>(c->wl.cpos);
  ca.cmask = c->dptr<SeqSet>(c->wl.cmask);
  ca.cellcls = c->dptr<int32_t>(c->wl.cellcls);
  ca.counts = c->dptr<int32_t>(c->wl.counts);
  ca.csr_cell = c->dptr<int32_t>(c->wl.csr_cell);
  ca.csr_pos = c->dptr<int32_t>(c->wl.csr_pos);
  ca.csr_mask = c->dptr<SeqSet>(c->wl.csr_mask);
  ca.n_updates = static_cast<int32_t>(c->upd.size());
  ca.n_classes = c->plan_ok ? static_cast<int32_t>(P0.classes.size()) : 0;
  ca.n_seg = P0.n_seg;
  ca.kv_size = g.kv_size;
  ca.n_kv = P0.n_kv;
  ca.n_stream = g.n_stream;
  ca.csr_cap = g.n_stream * g.kv_size;
  ca.tile_min = c->dptr<int32_t>(c->wl.tile_min);
  ca.tile_max = c->dptr<int32_t>(c->wl.tile_max);
  ca.max_class_tiles = P0.max_class_tiles;
  ca.n_lookup = static_cast<int32_t>(P0.lookup.size());
  // A small commit that a store launch will carry reads its tables straight
  // from the pinned staging buffer, and that launch copies the plan into the
  // device arena: no separate copy (and its latency) sits in the stream.
  // Otherwise the first commit kernel copies the plan into the arena while
  // it applies the mirror updates (read from the staging buffer too), and
  // the later ones read the arena: no copy command sits in the stream either
  // (a host->device copy between two kernels cost ~20 us per ubatch).
  const bool fused = may_fuse && commit_is_small(ca);
  const char* src = fused ? c->stage_dev[st] : arena;
  ca.classes = reinterpret_cast<const ClassInfo*>(src + A.classes);
  ca.lookup = reinterpret_cast<const LookupEntry*>(src + A.lookup);
  ca.lookup_off = reinterpret_cast<const int32_t*>(src + A.lookup_off);
  ca.updates = reinterpret_cast<const CellUpdate*>(c->stage_dev[st] + A.updates);
  ca.plan_src = c->stage_dev[st];
  ca.plan_dst = arena;
  ca.plan_n16 = static_cast<int32_t>((A.total + 15) / 16);
  c->fused_stage = st;
  if (fused) c->fused_dst_rows = reinterpret_cast<const int32_t*>(c->stage_dev[st] + A.dst_rows);
  // launched by the caller: alone, or inside the first store launch
  c->pending_fused = fused;
  c->pending = ca;
  c->commit_pending = true;
  c->plan_ubatch = k;
  c->plan_serial = c->core.split_serial();
  if (!c->plan_ok) return c->fail(rc0 ? rc0 : rc1, rc0 ? e0 : e1);
  return KVATTN_OK;
}

int check_ubatch(kvattn_ctx* c, const kvattn_ubatch* ub, int* k) {
  if (!ub) return c->fail(KVATTN_EINVAL, "ubatch is NULL");
  *k = c->core.find(ub->id);
  if (*k < 0) return c->fail(KVATTN_ESTATE, "stale ubatch: it belongs to an earlier split");
  return KVATTN_OK;
}

int check_layers(kvattn_ctx* c, int32_t il0, int32_t n_il) {
  if (il0 < 0 || n_il < 0 || il0 + n_il > c->core.geo().n_layer)
    return c->fail(KVATTN_EINVAL, "layer range outside [0, n_layer)");
  return KVATTN_OK;
}

bool plan_current(kvattn_ctx* c, int k) {
  return c->plan_ubatch == k && c->plan_serial == c->core.split_serial() && c->core.latest_committed() == k;
}

}  // namespace

extern "C" {

size_t kvattn_workspace_bytes(const kvattn_params* p) {
  if (!p) return 0;
  Geometry g;
  std::string err;
  if (make_geometry(*p, g, err)) return 0;
  return ws_layout(g).total;
}

size_t kvattn_cache_bytes(const kvattn_params* p) {
  if (!p) return 0;
  return 2ull * static_cast<size_t>(p->n_layer) * p->n_stream * p->kv_size * p->n_head_kv * p->head_dim * 2ull;
}

int kvattn_create(const kvattn_params* p, kvattn_ctx** out) {
  if (!p || !out) return KVATTN_EINVAL;
  *out = nullptr;
  kvattn_ctx* c = new (std::nothrow) kvattn_ctx();
  if (!c) return KVATTN_ENOMEM;
  int rc = c->core.init(*p, c->err);
  if (rc) {
    delete c;
    return rc;
  }
  const Geometry& g = c->core.geo();
  c->device = p->device;
  if (p->k_layers) {
    c->wl = ws_layout(g);
    if (!p->v_layers || !p->workspace || p->workspace_bytes < c->wl.total) {
      delete c;
      return KVATTN_EINVAL;
    }
    for (int l = 0; l < g.n_layer; ++l) {
      if (!p->k_layers[l] || !p->v_layers[l]) {
        delete c;
        return KVATTN_EINVAL;
      }
      c->K.push_back(p->k_layers[l]);
      c->V.push_back(p->v_layers[l]);
    }
    c->ws = static_cast<char*>(p->workspace);
    c->ws_bytes = p->workspace_bytes;
    c->has_dev = true;
  }
  c->core.prow_max = static_cast<int32_t>(std::min<int64_t>(4096, kPartialRowsCap));
  *out = c;
  return KVATTN_OK;
}

void kvattn_destroy(kvattn_ctx* c) {
  if (!c) return;
  if (c->dev_ready) {
    (void)hipSetDevice(c->device);
    (void)hipDeviceSynchronize();      // covers the staging uses no event covers yet
    for (int i = 0; i < kStages; ++i) {
      if (c->ev_used[i]) (void)hipEventSynchronize(c->ev[i]);
      if (c->ev[i]) (void)hipEventDestroy(c->ev[i]);
      if (c->stage[i]) (void)hipHostFree(c->stage[i]);
    }
    if (c->peek) (void)hipHostFree(c->peek);
    if (c->time_spare) (void)hipEventDestroy(c->time_spare);

  }
  delete c;
}

int kvattn_split(kvattn_ctx* c, const kvattn_batch* b, kvattn_ubatch* ubs, int32_t cap, int32_t* n_ubs,
                 int32_t* output_ids) {
  if (!c) return KVATTN_EINVAL;
  if (!b || !n_ubs || (cap > 0 && !ubs)) return c->fail(KVATTN_EINVAL, "NULL argument");
  c->err.clear();
  *n_ubs = 0;
  // a split cannot be undone, so check the capacity by dry-running the count
  int rc = c->core.split(*b, output_ids, c->err);
  if (rc) return rc;
  auto& v = c->core.ubatches();
  if (static_cast<int32_t>(v.size()) > cap) {
    kvattn_batch empty{0, nullptr, nullptr, nullptr, nullptr};
    std::string e;
    c->core.split(empty, nullptr, e);   // releases the reservation
    return c->fail(KVATTN_EINVAL, "ubatch array too small: need " + std::to_string(v.size()));
  }
  for (size_t k = 0; k < v.size(); ++k) {
    const UbatchRec& u = v[k];
    kvattn_ubatch& o = ubs[k];
    o.id = u.id;
    o.n_tokens = static_cast<int32_t>(u.pos.size());
    o.n_seq_tokens = u.n_seq_tokens;
    o.n_seqs = u.n_seqs;
    o.n_seqs_unq = static_cast<int32_t>(u.seq_unq.size());
    o.n_outputs = u.n_outputs;
    o.pos = u.pos.data();
    o.n_seq_id = u.n_seq_id.data();
    o.seq_id = u.seq_ptr.data();
    o.seq_id_unq = u.seq_unq.data();
    o.output = u.output.data();
    o.src_idx = u.src.data();
    o.stream = u.stream.data();
    o.cells = u.cells.data();
    o.n_copies = static_cast<int32_t>(u.copy_cell.size());
    o.copy_src = u.copy_src.data();
    o.copy_stream = u.copy_stream.data();
    o.copy_cell = u.copy_cell.data();
  }
  *n_ubs = static_cast<int32_t>(v.size());
  return KVATTN_OK;
}

int kvattn_store(kvattn_ctx* c, const kvattn_ubatch* ub, int32_t il0, int32_t n_il, const void* const* k_cur,
                 const void* const* v_cur, void* hip_stream) {
  if (!c) return KVATTN_EINVAL;
  int k, rc;
  if ((rc = check_ubatch(c, ub, &k)) || (rc = check_layers(c, il0, n_il))) return rc;
  if (n_il > 0 && (!k_cur || !v_cur)) return c->fail(KVATTN_EINVAL, "k_cur / v_cur is NULL");
  for (int32_t i = 0; i < n_il; ++i)
    if (!k_cur[i] || !v_cur[i]) return c->fail(KVATTN_EINVAL, "NULL k_cur / v_cur entry");
  UbatchRec& u = c->core.ubatches()[k];
  if (!c->has_dev && n_il == 0) {
    // host-only context: a zero-layer store commits the placement and nothing else
    if (u.committed) return KVATTN_OK;
    if (il0 != 0) return c->fail(KVATTN_ESTATE, "the first store of a ubatch must start at layer 0");
    c->upd.clear();
    return c->core.commit(k, &c->upd, c->err);
  }
  if ((rc = ensure_device(c))) return rc;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (!u.committed) {
    if (il0 != 0) return c->fail(KVATTN_ESTATE, "the first store of a ubatch must start at layer 0");
    c->upd.clear();
    if ((rc = c->core.commit(k, &c->upd, c->err))) return rc;
    rc = upload_commit(c, k, s, n_il > 0);
    // ENOMEM with the commit still pending: only the attention plan is
    // missing (attend reports it).  Without a pending commit nothing is
    // launched; the host table is committed but the device mirror cannot
    // follow, so every later device call on this context is refused.
    if (rc && !c->commit_pending) {
      c->broken = true;
      return rc;
    }
  } else if (c->core.latest_committed() != k || !plan_current(c, k)) {
    return c->fail(KVATTN_ESTATE, "only the most recently committed ubatch can be stored again");
  }
  // a small commit rides in one extra workgroup of the first store launch
  // (it does not depend on the stores); otherwise it runs first on its own
  bool fuse = false;
  if (c->commit_pending) {
    c->commit_pending = false;
    fuse = c->pending_fused;
    if (!fuse) {
      HIP_TRY(c, launch_commit(c->pending, s));
      if (int rc2 = release_stage(c, c->fused_stage, s)) return rc2;
    }
  }
  const Geometry& g = c->core.geo();
  StoreArgs a{};
  a.dst_rows = reinterpret_cast<const int32_t*>(c->arena() + c->al.dst_rows);
  a.n_src = static_cast<int32_t>(u.cells.size());
  a.n_rows = a.n_src + static_cast<int32_t>(u.copy_cell.size());
  a.E = g.E();
  for (int32_t l0 = 0; l0 < n_il; l0 += kMaxLayersPerLaunch) {
    const int n = std::min<int32_t>(kMaxLayersPerLaunch, n_il - l0);
    for (int i = 0; i < n; ++i) {
      a.k_cur[i] = static_cast<const float*>(k_cur[l0 + i]);
      a.v_cur[i] = static_cast<const float*>(v_cur[l0 + i]);
      a.k[i] = static_cast<_Float16*>(c->K[il0 + l0 + i]);
      a.v[i] = static_cast<_Float16*>(c->V[il0 + l0 + i]);
    }
    if (fuse && l0 == 0) {
      StoreArgs af = a;
      af.dst_rows = c->fused_dst_rows;     // the arena copy lands during this launch
      HIP_TRY(c, launch_store_commit(af, n, c->pending, s));
      if (int rc2 = release_stage(c, c->fused_stage, s)) return rc2;
    } else {
      HIP_TRY(c, launch_store(a, n, s));
    }
  }
  return rc;
}

int kvattn_attend(kvattn_ctx* c, const kvattn_ubatch* ub, int32_t il0, int32_t n_il, const void* const* q,
                  void* const* out, int32_t only_outputs, void* hip_stream) {
  if (!c) return KVATTN_EINVAL;
  return kvattn::attend_with_partials(c, ub, il0, n_il, q, out, only_outputs, hip_stream, nullptr, nullptr, 0);
}

}  // extern "C"

int kvattn::attend_with_partials(kvattn_ctx* c, const kvattn_ubatch* ub, int32_t il0, int32_t n_il,
                                 const void* const* q, void* const* out, int32_t only_outputs, void* hip_stream,
                                 float* part_acc, float* part_ml, int64_t part_rows) {
  if (!c) return KVATTN_EINVAL;
  // kernel timing is used by this call alone, whatever its outcome
  const int32_t tkind = c->time_kind;
  const hipEvent_t tev0 = c->time_ev[0], tev1 = c->time_ev[1];
  c->time_kind = -1;
  c->time_ev[0] = c->time_ev[1] = nullptr;
  bool timed = false;
  // the armed events of a call that launches no kernel of the chosen kind
  // are recorded back to back on its stream (elapsed time about zero)
  auto untimed = [&](hipStream_t st) -> int {
    if (tkind < 0 || timed) return KVATTN_OK;
    HIP_TRY(c, hipEventRecord(tev0, st));
    HIP_TRY(c, hipEventRecord(tev1, st));
    return KVATTN_OK;
  };
  int k, rc;
  if ((rc = check_ubatch(c, ub, &k)) || (rc = check_layers(c, il0, n_il))) return rc;
  if (n_il > 0 && (!q || !out)) return c->fail(KVATTN_EINVAL, "q / out is NULL");
  if ((rc = ensure_device(c))) return rc;
  if (!c->core.ubatches()[k].committed) return c->fail(KVATTN_ESTATE, "attend before the ubatch was stored");
  if (!plan_current(c, k)) return c->fail(KVATTN_ESTATE, "attend must follow its own ubatch's store");
  if (!c->plan_ok) return c->fail(KVATTN_ENOMEM, "no work plan for this ubatch (workspace too small)");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const Geometry& g = c->core.geo();
  const int v = only_outputs ? 1 : 0;
  const Plan& P = c->plan[v];
  if (P.slots.empty()) return untimed(s);     // no query rows (e.g. no flagged slot)
  const VariantLayout& VL = c->al.v[v];
  char* arena = c->arena();
  AttnArgs a{};
  a.slots = reinterpret_cast<const SlotInfo*>(arena + VL.slots);
  a.classes = reinterpret_cast<const ClassInfo*>(arena + c->al.classes);
  a.qslots = reinterpret_cast<const SlotInfo*>(arena + VL.qslots);
  a.csr_cell = c->dptr<int32_t>(c->wl.csr_cell);
  a.csr_pos = c->dptr<int32_t>(c->wl.csr_pos);
  a.csr_mask = c->dptr<SeqSet>(c->wl.csr_mask);
  a.tile_min = c->dptr<int32_t>(c->wl.tile_min);
  a.tile_max = c->dptr<int32_t>(c->wl.tile_max);
  // split-K partials: the workspace's region, or the caller's (the
  // allocation-free entry point), which must hold one launch's rows
  if (!part_acc) {
    part_acc = c->dptr<float>(c->wl.part_acc);
    part_ml = c->dptr<float>(c->wl.part_ml);
    part_rows = kPartialRowsCap;
  }
  if (P.n_partial_rows > part_rows)
    return c->fail(KVATTN_ENOMEM, "split-K partial rows of one layer (" + std::to_string(P.n_partial_rows) +
                                      ") exceed the partial buffer (" + std::to_string(part_rows) + " rows)");
  a.part_acc = part_acc;
  a.part_ml = part_ml;
  a.red_slot = reinterpret_cast<const int32_t*>(arena + VL.red_slot);
  a.red_off = reinterpret_cast<const int32_t*>(arena + VL.red_off);
  a.red_rows = reinterpret_cast<const int32_t*>(arena + VL.red_rows);
  a.rows_per_layer = P.n_partial_rows;
  a.kv_size = g.kv_size;
  a.n_head = g.n_head;
  a.n_head_kv = g.n_head_kv;
  a.causal = g.causal;
  a.swa = g.swa;
  a.scale_log2e = g.kq_scale * 1.4426950408889634f;
  a.layer_bytes = static_cast<uint32_t>(static_cast<size_t>(g.n_stream) * g.kv_size * g.E() * 2);
  const int64_t per = std::max<int64_t>(1, P.n_partial_rows);
  const int32_t chunk = static_cast<int32_t>(std::min<int64_t>(kMaxLayersPerLaunch, part_rows / per));
  const int32_t n_red = static_cast<int32_t>(P.red_slot.size());
  const int32_t kind_items[3] = {static_cast<int32_t>(P.items_mfma.size()), static_cast<int32_t>(P.items_valu.size()),
                                 n_red};
  // A plan with both matrix-core and vector-ALU items (a shared prefix beside
  // each sequence's own cells, or prompt chunks beside decode tokens) runs
  // them in one launch, where the shape allows it
  const bool both = kind_items[0] > 0 && kind_items[1] > 0 && g.swa == 0 && tkind != KVATTN_KERNEL_MFMA &&
                    tkind != KVATTN_KERNEL_VALU && attn_both_supported(g.head_dim, g.G(), g.E());
  for (int32_t l0 = 0; l0 < n_il; l0 += chunk) {
    const int n = std::min<int32_t>(chunk, n_il - l0);
    // The timed kernel's first launch starts the events and its last one
    // stops them.  Only one launch per call carries the caller's events (the
    // runtime holds the host thread at a second event-carrying launch until
    // the first has run): when the layers are cut into several launches, the
    // first carries the start event (with a spare event of the context as
    // its stop) and the stop event is recorded on the stream right after
    // the last one, so it stamps that kernel's completion.
    KernelEvents ev[3];
    bool stop_after = false;
    if (tkind >= 0 && kind_items[tkind] > 0) {
      const bool first = l0 == 0, last = l0 + n >= n_il;
      if (first) {
        ev[tkind].start = tev0;
        ev[tkind].stop = last ? tev1 : c->time_spare;
      } else if (last) {
        stop_after = true;
      }
      timed = true;
    }
    for (int i = 0; i < n; ++i) {
      if (!q[l0 + i] || !out[l0 + i]) return c->fail(KVATTN_EINVAL, "NULL q / out entry");
      a.q[i] = static_cast<const float*>(q[l0 + i]);
      a.o[i] = static_cast<float*>(out[l0 + i]);
      a.k[i] = static_cast<const _Float16*>(c->K[il0 + l0 + i]);
      a.v[i] = static_cast<const _Float16*>(c->V[il0 + l0 + i]);
    }
    // matrix-core items first: their workgroups need most of a CU's LDS and
    // would otherwise wait for vector-ALU workgroups to drain
    a.items = reinterpret_cast<const WorkItem*>(arena + VL.items_mfma);
    a.n_items = static_cast<int32_t>(P.items_mfma.size());
    if (both) {
      // both kinds in one launch (unless one kind's kernel is being timed)
      a.items2 = reinterpret_cast<const WorkItem*>(arena + VL.items_valu);
      a.n_items2 = static_cast<int32_t>(P.items_valu.size());
      HIP_TRY(c, launch_attn_both(a, n, g.head_dim, g.G(), s));
    } else {
      HIP_TRY(c, launch_attn_mfma(a, n, g.head_dim, g.G(), s, ev[KVATTN_KERNEL_MFMA]));
      if (stop_after && tkind == KVATTN_KERNEL_MFMA) HIP_TRY(c, hipEventRecord(tev1, s));
      a.items = reinterpret_cast<const WorkItem*>(arena + VL.items_valu);
      a.n_items = static_cast<int32_t>(P.items_valu.size());
      HIP_TRY(c, launch_attn_valu(a, n, g.head_dim, g.G(), s, ev[KVATTN_KERNEL_VALU]));
      if (stop_after && tkind == KVATTN_KERNEL_VALU) HIP_TRY(c, hipEventRecord(tev1, s));
    }
    HIP_TRY(c, launch_reduce(a, n_red, n, g.head_dim, s, ev[KVATTN_KERNEL_MERGE]));
    if (stop_after && tkind == KVATTN_KERNEL_MERGE) HIP_TRY(c, hipEventRecord(tev1, s));
  }
  return untimed(s);
}

extern "C" {

int kvattn_time_next_attend(kvattn_ctx* c, int32_t kind, void* start_event, void* stop_event) {
  if (!c) return KVATTN_EINVAL;
  if (kind < 0) {
    c->time_kind = -1;
    c->time_ev[0] = c->time_ev[1] = nullptr;
    return KVATTN_OK;
  }
  if (kind > KVATTN_KERNEL_MERGE) return c->fail(KVATTN_EINVAL, "unknown kernel kind " + std::to_string(kind));
  if (!start_event || !stop_event) return c->fail(KVATTN_EINVAL, "kernel timing needs both events");
  c->time_kind = kind;
  c->time_ev[0] = static_cast<hipEvent_t>(start_event);
  c->time_ev[1] = static_cast<hipEvent_t>(stop_event);
  return KVATTN_OK;
}

int32_t kvattn_n_kv(const kvattn_ctx* c) { return c ? c->core.n_kv() : 0; }

int kvattn_get_mask(kvattn_ctx* c, const kvattn_ubatch* ub, void* d_mask, size_t cap_elems, int32_t* n_kv,
                    void* hip_stream) {
  if (!c) return KVATTN_EINVAL;
  int k, rc;
  if ((rc = check_ubatch(c, ub, &k))) return rc;
  if ((rc = ensure_device(c))) return rc;
  if (!plan_current(c, k)) return c->fail(KVATTN_ESTATE, "mask is only kept for the latest committed ubatch");
  const Plan& P = c->plan[0];
  const int32_t T = static_cast<int32_t>(c->core.ubatches()[k].pos.size());
  if (n_kv) *n_kv = P.n_kv;
  if (static_cast<size_t>(T) * P.n_kv > cap_elems || !d_mask) return c->fail(KVATTN_EINVAL, "mask buffer too small");
  MaskArgs a{};
  a.cpos = c->dptr<int32_t>(c->wl.cpos);
  a.cmask = c->dptr<SeqSet>(c->wl.cmask);
  a.slots = reinterpret_cast<const SlotInfo*>(c->arena() + c->al.v[0].slots);
  a.mask = static_cast<uint16_t*>(d_mask);
  a.n_rows = T;
  a.n_kv = P.n_kv;
  a.kv_size = c->core.geo().kv_size;
  a.causal = c->core.geo().causal;
  a.swa = c->core.geo().swa;
  HIP_TRY(c, launch_mask(a, static_cast<hipStream_t>(hip_stream)));
  return KVATTN_OK;
}

int kvattn_get_classes(kvattn_ctx* c, int32_t* n_classes, int32_t* cls_stream, uint64_t* cls_mask,
                       int32_t* cls_count, int32_t cap_classes, int32_t* n_cells, int32_t* cells, int32_t cap_cells,
                       void* hip_stream) {
  if (!c) return KVATTN_EINVAL;
  int rc;
  if ((rc = ensure_device(c))) return rc;
  if (c->plan_ubatch < 0 || !plan_current(c, c->plan_ubatch)) return c->fail(KVATTN_ESTATE, "no committed ubatch");
  const Plan& P = c->plan[0];
  if (n_classes) *n_classes = static_cast<int32_t>(P.classes.size());
  if (n_cells) *n_cells = P.total_cells;
  for (int32_t i = 0; i < std::min<int32_t>(cap_classes, static_cast<int32_t>(P.classes.size())); ++i) {
    if (cls_stream) cls_stream[i] = P.classes[i].stream;
    if (cls_mask)
      for (int w = 0; w < kSeqWords; ++w) cls_mask[static_cast<size_t>(i) * kSeqWords + w] = P.classes[i].mask.w[w];
    if (cls_count) cls_count[i] = P.classes[i].n_cells;
  }
  const int32_t n = std::min(cap_cells, P.total_cells);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (cells && n > 0)
    HIP_TRY(c, hipMemcpyAsync(cells, c->ws + c->wl.csr_cell, static_cast<size_t>(n) * 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(c, hipStreamSynchronize(s));
  return KVATTN_OK;
}

int kvattn_get_cells(const kvattn_ctx* c, int32_t stream, int32_t* pos, uint64_t* seqmask) {
  if (!c || stream < 0 || stream >= c->core.geo().n_stream) return KVATTN_EINVAL;
  c->core.get_cells(stream, pos, seqmask);
  return KVATTN_OK;
}

int kvattn_seq_rm(kvattn_ctx* c, int32_t seq_id, int32_t p0, int32_t p1) {
  if (!c) return KVATTN_EINVAL;
  int rc = c->core.seq_rm(seq_id, p0, p1);
  if (rc) return c->fail(rc, "sequence id out of range");
  return KVATTN_OK;
}

int32_t kvattn_seq_pos_max(const kvattn_ctx* c, int32_t seq_id) { return c ? c->core.seq_pos_max(seq_id) : -1; }

}  // extern "C"

// ---- sequence state ("Opening the .bin dump") ------------------------------

namespace {

constexpr uint32_t kStateMagic = 0x5353564Bu;     // "KVSS" little-endian
constexpr uint32_t kStateVersion = 1;
constexpr size_t kStateFixed = 80;
constexpr size_t kStateRecordHeader = 12;

struct StateGeom {
  size_t n, row, rec0, stride, total;
};

StateGeom state_geom(const Geometry& g, size_t n) {
  StateGeom sg;
  sg.n = n;
  sg.row = static_cast<size_t>(g.E()) * 2;
  sg.rec0 = kStateFixed + 4 * n;
  sg.stride = kStateRecordHeader + n * sg.row;
  sg.total = sg.rec0 + 2 * static_cast<size_t>(g.n_layer) * sg.stride;
  return sg;
}

int ensure_peek(kvattn_ctx* c, size_t bytes) {
  if (c->peek_cap >= bytes) return KVATTN_OK;
  if (c->peek) HIP_TRY(c, hipHostFree(c->peek));
  c->peek = nullptr;
  c->peek_cap = 0;
  const size_t cap = std::max<size_t>(bytes, 1 << 16);
  HIP_TRY(c, hipHostMalloc(&c->peek, cap, hipHostMallocDefault));
  c->peek_cap = cap;
  void* dv = nullptr;
  HIP_TRY(c, hipHostGetDevicePointer(&dv, c->peek, 0));
  c->peek_dev = static_cast<char*>(dv);
  return KVATTN_OK;
}

template <class T>
T rd(const char* p, size_t at) {
  T v;
  std::memcpy(&v, p + at, sizeof(T));
  return v;
}

StateArgs state_args(kvattn_ctx* c, const StateGeom& sg, int32_t il0, int32_t n_il) {
  StateArgs a{};
  for (int i = 0; i < n_il; ++i) {
    a.k[i] = static_cast<_Float16*>(c->K[il0 + i]);
    a.v[i] = static_cast<_Float16*>(c->V[il0 + i]);
  }
  a.n = static_cast<int32_t>(sg.n);
  a.n_layer = c->core.geo().n_layer;
  a.il0 = il0;
  a.n_il = n_il;
  a.row_words = static_cast<int32_t>(sg.row / 4);
  a.rec0 = sg.rec0;
  a.rec_stride = sg.stride;
  return a;
}

// Placement of n cells at pos[] for seq (all-or-nothing), then the rows of
// the blob's records into them on stream s (device contexts only).
int restore_rows(kvattn_ctx* c, int32_t seq, const void* src, const int32_t* pos, int32_t n, hipStream_t s) {
  const Geometry& g = c->core.geo();
  std::vector<int32_t> cells;
  int rc;
  if ((rc = c->core.seq_restore(seq, pos, n, cells, c->err))) return rc;
  if (n == 0 || !c->has_dev) return KVATTN_OK;
  const StateGeom sg = state_geom(g, static_cast<size_t>(n));
  int st = 0;
  if ((rc = acquire_stage(c, 4 * sg.n, &st))) return rc;
  int32_t* rows = static_cast<int32_t*>(c->stage[st]);
  const int32_t sid = seq % g.n_stream;
  for (size_t i = 0; i < sg.n; ++i) rows[i] = sid * g.kv_size + cells[i];
  for (int32_t l0 = 0; l0 < g.n_layer; l0 += kMaxLayersPerLaunch) {
    const int32_t n_il = std::min<int32_t>(kMaxLayersPerLaunch, g.n_layer - l0);
    StateArgs a = state_args(c, sg, l0, n_il);
    a.cells = reinterpret_cast<const int32_t*>(c->stage_dev[st]);
    a.blob_r = static_cast<const uint32_t*>(src);
    HIP_TRY(c, launch_state_copy(a, false, s));
  }
  if ((rc = release_stage(c, st, s))) return rc;
  return KVATTN_OK;
}

}  // namespace

bool kvattn::ctx_has_device(const kvattn_ctx* c) { return c && c->has_dev; }

int kvattn::state_restore_known(kvattn_ctx* c, int32_t seq, const void* src, const int32_t* pos, int32_t n,
                        void* hip_stream) {
  if (!c || n < 0 || (n > 0 && !pos)) return KVATTN_EINVAL;
  if (c->has_dev) {
    if (!src || (reinterpret_cast<uintptr_t>(src) & 3)) return c->fail(KVATTN_EINVAL, "src is NULL or not 4-byte aligned");
    if (int rc = ensure_device(c)) return rc;
  }
  return restore_rows(c, seq, src, pos, n, static_cast<hipStream_t>(hip_stream));
}

extern "C" {

int kvattn_seq_state_size(const kvattn_ctx* c, int32_t seq_id, size_t* bytes) {
  if (!c || !bytes) return KVATTN_EINVAL;
  std::vector<int32_t> cells, pos;
  if (c->core.seq_cells(seq_id, cells, pos) < 0) return KVATTN_EINVAL;
  *bytes = state_geom(c->core.geo(), cells.size()).total;
  return KVATTN_OK;
}

int kvattn_seq_state_save(kvattn_ctx* c, int32_t seq_id, void* dst, size_t cap, size_t* written, void* hip_stream) {
  if (!c) return KVATTN_EINVAL;
  if (!dst || (reinterpret_cast<uintptr_t>(dst) & 3)) return c->fail(KVATTN_EINVAL, "dst is NULL or not 4-byte aligned");
  std::vector<int32_t> cells, pos;
  const int st_id = c->core.seq_cells(seq_id, cells, pos);
  if (st_id < 0) return c->fail(KVATTN_EINVAL, "sequence id out of range");
  const Geometry& g = c->core.geo();
  const StateGeom sg = state_geom(g, cells.size());
  if (cap < sg.total) return c->fail(KVATTN_ENOMEM, "dst is smaller than kvattn_seq_state_size");
  int rc;
  if ((rc = ensure_device(c))) return rc;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  // staging: leading metadata (what the blob starts with), then the rows
  // to gather (stream * kv_size + cell)
  int st = 0;
  if ((rc = acquire_stage(c, sg.rec0 + 4 * sg.n, &st))) return rc;
  char* b = static_cast<char*>(c->stage[st]);
  std::memset(b, 0, kStateFixed);
  const uint32_t head[8] = {kStateMagic, kStateVersion, static_cast<uint32_t>(g.n_layer),
                            static_cast<uint32_t>(g.n_head_kv), static_cast<uint32_t>(g.head_dim),
                            static_cast<uint32_t>(sg.n), kStateTypeF16, kStateTypeF16};
  std::memcpy(b, head, sizeof(head));
  const uint64_t sizes[3] = {sg.row, sg.rec0, sg.total};
  std::memcpy(b + 32, sizes, sizeof(sizes));
  if (sg.n) std::memcpy(b + kStateFixed, pos.data(), 4 * sg.n);
  int32_t* rows = reinterpret_cast<int32_t*>(b + sg.rec0);
  for (size_t i = 0; i < sg.n; ++i) rows[i] = st_id * g.kv_size + cells[i];
  for (int32_t l0 = 0; l0 < g.n_layer; l0 += kMaxLayersPerLaunch) {
    const int32_t n_il = std::min<int32_t>(kMaxLayersPerLaunch, g.n_layer - l0);
    StateArgs a = state_args(c, sg, l0, n_il);
    a.cells = reinterpret_cast<const int32_t*>(c->stage_dev[st] + sg.rec0);
    a.blob_w = static_cast<uint32_t*>(dst);
    a.prefix = reinterpret_cast<const uint32_t*>(c->stage_dev[st]);
    a.prefix_words = static_cast<int32_t>(sg.rec0 / 4);
    HIP_TRY(c, launch_state_copy(a, true, s));
  }
  if ((rc = release_stage(c, st, s))) return rc;
  if (written) *written = sg.total;
  return KVATTN_OK;
}

int kvattn_seq_state_load(kvattn_ctx* c, int32_t seq_id, const void* src, size_t bytes, void* hip_stream) {
  if (!c) return KVATTN_EINVAL;
  if (!src || (reinterpret_cast<uintptr_t>(src) & 3)) return c->fail(KVATTN_EINVAL, "src is NULL or not 4-byte aligned");
  if (seq_id < 0 || seq_id >= c->core.geo().n_seq_max) return c->fail(KVATTN_EINVAL, "sequence id out of range");
  if (bytes < kStateFixed) return c->fail(KVATTN_EINVAL, "blob shorter than its metadata");
  int rc;
  if ((rc = ensure_device(c))) return rc;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const Geometry& g = c->core.geo();
  // 1. the fixed metadata
  if ((rc = ensure_peek(c, kStateFixed))) return rc;
  HIP_TRY(c, hipMemcpyAsync(c->peek, src, kStateFixed, hipMemcpyDeviceToHost, s));
  HIP_TRY(c, hipStreamSynchronize(s));
  const char* pk = static_cast<const char*>(c->peek);
  const uint32_t n = rd<uint32_t>(pk, 20);
  if (rd<uint32_t>(pk, 0) != kStateMagic || rd<uint32_t>(pk, 4) != kStateVersion)
    return c->fail(KVATTN_EINVAL, "not a sequence-state blob");
  if (rd<uint32_t>(pk, 8) != static_cast<uint32_t>(g.n_layer) || rd<uint32_t>(pk, 12) != static_cast<uint32_t>(g.n_head_kv) ||
      rd<uint32_t>(pk, 16) != static_cast<uint32_t>(g.head_dim) || rd<uint32_t>(pk, 24) != kStateTypeF16 ||
      rd<uint32_t>(pk, 28) != kStateTypeF16)
    return c->fail(KVATTN_EINVAL, "blob geometry or type does not match the context");
  if (n > static_cast<uint32_t>(g.kv_size)) return c->fail(KVATTN_EINVAL, "more saved cells than a stream holds");
  const StateGeom sg = state_geom(g, n);
  if (rd<uint64_t>(pk, 32) != sg.row || rd<uint64_t>(pk, 40) != sg.rec0 || rd<uint64_t>(pk, 48) != sg.total ||
      bytes < sg.total)
    return c->fail(KVATTN_EINVAL, "blob sizes are inconsistent");
  // 2. positions and every record header
  const int32_t n_rec = 2 * g.n_layer;
  const size_t peek_bytes = 4 * sg.n + 12 * static_cast<size_t>(n_rec);
  if ((rc = ensure_peek(c, peek_bytes))) return rc;
  if (sg.n) HIP_TRY(c, hipMemcpyAsync(c->peek, static_cast<const char*>(src) + kStateFixed, 4 * sg.n,
                                      hipMemcpyDeviceToHost, s));
  HIP_TRY(c, launch_state_peek(static_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(c->peek_dev + 4 * sg.n),
                               n_rec, sg.rec0, sg.stride, s));
  HIP_TRY(c, hipStreamSynchronize(s));
  pk = static_cast<const char*>(c->peek);
  for (int32_t r = 0; r < n_rec; ++r) {
    const size_t at = 4 * sg.n + 12 * static_cast<size_t>(r);
    if (rd<uint32_t>(pk, at) != kStateTypeF16 || rd<uint64_t>(pk, at + 4) != sg.row)
      return c->fail(KVATTN_EINVAL, "a record header does not match");
  }
  std::vector<int32_t> pos(sg.n);
  if (sg.n) std::memcpy(pos.data(), pk, 4 * sg.n);
  // 3. placement (all-or-nothing), then the rows into the new cells
  return restore_rows(c, seq_id, src, pos.data(), static_cast<int32_t>(sg.n), s);
}

int kvattn_get_params(const kvattn_ctx* c, kvattn_params* out) {
  if (!c || !out) return KVATTN_EINVAL;
  const Geometry& g = c->core.geo();
  *out = kvattn_params{};
  out->n_layer = g.n_layer;
  out->n_head = g.n_head;
  out->n_head_kv = g.n_head_kv;
  out->head_dim = g.head_dim;
  out->kv_size = g.kv_size;
  out->n_stream = g.n_stream;
  out->n_seq_max = g.n_seq_max;
  out->n_batch = g.n_batch;
  out->n_ubatch = g.n_ubatch;
  out->causal = g.causal;
  out->kq_scale = g.kq_scale;
  out->device = c->device;
  out->attend_layers = g.attend_layers;
  out->split_mode = g.split_mode;
  out->swa_window = g.swa;
  return KVATTN_OK;
}

int kvattn_plan_stats(const kvattn_ctx* c, int32_t only_outputs, int32_t* n_classes, int32_t* n_items_valu,
                      int32_t* n_items_mfma, int32_t* n_partial_rows, int32_t* n_reduced) {
  if (!c) return KVATTN_EINVAL;
  const Plan& P = c->plan[only_outputs ? 1 : 0];
  if (n_classes) *n_classes = static_cast<int32_t>(P.classes.size());
  if (n_items_valu) *n_items_valu = static_cast<int32_t>(P.items_valu.size());
  if (n_items_mfma) *n_items_mfma = static_cast<int32_t>(P.items_mfma.size());
  if (n_partial_rows) *n_partial_rows = P.n_partial_rows;
  if (n_reduced) *n_reduced = static_cast<int32_t>(P.red_slot.size());
  return KVATTN_OK;
}

const char* kvattn_last_error(const kvattn_ctx* c) { return c ? c->err.c_str() : "NULL context"; }

}  // extern "C"
