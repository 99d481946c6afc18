/*
 * kvattn -- per-ubatch attention over a cell-granular F16 KV cache, for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (sources: "llama.cpp and the ubatch", joelfernandes.org;
 * "Batch、Ubatch 与解码主循环", jonathanding.github.io; "What does llama.cpp's
 * KV cache actually look like in memory?", joelfernandes.org):
 *
 *   1. a batch of token slots (position, sequence-id set, output flag) is
 *      validated and split into ubatches -- split_simple for one stream,
 *      split_equal for several, or split_seq on request ("Batch、Ubatch 与解码
 *      主循环", Part C);
 *   2. every slot of every ubatch is given a cache cell, all-or-nothing for
 *      the batch (same page, Part C "strategy choice"; Part F);
 *   3. each ubatch writes its K/V rows, rounded to F16, into per-layer
 *      tensors of shape [n_stream][kv_size][n_head_kv * head_dim] ("What
 *      does llama.cpp's KV cache ...", "The tensor's three dimensions");
 *   4. the KQ mask hides empty cells, cells of other sequences, future
 *      positions and, with a sliding window, positions outside it, the query
 *      masking with its first sequence id ("llama.cpp and the ubatch", "The
 *      mask is doing the work");
 *   5. masked-softmax grouped-query attention runs over the visible cells.
 *
 * Conventions for every entry point:
 *   - Return 0 on success, KVATTN_NO_SLOT (1) when the cache has no room for
 *     a batch (nothing is reserved), a negative KVATTN_E* code otherwise.
 *     No call aborts; kvattn_last_error() describes the last failure.
 *   - "device" pointers are HIP device addresses on params->device; "host"
 *     pointers are ordinary process memory.  The caller owns every buffer
 *     it passes; the library owns only its context and pinned staging.
 *   - All GPU work is enqueued on the hip_stream argument (a hipStream_t,
 *     NULL = the null stream) and nothing synchronises unless stated.  One
 *     context must be driven from one thread and one stream at a time.
 *   - Functions marked HOST-ONLY never touch the GPU and work on a machine
 *     without one (k_layers may then be NULL).
 */
#ifndef KVATTN_H
#define KVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVATTN_MAX_SEQ 256          /* sequence ids live in [0, 256): one bit each */
#define KVATTN_SEQ_WORDS 4          /* a sequence set is 4 uint64 words; id q is bit q % 64 of word q / 64 */
#define KVATTN_MAX_LAYERS_PER_LAUNCH 32

enum {
  KVATTN_OK = 0,
  KVATTN_NO_SLOT = 1,     /* no free cells for the whole batch; nothing reserved */
  KVATTN_EINVAL = -1,     /* an argument is out of range or inconsistent */
  KVATTN_ESTATE = -2,     /* call out of order (stale ubatch, attend before store, ...) */
  KVATTN_ENOMEM = -3,     /* workspace too small for this ubatch, or host allocation failed */
  KVATTN_EHIP = -4,       /* a HIP runtime call failed */
  KVATTN_ENODEV = -5      /* device work asked of a context created without device buffers */
};

typedef struct kvattn_ctx kvattn_ctx;

/* Context parameters.  Mirrors llama_context_params (n_batch, n_ubatch) and
 * the KV-cache constructor (layer count, head geometry, cells per stream,
 * stream count): "llama.cpp and the ubatch", "Three things called batch";
 * "What does llama.cpp's KV cache ...", "28 layers, 56 tensors" and
 * "Unified versus non-unified". */
typedef struct kvattn_params {
  int32_t n_layer;        /* layers owning a K and a V tensor */
  int32_t n_head;         /* query heads; a multiple of n_head_kv */
  int32_t n_head_kv;      /* KV heads */
  int32_t head_dim;       /* 16, 32, 64 or 128 */
  int32_t kv_size;        /* cells PER STREAM (tensor dimension 1); one layer's tensor,
                             n_stream * kv_size * n_head_kv * head_dim * 2 bytes, < 2 GiB */
  int32_t n_stream;       /* 1 = unified cache; a slot's stream is seq_id[0] % n_stream, its cell
                             holds the ids that live there (stream of id q: q % n_stream); a slot
                             whose ids span streams is also stored once in each other stream it
                             touches ("Unified versus non-unified": separate copies) */
  int32_t n_seq_max;      /* sequence ids must lie in [0, n_seq_max); <= KVATTN_MAX_SEQ */
  int32_t n_batch;        /* <= 0: 2048; clamped to kv_size*n_stream when causal */
  int32_t n_ubatch;       /* 0: n_batch; then clamped to n_batch */
  int32_t causal;         /* nonzero: hide cells with a later position */
  float kq_scale;         /* 0: 1/sqrt(head_dim) */
  const int32_t *cell_order; /* host, optional [n_stream][kv_size]: for each stream a permutation
                                of 0..kv_size-1; free cells are handed out in this order
                                (NULL = ascending).  Copied at create. */
  void *const *k_layers;  /* host array of n_layer device pointers, each F16
                             [n_stream][kv_size][n_head_kv*head_dim]; NULL = host-only context */
  void *const *v_layers;  /* same for V */
  void *workspace;        /* device, >= kvattn_workspace_bytes(); NULL with k_layers NULL */
  size_t workspace_bytes;
  int32_t device;         /* HIP device ordinal of every device pointer */
  int32_t attend_layers;  /* scheduling hint, no effect on results: layers per kvattn_attend
                             call the caller will use (0 = 1); sizes the work items */
  int32_t split_mode;     /* KVATTN_SPLIT_*: how kvattn_split cuts a batch into ubatches */
  int32_t swa_window;     /* sliding window in positions, 0 = none: a query at position p sees no
                             cell with position <= p - swa_window ("llama.cpp and the ubatch",
                             "The mask is doing the work", whose window rule is elided; this is
                             the reading taken) */
} kvattn_params;

/* Batch -> ubatch split strategies ("Batch、Ubatch 与解码主循环", Part C).
 * AUTO is the init_batch choice: split_simple for one stream, split_equal
 * (n_ubatch, sequential) for several.  SEQ is split_seq: every ubatch holds
 * the slots of one sequence set only (the set of the first unused slot, its
 * unused slots in submission order, at most n_ubatch). */
enum {
  KVATTN_SPLIT_AUTO = 0,
  KVATTN_SPLIT_SIMPLE = 1,  /* the next <= n_ubatch slots, sequence ids ignored */
  KVATTN_SPLIT_EQUAL = 2,   /* equal slot counts from pairwise-disjoint sequence sets */
  KVATTN_SPLIT_SEQ = 3
};

/* A batch as submitted: llama_batch without token/embd ("Batch、Ubatch 与解码主循环",
 * Part A).  pos, seq_id and output may each be NULL and are then filled:
 * seq_id -> {0}; pos -> continuing each first sequence id from one past its
 * largest cached position; output -> last slot only. */
typedef struct kvattn_batch {
  int32_t n_tokens;                 /* 0 <= n_tokens <= clamped n_batch */
  const int32_t *pos;               /* host [n_tokens] or NULL */
  const int32_t *n_seq_id;          /* host [n_tokens]; ignored when seq_id is NULL */
  const int32_t *const *seq_id;     /* host [n_tokens] lists, first id = the query's sequence */
  const int8_t *output;             /* host [n_tokens] or NULL */
} kvattn_batch;

/* One ubatch: llama_ubatch ("Batch、Ubatch 与解码主循环", Part B) plus its
 * placement.  All arrays are host memory owned by the context and stay
 * valid until the next kvattn_split or kvattn_destroy. */
typedef struct kvattn_ubatch {
  int32_t id;                       /* handle checked by store/attend */
  int32_t n_tokens;                 /* = n_seq_tokens * n_seqs */
  int32_t n_seq_tokens;
  int32_t n_seqs;
  int32_t n_seqs_unq;               /* distinct sequence ids in the ubatch */
  int32_t n_outputs;                /* flagged slots */
  const int32_t *pos;               /* [n_tokens] */
  const int32_t *n_seq_id;          /* [n_tokens] */
  const int32_t *const *seq_id;     /* [n_tokens] */
  const int32_t *seq_id_unq;        /* [n_seqs_unq], ascending */
  const int8_t *output;             /* [n_tokens] */
  const int32_t *src_idx;           /* [n_tokens] row of each slot in the submitted batch */
  const int32_t *stream;            /* [n_tokens] */
  const int32_t *cells;             /* [n_tokens] reserved cell within the stream */
  int32_t n_copies;                 /* separate copies (several streams only): extra cells of slots
                                       whose ids span streams, one per other stream they touch */
  const int32_t *copy_src;          /* [n_copies] slot (ubatch index) whose row the copy holds */
  const int32_t *copy_stream;       /* [n_copies] */
  const int32_t *copy_cell;         /* [n_copies] */
} kvattn_ubatch;

/* Device workspace the caller must provide: cell metadata mirror, the
 * per-ubatch visibility lists and work plan, and split-K partials, sized for
 * the clamped n_ubatch ("llama.cpp and the ubatch", "Where the memory
 * actually sits": the workspace is reserved once for the largest pass). */
size_t kvattn_workspace_bytes(const kvattn_params *p);

/* Total K+V cache bytes over all layers and streams: 2 * n_layer * n_stream
 * * kv_size * n_head_kv * head_dim * 2 ("What does llama.cpp's KV cache
 * ...", "One row, one token's keys": 448 MiB for 28 x 8 x 128 at 4096). */
size_t kvattn_cache_bytes(const kvattn_params *p);

/* HOST-ONLY.  Validates and copies *p.  Device buffers are only recorded;
 * the first call that needs the GPU initialises it. */
int kvattn_create(const kvattn_params *p, kvattn_ctx **out);
void kvattn_destroy(kvattn_ctx *ctx);

/* HOST-ONLY.  Validate + auto-fill the batch, split it into ubatches and
 * reserve a cell for every slot of every ubatch, all-or-nothing.  Follows
 * "Batch、Ubatch 与解码主循环", Part F (the decode loop validates and fills
 * the batch, then splits it) and Part C (split_simple / split_equal /
 * split_seq; every ubatch's cells are reserved before any runs); the
 * n_tokens <= n_batch check is "llama.cpp and the ubatch", "Three things
 * called batch", and output_ids the batch-row -> output-row map of "Where
 * the memory actually sits" on the same page.  Writes up
 * to cap ubatches to ubs[] and their count to *n_ubs (cap too small ->
 * KVATTN_EINVAL, nothing reserved).  output_ids, when not NULL, receives
 * n_batch entries: the rank of each flagged batch row among flagged rows,
 * -1 elsewhere.  Cells reserved by the previous split and never stored are
 * released; ubatches of the previous split become stale. */
int kvattn_split(kvattn_ctx *ctx, const kvattn_batch *b, kvattn_ubatch *ubs, int32_t cap,
                 int32_t *n_ubs, int32_t *output_ids);

/* Write K/V rows of layers il0 .. il0+n_il-1 ("Batch、Ubatch 与解码主循环",
 * Part D: a ubatch writes its keys and values into its cells, which later
 * ubatches read; the row layout is that of "What does llama.cpp's KV cache
 * actually look like in memory?", "The tensor's three dimensions").
 * k_cur/v_cur are host arrays
 * of n_il device pointers, each fp32 [n_tokens][n_head_kv*head_dim] in
 * ubatch slot order; rows are rounded to F16 (nearest-even) into the
 * ubatch's cells.  The first call with il0 == 0 commits the ubatch: its
 * cells become visible and the visibility lists for its attention are built
 * on the GPU.  Ubatches of one split commit in order.  Storing again is
 * idempotent.  On a host-only context, n_il == 0 commits the placement
 * without touching the GPU (any other call returns KVATTN_ENODEV). */
int kvattn_store(kvattn_ctx *ctx, const kvattn_ubatch *ub, int32_t il0, int32_t n_il,
                 const void *const *k_cur, const void *const *v_cur, void *hip_stream);

/* Attention of layers il0 .. il0+n_il-1 for the most recently committed
 * ubatch: masked-softmax attention of every query slot over the cells the
 * mask leaves visible ("llama.cpp and the ubatch", "The mask is doing the
 * work" and "Chunked prefill is the same mechanism": a chunk's queries see
 * the cached cells and their own ubatch's).  q/out are host arrays of n_il device pointers; q is fp32
 * [n_tokens][n_head*head_dim], out fp32 [n_tokens][n_head*head_dim] in
 * ubatch slot order -- or, with only_outputs, [n_outputs][...] holding the
 * flagged slots in slot order.  A slot with no visible cell yields zeros.
 * Repeatable.  Asynchronous on hip_stream. */
int kvattn_attend(kvattn_ctx *ctx, const kvattn_ubatch *ub, int32_t il0, int32_t n_il,
                  const void *const *q, void *const *out, int32_t only_outputs, void *hip_stream);

/* Size of the static device array kvattn_attend_noalloc keeps its split-K
 * partials in (one per GPU, held until the process ends). */
#define KVATTN_STATIC_SCRATCH_BYTES (16u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments and results as kvattn_attend, but the split-K partial
 * results live in a static device array of the library
 * (KVATTN_STATIC_SCRATCH_BYTES per GPU) instead of the context's workspace,
 * and the call allocates nothing (no hipMalloc / hipFree, no allocating
 * library routine).  The array is located at the context's device set-up
 * (its first store).  Limit: one layer's partial rows must fit the array --
 * 16 MiB / ((n_head * head_dim + 2 * n_head) * 4 B), 2016 rows for 16 heads
 * of 128 -- else KVATTN_ENOMEM and nothing is launched; layer ranges are cut
 * into as many launches as the array needs.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (two streams, two
 * threads) race and must be serialised by the caller. */
int kvattn_attend_noalloc(kvattn_ctx *ctx, const kvattn_ubatch *ub, int32_t il0, int32_t n_il,
                          const void *const *q, void *const *out, int32_t only_outputs, void *hip_stream);

/* ---- diagnostics (tests and benchmarks) ---------------------------------- */

/* The kernels of one attend call, for kvattn_time_next_attend. */
#define KVATTN_KERNEL_MFMA 0   /* matrix-core tile kernel (query blocks of 32+ rows) */
#define KVATTN_KERNEL_VALU 1   /* vector-ALU kernel (short query blocks, decode) */
#define KVATTN_KERNEL_MERGE 2  /* split-K merge of partial results */

/* Kernel timing for benchmarks and profilers (not an operation of the
 * method).  The next kvattn_attend or kvattn_attend_noalloc call on this
 * context launches kernel `kind` with hipExtLaunchKernel, which stamps
 * start_event with that kernel's own start time and stop_event with its end
 * time (kernel execution only, not the time the stream reached them, and
 * no marker packet of its own in the stream).  When the call cuts its
 * layers into several launches, start_event belongs to the first and
 * stop_event to the last (recorded on the stream right after it: one
 * launch per call carries events, since the runtime holds the host thread
 * at a second event-carrying launch).  Both are hipEvent_t created by
 * the caller on the context's device; the library keeps neither beyond the
 * next attend call, which uses the setting once and clears it.  A call that
 * launches no kernel of that kind records both events back to back on its
 * stream (elapsed time about zero); a call that fails before launching
 * records neither.  Create the events with hipEventDisableSystemFence: a kernel
 * bound to an event with the default flags ends with a system-scope cache
 * writeback and invalidation that slows the work after it (measured: a
 * shared-prefix decode step from 0.31 to 0.62 ms).  kind < 0 disarms.
 * KVATTN_EINVAL for an unknown kind or a NULL event. */
int kvattn_time_next_attend(kvattn_ctx *ctx, int32_t kind, void *start_event, void *stop_event);

/* HOST-ONLY.  n_kv reported for the current state ("llama.cpp and the
 * ubatch", "Prefill and decode are not the same shape"). */
int32_t kvattn_n_kv(const kvattn_ctx *ctx);

/* Dense F16 KQ mask of the most recently committed ubatch ("llama.cpp and
 * the ubatch", "The mask is doing the work"), built on the GPU from the
 * device cell mirror: 0x0000 visible, 0xFC00 (-inf) hidden,
 * row-major [n_tokens][n_kv].  d_mask is a device buffer of cap_elems F16;
 * *n_kv receives the row length.  Asynchronous on hip_stream. */
int kvattn_get_mask(kvattn_ctx *ctx, const kvattn_ubatch *ub, void *d_mask, size_t cap_elems,
                    int32_t *n_kv, void *hip_stream);

/* Visibility lists of the most recently committed ubatch, copied to host
 * (synchronises hip_stream): the mask of "llama.cpp and the ubatch", "The
 * mask is doing the work", kept in sparse form.  Cells are grouped in classes of equal
 * sequence sets; per class: stream, sequence set (KVATTN_SEQ_WORDS words at
 * cls_mask + KVATTN_SEQ_WORDS * class), number of cells, then the cells in
 * ascending index.  Fills up to cap_classes classes and cap_cells cells;
 * *n_classes / *n_cells receive the totals. */
int kvattn_get_classes(kvattn_ctx *ctx, int32_t *n_classes, int32_t *cls_stream,
                       uint64_t *cls_mask, int32_t *cls_count, int32_t cap_classes,
                       int32_t *n_cells, int32_t *cells, int32_t cap_cells, void *hip_stream);

/* HOST-ONLY.  Copy of the committed cell table of one stream: pos (-1 =
 * empty) and the sequence-set bitmask of each of the kv_size cells (the
 * per-cell metadata the mask reads, "llama.cpp and the ubatch", "The mask is
 * doing the work").  pos is a host array of kv_size entries, seqmask one of
 * KVATTN_SEQ_WORDS * kv_size words (cell c's set at seqmask + KVATTN_SEQ_WORDS * c). */
int kvattn_get_cells(const kvattn_ctx *ctx, int32_t stream, int32_t *pos, uint64_t *seqmask);

/* HOST-ONLY.  Remove sequence seq_id (every sequence when < 0) from cells
 * whose position lies in [p0, p1) (the retirement step of "Iteration-Level
 * Batching", "The loop that replaces the batch") (p0 < 0: from 0; p1 < 0: no end).  A cell
 * left without a sequence becomes free.  The device mirror follows at the
 * next commit. */
int kvattn_seq_rm(kvattn_ctx *ctx, int32_t seq_id, int32_t p0, int32_t p1);

/* HOST-ONLY.  Largest committed position of seq_id, -1 when none (what a
 * NULL pos continues from: "Batch、Ubatch 与解码主循环", Part A). */
int32_t kvattn_seq_pos_max(const kvattn_ctx *ctx, int32_t seq_id);

/* HOST-ONLY.  Work plan of the most recently committed ubatch (this
 * library's own decomposition; the pages give no kernel design): number of
 * visibility classes, vector-ALU work items, matrix-core work items (per
 * KV head), split-K partial rows and reduced slots.  Any pointer may be NULL. */
int kvattn_plan_stats(const kvattn_ctx *ctx, int32_t only_outputs, int32_t *n_classes,
                      int32_t *n_items_valu, int32_t *n_items_mfma, int32_t *n_partial_rows,
                      int32_t *n_reduced);

/* ---- sequence state: save / restore one sequence's cached K/V ------------
 *
 * The serialized form follows the .bin dump of "What does llama.cpp's KV
 * cache actually look like in memory?" ("Opening the .bin dump"): leading
 * metadata, then one record per layer for K (layers 0 .. n_layer-1), then
 * one per layer for V; each record is a 12-byte header followed by the
 * sequence's rows (n_head_kv * head_dim F16 values each).  The page fixes
 * only the sizes; the fields are this library's, all little-endian:
 *   bytes  0..79   "KVSS", u32 version 1, u32 n_layer, u32 n_head_kv,
 *                  u32 head_dim, u32 n_cells, u32 K type, u32 V type
 *                  (1 = F16), u64 row bytes, u64 offset of the first record
 *                  (80 + 4 n_cells), u64 total bytes, 24 zero bytes;
 *   then n_cells int32 positions, ascending;
 *   record header: u32 type (1 = F16), u64 row bytes.
 * Total = 80 + 4 n + 2 n_layer (12 + n row_bytes): 803,596 bytes for 7
 * cells of the page's 28-layer model, first K record at byte 108.
 * A sequence's cells are the committed cells whose sequence set holds it
 * (shared prefix cells included), ordered by position.  The blob holds
 * positions, not cell indices, so it restores into any free cells. */

/* HOST-ONLY.  Bytes kvattn_seq_state_save will write for seq_id. */
int kvattn_seq_state_size(const kvattn_ctx *ctx, int32_t seq_id, size_t *bytes);

/* Serialize seq_id into dst: a 4-byte aligned device buffer of cap bytes
 * (>= kvattn_seq_state_size, else KVATTN_ENOMEM).  *written (may be NULL)
 * receives the size.  Reads the cache rows on hip_stream, after the stores
 * enqueued there before; asynchronous. */
int kvattn_seq_state_save(kvattn_ctx *ctx, int32_t seq_id, void *dst, size_t cap, size_t *written,
                          void *hip_stream);

/* Restore a blob (4-byte aligned device buffer of `bytes`) as sequence
 * seq_id of this context: the blob's geometry must match (else
 * KVATTN_EINVAL, nothing changed); seq_id's cells are replaced by one new
 * cell per saved position in its stream (seq_id % n_stream), lowest free
 * rank first -- KVATTN_NO_SLOT, nothing changed, when the free cells plus
 * those only seq_id holds are too few.  The cells are committed at once
 * (the device cell mirror follows at the next ubatch commit, as after
 * kvattn_seq_rm).  Reads the metadata back first (synchronises
 * hip_stream), then copies the rows into the cells on hip_stream. */
int kvattn_seq_state_load(kvattn_ctx *ctx, int32_t seq_id, const void *src, size_t bytes, void *hip_stream);

/* HOST-ONLY.  The context's parameters as in effect: n_batch and n_ubatch
 * clamped, kq_scale and attend_layers defaulted, split_mode resolved (never
 * AUTO).  Pointer fields and workspace_bytes are zero. */
int kvattn_get_params(const kvattn_ctx *ctx, kvattn_params *out);

/* HOST-ONLY.  Text of the last error on this context ("" if none). */
const char *kvattn_last_error(const kvattn_ctx *ctx);

/* ---- machine ceilings (benchmarks; not part of the method) --------------- */

/* Read rate of the decode kernel's access: every wavefront reads whole 2 KiB
 * rows (1024 F16) of `rows` ([n_rows][1024], device) in the order of `index`
 * (n_index device int32; entries outside [0, n_rows) are clamped), each row
 * one 2 KiB wavefront access, four rows in flight per wavefront.  `out`
 * (device, n_wg * 256 floats, caller-owned) receives each thread's fp32 sum
 * of the numbers it read.  Asynchronous on hip_stream; KVATTN_EINVAL for a
 * NULL pointer or a non-positive size, KVATTN_EHIP if the launch fails. */
int kvattn_probe_gather(const void *rows, int64_t n_rows, const int32_t *index, int64_t n_index, float *out,
                        int32_t n_wg, void *hip_stream);

/* Matrix-core issue rate: n_wg workgroups of four wavefronts each run
 * `iters` rounds of four independent v_mfma_f32_32x32x16_f16 products (the
 * prefill kernel's instruction) on operands read from `ab` (device, 16 F16:
 * every lane's A fragment is ab[0..7], its B fragment ab[8..15]).  Each
 * product adds 2 * sum_j ab[j] * ab[8 + j] to each of its 1024 outputs, so
 * `out` (device, n_wg * 256 floats) receives 128 * iters * sum_j ab[j] *
 * ab[8 + j] per thread; one launch performs n_wg * 4 * iters * 4 * 32768
 * flop.  Asynchronous on hip_stream; errors as kvattn_probe_gather. */
int kvattn_probe_mfma(const void *ab, float *out, int32_t n_wg, int32_t iters, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* KVATTN_H */
