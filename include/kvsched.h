/*
 * kvsched -- the iteration-level (continuous) batching loop over a kvattn
 * context, in native code ("Iteration-Level Batching: Reforming the Batch at
 * Every Token", mercemay.com).
 *
 * Before every forward pass the loop rebuilds the batch ("The loop that
 * replaces the batch"):
 *
 *   1. finished sequences are retired and their cells released
 *      (kvattn_seq_rm on the context);
 *   2. under the paged policy, a stream whose free cells cannot cover one new
 *      cell for each sequence with a single pending position gives memory
 *      back: its most recently admitted sequence is preempted -- cells
 *      released, sampled tokens kept, back to the front of the waiting
 *      queue ("Where it breaks", cache exhaustion: swapping or
 *      recomputation).  KVATTN_PREEMPT_RECOMPUTE discards its progress, so
 *      it prefills prompt plus sampled tokens again.  KVATTN_PREEMPT_SWAP
 *      first saves its cells (kvattn_seq_state_save) into the swap arena, at
 *      the lowest offset where the blob fits (extents rounded up to 256
 *      bytes), and on re-admission restores them under its new sequence id
 *      before the batch is placed, so it resumes where it stopped; a victim
 *      whose blob does not fit is recomputed instead;
 *   3. waiting requests are admitted first come, first served while the
 *      token budget and the cache budget both allow ("The budget that
 *      actually binds"): the worst-case block reservation of the page's
 *      sketch (KVATTN_ADMIT_RESERVE) or, with a paged cache, the cells the
 *      new sequence's pending positions occupy, plus its restored cells
 *      when it was swapped out (KVATTN_ADMIT_PAGED);
 *   4. the batch is assembled: every running sequence with one pending
 *      position (a decoding sequence) contributes it; the remaining budget
 *      goes to pending prompt positions in admission order, split across
 *      iterations when chunked prefill is on.  The slot that completes a
 *      sequence's pending positions carries the output flag.
 *
 * The caller then runs the batch -- kvattn_split, and kvattn_store /
 * kvattn_attend for each ubatch -- and calls kvattn_sched_advance: a token
 * is taken as sampled for every flagged slot and every sequence moves on.
 * A request is finished once it has sampled n_generate tokens (its last
 * token is never fed back: n_prompt + n_generate - 1 cached positions).
 *
 * Sequence ids are the lowest free id in [0, n_seq_max) at admission; the
 * stream of a sequence is seq_id % n_stream, as in kvattn.
 *
 * The scheduler's tables are sized at kvattn_sched_create; submit, step and
 * advance allocate nothing of their own (the context's kvattn_seq_rm, which
 * step calls, keeps its own bookkeeping).  One scheduler drives one context
 * from one thread; the context must not be given other batches or seq_rm
 * calls meanwhile.
 * Return codes are kvattn's (KVATTN_OK, KVATTN_EINVAL, KVATTN_ESTATE,
 * KVATTN_ENOMEM); kvattn_sched_last_error() describes the last failure.
 */
#ifndef KVSCHED_H
#define KVSCHED_H

#include <stdint.h>

#include "kvattn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvattn_sched kvattn_sched;

enum {
  KVATTN_ADMIT_RESERVE = 0,   /* ceil((n_prompt + n_generate) / block_size) blocks held from admission */
  KVATTN_ADMIT_PAGED = 1      /* cells as positions are cached; preempt on exhaustion */
};

enum { KVATTN_REQ_WAITING = 0, KVATTN_REQ_RUNNING = 1, KVATTN_REQ_DONE = 2 };

enum {
  KVATTN_PREEMPT_RECOMPUTE = 0,   /* a preempted sequence prefills prompt + sampled tokens again */
  KVATTN_PREEMPT_SWAP = 1         /* its cells are saved to the swap arena and restored */
};

typedef struct kvattn_sched_params {
  int32_t token_budget;     /* positions per iteration; <= 0: the context's (clamped) n_batch.
                               max_running <= token_budget <= n_batch */
  int32_t max_running;      /* concurrent sequences; <= 0: n_seq_max */
  int32_t policy;           /* KVATTN_ADMIT_* */
  int32_t block_size;       /* cells per block for KVATTN_ADMIT_RESERVE (>= 1); kv_size / block_size
                               blocks per stream.  Ignored by KVATTN_ADMIT_PAGED */
  int32_t chunked;          /* nonzero: pending prompt positions may be split across iterations;
                               zero: a sequence runs all its pending positions or waits */
  int32_t max_requests;     /* capacity of the request table (requests ever submitted) */
  int32_t preempt;          /* KVATTN_PREEMPT_*; only the paged policy preempts */
  void *swap_space;         /* SWAP on a device context: device buffer of swap_bytes, 256-byte
                               aligned, owned by the caller; holds the saved states */
  size_t swap_bytes;
  void *hip_stream;         /* SWAP: the stream the batches run on; saves and restores are enqueued
                               there (a hipStream_t, NULL = the null stream) */
} kvattn_sched_params;

/* One iteration as assembled by kvattn_sched_step.  Every array is host
 * memory owned by the scheduler, valid until the next step or destroy. */
typedef struct kvattn_sched_iter {
  kvattn_batch batch;           /* pos, one sequence id per slot, output flags; pass to kvattn_split */
  const int32_t *req;           /* [batch.n_tokens] request id of each slot */
  int32_t n_retired;            /* requests retired this iteration, in admission order */
  const int32_t *retired;
  int32_t n_preempted;          /* requests preempted, in preemption order */
  const int32_t *preempted;
  int32_t n_admitted;           /* requests admitted, in admission order, with their sequence id */
  const int32_t *admitted;
  const int32_t *admitted_seq;
  int32_t n_swapped_out;        /* preempted requests whose cells went to the swap arena */
  const int32_t *swapped_out;
  int32_t n_swapped_in;         /* admitted requests whose cells were restored from it */
  const int32_t *swapped_in;
  int32_t n_running;            /* after admission */
  int32_t n_waiting;
  int32_t n_decode;             /* slots from sequences with a single pending position */
} kvattn_sched_iter;

/* HOST-ONLY.  A scheduler over ctx (borrowed; it must outlive the
 * scheduler).  Reads the context's kv_size, n_stream, n_seq_max and
 * n_batch through kvattn_get_params.  Bad parameters -> KVATTN_EINVAL. */
int kvattn_sched_create(kvattn_ctx *ctx, const kvattn_sched_params *p, kvattn_sched **out);
void kvattn_sched_destroy(kvattn_sched *s);

/* HOST-ONLY.  Queue a request of n_prompt positions that will sample
 * n_generate tokens; *req_id receives its id (0, 1, 2, ... in submission
 * order).  KVATTN_EINVAL for a request that could never finish alone: more
 * than kv_size cached positions, more blocks than a stream holds under
 * RESERVE, or -- without chunking -- a prompt (RESERVE) or a recomputation
 * of prompt plus sampled tokens (PAGED) longer than the token budget.
 * KVATTN_ENOMEM when max_requests have been submitted. */
int kvattn_sched_submit(kvattn_sched *s, int32_t n_prompt, int32_t n_generate, int32_t *req_id);

/* HOST-ONLY on a host-only context.  Steps 1-4 above: retire, relieve cache
 * pressure, admit, assemble into *it.  Calls kvattn_seq_rm on the context
 * for every retired or preempted sequence; with KVATTN_PREEMPT_SWAP on a
 * device context it also enqueues the saves and restores on hip_stream
 * (nothing synchronises; on a host-only context only the placement of
 * restored cells happens).  KVATTN_ESTATE when the previous iteration was not
 * advanced.  An empty batch (n_tokens 0) with n_running and n_waiting 0
 * means the loop is idle. */
int kvattn_sched_step(kvattn_sched *s, kvattn_sched_iter *it);

/* HOST-ONLY.  The assembled batch has run: every slot of it must have been
 * split and stored (committed) on the context -- the scheduler's cell
 * accounting assumes so and does not check.  KVATTN_ESTATE without a step. */
int kvattn_sched_advance(kvattn_sched *s);

/* HOST-ONLY.  State of request req_id (KVATTN_REQ_*), its sequence id (-1
 * when not running), cached positions and tokens sampled.  Any output
 * pointer may be NULL.  KVATTN_EINVAL for an unknown id. */
int kvattn_sched_request(const kvattn_sched *s, int32_t req_id, int32_t *state, int32_t *seq_id,
                         int32_t *n_cached, int32_t *n_sampled);

/* HOST-ONLY.  Text of the last error on this scheduler ("" if none). */
const char *kvattn_sched_last_error(const kvattn_sched *s);

#ifdef __cplusplus
}
#endif
#endif /* KVSCHED_H */
