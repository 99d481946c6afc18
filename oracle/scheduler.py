"""The iteration-level (continuous) batching loop, restated from "Iteration-Level Batching".

Test infrastructure only (see ``oracle/__init__.py``).

"Iteration-Level Batching", "The loop that replaces the batch": the scheduler keeps the sequences that
are generating (``running``) and the ones waiting to enter (``waiting``) and
rebuilds the batch before every forward pass.  One iteration

1. retires the finished sequences and releases their cache;
2. admits waiting sequences while the token budget and the cache budget both
   allow it (first come, first served: admission stops at the first request
   that does not fit);
3. assembles the batch: a new sequence contributes its prompt, a running one
   contributes one token;
4. runs the model; a sampler picks one token per sequence and each running
   sequence advances (``advance`` here).

"Iteration-Level Batching", "The budget that actually binds": the token budget counts positions per
iteration, and a prompt longer than what is left of it must wait or be split
(chunked prefill).  Cache budget: the sketch of "Iteration-Level Batching" reserves the worst case
``ceil((prompt_len + max_new) / block_size)`` blocks at admission (policy
``"reserve"``); with a paged cache admission only needs the cells the new
sequence's prompt will occupy and a running sequence grows one cell per step
(policy ``"paged"``, the policy "Iteration-Level Batching" says paged allocation makes possible).
"Iteration-Level Batching", "Where it breaks": when the cache runs out the loop takes memory back from
a running sequence; this oracle discards the progress of the most recently
admitted sequence of the exhausted stream and recomputes it later.

Readings where "Iteration-Level Batching" leaves a step open (each is a choice, stated once):

* A sequence is finished once it has sampled ``n_generate`` tokens; its last
  sampled token is never fed back, so a finished sequence has cached
  ``n_prompt + n_generate - 1`` positions.  It is retired (``seq_rm`` of all
  its cells) at the start of the next iteration.
* Positions of the token budget go first to every running sequence with one
  pending position (a decoding sequence, or a prompt with one position
  left), then to the remaining prompts in running order, each taking
  ``min(pending, left)``; without chunking a prompt takes all its pending
  positions or none.  The budget must be at least ``max_running``.
* The batch lists the running sequences in running (admission) order, each
  with its positions ascending; the position that completes a sequence's
  pending work carries the output flag (that is where the sampler picks).
* Sequence ids come from ``[0, n_seq_max)``: the lowest free id at admission;
  the stream of a sequence is ``seq_id % n_stream``.
* ``"paged"`` cache accounting per stream: a running sequence holds
  ``n_ctx`` cells and has promised ``pending`` more when it still has more
  than one pending position; each sequence with one pending position needs
  one new cell this iteration.  Before admission, while a stream's free cells
  fall short of that need, the last admitted running sequence of the stream
  is preempted: its cells are released, it returns to the front of the
  waiting queue keeping its sampled tokens, and on re-admission it prefills
  prompt plus sampled tokens.  A newcomer is admitted when its pending
  positions fit in the free cells left after that need.
* ``"reserve"``: ``kv_size // block_size`` blocks per stream; never preempts.
* Preemption by swapping (``preempt="swap"``, the other option "Iteration-Level Batching" names):
  the victim's cells are saved first (the sequence-state blob of "What does llama.cpp's KV cache actually look like in memory?", "Opening
  the .bin dump", ``blob_bytes``) into a swap arena of ``swap_bytes``, at the
  lowest offset where it fits (first fit, extents rounded up to 256 bytes);
  the victim keeps its cached positions and, when re-admitted, its cells
  are restored into its new sequence id before the batch is placed.  Its
  admission then needs its cached plus pending positions in free cells.  A
  victim whose blob does not fit the arena is recomputed instead.
* A request that can never finish alone (more than ``kv_size`` positions, or
  more blocks than a stream has; without chunking a prompt, or under
  ``"paged"`` a recomputation, longer than the budget) is rejected at
  submission.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass

WAITING, RUNNING, DONE = 0, 1, 2


class SchedError(ValueError):
    """A request or parameter the loop cannot serve."""


def blob_bytes(n_layer, row_bytes, n_cells):
    """Size of a saved sequence state: leading metadata (80 bytes + 4 per
    cell), then 2 * n_layer records of a 12-byte header and the rows."""
    return 80 + 4 * n_cells + 2 * n_layer * (12 + n_cells * row_bytes)


SWAP_ALIGN = 256


@dataclass
class Request:
    id: int
    n_prompt: int
    n_generate: int
    seq: int = -1
    n_ctx: int = 0         # positions stored in the cache
    generated: int = 0     # tokens sampled so far
    state: int = WAITING
    blocks: int = 0        # "reserve": blocks held
    swap: tuple = None     # (offset, bytes) of its saved state while swapped out
    blob: bytes = None

    @property
    def known(self):       # prompt plus sampled tokens
        return self.n_prompt + self.generated

    @property
    def pending(self):     # positions still to be run through the model
        return self.known - self.n_ctx

    @property
    def finished(self):
        return self.generated >= self.n_generate


def _ceil_div(a, b):
    return -(-a // b)


class OracleScheduler:
    """The loop of "Iteration-Level Batching" over one cache of ``n_stream`` streams of ``kv_size`` cells.

    ``release(seq_id)`` is called whenever a sequence's cells are released
    (retirement or preemption); pass the oracle engine's ``seq_rm`` so that
    its cell table follows.
    """

    def __init__(self, kv_size, n_stream, n_seq_max, token_budget, max_running=0,
                 policy="paged", block_size=1, chunked=True, release=None,
                 preempt="recompute", swap_bytes=0, n_layer=1, row_bytes=0, swap_out=None, swap_in=None):
        if policy not in ("paged", "reserve") or preempt not in ("recompute", "swap"):
            raise SchedError("policy")
        max_running = n_seq_max if max_running <= 0 else max_running
        if not (0 < max_running <= n_seq_max) or token_budget < max_running or block_size < 1:
            raise SchedError("bad parameters")
        self.kv_size, self.n_stream, self.n_seq_max = kv_size, n_stream, n_seq_max
        self.budget, self.max_running = token_budget, max_running
        self.policy, self.block_size, self.chunked = policy, block_size, bool(chunked)
        self.release = release
        self.preempt, self.swap_bytes = preempt, int(swap_bytes)
        self.n_layer, self.row_bytes = n_layer, row_bytes
        self.swap_out, self.swap_in = swap_out, swap_in   # callables: seq -> blob, (seq, blob) -> None
        self.swapped = []          # (offset, bytes, request id) of the arena's live extents, by offset
        self.requests = []
        self.waiting = deque()
        self.running = []
        self.seq_owner = [None] * n_seq_max
        self.free_blocks = [kv_size // block_size] * n_stream
        self.chunk = {}            # request id -> positions in the assembled batch
        self.assembled = False

    # -- submission ----------------------------------------------------------
    def submit(self, n_prompt, n_generate):
        if n_prompt < 1 or n_generate < 1 or n_prompt + n_generate - 1 > self.kv_size:
            raise SchedError("request can never fit the cache")
        if self.policy == "reserve" and \
                _ceil_div(n_prompt + n_generate, self.block_size) > self.kv_size // self.block_size:
            raise SchedError("request needs more blocks than a stream has")
        if not self.chunked:
            worst = n_prompt + n_generate - 1 if self.policy == "paged" else n_prompt
            if worst > self.budget:
                raise SchedError("prompt longer than the token budget and chunking is off")
        r = Request(len(self.requests), n_prompt, n_generate)
        self.requests.append(r)
        self.waiting.append(r)
        return r.id

    # -- cache accounting ("paged") ------------------------------------------
    def stream_of(self, seq):
        return seq % self.n_stream

    def _free_cells(self, s):
        held = 0
        for r in self.running:
            if self.stream_of(r.seq) == s:
                held += r.n_ctx + (r.pending if r.pending > 1 else 0)
        return self.kv_size - held

    def _need(self, s):
        return sum(1 for r in self.running if self.stream_of(r.seq) == s and r.pending == 1)

    def _drop(self, r):
        """Release r's cells and its sequence id."""
        if self.release is not None:
            self.release(r.seq)
        self.seq_owner[r.seq] = None
        if self.policy == "reserve":
            self.free_blocks[self.stream_of(r.seq)] += r.blocks
            r.blocks = 0
        self.running.remove(r)
        r.seq = -1

    def _take(self, want):
        """Positions a sequence with ``want`` pending positions gets from ``left``."""
        if self.chunked:
            return min(want, self._left)
        return want if want <= self._left else 0

    # -- swap arena (first fit) ---------------------------------------------
    def _swap_place(self, need):
        at = 0
        for off, size, _ in self.swapped:
            if off - at >= need:
                return at
            at = off + size
        return at if self.swap_bytes - at >= need else None

    def _swap_out(self, r):
        """Save r's state into the arena; False when it does not fit."""
        if self.preempt != "swap" or r.n_ctx == 0:
            return False
        need = -(-blob_bytes(self.n_layer, self.row_bytes, r.n_ctx) // SWAP_ALIGN) * SWAP_ALIGN
        at = self._swap_place(need)
        if at is None:
            return False
        r.blob = self.swap_out(r.seq) if self.swap_out is not None else None
        r.swap = (at, need)
        self.swapped.append((at, need, r.id))
        self.swapped.sort()
        return True

    def _swap_in(self, r):
        if self.swap_in is not None:
            self.swap_in(r.seq, r.blob)
        self.swapped.remove((r.swap[0], r.swap[1], r.id))
        r.swap, r.blob = None, None

    # -- one iteration -------------------------------------------------------
    def step(self):
        """Retire, relieve cache pressure, admit, assemble.  Returns the
        iteration record: retired / preempted / admitted request ids and the
        batch as parallel lists (request, seq id, position, output flag)."""
        if self.assembled:
            raise SchedError("advance() the previous batch first")
        retired, preempted, admitted, swapped_out, swapped_in = [], [], [], [], []

        for r in [r for r in self.running if r.finished]:
            self._drop(r)
            r.state = DONE
            retired.append(r.id)

        if self.policy == "paged":
            for s in range(self.n_stream):
                while self._free_cells(s) < self._need(s):
                    victim = [r for r in self.running if self.stream_of(r.seq) == s][-1]
                    if self._swap_out(victim):
                        swapped_out.append(victim.id)
                    else:
                        victim.n_ctx = 0
                    self._drop(victim)
                    victim.state = WAITING
                    self.waiting.appendleft(victim)
                    preempted.append(victim.id)

        self.chunk = {}
        self._left = self.budget
        for r in self.running:
            if r.pending == 1:
                self.chunk[r.id] = 1
                self._left -= 1
        for r in self.running:
            if r.pending > 1:
                self.chunk[r.id] = self._take(r.pending)
                self._left -= self.chunk[r.id]

        while self.waiting and len(self.running) < self.max_running:
            r = self.waiting[0]
            c = self._take(r.pending)
            if c == 0:
                break
            seq = self.seq_owner.index(None)
            s = self.stream_of(seq)
            if self.policy == "reserve":
                need = _ceil_div(r.n_prompt + r.n_generate, self.block_size)
                if need > self.free_blocks[s]:
                    break
            elif r.n_ctx + r.pending > self._free_cells(s) - self._need(s):
                break
            self.waiting.popleft()
            r.seq, r.state = seq, RUNNING
            self.seq_owner[seq] = r
            if self.policy == "reserve":
                r.blocks = need
                self.free_blocks[s] -= need
            if r.swap is not None:
                self._swap_in(r)
                swapped_in.append(r.id)
            self.running.append(r)
            admitted.append((r.id, seq))
            self.chunk[r.id] = c
            self._left -= c

        req, seq, pos, out = [], [], [], []
        for r in self.running:
            c = self.chunk.get(r.id, 0)
            for p in range(r.n_ctx, r.n_ctx + c):
                req.append(r.id)
                seq.append(r.seq)
                pos.append(p)
                out.append(1 if p == r.known - 1 else 0)
        self.assembled = True
        return {"retired": retired, "preempted": preempted, "admitted": admitted,
                "swapped_out": swapped_out, "swapped_in": swapped_in,
                "req": req, "seq": seq, "pos": pos, "output": out,
                "n_running": len(self.running), "n_waiting": len(self.waiting)}

    def advance(self):
        """The batch has run: each sequence's positions are cached and every
        sequence whose pending work completed samples one token."""
        if not self.assembled:
            raise SchedError("nothing assembled")
        for r in self.running:
            c = self.chunk.get(r.id, 0)
            if c:
                done = r.n_ctx + c == r.known
                r.n_ctx += c
                if done:
                    r.generated += 1
        self.assembled = False

    def idle(self):
        return not self.running and not self.waiting
