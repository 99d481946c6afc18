"""Seeded request streams for the iteration-level batching loop.

A stream is a list of requests, each with the iteration at which it arrives,
its prompt length and the number of tokens it will generate, drawn from
``default_rng(SeedSequence([seed, 3]))``: arrivals per iteration are Poisson
with mean ``rate`` (a burst of ``burst`` requests arrives at iteration 0),
prompt and generation lengths are uniform integers in the given closed
ranges.  The loop itself (who is admitted when) is not decided here.

K/V/Q rows are keyed by (request, layer, kind) and drawn once per request
for all of its positions from ``SeedSequence([seed, 4, request, layer,
kind])`` as fp32 standard normals, so a position recomputed after a
preemption gets the same rows it had the first time.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .workloads import QWEN3_06B, KIND_Q

PURPOSE_REQUESTS, PURPOSE_ROWS = 3, 4


@dataclass
class RequestStream:
    name: str
    n_layer: int
    n_head: int
    n_head_kv: int
    head_dim: int
    kv_size: int
    n_stream: int
    n_seq_max: int
    token_budget: int
    n_ubatch: int
    seed: int
    arrive: np.ndarray              # int32 [n_req] iteration of arrival, ascending
    n_prompt: np.ndarray            # int32 [n_req]
    n_generate: np.ndarray          # int32 [n_req]
    policy: str = "paged"
    block_size: int = 1
    chunked: bool = True
    max_running: int = 0
    split_mode: str = "auto"
    preempt: str = "recompute"
    swap_bytes: int = 0
    _rows: dict = field(default_factory=dict, repr=False)

    @property
    def n_requests(self):
        return int(len(self.arrive))

    @property
    def E(self):
        return self.n_head_kv * self.head_dim

    def width(self, kind):
        return self.n_head * self.head_dim if kind == KIND_Q else self.E

    def arrivals(self, it):
        """Request indices arriving at iteration ``it``."""
        lo, hi = np.searchsorted(self.arrive, [it, it + 1])
        return list(range(int(lo), int(hi)))

    def rows(self, req, layer, kind, pos):
        """fp32 [len(pos)][width] rows of request ``req`` at positions ``pos``."""
        key = (req, layer, kind)
        a = self._rows.get(key)
        if a is None:
            n = int(self.n_prompt[req] + self.n_generate[req] - 1)
            rng = np.random.default_rng(np.random.SeedSequence([self.seed, PURPOSE_ROWS, req, layer, kind]))
            a = rng.standard_normal((n, self.width(kind)), dtype=np.float32)
            self._rows[key] = a
        return a[np.asarray(pos, dtype=np.int64)]

    def batch_rows(self, reqs, pos, layer, kind):
        """Rows for a batch given per-slot request ids and positions."""
        out = np.empty((len(reqs), self.width(kind)), np.float32)
        reqs, pos = np.asarray(reqs), np.asarray(pos)
        for r in np.unique(reqs):
            m = reqs == r
            out[m] = self.rows(int(r), layer, kind, pos[m])
        return out

    def note(self):
        return (f"{self.n_requests} requests, prompts {self.n_prompt.min()}..{self.n_prompt.max()}, "
                f"generate {self.n_generate.min()}..{self.n_generate.max()}, {self.n_layer} layers, "
                f"{self.n_head}/{self.n_head_kv} heads x {self.head_dim}, kv_size {self.kv_size} x "
                f"{self.n_stream} streams, <= {self.max_running or self.n_seq_max} running, budget "
                f"{self.token_budget} positions, n_ubatch {self.n_ubatch}, {self.policy}")

    def sched_kwargs(self):
        return dict(kv_size=self.kv_size, n_stream=self.n_stream, n_seq_max=self.n_seq_max,
                    token_budget=self.token_budget, max_running=self.max_running, policy=self.policy,
                    block_size=self.block_size, chunked=self.chunked, preempt=self.preempt,
                    swap_bytes=self.swap_bytes, n_layer=self.n_layer, row_bytes=self.E * 2)


def request_stream(n_req=24, rate=1.0, burst=4, prompt_range=(4, 40), gen_range=(1, 12),
                   n_layer=2, n_head=4, n_head_kv=2, head_dim=64, kv_size=256, n_stream=1,
                   n_seq_max=8, token_budget=64, n_ubatch=32, policy="paged", block_size=1,
                   chunked=True, max_running=0, split_mode="auto", preempt="recompute", swap_bytes=0,
                   seed=2001, name="stream"):
    rng = np.random.default_rng(np.random.SeedSequence([seed, PURPOSE_REQUESTS]))
    arrive = [0] * min(burst, n_req)
    it = 0
    while len(arrive) < n_req:
        it += 1
        arrive += [it] * int(min(rng.poisson(rate), n_req - len(arrive)))
    n_prompt = rng.integers(prompt_range[0], prompt_range[1], size=n_req, endpoint=True)
    n_generate = rng.integers(gen_range[0], gen_range[1], size=n_req, endpoint=True)
    return RequestStream(name, n_layer, n_head, n_head_kv, head_dim, kv_size, n_stream, n_seq_max,
                         token_budget, n_ubatch, seed, np.asarray(arrive, np.int32),
                         n_prompt.astype(np.int32), n_generate.astype(np.int32), policy, block_size,
                         bool(chunked), max_running, split_mode, preempt, int(swap_bytes))


def qwen_serving(n_req=400, rate=2.0, burst=64, prompt_range=(128, 1024), gen_range=(64, 512),
                 n_layer=28, kv_size=131072, n_stream=1, n_seq_max=64, token_budget=2048, n_ubatch=512,
                 policy="paged", preempt="recompute", seed=2002):
    """Qwen3-0.6B-shaped serving stream: up to 64 concurrent sequences, a
    2048-position budget per iteration, prompts of 128..1024 positions and
    64..512 generated tokens, one unified cache of 131072 cells."""
    return request_stream(n_req=n_req, rate=rate, burst=burst, prompt_range=prompt_range,
                          gen_range=gen_range, n_layer=n_layer, n_head=QWEN3_06B["n_head"],
                          n_head_kv=QWEN3_06B["n_head_kv"], head_dim=QWEN3_06B["head_dim"],
                          kv_size=kv_size, n_stream=n_stream, n_seq_max=n_seq_max,
                          token_budget=token_budget, n_ubatch=n_ubatch, policy=policy, preempt=preempt,
                          seed=seed, name="qwen_serving")
