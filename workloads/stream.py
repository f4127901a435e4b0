"""Seeded multi-layer asynchronous stream for one expert-parallel rank (the C3 workload).

This is workload plumbing: queues, routing draws, straggler delays and the queue pick.
It computes none of the step's arithmetic; whichever executor runs the expert steps and
combine calls reports back the released tokens, which the stream then moves on.

Model (the pages' setting: per-layer attention and expert micro-queues, 2L of them, a
scheduler that picks one non-empty queue, [SEP] (marsggbo, "SOSP'26 | StreamEP") §3-§4;
stragglers per source message, §2 and §8):
  * T home tokens start in A_0.  An attention pick is instantaneous: every token in A_l
    gets a fresh activation (row (t * L + l) mod of a seeded N(0,1) bank, written into the
    token's pool slot t) and a top-K routing over E_total experts drawn from N(0,1)
    logits (softmax weights over the selected K).
  * Pairs whose expert is local (this rank owns experts [rank*E_loc, (rank+1)*E_loc)) go
    to X_l.  Results for the other experts come back from their owning rank s = e // E_loc
    as one message per (source, attention pick), after ceil(lognormal(0, 1)) time units;
    the result rows are rows of a seeded N(0,1) bank, taken round-robin.
  * Time advances by one unit per expert batch.  Each step first delivers the messages
    that are due, then picks a non-empty queue of the chain A_0, X_0, A_1, X_1, ... by the
    configured policy (ties go to the earliest queue of the chain):
      - "mtfs"   most tokens first: the deepest queue ([SEP] §4);
      - "flfs"   first layer first: the earliest non-empty queue of the chain ([SEP] §4);
      - "defrag" the defragmenting score of [SEP] §4,
                 S(s) = Q(s) + sum_{j=1..W} delta^j [Q(s_j) + H(s_j)],
                 with Q the queue depth, s_j the queue j places after s on the chain
                 (places past the last layer do not exist unless `wrap`), H(q) the tokens
                 drained from q over the last `hist` scheduling steps.
    An expert pick takes up to `cap` pairs in FIFO order.  If every queue is empty, time
    jumps to the next message.
  * A released token moves from layer l to A_{l+1} (after the last layer, to A_0); its
    generation, like the combine state's, advances by one per release.
"""
from __future__ import annotations

import heapq
from collections import deque
from dataclasses import dataclass, field

import numpy as np

from .gen import BASE_SEED


@dataclass
class StreamConfig:
    layers: int = 36
    E_total: int = 128
    E_loc: int = 8
    K: int = 4
    H: int = 2880
    I: int = 2880
    tokens: int = 4096
    cap: int = 512
    batches: int = 1000
    rank: int = 0
    row_bank: int = 16384   # remote-result rows
    x_bank: int = 8192      # attention-output rows
    seed: int = BASE_SEED + 3
    policy: str = "mtfs"    # "mtfs", "flfs" or "defrag"
    window: int = 2         # defrag lookahead W
    delta: float = 0.5      # defrag decay
    hist: int = 4           # defrag history: scheduling steps summed into H
    wrap: bool = False      # defrag lookahead wraps from the last layer to the first


@dataclass
class Message:
    due: int
    seq: int
    source: int
    layer: int
    tok: np.ndarray
    kslot: np.ndarray
    w: np.ndarray
    gen: np.ndarray
    row: np.ndarray         # row of the result bank carrying each result


@dataclass
class ExpertBatch:
    layer: int
    slot: np.ndarray
    expert: np.ndarray
    tok: np.ndarray
    kslot: np.ndarray
    w: np.ndarray
    gen: np.ndarray

    @property
    def n(self) -> int:
        return int(self.tok.shape[0])


@dataclass
class StreamSim:
    cfg: StreamConfig
    tau: int = 0
    batches_done: int = 0
    log: list = field(default_factory=list)

    def __post_init__(self):
        c = self.cfg
        self.rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([c.seed, 0])))
        self.A = [deque() for _ in range(c.layers)]
        self.X = [deque() for _ in range(c.layers)]
        self.A[0].extend(range(c.tokens))
        self.layer = np.zeros(c.tokens, np.int64)
        self.gen = np.zeros(c.tokens, np.uint32)
        self.msgs: list = []
        self.seq = 0
        self.bank_ptr = 0
        self.recent: deque = deque()                 # (chain position, tokens drained) per pick
        self.entered = np.zeros(c.tokens, np.int64)  # step at which a token entered its layer
        self.latency: list = []                      # steps from entering a layer to release

    # --------------------------------------------------------------------- banks
    def banks(self):
        """(result rows [row_bank][H], attention outputs [x_bank][H]) as fp32 N(0,1)."""
        c = self.cfg
        r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([c.seed, 1])))
        rows = r.standard_normal((c.row_bank, c.H), dtype=np.float32)
        xs = r.standard_normal((c.x_bank, c.H), dtype=np.float32)
        return rows, xs

    def x_row(self, t: np.ndarray, layer: int) -> np.ndarray:
        return (np.asarray(t, np.int64) * self.cfg.layers + layer) % self.cfg.x_bank

    # --------------------------------------------------------------------- steps
    def attention(self, l: int) -> np.ndarray:
        """Runs the attention pick of A_l; returns its tokens (in queue order)."""
        c = self.cfg
        toks = np.array(self.A[l], np.int64)
        self.A[l].clear()
        lg = self.rng.standard_normal((len(toks), c.E_total))
        top = np.argsort(-lg, axis=1, kind="stable")[:, : c.K]
        sel = np.take_along_axis(lg, top, axis=1)
        z = np.exp(sel - sel.max(axis=1, keepdims=True))
        w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
        lo, hi = c.rank * c.E_loc, (c.rank + 1) * c.E_loc
        remote: dict[int, list] = {}
        for i, t in enumerate(toks):
            g = self.gen[t]
            for j in range(c.K):
                e = int(top[i, j])
                if lo <= e < hi:
                    self.X[l].append((int(t), j, e, float(w[i, j]), int(g)))
                else:
                    remote.setdefault(e // c.E_loc, []).append((int(t), j, float(w[i, j]), int(g)))
        for s in sorted(remote):
            items = remote[s]
            d = int(np.ceil(self.rng.lognormal(0.0, 1.0)))
            m = len(items)
            rows = (self.bank_ptr + np.arange(m)) % c.row_bank
            self.bank_ptr += m
            msg = Message(self.tau + max(d, 1), self.seq, s, l, np.array([x[0] for x in items], np.int32),
                          np.array([x[1] for x in items], np.int32), np.array([x[2] for x in items], np.float32),
                          np.array([x[3] for x in items], np.uint32), rows.astype(np.int32))
            heapq.heappush(self.msgs, (msg.due, msg.seq, msg))
            self.seq += 1
        self.log.append(("A", l, len(toks)))
        self.note_drain("A", l, len(toks))
        return toks

    def due(self) -> list:
        out = []
        while self.msgs and self.msgs[0][0] <= self.tau:
            out.append(heapq.heappop(self.msgs)[2])
        return out

    def chain(self):
        """Queues in chain order A_0, X_0, A_1, X_1, ... as ((kind, layer), queue)."""
        for l in range(self.cfg.layers):
            yield ("A", l), self.A[l]
            yield ("X", l), self.X[l]

    def drained(self) -> np.ndarray:
        """H per chain position: tokens drained over the last `hist` scheduling steps."""
        h = np.zeros(2 * self.cfg.layers, np.int64)
        for pos, cnt in self.recent:
            h[pos] += cnt
        return h

    def pick(self):
        """The configured policy's queue over A_0, X_0, A_1, X_1, ...; None if all are empty."""
        c = self.cfg
        if c.policy == "flfs":
            for key, q in self.chain():
                if q:
                    return key
            return None
        if c.policy == "defrag":
            depth = [len(q) for _, q in self.chain()]
            h = self.drained()
            best, arg = None, None
            for pos, (key, q) in enumerate(self.chain()):
                if not q:
                    continue
                sc = defrag_score(depth, h, pos, c.window, c.delta, c.wrap)
                if best is None or sc > best:
                    best, arg = sc, key
            return arg
        best, arg = 0, None
        for key, q in self.chain():
            if len(q) > best:
                best, arg = len(q), key
        return arg

    def note_drain(self, kind: str, l: int, count: int) -> None:
        """Records one scheduling step's drain for the defrag history."""
        self.recent.append((2 * l + (kind == "X"), count))
        while len(self.recent) > self.cfg.hist:
            self.recent.popleft()

    def take(self, l: int) -> ExpertBatch:
        q = self.X[l]
        items = [q.popleft() for _ in range(min(self.cfg.cap, len(q)))]
        b = ExpertBatch(l, np.array([x[0] for x in items], np.int32), np.array([x[2] for x in items], np.int32),
                        np.array([x[0] for x in items], np.int32), np.array([x[1] for x in items], np.int32),
                        np.array([x[3] for x in items], np.float32), np.array([x[4] for x in items], np.uint32))
        self.log.append(("X", l, b.n))
        self.note_drain("X", l, b.n)
        return b

    def release(self, toks) -> None:
        """Released tokens (ascending) move to the next layer's attention queue."""
        for t in np.asarray(toks, np.int64):
            self.latency.append(self.tau - self.entered[t])
            self.entered[t] = self.tau
            self.layer[t] += 1
            self.gen[t] += 1
            if self.layer[t] == self.cfg.layers:
                self.layer[t] = 0
            self.A[self.layer[t]].append(int(t))

    def idle_jump(self) -> bool:
        """All queues empty: jump time to the next message; False if nothing is pending."""
        if not self.msgs:
            return False
        self.tau = max(self.tau, self.msgs[0][0])
        return True


def defrag_score(depth, drained, pos: int, window: int, delta: float, wrap: bool = False) -> float:
    """S(s) of the defragmenting scheduler ([SEP] §4) for the queue at chain position
    `pos`: depth[pos] + sum_{j=1..window} delta^j (depth[pos+j] + drained[pos+j]); chain
    positions past the end are absent unless `wrap`."""
    n = len(depth)
    score = float(depth[pos])
    for j in range(1, window + 1):
        q = pos + j
        if q >= n:
            if not wrap:
                break
            q %= n
        score += delta ** j * (depth[q] + drained[q])
    return score


def merge_messages(msgs: list) -> Message:
    """The messages due at one step, concatenated in delivery order (one combine call)."""
    cat = lambda f: np.concatenate([getattr(m, f) for m in msgs])  # noqa: E731
    return Message(msgs[0].due, msgs[0].seq, -1, -1, cat("tok"), cat("kslot"), cat("w"), cat("gen"), cat("row"))


def run_stream(sim: StreamSim, on_attention, on_messages, on_batch, max_batches: int | None = None,
               progress=None) -> None:
    """Drives the stream.  on_attention(layer, tokens); on_messages(merged message) ->
    released tokens; on_batch(batch) -> released tokens.  Stops after `max_batches` expert
    batches (default: the configured number)."""
    limit = sim.cfg.batches if max_batches is None else max_batches
    while sim.batches_done < limit:
        msgs = sim.due()
        if msgs:
            sim.release(on_messages(merge_messages(msgs)))
        p = sim.pick()
        if p is None:
            if not sim.idle_jump():
                raise RuntimeError("stream stalled: no queued work and no message in flight")
            continue
        kind, l = p
        if kind == "A":
            on_attention(l, sim.attention(l))
            continue
        b = sim.take(l)
        sim.release(on_batch(b))
        sim.batches_done += 1
        sim.tau += 1
        if progress is not None:
            progress(sim)
