"""When to launch the expert step on prefill waves of ready tokens (workload plumbing: arrival
times, the launch decision and the timeline; no arithmetic of the step itself).

CascadeEP (abstract) starts the expert FFN on whatever inputs are ready instead of waiting for
the slowest attention replica, trading an early start against FFN efficiency (streamFFN); ASAP
(summary) launches once a minimum batch is ready.  The pages give neither the gaps between
replica waves nor the threshold, so both are parameters here:

  * arrivals: wave 0 is ready at time 0 and each later wave a seeded Exponential(mean_gap)
    time after the one before (a memoryless stand-in for attention-replica imbalance);
  * policies, applied whenever the GPU is idle or a wave arrives:
      - "early":    launch the oldest waiting wave alone (one step per wave, in order);
      - "all":      wait for every wave, then launch them as one batch;
      - "minbatch": launch everything waiting as one batch once it holds at least
                    `min_batch` pairs, or once no wave is still to come;
  * the GPU runs one step at a time; a step's duration comes from the caller (measured on the
    device for the batch the policy formed).

A token's latency is the completion time of the step that carried it minus the arrival time
of its wave.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

POLICIES = ("early", "all", "minbatch")


def wave_arrivals(seed: int, n_waves: int, mean_gap_ms: float) -> np.ndarray:
    """Arrival time (ms) of each wave: 0 for the first, then Exponential(mean_gap_ms) gaps."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, n_waves])))
    gaps = rng.exponential(mean_gap_ms, size=max(n_waves - 1, 0)) if mean_gap_ms > 0 else np.zeros(n_waves - 1)
    return np.concatenate([[0.0], np.cumsum(gaps)])


@dataclass
class Launch:
    waves: tuple          # wave ids carried by this step, ascending
    start_ms: float
    end_ms: float
    pairs: int


@dataclass
class Timeline:
    launches: list = field(default_factory=list)

    def completion(self, n_waves: int) -> np.ndarray:
        done = np.full(n_waves, np.nan)
        for l in self.launches:
            for w in l.waves:
                done[w] = l.end_ms
        return done


def run_policy(policy: str, arrivals, sizes, step_ms, min_batch: int = 0) -> Timeline:
    """Discrete-event timeline of one policy.  step_ms(waves) -> duration of the step that
    carries those waves (the caller measures it); sizes[w] = pairs of wave w."""
    if policy not in POLICIES:
        raise ValueError(policy)
    n = len(sizes)
    order = np.argsort(arrivals, kind="stable")
    waiting: list = []
    nxt = 0          # next wave (in arrival order) not yet arrived
    t = 0.0          # time the GPU is free
    tl = Timeline()
    while nxt < n or waiting:
        # everything that has arrived by now is waiting
        while nxt < n and arrivals[order[nxt]] <= t:
            waiting.append(int(order[nxt]))
            nxt += 1
        ready = sorted(waiting)
        pairs = int(sum(sizes[w] for w in ready))
        if policy == "early":
            take = ready[:1] if ready else []
        elif policy == "all":
            take = ready if nxt == n else []
        else:
            take = ready if ready and (pairs >= min_batch or nxt == n) else []
        if not take:
            t = float(arrivals[order[nxt]])  # idle until the next wave arrives
            continue
        dur = float(step_ms(tuple(take)))
        tl.launches.append(Launch(tuple(take), t, t + dur, int(sum(sizes[w] for w in take))))
        for w in take:
            waiting.remove(w)
        t += dur
    return tl


def summarize(tl: Timeline, arrivals, sizes) -> dict:
    """Throughput over the whole timeline and per-token latency statistics (every token of a
    wave shares its wave's latency)."""
    n = len(sizes)
    done = tl.completion(n)
    lat = done - np.asarray(arrivals, float)
    per_tok = np.repeat(lat, np.asarray(sizes))
    total = int(sum(sizes))
    makespan = float(done.max())
    busy = float(sum(l.end_ms - l.start_ms for l in tl.launches))
    return {"steps": len(tl.launches), "batches": [list(l.waves) for l in tl.launches],
            "batch_pairs": [l.pairs for l in tl.launches], "makespan_ms": round(makespan, 4),
            "gpu_busy_ms": round(busy, 4),
            "pairs_per_s": round(total / (makespan * 1e-3), 1) if makespan > 0 else None,
            "pairs_per_gpu_s": round(total / (busy * 1e-3), 1) if busy > 0 else None,
            "token_latency_ms": {"mean": round(float(per_tok.mean()), 4),
                                 "p50": round(float(np.percentile(per_tok, 50)), 4),
                                 "p99": round(float(np.percentile(per_tok, 99)), 4),
                                 "max": round(float(per_tok.max()), 4)}}
