"""Benchmark: one expert-parallel rank's expert step on one MI355X.

Default workload (the largest single-GPU configuration): the prefill-shaped rank share.
256 experts, top-8, 32 local experts, hidden 4096, SwiGLU intermediate 2048, fp8 e4m3
weights (fp32 row scales) with bf16 activations and fp32 accumulation; 16384 token-expert
pairs with Zipf(1.0) routing arrive in four waves of 6554 / 4915 / 3277 / 1638 pairs, and
each wave is one step (CascadeEP's and ASAP's prefill setting: expert work starts on each
wave of ready tokens as attention replicas finish).

A step = moe_assemble + moe_expert_ffn_grouped + moe_combine_release on one ready batch,
all inputs resident in HBM.  Every step combines its local results into a combine-state
range of its own, whose results from the other ranks were delivered before the timed
region, so each step releases all of its tokens.  W warm-up steps, then exactly K steps are
timed back to back (synchronised on both sides); step s runs wave s mod 4.

The JSON line also carries: the roofline of the dominant kernel (the wave-0 gate/up GEMM,
timed by start/stop events its own dispatch records, in a separate pass), per-stage times
of each wave with the combine also measured after a 512 MiB cache-evicting write, the CPU
oracle on a bounded sample of whole experts, and the decode-shaped workload's own figures
(sub-object "decode").

Other workloads (--workload):
  decode   128 experts, top-4, 8 local, hidden 2880, intermediate 2880, bf16; 256 pairs
           from a 4096-slot pool (steps cycle through four copies of the weights)
  skewed   the decode layer shape with Zipf(1.2) routing over the 8 local experts: all 200
           batches of U{8..512} pairs, value = sum of pairs / sum of step times
  tiny     8 experts, top-2, hidden 64, intermediate 128, fp32 (launch-latency bound)
  stream   36 layers, 72 micro-queues, 16 simulated sources with lognormal delays, under a
           queue pick --policy (most tokens first, first layer first, defragmenting score)
  launch   the prefill waves arriving after seeded gaps (--gaps), launched by three policies:
           each wave early, all merged, or at a minimum batch (--min-batch); per-token latency
           and throughput from device-measured step times
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "expert tokens/sec per GPU (assemble+FFN+combine); % MFMA peak, % HBM BW"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILES = {"decode": os.path.join(PROFILES, "ffn_gateup_decode_traffic.md"),
                 "prefill": os.path.join(PROFILES, "ffn_gateup_prefill_traffic.md")}
CALIB_BYTES = 256 << 20
FLUSH_BYTES = 512 << 20
FFN_SRC = os.path.join(ROOT, "asynchronous_moe_expert_amd", "csrc", "ffn.hip")


class HipEvents:
    """Raw hipEvent_t handles (the library records some of them inside its own calls)."""

    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]

    def create(self) -> int:
        e = C.c_void_p()
        assert self.hip.hipEventCreate(C.byref(e)) == 0
        return e.value

    def record(self, ev: int, stream: int) -> None:
        assert self.hip.hipEventRecord(C.c_void_p(ev), C.c_void_p(stream)) == 0

    def ms(self, a: int, b: int) -> float:
        self.hip.hipEventSynchronize(C.c_void_p(b))
        out = C.c_float()
        assert self.hip.hipEventElapsedTime(C.byref(out), C.c_void_p(a), C.c_void_p(b)) == 0
        return float(out.value)


def stored_traffic(which: str):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3 counter
    summary, if its counters were taken on the kernel source as it is now (else None)."""
    try:
        text = open(TRAFFIC_FILES[which]).read()
        sha = re.search(r"ffn\.hip sha256: ([0-9a-f]{64})", text).group(1)
        val = re.search(r"traffic bytes per launch: ([0-9]+)", text).group(1)
        src = hashlib.sha256(open(FFN_SRC, "rb").read()).hexdigest()
        return float(val) if sha == src else None
    except (OSError, AttributeError, ValueError, KeyError):
        return None


def cpu_info() -> dict:
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def blas_threads() -> int:
    import threadpoolctl

    info = threadpoolctl.threadpool_info()
    return int(max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1]))


def calibration_copy(dev) -> None:
    """One device-to-device copy of CALIB_BYTES: the reference dispatch that scales the
    rocprofv3 byte counters of the same run to bytes."""
    import torch

    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# --------------------------------------------------------------------------- step runner
def _compact(b):
    """Token indices of a batch renumbered 0..T-1 (first appearance in the queue), and the
    remote arrivals' tokens through the same map: each step then needs a state range of T."""
    uniq, first = np.unique(b.tok, return_index=True)
    order = uniq[np.argsort(first, kind="stable")]
    lut = {int(t): i for i, t in enumerate(order)}
    tok = np.array([lut[int(t)] for t in b.tok], np.int32)
    r_tok = None if b.remote is None else np.array([lut[int(t)] for t in b.remote.tok], np.int32)
    return tok, r_tok, len(order)


class StepRunner:
    """Expert steps over a cycle of ready batches: step s runs batch s mod len(batches) on
    combine-state range s (its own tokens), whose remote results deliver() puts in first."""

    def __init__(self, batches, wts, act_code, w_code, n_steps: int, weight_copies: int = 1, weights_from=None):
        import torch

        import asynchronous_moe_expert_amd as M
        from workloads.device import tensor, weight_tensors

        self.M, self.torch = M, torch
        self.batches = batches
        b0 = batches[0]
        self.E, self.H, self.I, self.K = b0.E_loc, b0.H, wts.I, b0.K
        self.base = b0.expert_base
        comp = [_compact(b) for b in batches]
        self.T_step = max(c[2] for c in comp)
        n_steps = max(n_steps, len(batches))  # (the per-stage pass runs each batch once)
        self.n_steps = n_steps
        n_max = max(b.n for b in batches)
        self.st = M.ExpertStep(self.E, self.H, self.I, self.K, act_code, w_code, n_max, n_steps * self.T_step)
        if weights_from is None:
            wt = weight_tensors(wts)
            self.st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt.get("s_gate"), wt.get("s_up"), wt.get("s_down"))
            del wt
            # copies of the packed weights at distinct addresses; step s uses copy s % L, so no step
            # finds the weights the one before it streamed still in a cache
            L = max(1, weight_copies)
            self.w_copies = [(self.st.w_gu, self.st.w_d)] + [(self.st.w_gu.clone(), self.st.w_d.clone())
                                                             for _ in range(L - 1)]
        else:  # another runner's packed weights (read-only on the device), no second copy
            src = weights_from.st
            self.st.w_gu, self.st.w_d = src.w_gu, src.w_d
            self.st.s_gate, self.st.s_up, self.st.s_down = src.s_gate, src.s_up, src.s_down
            self.w_copies = weights_from.w_copies
        self.pool = tensor(b0.pool, b0.act)
        self.d = []
        for b, (tok, r_tok, _) in zip(batches, comp):
            x = dict(slot=tensor(b.slot), expert=tensor(b.expert), tok=tok, kslot=tensor(b.kslot), w=tensor(b.w),
                     gen=tensor(b.gen))
            if b.remote is not None and b.remote.m > 0:
                r = b.remote
                x.update(r_rows=tensor(r.rows, r.dtype), r_idx=tensor(r.row_idx), r_tok=r_tok,
                         r_kslot=tensor(r.kslot), r_w=tensor(r.w), r_gen=tensor(r.gen))
            self.d.append(x)
        # per-step token tensors (state range s), made before any timing
        self.tok = [tensor(self.d[s % len(batches)]["tok"] + s * self.T_step) for s in range(n_steps)]
        self.stream = torch.cuda.current_stream().cuda_stream

    def batch(self, s: int):
        return self.batches[s % len(self.batches)]

    def deliver(self, s: int) -> None:
        """The remote results of step s's tokens (untimed; the tokens' other K-1 positions)."""
        d = self.d[s % len(self.batches)]
        if "r_rows" in d:
            from workloads.device import tensor

            self.st.combine(d["r_rows"], d["r_idx"], tensor(d["r_tok"] + s * self.T_step), d["r_kslot"], d["r_w"],
                            d["r_gen"])

    def step(self, s: int) -> None:
        b, d = self.batch(s), self.d[s % len(self.batches)]
        self.st.w_gu, self.st.w_d = self.w_copies[s % len(self.w_copies)]
        self.st.run(d["slot"], d["expert"], self.base, self.pool, self.tok[s], d["kslot"], d["w"], d["gen"], n=b.n)

    def check(self, s: int) -> None:
        assert int(self.st.err.item()) == 0, "device error flags raised"
        assert int(self.st.rel_count.item()) == _compact(self.batch(s))[2], "a step did not release its tokens"

    def timed(self, W: int, K: int):
        """W warm-up steps, then K timed steps back to back; returns (ms, sum of pairs)."""
        torch = self.torch
        for s in range(W + K):
            self.deliver(s)
        torch.cuda.synchronize()
        assert int(self.st.rel_count.item()) == 0
        for s in range(W):
            self.step(s)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for s in range(W, W + K):
            self.step(s)
        t1.record()
        torch.cuda.synchronize()
        self.check(W + K - 1)
        return t0.elapsed_time(t1), sum(self.batch(s).n for s in range(W, W + K))

    def timed_graph(self, W: int, K: int):
        """The same K steps captured as one HIP graph (after W eager warm-up steps) and timed as
        one replay; a first replay warms the graph up, then the state is reset and the remote
        results delivered again, so the timed replay starts from the same state.  Returns (ms,
        sum of pairs)."""
        torch, M = self.torch, self.M
        M.moe_state_reset(self.st.state, 0)
        for s in range(W + K):
            self.deliver(s)
        for s in range(W):
            self.step(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(W, W + K):
                self.step(s)
        g.replay()
        torch.cuda.synchronize()
        self.check(W + K - 1)
        M.moe_state_reset(self.st.state, 0)
        for s in range(W, W + K):
            self.deliver(s)
        torch.cuda.synchronize()
        assert int(self.st.rel_count.item()) == 0
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        self.check(W + K - 1)
        del g
        return t0.elapsed_time(t1), sum(self.batch(s).n for s in range(W, W + K))

    def stages(self, ev: HipEvents, reps: int, flush: bool = False):
        """Per-stage HIP-event intervals of each batch of the cycle (state reset and delivery
        untimed before each step), plus the gate/up projection's own kernel time from the
        events its dispatch records, in a pass of its own so that they stay out of the stage
        intervals; with flush, the combine is also timed cold: after a 512 MiB write and two
        read passes over it, which leave the 256 MB last-level cache full of clean lines
        (combine_cold), and after the write alone (combine_cold_dirty: then every miss of the
        combine first writes back a dirty line of that buffer, which on its own took the same
        traffic pattern from ~43 to ~75 us in a probe)."""
        torch, M, st = self.torch, self.M, self.st
        nb = len(self.batches)
        names = ["assemble", "gate_up", "down", "combine"]
        evs = [ev.create() for _ in range(5)]
        gs, ge, c0, c1 = ev.create(), ev.create(), ev.create(), ev.create()
        scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") if flush else None
        times = {w: {k: [] for k in names + ["gate_up_kernel", "combine_cold", "combine_cold_dirty"]}
                 for w in range(nb)}
        for _ in range(reps):
            for w in range(nb):
                b, d = self.batches[w], self.d[w]
                self.st.w_gu, self.st.w_d = self.w_copies[w % len(self.w_copies)]
                for p in range(3 if flush else 2):
                    M.moe_state_reset(st.state, 0)
                    self.deliver(w)
                    tok = self.tok[w]
                    if p == 0:
                        # the calls of ExpertStep.run; where the queue index is derived inside the
                        # gate/up launch (queues of at most 256 pairs) the assemble interval holds
                        # no launch, elsewhere moe_assemble is timed on its own
                        ev.record(evs[0], self.stream)
                        index = (st.index_args(d["slot"], d["expert"], self.base, self.pool, b.n)
                                 if st.fuse_index and b.n <= 256 else None)
                        if index is None:
                            st.assemble(d["slot"], d["expert"], self.base, self.pool, n=b.n)
                        ev.record(evs[1], self.stream)
                        plan = st.local_combine_args(tok, d["kslot"], d["w"], d["gen"], b.n)
                        st.ffn(b.n, ev_mid=evs[2], plan=plan, index=index)
                        ev.record(evs[3], self.stream)
                        M.combine_call(plan, "apply")
                        ev.record(evs[4], self.stream)
                    else:
                        st.assemble(d["slot"], d["expert"], self.base, self.pool, n=b.n)
                        plan = st.local_combine_args(tok, d["kslot"], d["w"], d["gen"], b.n)
                        st.ffn(b.n, plan=plan, ev_gu=(gs, ge) if p == 1 else None)
                        if scratch is not None:
                            scratch.fill_(1.0)
                            if p == 2:
                                for _ in range(2):
                                    scratch.sum()
                        ev.record(c0, self.stream)
                        M.combine_call(plan, "apply")
                        ev.record(c1, self.stream)
                    torch.cuda.synchronize()
                    self.check(w)
                    if p == 0:
                        for k, nm in enumerate(names):
                            times[w][nm].append(ev.ms(evs[k], evs[k + 1]))
                    elif p == 1:
                        times[w]["gate_up_kernel"].append(ev.ms(gs, ge))
                        if scratch is not None:
                            times[w]["combine_cold_dirty"].append(ev.ms(c0, c1))
                    else:
                        times[w]["combine_cold"].append(ev.ms(c0, c1))
        return {w: {k: float(np.median(v)) for k, v in t.items() if v} for w, t in times.items()}


# ------------------------------------------------------------------------- CPU baselines
def cpu_baseline_decode(b, wts, seconds: float) -> dict:
    """The oracle (fp64 numpy) on the host: whole decode steps, repeated until `seconds`."""
    import oracle as O

    r = b.remote
    rows_remote = O.decode(r.rows, r.dtype)
    t0 = time.perf_counter()
    reps = 0
    while True:
        a = O.assemble(b.slot, b.expert, b.expert_base, b.E_loc, b.P)
        xb = O.decode(O.gather_rows(b.pool, b.slot, a["perm"], b.n), b.act)
        y = O.expert_ffn(xb, a["offsets"], wts)
        cs = O.CombineState(b.T, b.K)
        O.combine_release(cs, rows_remote, r.row_idx, r.tok, r.kslot, r.w, r.gen)
        O.combine_release(cs, y, a["pos"], b.tok, b.kslot, b.w, b.gen)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": b.n * reps / el, "unit": "expert tokens/s", "cores": blas_threads(), "kind": "oracle",
            **cpu_info(),
            "sample": f"{reps} whole decode steps of {b.n} token-expert pairs (assemble, fp64 SwiGLU FFN over "
                      f"8 experts, combine incl. the delivery of the remote results), {el:.1f} s"}


def cpu_baseline_batches(batches, wts, seconds: float, what: str) -> dict:
    """The oracle on whole steps of the given batches in order (assemble, FFN, combine with the
    delivery of their remote results), until `seconds`."""
    import oracle as O

    t0 = time.perf_counter()
    pairs = steps = 0
    for b in batches:
        a = O.assemble(b.slot, b.expert, b.expert_base, b.E_loc, b.P)
        xb = O.decode(O.gather_rows(b.pool, b.slot, a["perm"], b.n), b.act)
        y = O.expert_ffn(xb, a["offsets"], wts)
        cs = O.CombineState(b.T, b.K)
        if b.remote is not None:
            r = b.remote
            O.combine_release(cs, O.decode(r.rows, r.dtype), r.row_idx, r.tok, r.kslot, r.w, r.gen)
        O.combine_release(cs, y, a["pos"], b.tok, b.kslot, b.w, b.gen)
        pairs += b.n
        steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": pairs / el, "unit": "expert tokens/s", "cores": blas_threads(), "kind": "oracle", **cpu_info(),
            "sample": f"{steps} whole steps ({pairs} token-expert pairs) of the {what}, in order, {el:.1f} s"}


def _oracle_subqueue(b, wts, experts):
    """One oracle pass over the pairs of `experts` in batch b: assemble, gather, FFN (each
    expert's weights decoded once), combine of the local and remote results; returns pairs."""
    import oracle as O

    sel = np.isin(b.expert - b.expert_base, experts)
    slot, expert, tok = b.slot[sel], b.expert[sel], b.tok[sel]
    a = O.assemble(slot, expert, b.expert_base, b.E_loc, b.P)
    xb = O.decode(O.gather_rows(b.pool, slot, a["perm"], int(a["offsets"][-1])), b.act)
    y = O.expert_ffn(xb, a["offsets"], wts)
    r = b.remote
    rsel = np.isin(r.tok, tok)
    ridx = r.row_idx[rsel]
    uniq, inv = np.unique(ridx, return_inverse=True)
    cs = O.CombineState(b.T, b.K)
    O.combine_release(cs, O.decode(r.rows[uniq], r.dtype), inv.astype(np.int32), r.tok[rsel], r.kslot[rsel],
                      r.w[rsel], r.gen[rsel])
    _, rel, _ = O.combine_release(cs, y, a["pos"], tok, b.kslot[sel], b.w[sel], b.gen[sel])
    assert len(rel) == int(sel.sum())
    return int(sel.sum())


def cpu_baseline_prefill(b, wts, seconds: float, seconds_1core: float) -> dict:
    """The oracle on whole experts of the first prefill wave, in a seeded random order of
    experts, until `seconds` (all BLAS threads) and `seconds_1core` (one thread)."""
    import threadpoolctl

    order = list(np.random.default_rng(7).permutation(b.E_loc))

    def run(budget):
        pairs, done, t0 = 0, [], time.perf_counter()
        for e in order:
            pairs += _oracle_subqueue(b, wts, [e])
            done.append(int(e))
            if time.perf_counter() - t0 >= budget:
                break
        return pairs, done, time.perf_counter() - t0

    pairs, done, el = run(seconds)
    out = {"value": pairs / el, "unit": "expert tokens/s", "cores": blas_threads(), "kind": "oracle", **cpu_info(),
           "sample": f"whole local experts {done} of the first prefill wave ({pairs} of its {b.n} pairs): for "
                     f"each, assemble of its sub-queue, gather, fp64 SwiGLU FFN with the expert's fp8 weights "
                     f"decoded once, combine with the tokens' 7 remote results; {el:.1f} s"}
    if seconds_1core > 0:
        with threadpoolctl.threadpool_limits(1):
            p1, d1, e1 = run(seconds_1core)
        out["value_1core"] = p1 / e1
        out["sample_1core"] = f"whole local experts {d1} ({p1} pairs) with one BLAS thread, {e1:.1f} s"
    return out


# ------------------------------------------------------------------------------ workloads
def run_decode(args, W_steps: int, K_steps: int, cpu_seconds: float) -> dict:
    import torch

    import workloads as W

    b, wts = W.c1_decode()
    run = StepRunner([b], wts, 1, 1, W_steps + K_steps, args.weight_copies)
    if args.calibration_copy and args.workload == "decode":
        calibration_copy(torch.device("cuda:0"))
    total_ms, pairs = run.timed(W_steps, K_steps)
    ev = HipEvents()
    stg = run.stages(ev, max(1, min(K_steps, 20)))[0]
    g_ms, g_pairs = run.timed_graph(W_steps, K_steps)
    run2 = StepRunner([b], wts, 1, 1, W_steps + K_steps, weights_from=run)
    p_ms, p_pairs = timed_two_streams([run, run2], W_steps, K_steps)
    del run2
    counts = run.st.counts.cpu().numpy()
    active = int((counts > 0).sum())
    H, I, n = b.H, wts.I, b.n
    gu_bytes = active * 2 * H * I * 2 + n * H * 2 + n * I * 2
    gu_ms = stg["gate_up_kernel"]
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
    out = {
        "value": round(pairs / (total_ms * 1e-3), 1), "unit": "expert tokens/s", "steps": K_steps,
        "warmup": W_steps, "ms_per_step": round(total_ms / K_steps, 5), "dtype": "bf16",
        "config": {"workload": "decode-shaped EP rank share: 8 of 128 experts, top-4, hidden 2880, SwiGLU "
                               "intermediate 2880, 256 token-expert pairs from a 4096-slot token pool",
                   "E_loc": b.E_loc, "K": b.K, "H": H, "I": I, "pairs": n, "tokens": b.T, "pool_slots": b.P,
                   "weight_copies": len(run.w_copies)},
        "roofline": {"bound": "hbm", "kernel": "ffn_mfma_kernel<gate/up, bf16>", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic("decode"), "algorithmic_bytes": gu_bytes,
                     "kernel_us": round(gu_ms * 1e3, 2)},
        "stages_us": {k: round(v * 1e3, 2) for k, v in stg.items()},
        "graph": {"value": round(g_pairs / (g_ms * 1e-3), 1), "ms_per_step": round(g_ms / K_steps, 5),
                  "note": "the same K steps captured as one HIP graph and replayed once"},
        "two_streams": {"value": round(p_pairs / (p_ms * 1e-3), 1), "ms_per_step": round(p_ms / K_steps, 5),
                        "note": "the same K steps alternating between two sets of buffers and combine states "
                                "(the same weight copies) on two streams, so that consecutive steps overlap"},
    }
    out["cpu_baseline"] = cpu_baseline_decode(b, wts, cpu_seconds) if cpu_seconds > 0 else None
    return out


def timed_two_streams(runs, W: int, K: int):
    """Steps alternating between two runners (separate buffers and combine states, the same packed
    weights), step s on stream s % 2 after W warm-up steps: consecutive batches are independent
    (different tokens, different buffers), so one step's combine and launch gaps overlap the next
    step's kernels.  Every step is the whole hot path over its batch; both runners' last steps are
    checked.  Returns (ms, sum of pairs)."""
    torch, M = runs[0].torch, runs[0].M
    for i, r in enumerate(runs):
        M.moe_state_reset(r.st.state, 0)
        for s in range(i, W + K, 2):
            r.deliver(s)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in range(W):
        with torch.cuda.stream(streams[s % 2]):
            runs[s % 2].step(s)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for st in streams:
        st.wait_event(t0)
    for s in range(W, W + K):
        with torch.cuda.stream(streams[s % 2]):
            runs[s % 2].step(s)
    for st in streams:
        e = torch.cuda.Event()
        e.record(st)
        torch.cuda.current_stream().wait_event(e)
    t1.record()
    torch.cuda.synchronize()
    for i, r in enumerate(runs):
        mine = [s for s in range(W, W + K) if s % 2 == i]
        if mine:
            r.check(max(mine))
    return t0.elapsed_time(t1), sum(runs[0].batch(s).n for s in range(W, W + K))


def run_prefill(args) -> dict:
    import torch

    import workloads as W

    setup = W.c4_prefill_setup()
    g = args.merge
    waves = [W.merge_batches([W.c4_wave(setup, w) for w in range(i, i + g)]) for i in range(0, 4, g)]
    if args.waves is not None:  # a subset of the cycle (profiling one wave's kernels)
        waves = [waves[i] for i in args.waves]
    nw = len(waves)
    K_steps, W_steps = args.steps, args.warmup
    run = StepRunner(waves, setup.weights, 1, 2, W_steps + K_steps)
    E, H, I, K = run.E, run.H, run.I, run.K
    if args.calibration_copy:
        calibration_copy(torch.device("cuda:0"))
    total_ms, pairs = run.timed(W_steps, K_steps)
    ev = HipEvents()
    stg = run.stages(ev, max(1, min(K_steps // nw, 5)), flush=True)
    g_ms, g_pairs = run.timed_graph(W_steps, K_steps)
    run2 = StepRunner(waves, setup.weights, 1, 2, W_steps + K_steps, weights_from=run)
    p_ms, p_pairs = timed_two_streams([run, run2], W_steps, K_steps)
    del run2
    per_wave = []
    for w, b in enumerate(waves):
        m, n = stg[w], b.n
        fl = 6.0 * n * H * I
        c_bytes = n * H * 2 + n * H * (4 + 2) + 24 * n  # combine: result rows, held sums, released rows
        per_wave.append({"pairs": n, "us": {k: round(v * 1e3, 2) for k, v in m.items()},
                         "ffn_mfma_frac": round(fl / ((m["gate_up"] + m["down"]) * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "gate_up_mfma_frac": round(4.0 * n * H * I / (m["gate_up_kernel"] * 1e-3) / 1e12
                                                    / BF16_PEAK_TFLOPS, 4),
                         "combine_hbm_frac": round(c_bytes / (m["combine"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "combine_cold_hbm_frac": round(c_bytes / (m["combine_cold"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "combine_cold_dirty_hbm_frac": round(c_bytes / (m["combine_cold_dirty"] * 1e-3) / 1e9
                                                              / HBM_PEAK_GBS, 4)})
    b0 = waves[0]
    gu0_ms = stg[0]["gate_up_kernel"]
    gu_tf = 4.0 * b0.n * H * I / (gu0_ms * 1e-3) / 1e12
    counts = np.bincount(b0.expert - b0.expert_base, minlength=E)
    gu_alg = int((counts > 0).sum()) * 2 * I * H + b0.n * H * 2 + b0.n * I * 2
    out = {
        "metric": METRIC, "value": round(pairs / (total_ms * 1e-3), 1), "unit": "expert tokens/s", "n_gpus": 1,
        "steps": K_steps, "warmup": W_steps, "ms_per_step": round(total_ms / K_steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 activations, fp8 e4m3 weights, fp32 accumulate",
        "data": "synthetic (seeded; random-init expert weights)",
        "config": {"workload": "prefill-shaped EP rank share: 32 of 256 experts, top-8, hidden 4096, SwiGLU "
                               "intermediate 2048, 16384 pairs (Zipf 1.0) in waves of 6554/4915/3277/1638, "
                               "each wave one step",
                   "E_loc": E, "K": K, "H": H, "I": I, "pairs_per_cycle": sum(b.n for b in waves),
                   "pool_slots": b0.P, "waves_per_step": g},
        "roofline": {"bound": "mfma", "kernel": f"ffn gate/up GEMM, first wave ({b0.n} pairs)",
                     "achieved": round(gu_tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tf / BF16_PEAK_TFLOPS, 4), "traffic": stored_traffic("prefill"),
                     "algorithmic_bytes": gu_alg, "kernel_us": round(gu0_ms * 1e3, 2)},
        "graph": {"value": round(g_pairs / (g_ms * 1e-3), 1), "ms_per_step": round(g_ms / K_steps, 5),
                  "note": "the same K steps captured as one HIP graph and replayed once"},
        "two_streams": {"value": round(p_pairs / (p_ms * 1e-3), 1), "ms_per_step": round(p_ms / K_steps, 5),
                        "note": "the same K steps alternating between two sets of buffers and combine states "
                                "(shared weights) on two streams, so that consecutive waves overlap; every step "
                                "is the whole path over its batch, both sets checked"},
        "waves": per_wave,
        "note": "value: K steps timed back to back (step s = wave s mod 4, its remote results delivered before "
                "the timed region; each step's queue index also links its arrivals for the combine, in one "
                "launch); waves[].us: per-stage medians of HIP-event intervals, each step alone (there the index "
                "is timed on its own as assemble and the combine's link step runs at the start of gate_up); "
                "gate_up_kernel and roofline.kernel_us: the gate/up projection alone, from events its dispatch "
                "records; combine_cold: the combine after a 512 MiB write and two read passes over it (caches "
                "hold clean lines of another buffer); combine_cold_dirty: after the write alone (every miss then "
                "also writes back a dirty line)",
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline_prefill(W.c4_wave(setup, 0), setup.weights, args.cpu_seconds,
                                                   args.cpu_seconds / 2)
    else:
        out["cpu_baseline"] = None
    return out


def run_skewed(args) -> dict:
    import workloads as W

    pool = W.c2_pool()
    batches = [W.c2_skewed_batch(i, pool) for i in range(W.C2["batches"])]
    wts = W.c2_weights()
    nb = len(batches)
    run = StepRunner(batches, wts, 1, 1, nb + args.warmup, args.weight_copies)
    # warm-up on the first batches, then all 200 batches back to back: sum n / sum time
    W_steps = args.warmup
    for s in range(W_steps + nb):
        run.deliver(s)
    import torch

    torch.cuda.synchronize()
    for s in range(W_steps):
        run.step(s)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(W_steps, W_steps + nb):
        run.step(s)
    t1.record()
    torch.cuda.synchronize()
    assert int(run.st.err.item()) == 0
    ms = t0.elapsed_time(t1)
    # (step s runs batch s mod 200, so the timed steps cover every batch once)
    pairs = sum(run.batch(s).n for s in range(W_steps, W_steps + nb))
    sizes = np.array([b.n for b in batches])
    return {"metric": METRIC, "value": round(pairs / (ms * 1e-3), 1), "unit": "expert tokens/s", "n_gpus": 1,
            "steps": nb, "warmup": W_steps, "ms_per_step": round(ms / nb, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded)",
            "config": {"workload": "skewed ragged routing: decode layer shape, Zipf(1.2) over 8 local experts, "
                                   "200 batches of U{8..512} pairs", "pairs": int(sizes.sum()),
                       "batch_pairs_mean": float(sizes.mean()), "weight_copies": len(run.w_copies)},
            "roofline": None,
            "cpu_baseline": cpu_baseline_batches(batches, wts, args.cpu_seconds, "skewed batches")
            if args.cpu_seconds > 0 else None}


def run_tiny(args) -> dict:
    import workloads as W

    b, wts = W.c0_tiny()
    run = StepRunner([b], wts, 0, 0, args.warmup + args.steps)
    ms, pairs = run.timed(args.warmup, args.steps)
    return {"metric": METRIC, "value": round(pairs / (ms * 1e-3), 1), "unit": "expert tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms / args.steps, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded)",
            "config": {"workload": "tiny single MoE layer: 8 experts, top-2, hidden 64, intermediate 128, fp32, "
                                   "64 pairs", "pairs": b.n},
            "roofline": None,
            "cpu_baseline": cpu_baseline_batches([b] * 100000, wts, min(args.cpu_seconds, 5.0), "tiny layer")
            if args.cpu_seconds > 0 else None}


def run_launch(args) -> dict:
    """Prefill launch policies on the HIP path: seeded wave arrival times, the GPU running one
    step at a time, each step's duration measured on the device for the batch the policy
    formed (state reset and remote delivery untimed before it; median of 3 runs, cached per
    batch)."""
    import torch

    import asynchronous_moe_expert_amd as M
    import workloads as W
    from workloads.device import batch_tensors, tensor, weight_tensors
    from workloads.launch import run_policy, summarize, wave_arrivals

    setup = W.c4_prefill_setup()
    waves = [W.c4_wave(setup, w) for w in range(4)]
    sizes = [b.n for b in waves]
    E, H, I, K, P = setup.weights.E, setup.weights.H, setup.weights.I, waves[0].K, waves[0].P
    st = M.ExpertStep(E, H, I, K, M.MOE_BF16, M.MOE_FP8_E4M3, sum(sizes), P)
    wt = weight_tensors(setup.weights)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt["s_gate"], wt["s_up"], wt["s_down"])
    del wt
    pool = tensor(setup.pool, "bf16")
    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = ev.create(), ev.create()
    cache: dict = {}

    def step_ms(combo) -> float:
        if combo in cache:
            return cache[combo]
        b = W.merge_batches([waves[w] for w in combo])
        d = batch_tensors(b)
        d.pop("pool")
        ts = []
        for _ in range(3):
            M.moe_state_reset(st.state, 0)
            st.combine(d["r_rows"], d["r_idx"], d["r_tok"], d["r_kslot"], d["r_w"], d["r_gen"])
            ev.record(e0, stream)
            st.run(d["slot"], d["expert"], 0, pool, d["tok"], d["kslot"], d["w"], d["gen"], n=b.n)
            ev.record(e1, stream)
            torch.cuda.synchronize()
            assert int(st.err.item()) == 0 and int(st.rel_count.item()) == b.n
            ts.append(ev.ms(e0, e1))
        cache[combo] = float(np.median(ts))
        return cache[combo]

    results = {}
    for gap in args.gaps:
        arr = wave_arrivals(20261202 + 4, 4, gap)
        row = {"arrivals_ms": [round(float(a), 4) for a in arr]}
        for policy, mb in [("early", 0), ("all", 0)] + [("minbatch", b) for b in args.min_batch]:
            key = policy if policy != "minbatch" else f"minbatch_{mb}"
            row[key] = summarize(run_policy(policy, arr, sizes, step_ms, mb), arr, sizes)
        results[f"mean_gap_{gap}ms"] = row
    mid = results[f"mean_gap_{args.gaps[len(args.gaps) // 2]}ms"][f"minbatch_{args.min_batch[-1]}"]
    return {"metric": METRIC, "value": mid["pairs_per_gpu_s"], "unit": "expert tokens/s", "n_gpus": 1,
            "steps": None, "warmup": 0, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16 activations, fp8 e4m3 weights, fp32 accumulate", "data": "synthetic (seeded)",
            "config": {"workload": "prefill launch policies: the four prefill waves (6554/4915/3277/1638 "
                                   "pairs) arriving after seeded Exponential gaps; launch each wave early, "
                                   "merge all, or launch at a minimum batch", "mean_gaps_ms": args.gaps,
                       "min_batch": args.min_batch},
            "step_ms_by_batch": {"+".join(map(str, k)): round(v, 4) for k, v in sorted(cache.items())},
            "policies": results,
            "note": "value: pairs per GPU-second of the minimum-batch policy at the middle gap; pairs_per_s "
                    "divides by the makespan from the first arrival; token latency = completion of the "
                    "step carrying the token minus its wave's arrival"}


def run_stream_bench(args) -> dict:
    """The multi-layer stream on the HIP path under one queue-pick policy.  Every expert
    batch and message delivery is one combine call whose release list feeds the queues
    back, so the host waits for each call; GPU time is summed from HIP events around the
    calls, wall time is the whole loop."""
    import torch

    import asynchronous_moe_expert_amd as M
    import workloads as W
    from workloads.device import device_layer_weights
    from workloads.stream import StreamConfig, StreamSim, run_stream

    cfg = StreamConfig(policy=args.policy, batches=args.batches)
    sim = StreamSim(cfg)
    rows_f, xs_f = sim.banks()
    rows_t = torch.from_numpy(W.to_bf16_bits(rows_f).view(np.int16)).view(torch.bfloat16).cuda()
    xs_t = torch.from_numpy(W.to_bf16_bits(xs_f).view(np.int16)).view(torch.bfloat16).cuda()
    del rows_f, xs_f
    st = M.ExpertStep(cfg.E_loc, cfg.H, cfg.I, cfg.K, M.MOE_BF16, M.MOE_BF16, cfg.cap, cfg.tokens)
    packed = []
    for l in range(cfg.layers):
        w = device_layer_weights(cfg.seed, l, cfg.E_loc, cfg.H, cfg.I, 0.02)
        st.load_weights(w["wg"], w["wu"], w["wd"])
        packed.append((st.w_gu, st.w_d))
        del w
    pool = torch.empty((cfg.tokens, cfg.H), dtype=torch.bfloat16, device="cuda")
    base = cfg.rank * cfg.E_loc
    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = ev.create(), ev.create()
    acc = {"gpu_ms": 0.0, "pairs": 0, "msgs": 0}
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731

    def call(fn):
        ev.record(e0, stream)
        fn()
        ev.record(e1, stream)
        acc["gpu_ms"] += ev.ms(e0, e1)
        n_rel = int(st.rel_count.item())
        return st.rel_list[:n_rel].cpu().numpy()

    def on_attention(l, toks):
        t = torch.as_tensor(toks, device="cuda")
        pool[t] = xs_t[torch.as_tensor(sim.x_row(toks, l), device="cuda")]

    def on_messages(m):
        acc["msgs"] += 1
        args_ = (rows_t, i32(m.row), i32(m.tok), i32(m.kslot), torch.from_numpy(m.w).cuda(),
                 i32(m.gen.view(np.int32)))
        return call(lambda: st.combine(*args_, m=len(m.tok), n_rows=cfg.row_bank))

    def on_batch(b):
        st.w_gu, st.w_d = packed[b.layer]
        acc["pairs"] += b.n
        args_ = (i32(b.slot), i32(b.expert), base, pool, i32(b.tok), i32(b.kslot), torch.from_numpy(b.w).cuda(),
                 i32(b.gen.view(np.int32)))
        return call(lambda: st.run(*args_, n=b.n))

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_stream(sim, on_attention, on_messages, on_batch)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(st.err.item()) == 0, "device error flags raised"
    sizes = np.array([x[2] for x in sim.log if x[0] == "X"])
    lat = np.array(sim.latency)
    pct = lambda a, q: float(np.percentile(a, q)) if len(a) else None  # noqa: E731
    return {
        "metric": METRIC, "value": round(acc["pairs"] / (acc["gpu_ms"] * 1e-3), 1), "unit": "expert tokens/s",
        "n_gpus": 1, "steps": int(sim.batches_done), "warmup": 0, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded stream; random-init expert weights)",
        "config": {"workload": "multi-layer asynchronous stream: 36 layers (72 micro-queues), 8 of 128 experts, "
                               "top-4, hidden 2880, 4096 home tokens, 16 sources with lognormal(0,1) delays",
                   "policy": cfg.policy, "window": cfg.window, "delta": cfg.delta, "hist": cfg.hist,
                   "cap": cfg.cap, "expert_batches": int(sim.batches_done)},
        "stream": {"scheduler_steps": int(sim.tau), "layer_releases": int(len(lat)),
                   "layer_releases_per_batch": round(len(lat) / max(1, sim.batches_done), 2),
                   "batch_pairs": {"mean": round(float(sizes.mean()), 1), "p10": pct(sizes, 10),
                                   "p50": pct(sizes, 50), "p90": pct(sizes, 90), "max": int(sizes.max()),
                                   "under_64": int((sizes < 64).sum())},
                   "layer_latency_steps": {"p50": pct(lat, 50), "p90": pct(lat, 90), "p99": pct(lat, 99),
                                           "max": int(lat.max()) if len(lat) else None},
                   "message_deliveries": acc["msgs"], "gpu_ms": round(acc["gpu_ms"], 2),
                   "wall_s": round(wall, 2)},
        "note": "value = expert pairs / GPU time of the expert-step and delivery calls (HIP events); the host "
                "waits for each call's release list, so wall time includes the scheduler in Python",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle CPU-baseline budget (0 = skip)")
    ap.add_argument("--workload", choices=["prefill", "decode", "skewed", "tiny", "stream", "launch"],
                    default="prefill")
    ap.add_argument("--gaps", type=float, nargs="+", default=[0.1, 0.3, 1.0],
                    help="launch: mean gaps (ms) between prefill waves")
    ap.add_argument("--min-batch", type=int, nargs="+", default=[4096, 8192],
                    help="launch: minimum-batch thresholds (pairs)")
    ap.add_argument("--policy", choices=["mtfs", "flfs", "defrag"], default="mtfs",
                    help="queue pick of the stream workload")
    ap.add_argument("--batches", type=int, default=1000, help="expert batches of the stream workload")
    ap.add_argument("--merge", type=int, choices=[1, 2, 4], default=1,
                    help="prefill: consecutive waves merged into one ready batch (1 = each wave alone)")
    ap.add_argument("--weight-copies", type=int, default=4,
                    help="decode/skewed: packed copies of the layer's weights the steps cycle through (so that no "
                         "step finds weights left in the caches by the one before, as in a model of many layers)")
    ap.add_argument("--no-decode", action="store_true", help="prefill: skip the decode sub-object")
    ap.add_argument("--waves", type=int, nargs="+", default=None,
                    help="prefill: run only these steps of the cycle (e.g. 0 for the 6554-pair wave)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="copy 256 MiB device to device once before the warm-up (reference dispatch for "
                         "rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one expert-parallel rank's share on one GPU; there is no multi-GPU mode "
              "(run it with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import asynchronous_moe_expert_amd as M

    M.load()
    torch.cuda.set_device(0)
    if args.workload == "prefill":
        out = run_prefill(args)
        if not args.no_decode:
            out["decode"] = run_decode(args, 10, 50, min(args.cpu_seconds, 5.0))
    elif args.workload == "decode":
        d = run_decode(args, args.warmup, args.steps, args.cpu_seconds)
        out = {"metric": METRIC, "value": d.pop("value"), "unit": d.pop("unit"), "n_gpus": 1,
               "steps": d.pop("steps"), "warmup": d.pop("warmup"), "ms_per_step": d.pop("ms_per_step"),
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": d.pop("dtype"),
               "data": "synthetic (seeded; random-init expert weights)", **d}
    elif args.workload == "skewed":
        out = run_skewed(args)
    elif args.workload == "tiny":
        out = run_tiny(args)
    elif args.workload == "launch":
        out = run_launch(args)
    else:
        out = run_stream_bench(args)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
