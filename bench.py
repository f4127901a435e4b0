"""Benchmark: one expert-parallel rank's expert step on one MI355X.

Workload (decode-shaped rank share): 128 experts, top-4, 16 ranks -> 8 local experts,
hidden 2880, SwiGLU intermediate 2880, bf16; 256 token-expert pairs gathered from random
slots of a 4096-slot token pool, uniform routing, weights ~ N(0, 0.02).

A step = moe_assemble + moe_expert_ffn_grouped + moe_combine_release on one batch, all
inputs resident in HBM.  Each step combines its local results into tokens of its own
(distinct state indices per step), whose results from the other 15 ranks were delivered
before the timed region; every step therefore releases all of its tokens.

Prints one JSON line with the step throughput (expert tokens/s), the roofline of the
dominant kernel (the gate/up GEMM, timed with HIP events on the launch stream) and the
CPU oracle timed on a bounded sample on the host.

--workload stream runs the multi-layer asynchronous stream (36 layers, 72 micro-queues, 16
simulated sources with lognormal delays) for --batches expert batches under the queue pick
--policy (most tokens first, first layer first, or the defragmenting score) and reports the
batch-size distribution, steps, per-layer token latency and the GPU time of the calls.

--workload prefill times the prefill-shaped rank share instead (256 experts, top-8, 32
local experts, hidden 4096, intermediate 2048, fp8 e4m3 weights with bf16 activations,
16384 pairs with Zipf(1.0) routing arriving in four waves of 6554/4915/3277/1638, each
its own step).  Its line reports the FFN against the bf16 MFMA peak and the combine
against the HBM peak (the row gather is fused into the FFN's activation loads).
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

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_gateup_decode_traffic.md")
CALIB_BYTES = 256 << 20
FFN_SRC = os.path.join(ROOT, "asynchronous_moe_expert_amd", "csrc", "ffn.hip")


class HipEvents:
    """Raw hipEvent_t handles (the library records one between its two FFN kernels)."""

    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

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


def stored_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3 counter
    summary, if its counters were taken on the kernel source as it is now (else None)."""
    try:
        text = open(TRAFFIC_FILE).read()
        sha = re.search(r"ffn\.hip sha256: ([0-9a-f]{64})", text).group(1)
        val = re.search(r"traffic bytes per launch: ([0-9]+)", text).group(1)
        src = hashlib.sha256(open(FFN_SRC, "rb").read()).hexdigest()
        return float(val) if sha == src else None
    except (OSError, AttributeError, ValueError):
        return None


def cpu_baseline(b, wts, seconds: float) -> dict:
    """The oracle (fp64 numpy) on the host: whole decode steps, repeated until `seconds`."""
    import threadpoolctl

    import oracle as O

    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] or [1])
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
    return {"value": b.n * reps / el, "unit": "expert tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{reps} whole decode steps of {b.n} token-expert pairs (assemble, fp64 SwiGLU FFN over "
                      f"8 experts, combine incl. the delivery of the remote results), {el:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle CPU-baseline budget (0 = skip)")
    ap.add_argument("--workload", choices=["decode", "prefill", "stream"], default="decode")
    ap.add_argument("--policy", choices=["mtfs", "flfs", "defrag"], default="mtfs",
                    help="queue pick of the stream workload")
    ap.add_argument("--batches", type=int, default=1000, help="expert batches of the stream workload")
    ap.add_argument("--merge", type=int, choices=[1, 2, 4], default=1,
                    help="prefill: consecutive waves merged into one ready batch (1 = each wave alone)")
    ap.add_argument("--weight-copies", type=int, default=4,
                    help="decode: packed copies of the layer's weights the steps cycle through (so that no step "
                         "finds weights left in the caches by the one before, as in a model of many layers)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="copy 256 MiB device to device once before the warm-up (reference dispatch for "
                         "rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs one expert-parallel rank's share on a single GPU; it has no multi-GPU mode "
              "(use --gpus 1)", file=sys.stderr)
        return 2

    if args.workload == "prefill":
        return run_prefill(args)
    if args.workload == "stream":
        return run_stream_bench(args)
    import torch

    import asynchronous_moe_expert_amd as M
    import workloads as W
    from workloads.device import batch_tensors, weight_tensors

    M.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    b, wts = W.c1_decode()
    K_steps, W_steps = args.steps, args.warmup
    S = W_steps + 2 * K_steps  # warmup, the timed loop, then the loop timed per stage
    d = batch_tensors(b)
    wt = weight_tensors(wts)
    st = M.ExpertStep(b.E_loc, b.H, wts.I, b.K, M.MOE_BF16, M.MOE_BF16, b.n, S * b.T)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"])
    del wt
    # copies of the packed weights at distinct addresses; step s uses copy s % L, so the
    # weights a step streams (398 MB) were last read L steps earlier, with L x 398 MB of
    # other weights in between: more than the 256 MB last-level cache holds
    L = max(1, args.weight_copies)
    w_copies = [(st.w_gu, st.w_d)] + [(st.w_gu.clone(), st.w_d.clone()) for _ in range(L - 1)]
    # per-step token indices (each step completes tokens of its own) and the remote
    # results of every step's tokens, delivered before timing
    tok_steps = [d["tok"] + s * b.T for s in range(S)]
    r_tok = torch.cat([d["r_tok"] + s * b.T for s in range(S)])
    rep = lambda x: torch.cat([x] * S)  # noqa: E731
    st.combine(d["r_rows"], rep(d["r_idx"]), r_tok, rep(d["r_kslot"]), rep(d["r_w"]), rep(d["r_gen"]))
    torch.cuda.synchronize()
    assert int(st.rel_count.item()) == 0

    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    e_asm = [ev.create() for _ in range(S)]
    e_mid = [ev.create() for _ in range(S)]
    e_gs = [ev.create() for _ in range(S)]  # taken by the gate/up kernel's own dispatch
    e_ge = [ev.create() for _ in range(S)]
    e_ffn = [ev.create() for _ in range(S)]
    e_end = [ev.create() for _ in range(S)]
    e_start = ev.create()

    def step(s: int) -> None:
        st.w_gu, st.w_d = w_copies[s % L]
        st.run(d["slot"], d["expert"], b.expert_base, d["pool"], tok_steps[s], d["kslot"], d["w"], d["gen"], n=b.n)

    def step_timed(s: int) -> None:
        # the same calls as ExpertStep.run (the combine plan inside the FFN call, then the
        # apply) with HIP events between them on the launch stream
        st.w_gu, st.w_d = w_copies[s % L]
        st.assemble(d["slot"], d["expert"], b.expert_base, d["pool"])
        ev.record(e_asm[s], stream)
        plan = st.local_combine_args(tok_steps[s], d["kslot"], d["w"], d["gen"], b.n)
        st.ffn(b.n, ev_mid=e_mid[s], plan=plan, ev_gu=(e_gs[s], e_ge[s]))
        ev.record(e_ffn[s], stream)
        M.combine_call(plan, "apply")
        ev.record(e_end[s], stream)

    if args.calibration_copy:
        calibration_copy(dev)
    for s in range(W_steps):
        step(s)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(W_steps, W_steps + K_steps):
        step(s)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    assert int(st.err.item()) == 0, "device error flags raised"
    assert int(st.rel_count.item()) == b.T

    timed = range(W_steps + K_steps, S)
    ev.record(e_start, stream)
    for s in timed:
        step_timed(s)
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0 and int(st.rel_count.item()) == b.T
    prev = [e_start] + [e_end[s] for s in timed][:-1]
    asm_ms = np.mean([ev.ms(p, e_asm[s]) for p, s in zip(prev, timed)])
    gu_ms = np.mean([ev.ms(e_asm[s], e_mid[s]) for s in timed])
    gu_kernel_ms = np.mean([ev.ms(e_gs[s], e_ge[s]) for s in timed])  # the kernel alone
    dn_ms = np.mean([ev.ms(e_mid[s], e_ffn[s]) for s in timed])
    cb_ms = np.mean([ev.ms(e_ffn[s], e_end[s]) for s in timed])

    counts = st.counts.cpu().numpy()
    active = int((counts > 0).sum())
    H, I, n = b.H, wts.I, b.n
    gu_bytes = active * 2 * H * I * 2 + n * H * 2 + n * I * 2
    gu_flops = 4.0 * n * H * I
    achieved = gu_bytes / (gu_kernel_ms * 1e-3) / 1e9
    ms_step = total_ms / K_steps
    value = n * K_steps / (total_ms * 1e-3)
    out = {
        "metric": "expert tokens/sec per GPU (assemble+FFN+combine)",
        "value": round(value, 1),
        "unit": "expert tokens/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": W_steps,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init expert weights)",
        "config": {"workload": "decode-shaped EP rank share: 8 of 128 experts, top-4, hidden 2880, SwiGLU "
                               "intermediate 2880, 256 token-expert pairs from a 4096-slot token pool",
                   "E_loc": b.E_loc, "K": b.K, "H": H, "I": I, "pairs": n, "tokens": b.T, "pool_slots": b.P,
                   "weight_copies": L},
        "roofline": {"bound": "hbm", "kernel": "ffn_mfma_kernel<gate/up, bf16>", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(), "algorithmic_bytes": gu_bytes,
                     "kernel_us": round(gu_kernel_ms * 1e3, 2),
                     "mfma_frac": round(gu_flops / (gu_kernel_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 5)},
        "stages_us": {"assemble": round(asm_ms * 1e3, 2), "ffn_gate_up": round(gu_ms * 1e3, 2),
                      "ffn_down": round(dn_ms * 1e3, 2), "combine": round(cb_ms * 1e3, 2),
                      "note": "second K-step loop with HIP events between the calls (events add a "
                              "few us of launch latency to each interval, the gate/up one also its kernel's "
                              "own start/stop events); value is from the loop without; roofline.kernel_us is "
                              "the gate/up kernel alone"},
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(b, wts, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def run_stream_bench(args) -> int:
    """The multi-layer stream on the HIP path under one queue-pick policy.  Every expert
    batch and message delivery is one combine call whose release list feeds the queues
    back, so the host waits for each call; GPU time is summed from HIP events around the
    calls, wall time is the whole loop."""
    import torch

    import asynchronous_moe_expert_amd as M
    import workloads as W
    from workloads.device import device_layer_weights
    from workloads.stream import StreamConfig, StreamSim, run_stream

    M.load()
    torch.cuda.set_device(0)
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
    out = {
        "metric": "expert tokens/sec per GPU (assemble+FFN+combine)",
        "value": round(acc["pairs"] / (acc["gpu_ms"] * 1e-3), 1), "unit": "expert tokens/s", "n_gpus": 1,
        "steps": int(sim.batches_done), "warmup": 0, "higher_is_better": True, "scaling": "weak",
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
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline_prefill(setup, b, seconds: float) -> dict:
    """The oracle's FFN (fp64) on a seeded sample of the first wave's rows, for `seconds`."""
    import threadpoolctl

    import oracle as O

    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] or [1])
    rng = np.random.default_rng(7)
    rows, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        pick = rng.choice(b.n, 16, replace=False)
        x = O.decode(b.pool[b.slot[pick]], "bf16")
        O.ffn_rows(x, b.expert[pick] - b.expert_base, setup.weights)
        rows += len(pick)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": rows / el, "unit": "expert tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{rows} seeded rows of prefill wave 0 ({reps} draws of 16), fp64 SwiGLU FFN only "
                      f"(assemble and combine are a small share of the oracle's time), {el:.1f} s"}


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


def run_prefill(args) -> int:
    """Prefill-shaped rank share: each of the four waves is one step (assemble, FFN,
    combine of the local result into tokens whose 7 remote results were delivered first)."""
    import torch

    import asynchronous_moe_expert_amd as M
    import workloads as W
    from workloads.device import batch_tensors, weight_tensors

    M.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    setup = W.c4_prefill_setup()
    g = args.merge
    waves = [W.merge_batches([W.c4_wave(setup, w) for w in range(i, i + g)]) for i in range(0, 4, g)]
    nw = len(waves)
    E, H, I, K, P = setup.weights.E, setup.weights.H, setup.weights.I, waves[0].K, waves[0].P
    n_max = max(b.n for b in waves)
    wt = weight_tensors(setup.weights)
    st = M.ExpertStep(E, H, I, K, M.MOE_BF16, M.MOE_FP8_E4M3, n_max, P)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt["s_gate"], wt["s_up"], wt["s_down"])
    del wt
    pool = batch_tensors(waves[0])["pool"]
    dw = []
    for b in waves:
        d = batch_tensors(b)
        d.pop("pool")
        dw.append(d)
    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    reps = max(1, args.steps // nw)
    W_reps = max(1, args.warmup // nw)
    names = ["assemble", "gate_up", "down", "combine"]
    times = {w: {k: [] for k in names} for w in range(nw)}
    evs = [ev.create() for _ in range(5)]
    if args.calibration_copy:
        calibration_copy(dev)
    for rep in range(W_reps + reps):
        for w, b in enumerate(waves):
            d = dw[w]
            M.moe_state_reset(st.state, 0)
            st.combine(d["r_rows"], d["r_idx"], d["r_tok"], d["r_kslot"], d["r_w"], d["r_gen"])
            ev.record(evs[0], stream)
            st.assemble(d["slot"], d["expert"], b.expert_base, pool, n=b.n)
            ev.record(evs[1], stream)
            st.ffn(b.n, ev_mid=evs[2])
            ev.record(evs[3], stream)
            st.combine(st.y, st.pos, d["tok"], d["kslot"], d["w"], d["gen"], m=b.n, n_rows=b.n)
            ev.record(evs[4], stream)
            torch.cuda.synchronize()
            assert int(st.err.item()) == 0 and int(st.rel_count.item()) == b.n, "prefill step did not release"
            if rep >= W_reps:
                for k, nm in enumerate(names):
                    times[w][nm].append(ev.ms(evs[k], evs[k + 1]))
    # the gate/up projection's kernel time alone (start/stop events taken by its own
    # dispatches), in a pass of its own so that these events stay out of the intervals above
    gs, ge = ev.create(), ev.create()
    gu_kernel = {w: [] for w in range(nw)}
    for rep in range(reps):
        for w, b in enumerate(waves):
            d = dw[w]
            M.moe_state_reset(st.state, 0)
            st.combine(d["r_rows"], d["r_idx"], d["r_tok"], d["r_kslot"], d["r_w"], d["r_gen"])
            st.assemble(d["slot"], d["expert"], b.expert_base, pool, n=b.n)
            st.ffn(b.n, ev_gu=(gs, ge))
            st.combine(st.y, st.pos, d["tok"], d["kslot"], d["w"], d["gen"], m=b.n, n_rows=b.n)
            torch.cuda.synchronize()
            gu_kernel[w].append(ev.ms(gs, ge))
    med = {w: {nm: float(np.median(times[w][nm])) for nm in names} for w in range(nw)}
    step_ms = sum(sum(med[w].values()) for w in range(nw))
    n_tot = sum(b.n for b in waves)
    value = n_tot / (step_ms * 1e-3)
    per_wave = []
    for w, b in enumerate(waves):
        m = med[w]
        n = b.n
        fl_gu, fl_dn = 4.0 * n * H * I, 2.0 * n * H * I
        c_bytes = n * H * 2 + n * H * (4 + 2) + 24 * n   # combine: result rows, held sums, released rows
        # the row gather is fused into the gate/up GEMM's activation loads (the assemble
        # stage builds the index only), so it has no time of its own to price
        per_wave.append({"pairs": n, "us": {k: round(v * 1e3, 2) for k, v in m.items()},
                         "gate_up_kernel_us": round(float(np.median(gu_kernel[w])) * 1e3, 2),
                         "ffn_mfma_frac": round((fl_gu + fl_dn) / ((m["gate_up"] + m["down"]) * 1e-3) / 1e12
                                                / BF16_PEAK_TFLOPS, 4),
                         "combine_hbm_frac": round(c_bytes / (m["combine"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    b0, m0 = waves[0], med[0]
    gu0_ms = float(np.median(gu_kernel[0]))
    gu_tf = 4.0 * b0.n * H * I / (gu0_ms * 1e-3) / 1e12
    out = {
        "metric": "expert tokens/sec per GPU (assemble+FFN+combine)",
        "value": round(value, 1), "unit": "expert tokens/s", "n_gpus": 1, "steps": reps * nw, "warmup": W_reps * nw,
        "ms_per_step": round(step_ms / nw, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 activations, fp8 e4m3 weights, fp32 accumulate", "data": "synthetic (seeded; random-init expert weights)",
        "config": {"workload": "prefill-shaped EP rank share: 32 of 256 experts, top-8, hidden 4096, SwiGLU "
                               "intermediate 2048, 16384 pairs (Zipf 1.0) in waves of 6554/4915/3277/1638",
                   "E_loc": E, "K": K, "H": H, "I": I, "pairs": n_tot, "pool_slots": P, "waves_per_step": g},
        "roofline": {"bound": "mfma", "kernel": f"ffn gate/up GEMM, first step ({b0.n} pairs)", "achieved": round(gu_tf, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(gu_tf / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel_us": round(gu0_ms * 1e3, 2)},
        "waves": per_wave,
        "note": "per-stage medians of HIP-event intervals on the launch stream; each step is timed alone "
                "(state reset and remote delivery untimed before it); gate_up_kernel_us and roofline.kernel_us: "
                "the gate/up GEMM and its finalize alone, from events its dispatches record, in a separate pass",
    }
    out["cpu_baseline"] = cpu_baseline_prefill(setup, W.c4_wave(setup, 0, with_remote=False), args.cpu_seconds) \
        if args.cpu_seconds > 0 else None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
