"""Steps that run at the same time.  From several host threads: each thread runs decode steps on
its own stream and its own buffers while the other does the same (the library's only state kept
across calls on the host side is per-device kernel occupancy, cached with atomic stores, so the
calls need no lock).  From one thread on two streams: consecutive prefill steps alternate between
two sets of buffers that share the packed weights.  Every step gives the bits of the same steps
run one after another."""
import threading

import numpy as np
import pytest
import torch

import asynchronous_moe_expert_amd as M
import workloads as W
from gpu_helpers import dev
from workloads.device import batch_tensors, weight_tensors

pytestmark = pytest.mark.gpu


def test_steps_from_two_host_threads():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    print("decode steps from two host threads, each on its own stream", flush=True)
    b, wts = W.c1_decode()
    n, T, R = b.n, b.T, 4
    d = batch_tensors(b)
    wt = weight_tensors(wts)
    r = b.remote
    toks = [dev((b.tok + s * T).astype(np.int32)) for s in range(R)]
    rtoks = [dev((r.tok + s * T).astype(np.int32)) for s in range(R)]
    torch.cuda.synchronize()

    def new_step():
        st = M.ExpertStep(b.E_loc, b.H, wts.I, b.K, M.MOE_BF16, M.MOE_BF16, n, R * T)
        st.load_weights(wt["wg"], wt["wu"], wt["wd"])
        torch.cuda.synchronize()
        return st

    def steps(st, stream, out):
        with torch.cuda.stream(stream):
            for s in range(R):
                st.combine(d["r_rows"], d["r_idx"], rtoks[s], d["r_kslot"], d["r_w"], d["r_gen"])
                st.run(d["slot"], d["expert"], b.expert_base, d["pool"], toks[s], d["kslot"], d["w"], d["gen"])
                stream.synchronize()
                cnt = int(st.rel_count.item())
                rel = st.rel_list[:cnt]
                out.append(dict(err=int(st.err.item()), y=st.y[:n].view(torch.int16).cpu().numpy(),
                                rel=rel.cpu().numpy(), out=st.out[rel.long()].view(torch.int16).cpu().numpy(),
                                mask=st.state.mask[s * T:(s + 1) * T].cpu().numpy()))

    ref = []
    steps(new_step(), torch.cuda.Stream(), ref)
    assert all(x["err"] == 0 and len(x["rel"]) > 0 for x in ref)
    sts = [new_step(), new_step()]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    errors = []

    def worker(i):
        try:
            steps(sts[i], streams[i], outs[i])
        except Exception as e:  # re-raised in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    if errors:
        raise errors[0]
    for i in range(2):
        assert len(outs[i]) == R
        for s in range(R):
            for k in ("err", "y", "rel", "out", "mask"):
                assert np.array_equal(outs[i][s][k], ref[s][k]), f"thread {i}, step {s}: {k} differs"
    print(f"  2 threads x {R} steps: the bits of the single-thread run", flush=True)


def test_prefill_steps_on_two_streams():
    """Prefill-sized steps (4915 and 3277 pairs, fp8 weights) alternating between two sets of
    buffers on two streams, so that consecutive steps' kernels run at the same time and share the
    packed weights: every step gives the bits of the same steps run one after another."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    print("prefill steps on two streams", flush=True)
    setup = W.c4_prefill_setup()
    waves = [W.c4_wave(setup, 1), W.c4_wave(setup, 2)]
    R, Tt = 4, 16384  # steps; token indices span the whole pool
    ds = [batch_tensors(b) for b in waves]
    wt = weight_tensors(setup.weights)
    nmax = max(b.n for b in waves)

    def new_step(src=None):
        st = M.ExpertStep(32, 4096, setup.weights.I, 8, M.MOE_BF16, M.MOE_FP8_E4M3, nmax, R * Tt)
        if src is None:
            st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt["s_gate"], wt["s_up"], wt["s_down"])
        else:
            st.w_gu, st.w_d = src.w_gu, src.w_d
            st.s_gate, st.s_up, st.s_down = src.s_gate, src.s_up, src.s_down
        return st

    def deliver(st, s):
        b, d = waves[s % 2], ds[s % 2]
        r = b.remote
        st.combine(d["r_rows"], d["r_idx"], dev((r.tok + s * Tt).astype(np.int32)), d["r_kslot"], d["r_w"], d["r_gen"])

    def step(st, s):
        b, d = waves[s % 2], ds[s % 2]
        st.run(d["slot"], d["expert"], b.expert_base, d["pool"], dev((b.tok + s * Tt).astype(np.int32)), d["kslot"],
               d["w"], d["gen"])

    def result(st, s):
        n = waves[s % 2].n
        cnt = int(st.rel_count.item())
        rel = st.rel_list[:cnt]
        return dict(err=int(st.err.item()), y=st.y[:n].view(torch.int16).cpu().numpy(), rel=rel.cpu().numpy(),
                    out=st.out[rel.long()].view(torch.int16).cpu().numpy(),
                    mask=st.state.mask[s * Tt:(s + 1) * Tt].cpu().numpy())

    ref_st = new_step()
    ref = []
    for s in range(R):
        deliver(ref_st, s)
        step(ref_st, s)
        torch.cuda.synchronize()
        ref.append(result(ref_st, s))
    assert all(x["err"] == 0 and len(x["rel"]) == waves[s % 2].n for s, x in enumerate(ref))
    sts = [new_step(ref_st), new_step(ref_st)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in range(R):
        with torch.cuda.stream(streams[s % 2]):
            deliver(sts[s % 2], s)
    torch.cuda.synchronize()
    got = []
    # steps s and s+1 run together; each pair is read back after both streams finish
    for s0 in range(0, R, 2):
        for s in (s0, s0 + 1):
            with torch.cuda.stream(streams[s % 2]):
                step(sts[s % 2], s)
        torch.cuda.synchronize()
        got += [result(sts[s % 2], s) for s in (s0, s0 + 1)]
    for s in range(R):
        for k in ("err", "y", "rel", "out", "mask"):
            assert np.array_equal(got[s][k], ref[s][k]), f"step {s}: {k} differs"
    print(f"  {R} steps on two streams: the bits of the steps run one after another", flush=True)
