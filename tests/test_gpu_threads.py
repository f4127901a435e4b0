"""Calls from several host threads at once: each thread runs decode steps on its own stream and
its own buffers while the other does the same, and every step gives the bits of the same steps
run from one thread.  The library's only state kept across calls on the host side is per-device
kernel occupancy, cached with atomic stores, so the calls need no lock."""
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
