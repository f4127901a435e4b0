"""A whole step captured once as a HIP graph and replayed on fixed buffers ([SEP] section 6:
per-layer graphs with intermediate buffers shared across steps).  Each replay runs the whole
step on inputs written into the captured buffers beforehand: a differently ordered queue and a
fresh range of combine-state tokens per replay.  The decode step (moe_assemble inside the gate/up
launch with the combine plan, moe_combine_apply) must match the oracle on every replay (integer
outputs bit for bit, released rows within the bf16 tolerance); the prefill-sized step must give
the bits of the same step run eagerly."""
import numpy as np
import pytest
import torch

import asynchronous_moe_expert_amd as M
import oracle as O
import workloads as W
from gpu_helpers import TOL, decode_tensor, dev, row_rel_err, sync_err
from workloads.device import batch_tensors, weight_tensors

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replay():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    print("decode step as a captured graph, 4 replays", flush=True)
    b, wts = W.c1_decode()
    n, T, S = b.n, b.T, 4
    d = batch_tensors(b)
    wt = weight_tensors(wts)
    st = M.ExpertStep(b.E_loc, b.H, wts.I, b.K, M.MOE_BF16, M.MOE_BF16, n, (S + 1) * T)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"])
    rng = np.random.default_rng(2024)
    perms = [rng.permutation(n) for _ in range(S + 1)]
    # the remote results of every replay's tokens (token range s), delivered eagerly first
    r = b.remote
    for s in range(S + 1):
        st.combine(d["r_rows"], d["r_idx"], dev(r.tok + s * T), d["r_kslot"], d["r_w"], d["r_gen"])
    torch.cuda.synchronize()
    assert int(st.rel_count.item()) == 0
    # the captured buffers
    bufs = {k: torch.empty(n, dtype=torch.int32, device="cuda") for k in ("slot", "expert", "tok", "kslot", "gen")}
    bufs["w"] = torch.empty(n, dtype=torch.float32, device="cuda")

    def stage(s):
        p = perms[s]
        bufs["slot"].copy_(dev(b.slot[p]))
        bufs["expert"].copy_(dev(b.expert[p]))
        bufs["tok"].copy_(dev((b.tok[p] + s * T).astype(np.int32)))
        bufs["kslot"].copy_(dev(b.kslot[p]))
        bufs["gen"].copy_(dev(b.gen[p]))
        bufs["w"].copy_(dev(b.w[p]))

    def step():
        st.run(bufs["slot"], bufs["expert"], b.expert_base, d["pool"], bufs["tok"], bufs["kslot"], bufs["w"],
               bufs["gen"], n=n)

    # one eager step first (token range S), so that the library's one-time host queries are done
    stage(S)
    step()
    torch.cuda.synchronize()
    assert int(st.rel_count.item()) == T and sync_err(st.err) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    assert int(st.rel_count.item()) == T, "capture must not run the step"
    a0 = O.assemble(b.slot, b.expert, b.expert_base, b.E_loc, b.P)
    y0 = O.expert_ffn(O.decode(O.gather_rows(b.pool, b.slot, a0["perm"], n), "bf16"), a0["offsets"], wts)
    y_of_pair = np.empty_like(y0)
    y_of_pair[a0["perm"]] = y0  # FFN output of queue entry i of the unpermuted queue
    rem = O.decode(r.rows, r.dtype)
    for s in range(S):
        stage(s)
        g.replay()
        torch.cuda.synchronize()
        p = perms[s]
        a = O.assemble(b.slot[p], b.expert[p], b.expert_base, b.E_loc, b.P)
        assert sync_err(st.err) == 0 == a["err"]
        assert np.array_equal(st.perm.cpu().numpy()[:n], a["perm"]), f"perm differs on replay {s}"
        assert np.array_equal(st.pos.cpu().numpy()[:n], a["pos"]), f"pos differs on replay {s}"
        assert np.array_equal(st.offsets.cpu().numpy(), a["offsets"]), f"offsets differ on replay {s}"
        ocs = O.CombineState(T, b.K)
        O.combine_release(ocs, rem, r.row_idx, r.tok, r.kslot, r.w, r.gen)
        y_rows = y_of_pair[p][a["perm"]]  # batch row r holds entry perm[r] of this replay's queue
        out, rel, oerr = O.combine_release(ocs, y_rows, a["pos"], b.tok[p], b.kslot[p], b.w[p], b.gen[p])
        n_rel = int(st.rel_count.item())
        assert oerr == 0 and n_rel == T
        assert np.array_equal(st.rel_list[:n_rel].cpu().numpy(), rel + s * T), f"release list differs on replay {s}"
        ey = row_rel_err(decode_tensor(st.y[:n]), y_rows)
        g_out = decode_tensor(st.out[torch.as_tensor(rel + s * T, device="cuda").long()])
        eo = row_rel_err(g_out, np.array([out[t] for t in rel]))
        print(f"  replay {s}: Y row err {ey:.3e}, combined row err {eo:.3e}, released {n_rel}", flush=True)
        assert ey <= TOL["bf16"] and eo <= TOL["bf16"]


def test_prefill_step_graph_replay():
    """A prefill-sized step (3277 pairs, fp8 weights: the index launch that also links the
    combine's arrivals, the 256-row GEMM for both projections, the list-path merge and release)
    captured once and replayed on differently ordered queues and fresh token ranges: every replay
    gives the same bits as the same step run eagerly (index outputs, FFN rows, error word, release
    list, released rows, masks and generations)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    print("prefill step as a captured graph, 3 replays", flush=True)
    setup = W.c4_prefill_setup()
    b = W.c4_wave(setup, 2)
    n, T, S = b.n, b.T, 3
    d = batch_tensors(b)
    wt = weight_tensors(setup.weights)
    r = b.remote

    def new_step():
        st = M.ExpertStep(b.E_loc, b.H, setup.weights.I, b.K, M.MOE_BF16, M.MOE_FP8_E4M3, n, (S + 1) * T)
        st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt["s_gate"], wt["s_up"], wt["s_down"])
        for s in range(S + 1):  # every token range's remote results, delivered eagerly first
            st.combine(d["r_rows"], d["r_idx"], dev(r.tok + s * T), d["r_kslot"], d["r_w"], d["r_gen"])
        return st

    gs, es = new_step(), new_step()
    torch.cuda.synchronize()
    assert int(gs.rel_count.item()) == 0 == int(es.rel_count.item())
    rng = np.random.default_rng(7)
    perms = [rng.permutation(n) for _ in range(S + 1)]
    bufs = {k: torch.empty(n, dtype=torch.int32, device="cuda") for k in ("slot", "expert", "tok", "kslot", "gen")}
    bufs["w"] = torch.empty(n, dtype=torch.float32, device="cuda")

    def inputs(s):
        p = perms[s]
        return dict(slot=b.slot[p], expert=b.expert[p], tok=(b.tok[p] + s * T).astype(np.int32), kslot=b.kslot[p],
                    gen=b.gen[p], w=b.w[p])

    def run(st, x):
        st.run(x["slot"], x["expert"], b.expert_base, d["pool"], x["tok"], x["kslot"], x["w"], x["gen"], n=n)

    def result(st, s):
        cnt = int(st.rel_count.item())
        rel = st.rel_list[:cnt]
        lo, hi = s * T, (s + 1) * T
        return dict(err=sync_err(st.err), perm=st.perm[:n].cpu().numpy(), pos=st.pos[:n].cpu().numpy(),
                    offsets=st.offsets.cpu().numpy(), y=st.y[:n].view(torch.int16).cpu().numpy(),
                    rel=rel.cpu().numpy(), out=st.out[rel.long()].view(torch.int16).cpu().numpy(),
                    mask=st.state.mask[lo:hi].cpu().numpy(), tgen=st.state.tgen[lo:hi].cpu().numpy())

    # one eager step on the graph's buffers first (token range S), then the capture
    for k, v in inputs(S).items():
        bufs[k].copy_(dev(v))
    run(gs, bufs)
    torch.cuda.synchronize()
    # (token indices span the whole pool, T = 16384; each of the wave's tokens has one local pair)
    assert int(gs.rel_count.item()) == n and sync_err(gs.err) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(gs, bufs)
    torch.cuda.synchronize()
    for s in range(S):
        x = inputs(s)
        for k, v in x.items():
            bufs[k].copy_(dev(v))
        g.replay()
        torch.cuda.synchronize()
        got = result(gs, s)
        run(es, {k: dev(v) for k, v in x.items()})
        torch.cuda.synchronize()
        want = result(es, s)
        assert got["err"] == 0 == want["err"]
        assert len(got["rel"]) == n, f"replay {s} released {len(got['rel'])} of {n}"
        for k in ("perm", "pos", "offsets", "y", "rel", "out", "mask", "tgen"):
            assert np.array_equal(got[k], want[k]), f"{k} differs on replay {s}"
        print(f"  replay {s}: {n} released, same bits as the eager step", flush=True)
