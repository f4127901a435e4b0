"""GPU parity on the multi-layer asynchronous stream (36 layers, 72 queues, 16 simulated
sources with lognormal message delays): 1000 expert batches under the most-tokens-first
pick, and 300 under each of the first-layer-first pick (which fragments the expert batches:
most of them under 64 pairs) and the defragmenting score ([SEP] section 4).

The stream drives the HIP path and the oracle in lockstep: after every combine call (the
messages due at a step, or an expert batch) the release lists must be identical, and the
error words zero; the combine state (masks, generations) is compared every 100 batches and
at the end.  On a few sampled batches the FFN rows and the combined rows of the tokens the
batch released are compared with the oracle within the bf16 tolerance."""
import numpy as np
import pytest
import torch

import asynchronous_moe_expert_amd as M
import oracle as O
import workloads as W
from gpu_helpers import TOL, decode_tensor, dev, row_rel_err, sync_err
from workloads.device import device_layer_weights, to_numpy_bits
from workloads.stream import StreamConfig, StreamSim, run_stream

pytestmark = pytest.mark.gpu


class _LayerW:  # host copy of one layer's weights in the oracle's input form
    def __init__(self, d):
        self.dtype = "bf16"
        self.wg, self.wu, self.wd = (to_numpy_bits(d[k]) for k in ("wg", "wu", "wd"))


@pytest.fixture(scope="module")
def packed_layers():
    """The 36 layers' packed expert weights (the same seeded draws for every policy)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    cfg = StreamConfig()
    st = M.ExpertStep(cfg.E_loc, cfg.H, cfg.I, cfg.K, M.MOE_BF16, M.MOE_BF16, 1, 1)
    packed = []
    for l in range(cfg.layers):
        w = device_layer_weights(cfg.seed, l, cfg.E_loc, cfg.H, cfg.I, 0.02)
        st.load_weights(w["wg"], w["wu"], w["wd"])
        packed.append((st.w_gu, st.w_d))
        del w
    torch.cuda.synchronize()
    print("  weights packed for all layers", flush=True)
    return packed


@pytest.mark.parametrize("policy,batches", [("mtfs", 1000), ("flfs", 300), ("defrag", 300)])
def test_c3_stream_lockstep(packed_layers, policy, batches):
    cfg = StreamConfig(policy=policy, batches=batches)
    print(f"C3 stream ({policy}): {cfg.layers} layers, {cfg.tokens} tokens, {cfg.batches} expert batches",
          flush=True)
    sim = StreamSim(cfg)
    rows_f, xs_f = sim.banks()
    rows_bits, xs_bits = W.to_bf16_bits(rows_f), W.to_bf16_bits(xs_f)
    rows_t, xs_t = dev(rows_bits, "bf16"), dev(xs_bits, "bf16")
    del rows_f, xs_f
    st = M.ExpertStep(cfg.E_loc, cfg.H, cfg.I, cfg.K, M.MOE_BF16, M.MOE_BF16, cfg.cap, cfg.tokens)
    packed = packed_layers
    pool = torch.empty((cfg.tokens, cfg.H), dtype=torch.bfloat16, device="cuda")
    base = cfg.rank * cfg.E_loc
    ocs = O.CombineState(cfg.tokens, cfg.K)
    zr = np.zeros((cfg.row_bank, 1))
    zb = np.zeros((cfg.cap, 1))
    sample = {0, 1, cfg.batches // 3, 2 * cfg.batches // 3, cfg.batches - 1}
    parts: dict[int, list] = {}  # token -> [(j, w, row64 or None)] of its current layer
    counters = dict(calls=0, checked_rows=0, checked_tokens=0)

    def gpu_combine(rows, idx, tok, ks, w, gen, m, n_rows):
        st.err.zero_()
        st.combine(rows, dev(idx), dev(tok), dev(ks), dev(w), dev(gen), m=m, n_rows=n_rows)
        e = sync_err(st.err)
        n_rel = int(st.rel_count.item())
        return e, st.rel_list[:n_rel].cpu().numpy()

    def on_attention(l, toks):
        t = torch.as_tensor(toks, device="cuda")
        pool[t] = xs_t[torch.as_tensor(sim.x_row(toks, l), device="cuda")]

    def on_messages(m):
        e, rel_g = gpu_combine(rows_t, m.row, m.tok, m.kslot, m.w, m.gen, len(m.tok), cfg.row_bank)
        out, rel_o, oerr = O.combine_release(ocs, zr, m.row, m.tok, m.kslot, m.w, m.gen)
        counters["calls"] += 1
        assert e == 0 == oerr, f"error flags {e:#x} at step {sim.tau}"
        assert np.array_equal(rel_g, rel_o), f"release lists diverge at step {sim.tau} (message delivery)"
        for t, j, w, r in zip(m.tok, m.kslot, m.w, m.row):
            parts.setdefault(int(t), []).append((int(j), float(w), ("r", int(r))))
        for t in rel_o:
            parts.pop(int(t), None)
        return rel_o

    def on_batch(b):
        k = sim.batches_done
        st.w_gu, st.w_d = packed[b.layer]
        st.err.zero_()
        st.run(dev(b.slot), dev(b.expert), base, pool, dev(b.tok), dev(b.kslot), dev(b.w), dev(b.gen), n=b.n)
        e = sync_err(st.err)
        n_rel = int(st.rel_count.item())
        rel_g = st.rel_list[:n_rel].cpu().numpy()
        a = O.assemble(b.slot, b.expert, base, cfg.E_loc, cfg.tokens)
        out, rel_o, oerr = O.combine_release(ocs, zb[: b.n], a["pos"], b.tok, b.kslot, b.w, b.gen)
        counters["calls"] += 1
        assert e == 0 == oerr == a["err"], f"error flags {e:#x} at batch {k}"
        assert np.array_equal(st.perm.cpu().numpy()[: b.n], a["perm"]), f"perm diverges at batch {k}"
        assert np.array_equal(st.offsets.cpu().numpy(), a["offsets"]), f"offsets diverge at batch {k}"
        assert np.array_equal(rel_g, rel_o), f"release lists diverge at batch {k}"
        for i in range(b.n):
            parts.setdefault(int(b.tok[i]), []).append((int(b.kslot[i]), float(b.w[i]), ("l", k, i)))
        if k in sample:
            wl = _LayerW(device_layer_weights(cfg.seed, b.layer, cfg.E_loc, cfg.H, cfg.I, 0.02))
            x = O.decode_bf16(xs_bits[sim.x_row(b.slot[a["perm"]], b.layer)])
            y = O.expert_ffn(x, a["offsets"], wl)
            ey = row_rel_err(decode_tensor(st.y[: b.n]), y)
            refs, toks = [], []
            for t in rel_o:
                ps = parts.get(int(t), [])
                if len(ps) != cfg.K or any(p[2][0] == "l" and p[2][1] != k for p in ps):
                    continue  # a local result of an earlier batch: its oracle row is not at hand
                rows64 = []
                for j, w, ref in sorted(ps):
                    r = O.decode_bf16(rows_bits[ref[1]]) if ref[0] == "r" else y[a["pos"][ref[2]]]
                    rows64.append((w, r))
                refs.append(O.combine_token(rows64))
                toks.append(int(t))
            eo = row_rel_err(decode_tensor(st.out[torch.as_tensor(toks, device="cuda").long()]), np.array(refs)) \
                if toks else 0.0
            counters["checked_rows"] += b.n
            counters["checked_tokens"] += len(toks)
            if not toks and k + 1 < cfg.batches:
                sample.add(k + 1)  # nothing to compare in this batch: sample the next one too
            print(f"  batch {k} layer {b.layer} n={b.n}: Y row err {ey:.3e}, {len(toks)} combined rows err {eo:.3e}",
                  flush=True)
            assert ey <= TOL["bf16"] and eo <= TOL["bf16"]
        for t in rel_o:
            parts.pop(int(t), None)
        return rel_o

    def progress(s):
        if s.batches_done % 100 == 0:
            assert np.array_equal(st.state.mask.cpu().numpy().view(np.uint32), ocs.mask)
            assert np.array_equal(st.state.tgen.cpu().numpy().view(np.uint32), ocs.tgen)
            print(f"  {s.batches_done} batches, step {s.tau}, {counters['calls']} combine calls: state matches",
                  flush=True)

    run_stream(sim, on_attention, on_messages, on_batch, progress=progress)
    assert np.array_equal(st.state.mask.cpu().numpy().view(np.uint32), ocs.mask)
    assert np.array_equal(st.state.tgen.cpu().numpy().view(np.uint32), ocs.tgen)
    assert counters["checked_tokens"] > 0
    sizes = [x[2] for x in sim.log if x[0] == "X"]
    print(f"  done: {counters['calls']} calls; expert batch size mean {np.mean(sizes):.1f}, max {max(sizes)}",
          flush=True)
