"""CPU checks of the multi-layer stream workload, driven with the oracle as executor."""
import numpy as np

import oracle as O
from workloads.stream import StreamConfig, StreamSim, run_stream


def _run(cfg, batches):
    sim = StreamSim(cfg)
    cs = O.CombineState(cfg.tokens, cfg.K)
    zr = np.zeros((cfg.row_bank, 1))
    zb = np.zeros((cfg.cap, 1))
    trace = []

    def on_messages(m):
        out, rel, err = O.combine_release(cs, zr, m.row, m.tok, m.kslot, m.w, m.gen)
        assert err == 0
        trace.append(("m", tuple(rel)))
        return rel

    def on_batch(b):
        a = O.assemble(b.slot, b.expert, cfg.rank * cfg.E_loc, cfg.E_loc, cfg.tokens)
        assert a["err"] == 0
        out, rel, err = O.combine_release(cs, zb[: b.n], a["pos"], b.tok, b.kslot, b.w, b.gen)
        assert err == 0
        trace.append(("b", b.layer, b.n, tuple(rel)))
        return rel

    run_stream(sim, lambda l, t: None, on_messages, on_batch, max_batches=batches)
    return sim, cs, trace


def test_small_stream_is_deterministic_and_conserves_results():
    cfg = StreamConfig(layers=3, E_total=16, E_loc=4, K=2, H=8, I=8, tokens=64, cap=32, batches=60,
                       row_bank=256, x_bank=64)
    s1, cs1, t1 = _run(cfg, 60)
    s2, cs2, t2 = _run(cfg, 60)
    assert t1 == t2 and s1.log == s2.log
    # every release moved a token one layer on; held partial results match the tokens in flight
    assert np.array_equal(cs1.tgen, s1.gen)
    held = sum(bin(int(m)).count("1") for m in cs1.mask)
    in_flight = sum(len(q) for q in s1.X) + sum(len(msg.tok) for _, _, msg in s1.msgs)
    waiting = sum(len(q) for q in s1.A)
    assert held + in_flight == cfg.K * (cfg.tokens - waiting)


def test_most_tokens_first_pick_and_tie_break():
    cfg = StreamConfig(layers=3, E_total=16, E_loc=4, K=2, H=8, I=8, tokens=8, cap=4, batches=1,
                       row_bank=16, x_bank=8)
    sim = StreamSim(cfg)
    sim.A[0].clear()
    assert sim.pick() is None
    sim.A[2].extend([1, 2])
    sim.X[1].extend([(0, 0, 0, 1.0, 0)] * 2)
    assert sim.pick() == ("X", 1)  # equal sizes: X_1 comes before A_2 in the chain
    sim.A[2].append(3)
    assert sim.pick() == ("A", 2)


def test_release_moves_token_to_next_layer_attention(golden):
    g = golden("streamep_request37_queue.json")
    cfg = StreamConfig(layers=4, E_total=16, E_loc=4, K=2, H=8, I=8, tokens=64, cap=4, batches=1,
                       row_bank=16, x_bank=8)
    sim = StreamSim(cfg)
    t = 37
    sim.A[0].remove(t)
    sim.layer[t] = g["label_before"][0]
    sim.release([t])
    assert sim.layer[t] == g["label_after"][0] and t in sim.A[g["label_after"][0]] and sim.gen[t] == 1
    # the expert of the next hop is not chosen until that layer's attention pick
    assert all(x[0] != t for q in sim.X for x in q)
