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


# ---------------------------------------------------------------- queue-pick policies
from workloads.stream import defrag_score  # noqa: E402


def test_defrag_score_worked_example(golden):
    """The page's worked example: 20 + 0.5 * 100 + 0.25 * 80 = 90 beats an isolated 60."""
    g = golden("streamep_defrag_score.json")
    a, (n1, n2) = g["candidate_depth"], g["candidate_next_depth_plus_history"]
    # chain: [A, next1, next2, isolated, <empty>...]; next1 = 70 queued + 30 drained,
    # next2 = 80 queued; nothing follows the isolated queue within the window
    depth = [a, 70, 80, g["isolated_depth"], 0, 0]
    drained = [0, n1 - 70, n2 - 80, 0, 0, 0]
    assert defrag_score(depth, drained, 0, g["window"], g["delta"]) == g["candidate_score"]
    assert defrag_score(depth, drained, 3, g["window"], g["delta"]) == g["isolated_score"]
    # The same situation in a stream.  Chain: A_0 empty, X_0 = candidate (20 queued),
    # A_1 = 10 queued + 90 drained in recent steps, X_1 = 10 queued + 70 drained,
    # A_2 = the isolated queue (60 queued, nothing after it).  Scores: X_0 = 20 + 0.5 * 100
    # + 0.25 * 80 = 90, A_1 = 10 + 0.5 * 80 + 0.25 * 60 = 65, X_1 = 10 + 0.5 * 60 = 40,
    # A_2 = 60.  The defrag pick takes the candidate, most-tokens-first the isolated queue.
    for policy, want in (("defrag", ("X", 0)), ("mtfs", ("A", 2))):
        cfg = StreamConfig(layers=3, E_total=16, E_loc=4, K=2, H=8, I=8, tokens=200, cap=256, batches=1,
                           row_bank=16, x_bank=8, policy=policy, window=g["window"], delta=g["delta"])
        sim = StreamSim(cfg)
        sim.A[0].clear()
        sim.X[0].extend([(0, 0, 0, 1.0, 0)] * a)
        sim.A[1].extend(range(10))
        sim.X[1].extend([(0, 0, 0, 1.0, 0)] * 10)
        sim.A[2].extend(range(100, 160))
        sim.recent.extend([(2, 90), (3, 70)])
        depth, h = [len(q) for _, q in sim.chain()], sim.drained()
        assert [defrag_score(depth, h, pos, 2, 0.5) for pos in (1, 2, 3, 4)] == [90, 65, 40, 60]
        assert sim.pick() == want, policy


def test_defrag_reduces_to_most_tokens_first_without_lookahead():
    rng = np.random.default_rng(3)
    for window, delta in ((0, 0.5), (2, 0.0)):
        cfg = StreamConfig(layers=5, E_total=16, E_loc=4, K=2, H=8, I=8, tokens=8, cap=4, batches=1,
                           row_bank=16, x_bank=8, policy="defrag", window=window, delta=delta)
        ref = StreamConfig(**{**cfg.__dict__, "policy": "mtfs"})
        for _ in range(50):
            sims = [StreamSim(cfg), StreamSim(ref)]
            depths = rng.integers(0, 6, 10)
            for sim in sims:
                sim.A[0].clear()
                for pos, d in enumerate(depths):
                    q = sim.A[pos // 2] if pos % 2 == 0 else sim.X[pos // 2]
                    q.extend([(0, 0, 0, 1.0, 0)] * int(d))
                sim.recent.extend([(int(rng.integers(0, 10)), int(rng.integers(1, 9)))])
            assert sims[0].pick() == sims[1].pick()


def test_defrag_lookahead_truncates_or_wraps_at_the_last_layer():
    depth, drained = [1, 2, 3, 4], [0, 0, 0, 10]
    assert defrag_score(depth, drained, 3, 2, 0.5) == 4                       # nothing after the end
    assert defrag_score(depth, drained, 3, 2, 0.5, wrap=True) == 4 + 0.5 * 1 + 0.25 * 2
    assert defrag_score(depth, drained, 2, 2, 0.5) == 3 + 0.5 * 14


def test_first_layer_first_pick():
    cfg = StreamConfig(layers=3, E_total=16, E_loc=4, K=2, H=8, I=8, tokens=8, cap=4, batches=1,
                       row_bank=16, x_bank=8, policy="flfs")
    sim = StreamSim(cfg)
    sim.A[0].clear()
    assert sim.pick() is None
    sim.A[2].extend(range(8))
    sim.X[1].append((0, 0, 0, 1.0, 0))
    assert sim.pick() == ("X", 1)


def test_every_policy_conserves_results_and_is_deterministic():
    for policy in ("mtfs", "flfs", "defrag"):
        cfg = StreamConfig(layers=3, E_total=16, E_loc=4, K=2, H=8, I=8, tokens=64, cap=32, batches=60,
                           row_bank=256, x_bank=64, policy=policy)
        s1, cs1, t1 = _run(cfg, 60)
        s2, cs2, t2 = _run(cfg, 60)
        assert t1 == t2 and s1.log == s2.log, policy
        assert np.array_equal(cs1.tgen, s1.gen), policy
        held = sum(bin(int(m)).count("1") for m in cs1.mask)
        in_flight = sum(len(q) for q in s1.X) + sum(len(msg.tok) for _, _, msg in s1.msgs)
        waiting = sum(len(q) for q in s1.A)
        assert held + in_flight == cfg.K * (cfg.tokens - waiting), policy
        assert len(s1.latency) == int(s1.gen.sum()), policy   # one latency sample per release
