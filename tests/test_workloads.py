"""Host-side checks of the seeded input generators (shapes, seeding, structure)."""
import numpy as np

import workloads as W


def _covers_each_position_once(b):
    """Local pairs plus remote arrivals give every token each of its K positions once,
    and the router weights of a token sum to 1."""
    seen = {}
    for t, j, w in zip(b.tok, b.kslot, b.w):
        seen.setdefault(int(t), {})[int(j)] = float(w)
    if b.remote is not None:
        for t, j, w in zip(b.remote.tok, b.remote.kslot, b.remote.w):
            assert int(j) not in seen.setdefault(int(t), {})
            seen[int(t)][int(j)] = float(w)
    assert len(seen) == b.T
    for t, d in seen.items():
        assert sorted(d) == list(range(b.K))
        assert abs(sum(d.values()) - 1.0) < 1e-5


def test_c0_shape_and_determinism():
    b, w = W.c0_tiny()
    assert (b.n, b.T, b.K, b.H, b.P) == (64, 32, 2, 64, 128)
    assert len(set(b.slot.tolist())) == 32 and w.wg.shape == (8, 128, 64) and w.wd.shape == (8, 64, 128)
    b2, w2 = W.c0_tiny()
    assert np.array_equal(b.slot, b2.slot) and np.array_equal(w.wd, w2.wd)
    _covers_each_position_once(b)


def test_c1_exactly_256_pairs_at_distinct_slots():
    b, _ = W.c1_decode(with_weights=False)
    assert b.n == 256 and b.pool.shape == (4096, 2880) and b.pool.dtype == np.uint16
    slots_of_tok = {}
    for s, t in zip(b.slot, b.tok):
        assert slots_of_tok.setdefault(int(t), int(s)) == int(s)
    assert len(set(slots_of_tok.values())) == b.T
    assert np.all((b.expert >= 0) & (b.expert < 8))
    _covers_each_position_once(b)
    b3, _ = W.c1_decode(rank=3, with_weights=False)
    assert np.all((b3.expert >= 24) & (b3.expert < 32)) and b3.expert_base == 24


def test_c2_batches_sizes_and_skew():
    pool = np.zeros((4096, 2880), np.uint16)
    ns, counts = [], np.zeros(8)
    for bi in range(40):
        b = W.c2_skewed_batch(bi, pool)
        assert 8 <= b.n <= 512 and b.T == b.n and len(set(b.slot.tolist())) == b.n
        ns.append(b.n)
        counts += np.bincount(b.expert, minlength=8)
        if bi < 3:
            _covers_each_position_once(b)
    frac = counts / counts.sum()
    assert frac[0] > 0.35 and frac[7] < 0.06  # Zipf(1.2): hot ~0.43, coldest ~0.035
    assert abs(W.ZIPF_P[1.2][0] - 0.4287) < 1e-3


def test_c4_waves_partition_tokens():
    s = W.c4_prefill_setup(with_weights=False)
    assert W.C4["waves"] == (6554, 4915, 3277, 1638) and sum(W.C4["waves"]) == 16384
    allt = []
    for wv in range(4):
        b = W.c4_wave(s, wv, with_remote=(wv == 3))
        assert b.n == W.C4["waves"][wv]
        allt += b.tok.tolist()
        assert np.array_equal(b.tok, b.slot)
    assert sorted(allt) == list(range(16384))
    b = W.c4_wave(s, 3)
    assert b.remote.m == 7 * b.n
    frac = np.bincount(s.expert, minlength=32) / 16384
    assert 0.22 < frac[0] < 0.27


def test_fp8_weight_quantisation_round_trip():
    rng = np.random.default_rng(0)
    lw = W.make_layer_weights(rng, 2, 64, 32, 0.02, "fp8")
    codes = lw.wg[0].astype(np.int64)
    assert lw.sg.shape == (2, 32) and lw.sd.shape == (2, 64)
    assert np.all((codes & 0x7F) != 0x7F)  # never NaN
    assert np.any((codes & 0x7F) == 0x7E)  # each row's amax maps to 448


def test_merged_prefill_waves_keep_every_pair_and_remote_row():
    s = W.c4_prefill_setup(with_weights=False)
    a = [W.c4_wave(s, w) for w in (2, 3)]
    m = W.merge_batches(a)
    assert m.n == a[0].n + a[1].n and m.remote.m == a[0].remote.m + a[1].remote.m
    assert np.array_equal(m.tok, np.concatenate([a[0].tok, a[1].tok]))
    r0, r1, r = a[0].remote, a[1].remote, m.remote
    for k in (0, r0.m - 1, r0.m, r.m - 1):
        src, i = (r0, k) if k < r0.m else (r1, k - r0.m)
        assert np.array_equal(r.rows[r.row_idx[k]], src.rows[src.row_idx[i]])
        assert (r.tok[k], r.kslot[k], r.w[k]) == (src.tok[i], src.kslot[i], src.w[i])
    assert W.merge_batches([a[0]]) is a[0]
