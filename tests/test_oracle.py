"""Pins for the CPU oracle: each check ties it to something other than itself
(the pages' worked examples, closed forms, exact rational arithmetic, library routines
on special cases, brute force on tiny inputs), so that a dropped term, a wrong index or
sign, or a transposed operand anywhere in the oracle fails at least one of them."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O


# ------------------------------------------------------------------ storage decoding
def test_decode_bf16_all_codes_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_decode_e4m3_all_codes_match_torch_and_spec_values():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 for both signs
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    # OCP FP8 E4M3 table values: max normal, min normal, min subnormal, one
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0x38] == 1.0 and got[0xB8] == -1.0 and got[0x00] == 0.0


# ------------------------------------------------------------------------- assemble
def _brute_assemble(slot, expert, base, E_loc, P):
    """Filter-based grouping: for each expert, the valid pairs in queue order."""
    valid = [0 <= s < P and base <= e < base + E_loc for s, e in zip(slot, expert)]
    groups = [[i for i in range(len(slot)) if valid[i] and expert[i] - base == e] for e in range(E_loc)]
    perm = [i for g in groups for i in g]
    return [len(g) for g in groups], perm


@pytest.mark.parametrize("seed", range(12))
def test_assemble_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    E_loc, base, P = int(rng.integers(1, 7)), int(rng.integers(0, 20)), int(rng.integers(1, 40))
    n = int(rng.integers(0, 60))
    slot = rng.integers(-3, P + 3, size=n)
    expert = rng.integers(base - 2, base + E_loc + 2, size=n)
    a = O.assemble(slot, expert, base, E_loc, P)
    counts, perm = _brute_assemble(list(slot), list(expert), base, E_loc, P)
    assert list(a["counts"]) == counts
    assert list(a["offsets"]) == [0] + list(np.cumsum(counts))
    nv = len(perm)
    assert list(a["perm"][:nv]) == perm and all(a["perm"][nv:] == -1)
    for r, i in enumerate(perm):
        assert a["pos"][i] == r
    assert sum(a["pos"] >= 0) == nv
    exp_err = (O.ERR_SLOT_RANGE if any((slot < 0) | (slot >= P)) else 0) | \
              (O.ERR_EXPERT_NONLOCAL if any((expert < base) | (expert >= base + E_loc)) else 0)
    assert a["err"] == exp_err


def test_assemble_matches_numpy_stable_argsort():
    rng = np.random.default_rng(7)
    n, E_loc = 5000, 32
    expert = rng.integers(0, E_loc, size=n)
    slot = rng.integers(0, 100, size=n)
    a = O.assemble(slot, expert, 0, E_loc, 100)
    assert np.array_equal(a["perm"], np.argsort(expert, kind="stable"))
    assert np.array_equal(a["counts"], np.bincount(expert, minlength=E_loc))


def test_assemble_queue_permutation_keeps_per_expert_multisets():
    rng = np.random.default_rng(3)
    n, E_loc, P = 200, 8, 64
    slot = rng.integers(0, P, size=n)
    expert = rng.integers(0, E_loc, size=n)
    a = O.assemble(slot, expert, 0, E_loc, P)
    q = rng.permutation(n)
    b = O.assemble(slot[q], expert[q], 0, E_loc, P)
    assert np.array_equal(a["counts"], b["counts"]) and np.array_equal(a["offsets"], b["offsets"])
    for e in range(E_loc):
        lo, hi = a["offsets"][e], a["offsets"][e + 1]
        sa = sorted(slot[a["perm"][lo:hi]])
        sb = sorted(slot[q][b["perm"][lo:hi]])
        assert sa == sb


def test_gather_is_byte_exact_and_page_payload_size(golden):
    g = golden("streamep_payload_bytes.json")
    rng = np.random.default_rng(0)
    P, H = 512, g["hidden"]
    pool = rng.integers(0, 65536, size=(P, H)).astype(np.uint16)  # arbitrary bf16 bit patterns
    slot = rng.permutation(P)[: g["tokens"]]
    a = O.assemble(slot, np.zeros(g["tokens"], int), 0, 1, P)
    xb = O.gather_rows(pool, slot, a["perm"], int(a["offsets"][-1]))
    assert xb.nbytes == g["payload_bytes"] == g["tokens"] * g["hidden"] * g["bytes_per_element"]
    assert np.array_equal(xb, pool[slot])


def test_gather_follows_perm_for_a_scrambled_multi_expert_queue():
    """[SEP] section 3: the scattered token vectors of a queue become one contiguous batch,
    here grouped by expert.  With several experts in a shuffled queue the batch order is far
    from the queue order, so a gather that ignored perm (rows in queue order) fails."""
    rng = np.random.default_rng(11)
    P, H, E_loc, n = 96, 6, 5, 40
    pool = rng.integers(0, 65536, size=(P, H)).astype(np.uint16)
    slot = rng.permutation(P)[:n]
    expert = rng.integers(0, E_loc, size=n)
    a = O.assemble(slot, expert, 0, E_loc, P)
    _, perm = _brute_assemble(list(slot), list(expert), 0, E_loc, P)
    expected = np.stack([pool[slot[i]] for i in perm])  # expert ascending, queue order inside
    assert not np.array_equal(pool[slot], expected)
    assert np.array_equal(O.gather_rows(pool, slot, a["perm"], int(a["offsets"][-1])), expected)
    # the row index is slot[perm[r]] for any perm (here a reversal of the queue)
    rev = np.arange(n)[::-1]
    assert np.array_equal(O.gather_rows(pool, slot, rev, n), pool[slot[::-1]])


def test_request37_queue_assembles_in_queue_order(golden):
    g = golden("streamep_request37_queue.json")
    rng = np.random.default_rng(37)
    P, H = 64, 8
    pool = rng.standard_normal((P, H)).astype(np.float32)
    slots = np.array([41, 5, 17])  # scattered pool slots of requests 23, 33, 37
    a = O.assemble(slots, [g["expert"]] * 3, 0, 4, P)
    assert list(a["counts"]) == [0, 3, 0, 0]
    xb = O.gather_rows(pool, slots, a["perm"], 3)
    assert np.array_equal(xb, pool[slots])  # one contiguous batch, queue order kept


# ----------------------------------------------------------------------- expert FFN
def test_silu_matches_library_logistic():
    z = np.linspace(-40, 40, 2001)
    assert np.allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-15, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


def test_swiglu_hand_derived_closed_form(golden):
    g = golden("swiglu_handcalc.json")
    ln3 = math.log(3.0)
    x = np.array([g["x"]])
    y = O.swiglu(x, np.array(g["wg_over_ln3"]) * ln3, np.array(g["wu"]), np.array(g["wd"]))
    assert np.allclose(y[0], np.array(g["y_over_ln3"]) * ln3, rtol=1e-14, atol=0)


def test_swiglu_special_cases():
    rng = np.random.default_rng(1)
    H, I, m = 16, 24, 5
    x = rng.standard_normal((m, H))
    wg, wu, wd = rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))
    assert np.all(O.swiglu(np.zeros((m, H)), wg, wu, wd) == 0.0)
    assert np.all(O.swiglu(x, wg, np.zeros((I, H)), wd) == 0.0)
    assert np.all(O.swiglu(x, np.zeros((I, H)), wu, wd) == 0.0)  # silu(0) = 0
    # homogeneity in Wu and Wd (exact for powers of two)
    y = O.swiglu(x, wg, wu, wd)
    assert np.array_equal(O.swiglu(x, wg, 2 * wu, wd), 2 * y)
    assert np.array_equal(O.swiglu(x, wg, wu, 0.5 * wd), 0.5 * y)
    # with a huge positive gate, silu(g) = g to double precision: a bilinear form
    big = np.abs(wg) * 0 + 1.0
    xp = np.abs(x) + 1.0
    y2 = O.swiglu(xp, 1e3 * big, wu, wd)
    bil = np.einsum("oi,mi,mi->mo", wd, xp @ (1e3 * big).T, xp @ wu.T)
    assert np.allclose(y2, bil, rtol=1e-12)


def test_swiglu_rows_independent():
    rng = np.random.default_rng(2)
    H, I, m = 8, 12, 9
    x = rng.standard_normal((m, H))
    W = (rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I)))
    y = O.swiglu(x, *W)
    q = rng.permutation(m)
    assert np.allclose(O.swiglu(x[q], *W), y[q], rtol=1e-14, atol=1e-14)
    for r in range(m):
        assert np.allclose(O.swiglu(x[r:r + 1], *W)[0], y[r], rtol=1e-14, atol=1e-14)


class _W:  # minimal stand-in for workloads.LayerWeights
    def __init__(self, dtype, wg, wu, wd, sg=None, su=None, sd=None):
        self.dtype, self.wg, self.wu, self.wd, self.sg, self.su, self.sd = dtype, wg, wu, wd, sg, su, sd


def test_expert_ffn_dispatches_rows_to_their_experts():
    rng = np.random.default_rng(4)
    E, H, I = 3, 8, 16
    wts = _W("f32", rng.standard_normal((E, I, H)).astype(np.float32),
             rng.standard_normal((E, I, H)).astype(np.float32), rng.standard_normal((E, H, I)).astype(np.float32))
    offsets = [0, 2, 2, 7]  # expert 1 empty
    xb = rng.standard_normal((7, H))
    y = O.expert_ffn(xb, offsets, wts)
    for r, e in enumerate([0, 0, 2, 2, 2, 2, 2]):
        W = [np.asarray(a[e], np.float64) for a in (wts.wg, wts.wu, wts.wd)]
        assert np.allclose(y[r], O.swiglu(xb[r:r + 1], *W)[0], rtol=1e-14)
    assert np.allclose(O.ffn_rows(xb, [0, 0, 2, 2, 2, 2, 2], wts), y, rtol=1e-14)


def test_fp8_weights_are_code_times_row_scale():
    # expert 1: rows (-1, 448) and (1, 2) with row scales 0.25 and 4 (exact in binary)
    codes = np.array([[[0x38, 0x40], [0x38, 0x38]], [[0xB8, 0x7E], [0x38, 0x40]]], np.uint8)
    sc = np.array([[0.5, 1.0], [0.25, 4.0]], np.float32)
    wts = _W("fp8", codes, codes, codes, sc, 2 * sc, 4 * sc)
    wg, wu, wd = O.expert_weights(wts, 1)
    assert np.array_equal(wg, np.array([[-0.25, 112.0], [4.0, 8.0]]))
    assert np.array_equal(wu, 2 * wg) and np.array_equal(wd, 4 * wg)


# ------------------------------------------------------------------ combine/release
def _one_call(K, T, arrivals, H=4, rows=None, state=None):
    st = state or O.CombineState(T, K)
    rows = rows if rows is not None else np.eye(len(arrivals), H)
    ri = [a[0] for a in arrivals]
    out, rel, err = O.combine_release(st, rows, ri, [a[1] for a in arrivals], [a[2] for a in arrivals],
                                      [a[3] for a in arrivals], [a[4] for a in arrivals])
    return st, out, rel, err


def test_page_example_fourth_result_releases(golden):
    g = golden("streamep_topk_release.json")
    K = g["K"]
    st = O.CombineState(1, K)
    rows = np.arange(K * 3, dtype=np.float64).reshape(K, 3)
    seen = []
    for j in range(K):
        out, rel, err = O.combine_release(st, rows, [j], [0], [j], [0.25], [0])
        assert err == 0
        seen.append(len(rel) == 1)
    assert seen == g["released_after_arrival"]
    assert st.mask[0] == 0 and st.tgen[0] == 1


def test_page_example_combine_cardinality(golden):
    g = golden("streamep_combine_cardinality.json")
    T, K, H = g["tokens"], g["K"], 16  # hidden shrunk; only the counts are pinned here
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((T * K, H))
    st = O.CombineState(T, K)
    tok = np.repeat(np.arange(T), K)
    ks = np.tile(np.arange(K), T)
    out, rel, err = O.combine_release(st, rows, np.arange(T * K), tok, ks, np.full(T * K, 0.25), np.zeros(T * K))
    assert len(tok) == g["expert_results"] and len(out) == len(rel) == g["combined_vectors"]
    assert list(rel) == list(range(T))


def test_one_hot_weights_reproduce_single_expert():
    rng = np.random.default_rng(6)
    K, H = 4, 32
    rows = rng.standard_normal((K, H))
    for jhot in range(K):
        st = O.CombineState(1, K)
        w = [1.0 if j == jhot else 0.0 for j in range(K)]
        out, rel, _ = O.combine_release(st, rows, range(K), [0] * K, range(K), w, [0] * K)
        assert np.array_equal(out[0], rows[jhot])


def test_identical_experts_with_unit_weight_sum_reproduce_expert():
    rng = np.random.default_rng(7)
    H, I, K = 8, 12, 4
    x = rng.standard_normal((1, H))
    W = (rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I)))
    ex = O.swiglu(x, *W)[0]
    w = np.float32(rng.dirichlet(np.ones(K)))
    st = O.CombineState(1, K)
    out, rel, _ = O.combine_release(st, np.tile(ex, (K, 1)), range(K), [0] * K, range(K), w, [0] * K)
    assert np.allclose(out[0], ex * float(np.sum(w.astype(np.float64))), rtol=1e-14)
    assert abs(float(np.sum(w.astype(np.float64))) - 1.0) < 1e-6


def test_integer_toy_combine_is_exact_rational_sum():
    rng = np.random.default_rng(8)
    T, K, H = 6, 4, 5
    rows = rng.integers(-50, 50, size=(T * K, H)).astype(np.float64)
    w = [2.0 ** -int(e) for e in rng.integers(0, 6, size=T * K)]
    tok = np.repeat(np.arange(T), K)
    ks = np.tile(np.arange(K), T)
    st = O.CombineState(T, K)
    out, rel, err = O.combine_release(st, rows, range(T * K), tok, ks, w, [0] * (T * K))
    for t in range(T):
        exp = [sum(Fraction(w[i]) * Fraction(int(rows[i, h])) for i in range(T * K) if tok[i] == t)
               for h in range(H)]
        assert [Fraction(v) for v in out[t]] == exp


def test_arrival_order_permutation_keeps_results():
    rng = np.random.default_rng(9)
    T, K, H = 10, 3, 6
    n = T * K - 4  # some tokens stay incomplete
    arr = [(i, t, j, float(rng.random()), 0) for i, (t, j) in enumerate(itertools.product(range(T), range(K)))][:n]
    rows = rng.integers(-9, 9, size=(T * K, H)).astype(np.float64)
    s1, o1, r1, _ = _one_call(K, T, arr, rows=rows)
    q = rng.permutation(n)
    s2, o2, r2, _ = _one_call(K, T, [arr[i] for i in q], rows=rows)
    assert list(r1) == list(r2) and np.array_equal(s1.mask, s2.mask)
    for t in o1:
        assert np.array_equal(o1[t], o2[t])


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_release_exactly_once_at_last_arrival_over_all_splits_and_orders(K):
    rows = np.eye(K, 2 * K)
    for order in itertools.permutations(range(K)):
        for cuts in itertools.product([0, 1], repeat=K - 1):  # cut after position p?
            calls, cur = [], [order[0]]
            for p in range(1, K):
                if cuts[p - 1]:
                    calls.append(cur)
                    cur = []
                cur.append(order[p])
            calls.append(cur)
            st = O.CombineState(1, K)
            released = 0
            for c, js in enumerate(calls):
                out, rel, err = O.combine_release(st, rows, list(js), [0] * len(js), list(js), [1.0] * len(js), [0] * len(js))
                assert err == 0
                last = c == len(calls) - 1
                assert (len(rel) == 1) == last
                assert bin(int(st.mask[0])).count("1") == (0 if last else sum(len(x) for x in calls[: c + 1]))
                released += len(rel)
            assert released == 1
            assert np.array_equal(out[0], rows.sum(axis=0))


def test_duplicates_and_stale_generations_are_rejected():
    K, T, H = 2, 3, 4
    rows = np.arange(5 * H, dtype=np.float64).reshape(5, H)
    st = O.CombineState(T, K)
    # token 0 position 0 twice in one call: the first is accepted, the retry is not
    out, rel, err = O.combine_release(st, rows, [0, 1], [0, 0], [0, 0], [1.0, 1.0], [0, 0])
    assert err == O.ERR_DUPLICATE and len(rel) == 0 and st.mask[0] == 1
    # a retry in a later call is rejected too; the missing position completes the token
    out, rel, err = O.combine_release(st, rows, [2, 3], [0, 0], [0, 1], [1.0, 1.0], [0, 0])
    assert err == O.ERR_DUPLICATE and list(rel) == [0]
    assert np.array_equal(out[0], rows[0] + rows[3])
    # a late result from the released generation is stale
    out, rel, err = O.combine_release(st, rows, [4], [0], [0], [1.0], [0])
    assert err == O.ERR_STALE_GEN and st.mask[0] == 0 and st.tgen[0] == 1
    # range checks
    _, _, err = O.combine_release(st, rows, [9, 0, 0], [0, 5, 0], [0, 0, 7], [1.0] * 3, [1, 0, 0])
    assert err == O.ERR_ROW_RANGE | O.ERR_TOKEN_RANGE | O.ERR_KSLOT_RANGE
    assert st.mask[0] == 0


def test_weights_not_renormalised_over_arrived_results():
    # the token is released only with all K results; each keeps its own router weight
    K = 3
    rows = np.ones((K, 2))
    st = O.CombineState(1, K)
    O.combine_release(st, rows, [0, 1], [0, 0], [0, 1], [0.5, 0.25], [0, 0])
    out, rel, _ = O.combine_release(st, rows, [2], [0], [2], [0.125], [0])
    assert np.array_equal(out[0], np.full(2, 0.875))


def test_combine_token_matches_release_path():
    rng = np.random.default_rng(10)
    K, H = 4, 7
    rows = rng.standard_normal((K, H))
    w = rng.random(K).astype(np.float32)
    st = O.CombineState(1, K)
    out, _, _ = O.combine_release(st, rows, range(K), [0] * K, range(K), w, [0] * K)
    assert np.array_equal(out[0], O.combine_token([(w[j], rows[j]) for j in range(K)]))
