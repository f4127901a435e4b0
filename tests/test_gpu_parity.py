"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element
on the same seeded inputs.  Integer outputs bit-exact; rows within the per-dtype tolerance
(max over rows of ||gpu - ref||_inf / ||ref||_inf: 1e-5 fp32, 2e-2 bf16, 6e-2 fp8)."""
import numpy as np
import pytest
import torch

import asynchronous_moe_expert_amd as M
import oracle as O
import workloads as W
from gpu_helpers import TOL, HipEvents, decode_tensor, dev, elem_rel_err, row_rel_err, sync_err
from workloads.device import batch_tensors, to_numpy_bits, weight_tensors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()


def _say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------- assemble
ASM_CASES = [
    # (n, E_loc, base, P, H, act, pitch_extra, bad_frac)
    (0, 4, 0, 16, 64, "bf16", 0, 0.0),
    (1, 1, 3, 8, 64, "f32", 0, 0.0),
    (7, 5, 10, 40, 8, "f32", 4, 0.3),
    (1023, 8, 0, 2048, 192, "bf16", 8, 0.0),
    (1024, 8, 16, 1024, 64, "bf16", 0, 0.05),
    (1025, 3, 0, 300, 64, "bf16", 0, 0.1),
    (3000, 256, 0, 5000, 64, "bf16", 0, 0.02),
    (5000, 32, 64, 9000, 2880, "bf16", 0, 0.0),
    (9000, 16, 0, 12000, 64, "bf16", 0, 0.05),   # past the 8 chunks whose keys stay in registers
]


@pytest.mark.parametrize("case", ASM_CASES, ids=[f"n{c[0]}_E{c[1]}_H{c[4]}" for c in ASM_CASES])
def test_assemble_matches_oracle(case):
    n, E, base, P, H, act, extra, bad = case
    _say("assemble case", case)
    rng = np.random.default_rng(n * 7 + E)
    slot = rng.integers(0, P, size=n).astype(np.int32)
    expert = (base + rng.integers(0, E, size=n)).astype(np.int32)
    nb = int(bad * n)
    if nb:
        idx = rng.choice(n, size=nb, replace=False)
        slot[idx[: nb // 2]] = rng.choice([-1, P, P + 5], size=nb // 2)
        expert[idx[nb // 2:]] = rng.choice([base - 1, base + E, -7], size=nb - nb // 2)
    raw = rng.standard_normal((P, H + extra)).astype(np.float32)
    pool_np = W.to_bf16_bits(raw) if act == "bf16" else raw
    pool_full = dev(pool_np, act)
    pool = pool_full[:, :H]
    st_xb = torch.empty((max(n, 1), H), dtype=pool.dtype, device="cuda")
    perm = torch.full((max(n, 1),), -9, dtype=torch.int32, device="cuda")
    pos = torch.full((max(n, 1),), -9, dtype=torch.int32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    row_slot = torch.full((max(n, 1),), -9, dtype=torch.int32, device="cuda")
    M.moe_assemble(dev(slot), dev(expert), base, E, pool, perm, pos, counts, offsets, st_xb, err, n=n,
                   row_slot=row_slot)
    e = sync_err(err)
    a = O.assemble(slot, expert, base, E, P)
    assert e == a["err"]
    assert np.array_equal(counts.cpu().numpy(), a["counts"])
    assert np.array_equal(offsets.cpu().numpy(), a["offsets"])
    if n:
        assert np.array_equal(perm.cpu().numpy()[:n], a["perm"])
        assert np.array_equal(pos.cpu().numpy()[:n], a["pos"])
        nv = int(a["offsets"][-1])
        # row_slot: the pool slot of each batch row, -1 past the accepted pairs
        rs = row_slot.cpu().numpy()[:n]
        assert np.array_equal(rs[:nv], slot[a["perm"][:nv]]) and np.all(rs[nv:] == -1)
        ref = O.gather_rows(pool_np[:, :H], slot, a["perm"], nv)
        got = to_numpy_bits(st_xb[:nv])
        assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8))


# ------------------------------------------------------------------------------- FFN
FFN_CASES = [
    # (act/weight dtype, E, H, I, counts)
    ("f32", 3, 64, 128, [5, 0, 17]),
    ("bf16", 4, 128, 192, [1, 64, 0, 130]),
    ("bf16", 2, 2880, 2880, [37, 70]),
    ("bf16", 5, 256, 128, [0, 0, 200, 1, 16]),
    ("fp8", 3, 256, 128, [65, 3, 0]),
    ("fp8", 2, 4096, 2048, [129, 40]),
    # >= 96 rows per expert on average: the 128-row tiled kernel, with partial row chunks,
    # an empty expert, partial 256-column blocks and contractions of 3, 10 and 45 k-steps
    ("bf16", 4, 512, 256, [300, 0, 5, 130]),
    ("fp8", 3, 640, 192, [257, 1, 130]),
    ("bf16", 2, 2880, 2880, [200, 190]),
    ("fp8", 2, 4096, 2048, [300, 60]),
    # last chunks of 70, 96 and 97 rows: 3, 3 and 4 executed 32-row tiles (the fp8 kernel skips the rest)
    ("fp8", 3, 512, 256, [198, 96, 353]),
]


@pytest.mark.parametrize("case", FFN_CASES, ids=[f"{c[0]}_E{c[1]}_H{c[2]}_I{c[3]}" for c in FFN_CASES])
def test_ffn_matches_oracle(case):
    wdt, E, H, I, counts = case
    _say("ffn case", case)
    rng = np.random.default_rng(E * 1000 + H + I)
    act = "f32" if wdt == "f32" else "bf16"
    wts = W.make_layer_weights(rng, E, H, I, 0.05, wdt)
    n = int(sum(counts))
    x_raw = rng.standard_normal((n, H)).astype(np.float32)
    x_np = x_raw if act == "f32" else W.to_bf16_bits(x_raw)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    codes = {"f32": M.MOE_F32, "bf16": M.MOE_BF16, "fp8": M.MOE_FP8_E4M3}
    st = M.ExpertStep(E, H, I, 2, codes[act], codes[wdt], n, 4)
    wt = weight_tensors(wts)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt.get("s_gate"), wt.get("s_up"), wt.get("s_down"))
    st.xb[:n].copy_(dev(x_np, act))
    st.offsets.copy_(dev(offsets))
    st.ffn(n)
    torch.cuda.synchronize()
    y_ref = O.expert_ffn(O.decode(x_np, act), offsets, wts)
    err = row_rel_err(decode_tensor(st.y[:n]), y_ref)
    _say(f"  row rel err {err:.3e}")
    assert err <= TOL[wdt]


MANY_EXPERT_CASES = [
    # (weight dtype, E_loc, H, I, mean rows per expert): expert tables of 2-4 groups of 64 on
    # every FFN path: both weight-streaming kernels (bf16), streaming gate/up with the fp8 down
    # on the 256-row GEMM, the 256-row fp8 GEMM, the 128-row bf16 GEMM
    ("bf16", 200, 128, 64, 20),
    ("fp8", 256, 128, 64, 60),
    ("fp8", 130, 256, 128, 110),
    ("bf16", 256, 128, 128, 100),
]


@pytest.mark.parametrize("case", MANY_EXPERT_CASES, ids=[f"{c[0]}_E{c[1]}_m{c[4]}" for c in MANY_EXPERT_CASES])
def test_ffn_many_local_experts(case):
    """Up to 256 local experts, Zipf-skewed row counts with about a tenth of the experts empty:
    every row against the oracle."""
    wdt, E, H, I, mean = case
    _say("ffn many experts", case)
    rng = np.random.default_rng(E * 7 + H + mean)
    wts = W.make_layer_weights(rng, E, H, I, 0.05, wdt)
    p = 1.0 / np.arange(1, E + 1) ** 0.8
    p[rng.choice(E, E // 10, replace=False)] = 0.0
    p = rng.permutation(p / p.sum())
    n = mean * E
    counts = rng.multinomial(n, p)
    assert (counts == 0).sum() >= E // 10 and counts.max() > 2 * mean
    x_np = W.to_bf16_bits(rng.standard_normal((n, H)).astype(np.float32))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    codes = {"bf16": M.MOE_BF16, "fp8": M.MOE_FP8_E4M3}
    st = M.ExpertStep(E, H, I, 2, M.MOE_BF16, codes[wdt], n, 4)
    wt = weight_tensors(wts)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt.get("s_gate"), wt.get("s_up"), wt.get("s_down"))
    st.xb[:n].copy_(dev(x_np, "bf16"))
    st.offsets.copy_(dev(offsets))
    st.ffn(n)
    torch.cuda.synchronize()
    y_ref = O.expert_ffn(O.decode(x_np, "bf16"), offsets, wts)
    y_gpu = decode_tensor(st.y[:n])
    err, ee = row_rel_err(y_gpu, y_ref), elem_rel_err(y_gpu, y_ref)
    _say(f"  {n} rows: row rel err {err:.3e} (elementwise {ee:.3e})")
    assert err <= TOL[wdt]


def test_ffn_empty_batch_is_a_no_op():
    st = M.ExpertStep(2, 64, 64, 2, M.MOE_BF16, M.MOE_BF16, 4, 4)
    z = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device="cuda")
    st.load_weights(z, z, z)
    st.y.fill_(3.0)
    st.offsets.zero_()
    st.ffn(0)
    torch.cuda.synchronize()
    assert torch.all(st.y == 3.0)


@pytest.mark.parametrize("fuse_plan", [True, False])
def test_empty_step_releases_nothing(fuse_plan):
    """A whole step on an empty queue (n = 0): the FFN call still enqueues the (empty)
    combine plan; nothing is accepted or released and the token state is unchanged."""
    st = M.ExpertStep(2, 64, 64, 2, M.MOE_BF16, M.MOE_BF16, 4, 8, fuse_plan=fuse_plan)
    z = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device="cuda")
    st.load_weights(z, z, z)
    M.moe_state_reset(st.state, 5)
    st.err.zero_()
    st.rel_count.fill_(-1)
    mask0, tgen0 = st.state.mask.clone(), st.state.tgen.clone()
    pool = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    i32 = lambda: torch.zeros(0, dtype=torch.int32, device="cuda")  # noqa: E731
    st.run(i32(), i32(), 0, pool, i32(), i32(), torch.zeros(0, dtype=torch.float32, device="cuda"), i32())
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0 and int(st.rel_count.item()) == 0
    assert torch.equal(st.state.mask, mask0) and torch.equal(st.state.tgen, tgen0)


# --------------------------------------------------------------------------- combine
def _combine_call(st, rows_t, rows64, arr, ocs, K):
    """Run one combine call on GPU and oracle; compare err, rel list and state."""
    row_idx, tok, ks, w, gen = (np.array(c) for c in zip(*arr)) if arr else [np.zeros(0, np.int32)] * 5
    m = len(arr)
    st.err.zero_()
    d = [dev(np.asarray(v, dt)) for v, dt in ((row_idx, np.int32), (tok, np.int32), (ks, np.int32),
                                               (w, np.float32), (gen, np.uint32))]
    st.combine(rows_t, *d, m=m, n_rows=rows_t.shape[0])
    e = sync_err(st.err)
    out, rel, oerr = O.combine_release(ocs, rows64, row_idx, tok, ks, np.asarray(w, np.float32), gen)
    n_rel = int(st.rel_count.item())
    assert e == oerr, (e, oerr)
    assert np.array_equal(st.rel_list[:n_rel].cpu().numpy(), rel)
    assert np.array_equal(st.state.mask.cpu().numpy().view(np.uint32), ocs.mask)
    assert np.array_equal(st.state.tgen.cpu().numpy().view(np.uint32), ocs.tgen)
    assert np.all(st.state.head.cpu().numpy() == -1)  # per-call lists are torn down
    assert np.all(st.state.rflag.cpu().numpy() == 0)
    return out, rel


@pytest.mark.parametrize("rdt", ["f32", "bf16"])
def test_combine_integer_toy_is_bit_exact_over_split_calls(rdt):
    _say("combine integer toy", rdt)
    rng = np.random.default_rng(11)
    T, K, H = 200, 4, 64
    # small integers and power-of-two weights: every partial sum is exact in fp32 and bf16
    rows_np = rng.integers(-8, 8, size=(T * K + 10, H)).astype(np.float32)
    rows64 = rows_np.astype(np.float64)
    rows_t = dev(W.to_bf16_bits(rows_np), "bf16") if rdt == "bf16" else dev(rows_np)
    arrivals = [(t * K + j, t, j, 2.0 ** -int(rng.integers(0, 3)), 0) for t in range(T) for j in range(K)]
    order = rng.permutation(len(arrivals))
    arrivals = [arrivals[i] for i in order]
    st = M.ExpertStep(1, H, 64, K, M.MOE_BF16 if rdt == "bf16" else M.MOE_F32, M.MOE_BF16, 1, T)
    ocs = O.CombineState(T, K)
    cuts = [0, 250, 251, 520, len(arrivals)]
    released = []
    for c in range(4):
        chunk = arrivals[cuts[c]:cuts[c + 1]]
        if c == 1:  # a retry of an earlier result and a stale result ride along
            chunk = chunk + [arrivals[3], (T * K + 1, arrivals[5][1], arrivals[5][2], 1.0, 7)]
        out, rel = _combine_call(st, rows_t, rows64, chunk, ocs, K)
        g = st.out.cpu()
        g = O.decode_bf16(to_numpy_bits(g)) if rdt == "bf16" else g.numpy().astype(np.float64)
        for t in rel:
            assert np.array_equal(g[t], out[t])  # exact
        released += list(rel)
    assert sorted(released) == list(range(T))


def test_combine_errors_duplicates_and_generations():
    _say("combine errors")
    K, T, H = 2, 6, 64
    rows_np = np.arange(10 * H, dtype=np.float32).reshape(10, H) / 64
    rows_t, rows64 = dev(rows_np), rows_np.astype(np.float64)
    st = M.ExpertStep(1, H, 64, K, M.MOE_F32, M.MOE_F32, 1, T)
    ocs = O.CombineState(T, K)
    # in-call duplicate with different rows: the lower arrival index wins, as in the oracle
    _combine_call(st, rows_t, rows64, [(0, 0, 0, 1.0, 0), (1, 0, 0, 1.0, 0)], ocs, K)
    out, rel = _combine_call(st, rows_t, rows64, [(2, 0, 1, 1.0, 0)], ocs, K)  # releases token 0
    assert list(rel) == [0]
    assert np.array_equal(st.out.cpu().numpy()[0].astype(np.float64), out[0])
    _combine_call(st, rows_t, rows64, [(3, 0, 0, 1.0, 0)], ocs, K)  # stale generation
    _combine_call(st, rows_t, rows64, [(3, 9, 0, 1.0, 0), (3, 1, 5, 1.0, 0), (99, 1, 0, 1.0, 0), (-1, 2, 1, 1, 0)],
                  ocs, K)
    _combine_call(st, rows_t, rows64, [], ocs, K)  # empty call
    out, rel = _combine_call(st, rows_t, rows64, [(4, 5, 0, 0.5, 0), (4, 5, 0, 0.5, 0), (5, 5, 1, 0.25, 0)], ocs, K)
    assert list(rel) == [5]
    g = st.out.cpu().numpy().astype(np.float64)
    assert np.array_equal(g[5], out[5])  # identical duplicate rows: result independent of the winner


def test_combine_long_chain_for_one_token():
    """More arrivals for one token in one call than the merge takes per pass (64): retries
    of position 0 interleaved with the other positions, the last position at the end."""
    _say("combine long chain")
    K, T, H = 4, 3, 64
    rng = np.random.default_rng(5)
    rows_np = rng.integers(-4, 4, size=(200, H)).astype(np.float32)
    rows_t, rows64 = dev(rows_np), rows_np.astype(np.float64)
    st = M.ExpertStep(1, H, 64, K, M.MOE_F32, M.MOE_F32, 1, T)
    ocs = O.CombineState(T, K)
    arr = [(q, 1, 0, 0.5, 0) for q in range(130)]                 # 130 claims of position 0
    arr[40] = (40, 1, 1, 0.25, 0)
    arr[100] = (100, 1, 2, 2.0, 0)
    arr += [(150, 2, 0, 1.0, 0), (151, 1, 3, 1.0, 0)]             # token 2 stays partial
    out, rel = _combine_call(st, rows_t, rows64, arr, ocs, K)
    assert list(rel) == [1]
    assert np.array_equal(st.out.cpu().numpy()[1].astype(np.float64), out[1])


@pytest.mark.parametrize("K", [1, 3, 32])
def test_combine_k_extremes(K):
    _say("combine K", K)
    rng = np.random.default_rng(K)
    T, H = 40, 128
    rows_np = rng.standard_normal((T * K, H)).astype(np.float32)
    rows_t, rows64 = dev(rows_np), rows_np.astype(np.float64)
    st = M.ExpertStep(1, H, 64, K, M.MOE_F32, M.MOE_F32, 1, T)
    ocs = O.CombineState(T, K)
    arr = [(t * K + j, t, j, float(rng.random()), 0) for t in range(T) for j in range(K)]
    arr = [arr[i] for i in rng.permutation(len(arr))]
    h = len(arr) // 2
    _combine_call(st, rows_t, rows64, arr[:h], ocs, K)
    out, rel = _combine_call(st, rows_t, rows64, arr[h:], ocs, K)
    g = st.out.cpu().numpy().astype(np.float64)
    all_out = {**out}
    assert row_rel_err(g[list(all_out)], np.array([all_out[t] for t in all_out])) <= 1e-6


# --------------------------------------------------------------------- whole configs
def _run_config_step(b, wts, act_code, w_code, check_rows=True, sample_rows=None, T_cap=None, overlap=False):
    """Deliver the remote results (one call), then run the step on the local pairs.
    Returns the GPU step and the oracle pieces for comparison."""
    d = batch_tensors(b)
    wt = weight_tensors(wts)
    st = M.ExpertStep(b.E_loc, b.H, wts.I, b.K, act_code, w_code, b.n, T_cap or b.T, overlap=overlap)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt.get("s_gate"), wt.get("s_up"), wt.get("s_down"))
    if "r_rows" in d:
        st.combine(d["r_rows"], d["r_idx"], d["r_tok"], d["r_kslot"], d["r_w"], d["r_gen"])
        torch.cuda.synchronize()
        assert int(st.rel_count.item()) == 0
    st.run(d["slot"], d["expert"], b.expert_base, d["pool"], d["tok"], d["kslot"], d["w"], d["gen"])
    e = sync_err(st.err)
    return st, e


def test_c0_tiny_full_step():
    b, wts = W.c0_tiny()
    _say("C0 tiny fp32 step")
    st, e = _run_config_step(b, wts, M.MOE_F32, M.MOE_F32)
    a = O.assemble(b.slot, b.expert, b.expert_base, b.E_loc, b.P)
    assert e == 0 == a["err"]
    assert np.array_equal(st.perm.cpu().numpy(), a["perm"])
    y = O.expert_ffn(O.decode(O.gather_rows(b.pool, b.slot, a["perm"], b.n), "f32"), a["offsets"], wts)
    assert row_rel_err(st.y.cpu().numpy(), y) <= TOL["f32"]
    ocs = O.CombineState(b.T, b.K)
    out, rel, oerr = O.combine_release(ocs, y, a["pos"], b.tok, b.kslot, b.w, b.gen)
    n_rel = int(st.rel_count.item())
    assert np.array_equal(st.rel_list[:n_rel].cpu().numpy(), rel) and n_rel == b.T == 32
    g = st.out.cpu().numpy()
    assert row_rel_err(g[rel], np.array([out[t] for t in rel])) <= TOL["f32"]


def _oracle_step(b, wts, y_rows=None):
    a = O.assemble(b.slot, b.expert, b.expert_base, b.E_loc, b.P)
    xb = O.decode(O.gather_rows(b.pool, b.slot, a["perm"], b.n), b.act)
    y = O.expert_ffn(xb, a["offsets"], wts) if y_rows is None else y_rows
    return a, y


def _check_step(st, e, b, wts, a, y, tol):
    assert e == a["err"] == 0
    assert np.array_equal(st.perm.cpu().numpy()[: b.n], a["perm"])
    assert np.array_equal(st.pos.cpu().numpy()[: b.n], a["pos"])
    assert np.array_equal(st.offsets.cpu().numpy(), a["offsets"])
    assert np.array_equal(st.counts.cpu().numpy(), a["counts"])
    ey = row_rel_err(decode_tensor(st.y[: b.n]), y)
    ocs = O.CombineState(b.T, b.K)
    r = b.remote
    O.combine_release(ocs, O.decode(r.rows, r.dtype), r.row_idx, r.tok, r.kslot, r.w, r.gen)
    out, rel, oerr = O.combine_release(ocs, y, a["pos"], b.tok, b.kslot, b.w, b.gen)
    n_rel = int(st.rel_count.item())
    assert oerr == 0 and np.array_equal(st.rel_list[:n_rel].cpu().numpy(), rel) and n_rel == b.T
    g = decode_tensor(st.out[torch.as_tensor(rel, device="cuda").long()])
    eo = row_rel_err(g, np.array([out[t] for t in rel]))
    _say(f"  Y row err {ey:.3e}, combined row err {eo:.3e}, released {n_rel}")
    assert ey <= tol and eo <= tol


def test_c1_decode_full_step():
    _say("C1 decode bf16 step")
    b, wts = W.c1_decode()
    st, e = _run_config_step(b, wts, M.MOE_BF16, M.MOE_BF16)
    a, y = _oracle_step(b, wts)
    _check_step(st, e, b, wts, a, y, TOL["bf16"])


def test_c1_decode_overlapped_step():
    """The same step with the combine's plan half on a side stream during the FFN."""
    _say("C1 decode bf16 step, plan overlapped with the FFN")
    b, wts = W.c1_decode()
    st, e = _run_config_step(b, wts, M.MOE_BF16, M.MOE_BF16, overlap=True)
    a, y = _oracle_step(b, wts)
    _check_step(st, e, b, wts, a, y, TOL["bf16"])


def test_gate_up_dispatch_events():
    """The gate/up kernel's own start/stop events (moe_ffn_args.ev_gu_start / ev_gu_stop):
    the FFN gives the same bits with and without them, and the duration they record is
    positive and inside the interval of events recorded around the whole call."""
    _say("C1 decode FFN with the gate/up dispatch events")
    b, wts = W.c1_decode()
    d = batch_tensors(b)
    wt = weight_tensors(wts)
    st = M.ExpertStep(b.E_loc, b.H, wts.I, b.K, M.MOE_BF16, M.MOE_BF16, b.n, b.T)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"])
    st.assemble(d["slot"], d["expert"], b.expert_base, d["pool"])
    st.ffn(b.n)
    torch.cuda.synchronize()
    y0 = to_numpy_bits(st.y[: b.n])
    hip = HipEvents()
    ev = [hip.create() for _ in range(4)]
    stream = torch.cuda.current_stream().cuda_stream
    hip.record(ev[0], stream)
    st.ffn(b.n, ev_gu=(ev[1], ev[2]))
    hip.record(ev[3], stream)
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_bits(st.y[: b.n]), y0)
    kernel, whole = hip.ms(ev[1], ev[2]), hip.ms(ev[0], ev[3])
    _say(f"  gate/up kernel {kernel * 1e3:.1f} us of {whole * 1e3:.1f} us")
    assert 0.0 < kernel < whole
    for e in ev:
        hip.destroy(e)


def test_c1_decode_other_rank():
    _say("C1 decode bf16 step, rank 5")
    b, wts = W.c1_decode(rank=5)
    st, e = _run_config_step(b, wts, M.MOE_BF16, M.MOE_BF16)
    a, y = _oracle_step(b, wts)
    _check_step(st, e, b, wts, a, y, TOL["bf16"])


def test_c2_skewed_batches():
    """All 200 batches: integer parts bit-exact; rows checked on every 20th batch and on
    the smallest and largest batch."""
    _say("C2 skewed ragged, 200 batches")
    wts = W.c2_weights()
    pool = W.c2_pool()
    wt = weight_tensors(wts)
    st = M.ExpertStep(8, 2880, 2880, 4, M.MOE_BF16, M.MOE_BF16, 512, 512)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"])
    pool_t = dev(pool, "bf16")
    batches = [W.c2_skewed_batch(i, pool) for i in range(200)]
    ns = [bb.n for bb in batches]
    float_check = set(range(0, 200, 20)) | {int(np.argmin(ns)), int(np.argmax(ns))}
    for i, b in enumerate(batches):
        d = batch_tensors(b)
        d["pool"] = pool_t
        M.moe_state_reset(st.state, 0)
        st.err.zero_()
        st.combine(d["r_rows"], d["r_idx"], d["r_tok"], d["r_kslot"], d["r_w"], d["r_gen"])
        st.run(d["slot"], d["expert"], 0, d["pool"], d["tok"], d["kslot"], d["w"], d["gen"])
        e = sync_err(st.err)
        a = O.assemble(b.slot, b.expert, 0, 8, b.P)
        assert e == 0
        assert np.array_equal(st.perm.cpu().numpy()[: b.n], a["perm"]), i
        assert np.array_equal(st.offsets.cpu().numpy(), a["offsets"]), i
        n_rel = int(st.rel_count.item())
        assert np.array_equal(st.rel_list[:n_rel].cpu().numpy(), np.arange(b.n)), i
        if i in float_check:
            _say(f" batch {i} n={b.n}")
            a, y = _oracle_step(b, wts)
            _check_step(st, e, b, wts, a, y, TOL["bf16"])


def test_fused_plan_matches_separate_plan():
    """The combine plan run by moe_expert_ffn_grouped (in a spare workgroup of the gate/up
    launch for up to 256 arrivals, else launched before the FFN) gives the same bits as
    moe_combine_plan launched on its own: combined rows, release list and count, error
    word, masks, generations and held partial sums, with stale and duplicate arrivals."""
    wts = W.c2_weights()
    pool = W.c2_pool()
    wt = weight_tensors(wts)
    steps = []
    for fuse in (True, False):
        st = M.ExpertStep(8, 2880, 2880, 4, M.MOE_BF16, M.MOE_BF16, 512, 512, fuse_plan=fuse)
        st.load_weights(wt["wg"], wt["wu"], wt["wd"])
        steps.append(st)
    pool_t = dev(pool, "bf16")
    batches = [W.c2_skewed_batch(i, pool) for i in range(60)]
    ns = np.array([bb.n for bb in batches])
    pick = [int(np.argmin(ns)), int(np.flatnonzero((ns > 100) & (ns <= 256))[0]),
            int(np.argmax(np.where(ns <= 256, ns, 0))), int(np.flatnonzero(ns > 256)[0])]
    rng = np.random.default_rng(7)
    for i in pick:
        b = batches[i]
        _say(f"fused plan: batch {i} n={b.n}")
        d = batch_tensors(b)
        d["pool"] = pool_t
        gen, ks = b.gen.copy(), b.kslot.copy()
        bad = rng.choice(b.n, min(4, b.n), replace=False)
        gen[bad[:2]] += 1                              # stale generation
        ks[bad[2:]] = (ks[bad[2:]] + 1) % b.K          # a position the token already holds
        d["gen"], d["kslot"] = dev(gen.astype(np.uint32)), dev(ks.astype(np.int32))
        res = []
        for st in steps:
            M.moe_state_reset(st.state, 0)
            st.err.zero_()
            st.out.zero_()
            st.combine(d["r_rows"], d["r_idx"], d["r_tok"], d["r_kslot"], d["r_w"], d["r_gen"])
            st.run(d["slot"], d["expert"], 0, d["pool"], d["tok"], d["kslot"], d["w"], d["gen"])
            torch.cuda.synchronize()
            cnt = int(st.rel_count.item())
            mask = st.state.mask.cpu().numpy()
            held = np.flatnonzero(mask)
            res.append(dict(err=int(st.err.item()), cnt=cnt, rel=st.rel_list[:cnt].cpu().numpy(), mask=mask,
                            tgen=st.state.tgen.cpu().numpy(), out=to_numpy_bits(st.out), held=held,
                            acc=st.state.acc[torch.as_tensor(held, device="cuda").long()].cpu().numpy()))
        f, u = res
        assert f["err"] == u["err"] != 0
        assert f["cnt"] == u["cnt"] and np.array_equal(f["rel"], u["rel"])
        assert np.array_equal(f["mask"], u["mask"]) and np.array_equal(f["tgen"], u["tgen"])
        assert np.array_equal(f["out"], u["out"])
        assert np.array_equal(f["held"], u["held"]) and len(f["held"]) > 0
        assert np.array_equal(f["acc"].view(np.uint32), u["acc"].view(np.uint32))


def test_linked_index_matches_separate_link(c4_ref):
    """Queues of more than 1024 pairs: the index launch that also links the call's arrivals
    (the combine's link step; ExpertStep with the plan in the FFN call) gives the same bits as
    the link launched on its own (the step without a fused plan), with stale generations,
    repeated positions and rejected queue entries: release list and count, error word, masks,
    generations, held partial sums and the combined rows."""
    s, _ = c4_ref
    b = W.c4_wave(s, 3)  # 1638 pairs, each token's seven remote results delivered first
    _say(f"linked index: {b.n} pairs")
    wt = weight_tensors(s.weights)
    d = batch_tensors(b)
    rng = np.random.default_rng(11)
    bad = rng.choice(b.n, 12, replace=False)
    gen, ks, slot = b.gen.copy(), b.kslot.copy(), b.slot.copy()
    gen[bad[:4]] += 1                          # stale generation
    ks[bad[4:8]] = (ks[bad[4:8]] + 1) % b.K    # a position the token already holds (remote)
    slot[bad[8:]] = -1                          # rejected by the index: no batch row
    d["gen"], d["kslot"], d["slot"] = dev(gen.astype(np.uint32)), dev(ks.astype(np.int32)), dev(slot.astype(np.int32))
    res = []
    for fuse in (True, False):
        st = M.ExpertStep(b.E_loc, b.H, s.weights.I, b.K, M.MOE_BF16, M.MOE_FP8_E4M3, b.n, b.T, fuse_plan=fuse)
        st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt["s_gate"], wt["s_up"], wt["s_down"])
        st.combine(d["r_rows"], d["r_idx"], d["r_tok"], d["r_kslot"], d["r_w"], d["r_gen"])
        st.run(d["slot"], d["expert"], b.expert_base, d["pool"], d["tok"], d["kslot"], d["w"], d["gen"])
        torch.cuda.synchronize()
        cnt = int(st.rel_count.item())
        mask = st.state.mask.cpu().numpy()
        held = np.flatnonzero(mask)
        res.append(dict(err=int(st.err.item()), cnt=cnt, rel=st.rel_list[:cnt].cpu().numpy(), mask=mask,
                        tgen=st.state.tgen.cpu().numpy(), out=to_numpy_bits(st.out), held=held,
                        acc=st.state.acc[torch.as_tensor(held, device="cuda").long()].cpu().numpy(),
                        pos=st.pos[: b.n].cpu().numpy()))
        del st
    f, u = res
    want = M.ERR_STALE_GEN | M.ERR_DUPLICATE | M.ERR_SLOT_RANGE | M.ERR_ROW_RANGE
    assert f["err"] == u["err"] and (f["err"] & want) == want, (hex(f["err"]), hex(u["err"]))
    assert np.array_equal(f["pos"], u["pos"]) and (f["pos"][bad[8:]] == -1).all()
    assert f["cnt"] == u["cnt"] and np.array_equal(f["rel"], u["rel"]) and 0 < f["cnt"] < b.n
    assert np.array_equal(f["mask"], u["mask"]) and np.array_equal(f["tgen"], u["tgen"])
    assert np.array_equal(f["out"], u["out"])
    assert np.array_equal(f["held"], u["held"]) and len(f["held"]) > 0
    assert np.array_equal(f["acc"].view(np.uint32), u["acc"].view(np.uint32))


LINK_CASES = [
    # (n, E_loc, H, I, weight dtype): one pair past the first 1024-pair index workgroup, and
    # three workgroups with a ragged last one
    (1025, 8, 128, 64, "bf16"),
    (2600, 8, 256, 128, "fp8"),
]


@pytest.mark.parametrize("case", LINK_CASES, ids=[f"n{c[0]}_{c[4]}" for c in LINK_CASES])
def test_linked_index_multi_arrival_tokens(case):
    """The index launch that links the call's arrivals, on queues where most tokens have two to
    four arrivals in the call (the merge walks and sorts their lists) and a few have more than K
    (repeated positions), with stale generations and rejected queue entries: the same bits as the
    link launched on its own (index outputs, error word, release list, masks, generations, held
    partial sums, released rows)."""
    n, E, H, I, wdt = case
    K, P = 4, 4096
    T = n // 2
    _say("linked index, multi-arrival tokens", case)
    rng = np.random.default_rng(n + H)
    wts = W.make_layer_weights(rng, E, H, I, 0.05, wdt)
    wt = weight_tensors(wts)
    pool = dev(W.to_bf16_bits(rng.standard_normal((P, H)).astype(np.float32)), "bf16")
    slot = rng.integers(0, P, n).astype(np.int32)
    expert = rng.integers(0, E, n).astype(np.int32)
    tok = rng.integers(0, T, n).astype(np.int32)
    # each token's arrivals take distinct positions from a random order; a fifth or later
    # arrival repeats one (a duplicate)
    kslot = np.zeros(n, np.int32)
    seen = {}
    for i in range(n):
        order = seen.setdefault(int(tok[i]), list(rng.permutation(K)))
        kslot[i] = order.pop(0) if order else int(rng.integers(0, K))
    gen = np.zeros(n, np.uint32)
    w = rng.standard_normal(n).astype(np.float32)
    bad = rng.choice(n, 16, replace=False)
    gen[bad[:8]] = 1          # stale generation
    slot[bad[8:]] = -1        # rejected by the index: no batch row
    per_tok = np.bincount(tok, minlength=T)
    assert (per_tok >= 2).sum() > T // 3 and (per_tok >= K).any() and (per_tok > K).any()
    codes = {"bf16": M.MOE_BF16, "fp8": M.MOE_FP8_E4M3}
    d = dict(slot=dev(slot), expert=dev(expert), tok=dev(tok), kslot=dev(kslot), w=dev(w), gen=dev(gen))
    res = []
    for fuse in (True, False):
        st = M.ExpertStep(E, H, I, K, M.MOE_BF16, codes[wdt], n, T, fuse_plan=fuse)
        st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt.get("s_gate"), wt.get("s_up"), wt.get("s_down"))
        st.run(d["slot"], d["expert"], 0, pool, d["tok"], d["kslot"], d["w"], d["gen"])
        torch.cuda.synchronize()
        cnt = int(st.rel_count.item())
        mask = st.state.mask.cpu().numpy()
        held = np.flatnonzero(mask)
        res.append(dict(err=int(st.err.item()), cnt=cnt, rel=st.rel_list[:cnt].cpu().numpy(), mask=mask,
                        tgen=st.state.tgen.cpu().numpy(), out=to_numpy_bits(st.out), held=held,
                        acc=st.state.acc[torch.as_tensor(held, device="cuda").long()].cpu().numpy(),
                        pos=st.pos[:n].cpu().numpy(), perm=st.perm[:n].cpu().numpy(),
                        offsets=st.offsets.cpu().numpy(), y=to_numpy_bits(st.y[:n])))
        del st
    f, u = res
    want = M.ERR_STALE_GEN | M.ERR_DUPLICATE | M.ERR_SLOT_RANGE | M.ERR_ROW_RANGE
    assert f["err"] == u["err"] and (f["err"] & want) == want, (hex(f["err"]), hex(u["err"]))
    for k in ("pos", "perm", "offsets", "mask", "tgen", "held", "y"):
        assert np.array_equal(f[k], u[k]), k
    assert (f["pos"][bad[8:]] == -1).all()
    assert f["cnt"] == u["cnt"] and np.array_equal(f["rel"], u["rel"]) and 0 < f["cnt"] < T
    assert len(f["held"]) > 0
    assert np.array_equal(f["acc"].view(np.uint32), u["acc"].view(np.uint32))
    assert np.array_equal(f["out"], u["out"])
    # against the oracle, on the GPU's FFN rows: its assemble gives the batch rows, its combine
    # the acceptance, the release list, masks, generations and the error bits; released rows
    # within bf16 rounding, held partial sums within fp32 rounding
    a = O.assemble(slot, expert, 0, E, P)
    assert np.array_equal(f["pos"], a["pos"]) and np.array_equal(f["offsets"], a["offsets"])
    ocs = O.CombineState(T, K)
    out, rel, oerr = O.combine_release(ocs, O.decode_bf16(f["y"]), a["pos"], tok, kslot, w, gen)
    assert f["err"] == (a["err"] | oerr), (hex(f["err"]), hex(a["err"] | oerr))
    assert np.array_equal(f["rel"], rel)
    assert np.array_equal(f["mask"], ocs.mask) and np.array_equal(f["tgen"], ocs.tgen)
    got = O.decode_bf16(f["out"][rel])
    assert row_rel_err(got, np.stack([out[int(t)] for t in rel])) <= TOL["bf16"]
    ref_held = np.stack([sum(ocs.parts[int(t)].values()) for t in f["held"]])
    assert row_rel_err(f["acc"].astype(np.float64), ref_held) <= 1e-5


@pytest.fixture(scope="module")
def c4_ref():
    """The prefill setup and the oracle's FFN output of every one of its 16384 tokens
    (token index = pool slot; each token has one local pair, so E_{expert[t]}(x_t) is fixed
    per token and serves every wave and every merge of waves).  ffn_rows decodes each
    expert's fp8 weights once."""
    s = W.c4_prefill_setup()
    y = O.ffn_rows(O.decode(s.pool, "bf16"), s.expert, s.weights)
    return s, y


def _check_c4_batch(b, wts, y_ref_all, tol):
    """Runs one prefill-shaped batch (remote results delivered first) and checks it against
    the oracle: integer parts bit-exact, every FFN row and every combined row within tol."""
    st, e = _run_config_step(b, wts, M.MOE_BF16, M.MOE_FP8_E4M3, T_cap=b.T)
    a = O.assemble(b.slot, b.expert, 0, b.E_loc, b.P)
    assert e == 0 == a["err"]
    assert np.array_equal(st.perm.cpu().numpy()[: b.n], a["perm"])
    assert np.array_equal(st.pos.cpu().numpy()[: b.n], a["pos"])
    assert np.array_equal(st.offsets.cpu().numpy(), a["offsets"])
    assert np.array_equal(st.counts.cpu().numpy(), a["counts"])
    n_rel = int(st.rel_count.item())
    assert np.array_equal(st.rel_list[:n_rel].cpu().numpy(), np.sort(b.tok))
    # every batch row: row r holds the pair perm[r], whose token (= pool slot) fixes its output
    y_ref = y_ref_all[b.tok[a["perm"]]]
    y_gpu = decode_tensor(st.y[: b.n])
    ey, ee = row_rel_err(y_gpu, y_ref), elem_rel_err(y_gpu, y_ref)
    del y_gpu
    # every released token: its remote results plus the local one, in position order
    r = b.remote
    parts = {}
    for k in range(r.m):
        parts.setdefault(int(r.tok[k]), {})[int(r.kslot[k])] = (r.w[k], r.row_idx[k])
    refs = np.empty((b.n, b.H))
    for i in range(b.n):
        t = int(b.tok[i])
        full = {j: (w, O.decode_bf16(r.rows[ri])) for j, (w, ri) in parts[t].items()}
        full[int(b.kslot[i])] = (b.w[i], y_ref_all[t])
        refs[i] = O.combine_token([full[j] for j in range(b.K)])
    out_gpu = decode_tensor(st.out[torch.as_tensor(b.tok, device="cuda").long()])
    eo, eoe = row_rel_err(out_gpu, refs), elem_rel_err(out_gpu, refs)
    _say(f"  all {b.n} Y rows: row err {ey:.3e} (elementwise {ee:.3e}); all {n_rel} combined rows: "
         f"row err {eo:.3e} (elementwise {eoe:.3e})")
    assert ey <= tol and eo <= tol


@pytest.mark.parametrize("wave", [0, 1, 2, 3])
def test_c4_prefill_wave(c4_ref, wave):
    """Full-size prefill waves (6554 / 4915 / 3277 / 1638 pairs, 32 experts, fp8 weights):
    integer parts bit-exact; every FFN row and every combined row against the oracle."""
    _say(f"C4 prefill fp8 wave {wave}")
    s, y_all = c4_ref
    _check_c4_batch(W.c4_wave(s, wave), s.weights, y_all, TOL["fp8"])


@pytest.mark.parametrize("waves", [(0, 1), (1, 2), (2, 3), (0, 1, 2), (1, 2, 3), (0, 1, 2, 3)],
                         ids=lambda w: "waves" + "".join(map(str, w)))
def test_c4_merged_waves(c4_ref, waves):
    """Prefill waves merged into one ready batch (every run of consecutive waves a launch policy
    can form, up to all 16384 pairs: more row chunks per expert and a longer index pass than
    any single wave): integer parts bit-exact, every FFN row and every combined row against
    the oracle."""
    _say(f"C4 prefill fp8, merged waves {waves}")
    s, y_all = c4_ref
    _check_c4_batch(W.merge_batches([W.c4_wave(s, w) for w in waves]), s.weights, y_all, TOL["fp8"])


GATHER_CASES = [
    # (act/weight dtype, E, H, I, n, P, pitch padding): streaming kernel, 256-row fp8 GEMM,
    # 128-row GEMM kernel, fp32 path; pools whose rows are wider than H
    ("bf16", 8, 2880, 2880, 256, 4096, 0),
    ("fp8", 3, 640, 192, 700, 900, 0),
    ("bf16", 4, 512, 256, 600, 1000, 0),
    ("f32", 3, 64, 128, 40, 64, 0),
    ("bf16", 8, 2880, 2880, 256, 4096, 8),
    ("fp8", 3, 640, 192, 700, 900, 64),
]


@pytest.mark.parametrize("case", GATHER_CASES,
                         ids=[f"{c[0]}_E{c[1]}_H{c[2]}_n{c[4]}" + (f"_pad{c[6]}" if c[6] else "") for c in GATHER_CASES])
def test_gather_on_load_matches_explicit_gather(case):
    """The FFN reading pool rows through slot[perm[r]] gives the same bits as the FFN on the
    batch moe_assemble copied out, and both match the oracle; queue entries with invalid
    slots or non-local experts are rejected the same way.  The pool may be a view of wider
    rows (pitch H + padding)."""
    wdt, E, H, I, n, P, pad = case
    _say("gather-on-load case", case)
    rng = np.random.default_rng(n + H)
    act = "f32" if wdt == "f32" else "bf16"
    wts = W.make_layer_weights(rng, E, H, I, 0.05, wdt)
    pool_raw = rng.standard_normal((P, H + pad)).astype(np.float32)
    pool_full = pool_raw if act == "f32" else W.to_bf16_bits(pool_raw)
    pool_np = pool_full[:, :H]
    slot = rng.integers(0, P, n).astype(np.int32)
    expert = rng.integers(0, E, n).astype(np.int32)
    slot[:: 17] = P + 3          # rejected: slot out of range
    expert[5:: 29] = E + 1       # rejected: non-local expert
    codes = {"f32": M.MOE_F32, "bf16": M.MOE_BF16, "fp8": M.MOE_FP8_E4M3}
    wt = weight_tensors(wts)
    pool = dev(pool_full, act)[:, :H]
    assert pool.stride(0) == H + pad
    ys = []
    # gather through row_slot (the default), through perm and slot, and the explicit copy
    for mode in ("row_slot", "perm_slot", "explicit"):
        st = M.ExpertStep(E, H, I, 2, codes[act], codes[wdt], n, 4, gather_on_load=mode != "explicit")
        st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt.get("s_gate"), wt.get("s_up"), wt.get("s_down"))
        st.assemble(dev(slot), dev(expert), 0, pool)
        if mode == "perm_slot":
            st._gather = st._gather[:3]
        st.ffn(n)
        assert sync_err(st.err) == (M.ERR_SLOT_RANGE | M.ERR_EXPERT_NONLOCAL)
        ys.append(to_numpy_bits(st.y))
        offsets = st.offsets.cpu().numpy()
    nv = int(offsets[-1])
    assert np.array_equal(ys[0][:nv], ys[2][:nv]), "gather through row_slot differs from the explicit gather"
    assert np.array_equal(ys[1][:nv], ys[2][:nv]), "gather through perm/slot differs from the explicit gather"
    a = O.assemble(slot, expert, 0, E, P)
    assert np.array_equal(offsets, a["offsets"])
    y_ref = O.expert_ffn(O.decode(O.gather_rows(pool_np, slot, a["perm"], nv), act), a["offsets"], wts)
    err = row_rel_err(O.decode(ys[0][:nv], act), y_ref)
    _say(f"  row rel err {err:.3e}")
    assert err <= TOL[wdt]


def test_combine_plan_and_list_paths_agree():
    """Calls of up to 1024 arrivals on states under 2^20 tokens take the two-kernel plan
    path; other calls take the linked-list path.  The same calls on a small state (plan
    path) and on a 2^20-token state (list path) give the same bits: error words, release
    lists, released rows, partial sums and token state, including retries, stale and
    out-of-range arrivals and one token with more arrivals than a merge pass takes."""
    _say("combine plan vs list path")
    rng = np.random.default_rng(21)
    K, H, T_small = 4, 64, 300
    rows_np = rng.standard_normal((2000, H)).astype(np.float32)
    rows_t = dev(rows_np)
    sts = [M.ExpertStep(1, H, 64, K, M.MOE_F32, M.MOE_F32, 1, T) for T in (T_small, 1 << 20)]
    calls = []
    for c in range(3):
        m = int(rng.integers(200, 900))
        tok = rng.integers(0, 250, m)
        ks = rng.integers(0, K, m)
        gen = np.where(rng.random(m) < 0.03, 5, 0)              # stale
        row = rng.integers(0, 2000, m)
        row[rng.random(m) < 0.02] = 2500                          # row out of range
        ks[rng.random(m) < 0.02] = K + 2                          # position out of range
        if c == 1:                                                # a long chain for token 7
            tok[:150], ks[:150] = 7, np.arange(150) % K
        calls.append((row, tok, ks, rng.random(m).astype(np.float32), gen))
    res = []
    for st in sts:
        out = []
        for (row, tok, ks, w, gen) in calls:
            # generations advance as tokens release; re-tag the non-stale arrivals to the
            # token's current generation so that most arrivals are live
            tg = st.state.tgen.cpu().numpy().view(np.uint32)
            g = np.where(gen == 0, tg[tok], tg[tok] + 5).astype(np.uint32)
            st.err.zero_()
            st.combine(rows_t, dev(row.astype(np.int32)), dev(tok.astype(np.int32)), dev(ks.astype(np.int32)),
                       dev(w), dev(g))
            e = sync_err(st.err)
            n = int(st.rel_count.item())
            rel = st.rel_list[:n].cpu().numpy().copy()
            o = st.out[torch.as_tensor(rel, device="cuda").long()].cpu().numpy().copy() if n else np.zeros((0, H))
            out.append((e, rel, o))
        acc = st.state.acc[:T_small].cpu().numpy()
        mask = st.state.mask[:T_small].cpu().numpy()
        tgen = st.state.tgen[:T_small].cpu().numpy()
        res.append((out, acc, mask, tgen))
    (oa, acc_a, mask_a, tg_a), (ob, acc_b, mask_b, tg_b) = res
    for (ea, ra, xa), (eb, rb, xb) in zip(oa, ob):
        assert ea == eb and ea != 0
        assert np.array_equal(ra, rb) and len(ra) > 0
        assert np.array_equal(xa.view(np.uint32), xb.view(np.uint32))
    assert np.array_equal(mask_a, mask_b) and np.array_equal(tg_a, tg_b)
    held = mask_a != 0
    assert held.any()
    assert np.array_equal(acc_a[held].view(np.uint32), acc_b[held].view(np.uint32))


@pytest.mark.parametrize("shared_first", [False, True])
def test_shared_expert_joins_the_combine(shared_first):
    """Decode step with a shared expert at the home rank: every home token also goes through
    a dense SwiGLU whose result is combine position K with weight 1.  No token is released
    before both its routed and its shared results are in; the released rows match the
    oracle's sum_j w_j E_j(x) + E_shared(x); the order of the two calls does not matter."""
    _say("shared expert", "first" if shared_first else "last")
    b, wts = W.c1_decode()
    K, H, T = b.K, b.H, b.T
    rng = np.random.default_rng(77)
    sw = W.make_layer_weights(rng, 1, H, 1536, 0.02, "bf16")
    d = batch_tensors(b)
    wt, swt = weight_tensors(wts), weight_tensors(sw)
    st = M.ExpertStep(b.E_loc, H, wts.I, K + 1, M.MOE_BF16, M.MOE_BF16, b.n, T)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"])
    sh = M.SharedExpert(H, 1536, M.MOE_BF16, M.MOE_BF16, T)
    sh.load_weights(swt["wg"], swt["wu"], swt["wd"])
    # the home tokens: one pool slot per token index
    t_slot = np.zeros(T, np.int32)
    t_slot[b.tok] = b.slot
    toks = np.arange(T, dtype=np.int32)
    gens = np.zeros(T, np.uint32)
    st.combine(d["r_rows"], d["r_idx"], d["r_tok"], d["r_kslot"], d["r_w"], d["r_gen"])
    torch.cuda.synchronize()
    assert int(st.rel_count.item()) == 0

    def shared():
        sh.run(st, dev(t_slot), d["pool"], dev(toks), dev(gens), kslot=K)
        torch.cuda.synchronize()
        return int(st.rel_count.item())

    def routed():
        st.run(d["slot"], d["expert"], b.expert_base, d["pool"], d["tok"], d["kslot"], d["w"], d["gen"])
        torch.cuda.synchronize()
        return int(st.rel_count.item())

    first, second = (shared, routed) if shared_first else (routed, shared)
    assert first() == 0          # a result is still missing for every token
    n_rel = second()
    assert n_rel == T and sync_err(st.err) == 0 and sync_err(sh.step.err) == 0
    assert np.array_equal(st.rel_list[:n_rel].cpu().numpy(), toks)
    # oracle: routed results, remote results, shared result at position K with weight 1
    a, y = _oracle_step(b, wts)
    y_sh = O.expert_ffn(O.decode(b.pool[t_slot], "bf16"), np.array([0, T]), sw)
    ocs = O.CombineState(T, K + 1)
    r = b.remote
    O.combine_release(ocs, O.decode(r.rows, r.dtype), r.row_idx, r.tok, r.kslot, r.w, r.gen)
    calls = [(y, a["pos"], b.tok, b.kslot, b.w, b.gen),
             (y_sh, toks, toks, np.full(T, K, np.int32), np.ones(T, np.float32), gens)]
    if shared_first:
        calls.reverse()
    out = {}
    for args_ in calls:
        o, rel, err = O.combine_release(ocs, *args_)
        assert err == 0
        out.update(o)
    assert sorted(out) == list(range(T))
    g = decode_tensor(st.out[:T])
    err = row_rel_err(g, np.array([out[t] for t in range(T)]))
    _say(f"  combined rows with the shared expert: err {err:.3e}")
    assert err <= TOL["bf16"]


def _gemm_split_plan(counts, Nw, Kd, G_res):
    """Host model of the tiled kernel's work split (128-row chunks, 256 columns, 8 XCD ranges
    of chunk-major units, a tail of T <= Gx/2 units split into S k-ranges): the tail units'
    chunks of each XCD, with S, or an empty list when no tail is split."""
    E, n = len(counts), int(sum(counts))
    nbN = -(-Nw // 256)
    U = sum(-(-c // 128) for c in counts) * nbN
    G = min((n + 127 * E) // 128 * nbN, G_res)
    G = -(-G // 8) * 8
    Gx, KS = G // 8, Kd // 64
    out = []
    for x in range(8):
        u0 = U * x // 8
        nx = U * (x + 1) // 8 - u0
        R, T = divmod(nx, Gx)
        S = max(1, min(Gx // T, 8, KS // 4)) if T else 1
        if S > 1:
            out += [((u0 + R * Gx + t) // nbN, S) for t in range(T)]
    return out


GEMM256_CASES = [
    # (E, H, I, counts): 256-row units over every tile-count variant (last chunks of 88, 40,
    # 150, 230 and 1 rows: 3, 2, 5, 8 and 1 tiles of 32 rows), an empty expert, full chunks, a
    # partial last column block (Nw = 640: two of four waves active), contractions of 10 and 5
    # k-steps (not a multiple of the ring depth) ...
    (6, 640, 320, [600, 0, 40, 150, 230, 513]),
    # ... the other tile counts (4, 6, 7: chunks of 100, 170 and 200 rows) ...
    (3, 512, 256, [100, 170, 200]),
    # ... and more units than workgroups (18 chunks x 16 gate/up column blocks: two rounds)
    (2, 512, 2048, [3000, 1500]),
    # ... and more full rounds than the cost-ranked last round covers (159 chunks x 16 gate/up
    # column blocks: 9 full rounds and a tail in plain snake order)
    (4, 256, 2048, [20000, 12000, 6000, 2200]),
    # ... and workgroups left out of the later rounds: gate/up round 0 holds 128 units of 9 tiles'
    # cost (8 full chunks) and 128 of one tile; the later units of one tile go only to those 128:
    # one snaked round (139 rows per expert on average) ...
    (17, 256, 2048, [2048] + [20] * 16),
    # ... and one snaked round and a cost-ranked tail of 32
    (19, 256, 2048, [2048] + [20] * 18),
]


@pytest.mark.parametrize("case", GEMM256_CASES, ids=[f"E{c[0]}_H{c[1]}_I{c[2]}" for c in GEMM256_CASES])
def test_gemm256_fp8_units(case):
    """The fp8 tiled FFN (256-row units in cost order): every row against the oracle, the same
    bits on a second run, and the same bits with a workspace holding only h."""
    E, H, I, counts = case
    n = int(sum(counts))
    _say("gemm256 case", case)
    rng = np.random.default_rng(H + I + n)
    wts = W.make_layer_weights(rng, E, H, I, 0.05, "fp8")
    x_np = W.to_bf16_bits(rng.standard_normal((n, H)).astype(np.float32))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    st = M.ExpertStep(E, H, I, 2, M.MOE_BF16, M.MOE_FP8_E4M3, n, 4)
    wt = weight_tensors(wts)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt["s_gate"], wt["s_up"], wt["s_down"])
    st.xb[:n].copy_(dev(x_np, "bf16"))
    st.offsets.copy_(dev(offsets))
    h_bytes = (n * I * 2 + 255) // 256 * 256
    ys = []
    for ws in (st.workspace, st.workspace, st.workspace[:h_bytes]):
        st.y.zero_()
        M.moe_expert_ffn_grouped(n, E, H, I, M.MOE_BF16, M.MOE_FP8_E4M3, st.xb, st.offsets, st.w_gu, st.w_d, st.y,
                                 ws, st.s_gate, st.s_up, st.s_down)
        torch.cuda.synchronize()
        ys.append(to_numpy_bits(st.y[:n]))
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
    y_ref = O.expert_ffn(O.decode(x_np, "bf16"), offsets, wts)
    y_gpu = O.decode_bf16(ys[0])
    err, ee = row_rel_err(y_gpu, y_ref), elem_rel_err(y_gpu, y_ref)
    _say(f"  all {n} rows: row rel err {err:.3e} (elementwise {ee:.3e})")
    assert err <= TOL["fp8"]


@pytest.mark.parametrize("wdt", ["bf16"])
def test_gemm_split_tail_matches_whole_units(wdt):
    """Tiled FFN kernel for bf16 weights with each XCD's last partial round split along the
    contraction: the result is deterministic, matches the run with whole tail units (workspace
    without the partial area) to rounding, and matches the oracle on rows of the split units."""
    # 67 chunks x 16 gate/up column blocks = 134 units per XCD: a tail of 6 whether the kernel
    # runs one workgroup per CU (4 full rounds of 32) or two (2 full rounds of 64)
    E, H, I = 8, 1024, 2048
    counts = [2400, 1900, 1250, 1000, 850, 600, 250, 50]
    n = int(sum(counts))
    _say("gemm split case", wdt, counts)
    rng = np.random.default_rng(4242)
    wts = W.make_layer_weights(rng, E, H, I, 0.05, wdt)
    x_np = W.to_bf16_bits(rng.standard_normal((n, H)).astype(np.float32))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    code = {"bf16": M.MOE_BF16, "fp8": M.MOE_FP8_E4M3}[wdt]
    st = M.ExpertStep(E, H, I, 2, M.MOE_BF16, code, n, 4)
    wt = weight_tensors(wts)
    st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt.get("s_gate"), wt.get("s_up"), wt.get("s_down"))
    st.xb[:n].copy_(dev(x_np, "bf16"))
    st.offsets.copy_(dev(offsets))
    h_bytes = (n * I * 2 + 255) // 256 * 256
    assert st.workspace.numel() >= h_bytes + 256 * 128 * 1024
    ys = []
    for ws in (st.workspace, st.workspace, st.workspace[:h_bytes]):
        st.y.zero_()
        M.moe_expert_ffn_grouped(n, E, H, I, M.MOE_BF16, code, st.xb, st.offsets, st.w_gu, st.w_d, st.y, ws,
                                 st.s_gate, st.s_up, st.s_down)
        torch.cuda.synchronize()
        ys.append(to_numpy_bits(st.y[:n]))
    assert np.array_equal(ys[0], ys[1]), "split run is not deterministic"
    d = row_rel_err(O.decode_bf16(ys[0]), O.decode_bf16(ys[2]))
    _say(f"  split vs whole-unit row rel diff {d:.3e}")
    assert d <= 1e-2
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plans = [_gemm_split_plan(counts, 2 * I, H, cus * occ) for occ in (1, 2)]
    plan = plans[0]
    if cus == 256 and all(plans):
        assert not np.array_equal(ys[0], ys[2]), "no split was taken where the launch model predicts one"
    # oracle on rows of the split units' chunks (gate/up plan) plus a random sample
    starts = np.concatenate([[0], np.cumsum([-(-c // 128) for c in counts])])
    rows = list(rng.choice(n, 24, replace=False))
    for c, _S in plan[::3]:
        e = int(np.searchsorted(starts, c, side="right") - 1)
        r0 = offsets[e] + (c - starts[e]) * 128
        r1 = min(r0 + 128, offsets[e + 1])
        rows += [r0, (r0 + r1) // 2, r1 - 1]
    rows = np.unique(np.array(rows, dtype=np.int64))
    le = np.searchsorted(offsets, rows, side="right") - 1
    y_ref = O.ffn_rows(O.decode(x_np[rows], "bf16"), le, wts)
    err = row_rel_err(O.decode_bf16(ys[0][rows]), y_ref)
    _say(f"  {len(plan)} split tail units; oracle row rel err on {len(rows)} rows {err:.3e}")
    assert err <= TOL[wdt]


def _fused_index_batch(case):
    if case.startswith("many"):
        # 200 (bf16) or 256 (fp8) local experts from a nonzero base, most with one or two pairs
        # or none; two local pairs per token at distinct positions
        E, wdt, n = (200, "bf16", 256) if case == "many_bf16" else (256, "fp8", 250)
        rng = np.random.default_rng(E + n)
        H, I, K, P, base = 256, 128, 4, 512, 56
        T = (n + 1) // 2
        wts = W.make_layer_weights(rng, E, H, I, 0.05, wdt)
        tok = np.repeat(np.arange(T, dtype=np.int32), 2)[:n]
        kslot = np.concatenate([rng.permutation(K)[:2] for _ in range(T)]).astype(np.int32)[:n]
        b = W.Batch(act="bf16", H=H, K=K, E_loc=E, expert_base=base, P=P,
                    pool=W.to_bf16_bits(rng.standard_normal((P, H)).astype(np.float32)),
                    slot=rng.integers(0, P, n).astype(np.int32),
                    expert=(base + rng.integers(0, E, n)).astype(np.int32), tok=tok, kslot=kslot,
                    w=rng.standard_normal(n).astype(np.float32), gen=np.zeros(n, np.uint32), T=T)
        return b, wts, M.MOE_BF16, (M.MOE_BF16 if wdt == "bf16" else M.MOE_FP8_E4M3)
    if case.startswith("c1"):
        b, wts = W.c1_decode()
        act, wc = M.MOE_BF16, M.MOE_BF16
    else:  # fp8 weights on the weight-streaming path: the first 256 pairs of the last prefill wave
        setup = W.c4_prefill_setup()
        b = W.merge_batches([W.c4_wave(setup, 3)])
        wts = setup.weights
        act, wc = M.MOE_BF16, M.MOE_FP8_E4M3
        keep = np.arange(256)
        b = W.subset_batch(b, keep)
    if case == "c1_bad_ragged":
        keep = np.arange(200)
        b = W.subset_batch(b, keep)
        b.slot = b.slot.copy()
        b.expert = b.expert.copy()
        b.slot[[3, 77, 150]] = [b.P, -1, b.P + 9]          # slots outside the pool
        b.expert[[10, 120]] = [b.expert_base - 1, b.expert_base + b.E_loc]  # experts of another rank
    return b, wts, act, wc


@pytest.mark.parametrize("case", ["c1_bf16", "c1_bad_ragged", "c4_fp8_256", "many_bf16", "many_fp8"])
def test_fused_queue_index(case):
    """moe_ffn_args.index: the queue index derived inside the gate/up launch gives the same bits
    as moe_assemble followed by the FFN (index outputs, error word, FFN rows, release list,
    released rows and combine state), and its integer outputs match the oracle; also with no
    combine plan in the call."""
    _say(f"fused queue index vs separate moe_assemble: {case}")
    b, wts, act, wc = _fused_index_batch(case)
    d = batch_tensors(b)
    wt = weight_tensors(wts)
    n = b.n
    steps = []
    for fuse in (True, False):
        st = M.ExpertStep(b.E_loc, b.H, wts.I, b.K, act, wc, n, b.T, fuse_index=fuse)
        st.load_weights(wt["wg"], wt["wu"], wt["wd"], wt.get("s_gate"), wt.get("s_up"), wt.get("s_down"))
        if "r_rows" in d:
            st.combine(d["r_rows"], d["r_idx"], d["r_tok"], d["r_kslot"], d["r_w"], d["r_gen"])
        st.err.zero_()
        st.run(d["slot"], d["expert"], b.expert_base, d["pool"], d["tok"], d["kslot"], d["w"], d["gen"])
        torch.cuda.synchronize()
        steps.append(st)
    f, s = steps
    a = O.assemble(b.slot, b.expert, b.expert_base, b.E_loc, b.P)
    ef, es = sync_err(f.err), sync_err(s.err)
    assert ef == es and (ef & 3) == a["err"], (ef, es, a["err"])
    assert np.array_equal(f.perm.cpu().numpy()[:n], a["perm"])
    assert np.array_equal(f.pos.cpu().numpy()[:n], a["pos"])
    assert np.array_equal(f.counts.cpu().numpy(), a["counts"])
    assert np.array_equal(f.offsets.cpu().numpy(), a["offsets"])
    nv = int(a["offsets"][-1])
    rs = f.row_slot.cpu().numpy()[:n]
    assert np.array_equal(rs[:nv], b.slot[a["perm"][:nv]]) and (rs[nv:] == -1).all()
    for name in ("perm", "pos", "counts", "offsets", "row_slot"):
        assert np.array_equal(getattr(f, name).cpu().numpy()[:n], getattr(s, name).cpu().numpy()[:n]), name
    assert np.array_equal(to_numpy_bits(f.y[:nv]), to_numpy_bits(s.y[:nv])), "FFN rows differ"
    nr = int(f.rel_count.item())
    assert nr == int(s.rel_count.item())
    rel = f.rel_list[:nr]
    assert torch.equal(rel, s.rel_list[:nr])
    if nr:
        assert np.array_equal(to_numpy_bits(f.out[rel.long()]), to_numpy_bits(s.out[rel.long()]))
    assert torch.equal(f.state.mask, s.state.mask) and torch.equal(f.state.tgen, s.state.tgen)
    # the FFN call with the index and no combine plan
    f.err.zero_()
    f.y.zero_()
    ix = f.index_args(d["slot"], d["expert"], b.expert_base, d["pool"], n)
    f.ffn(n, index=ix)
    torch.cuda.synchronize()
    assert sync_err(f.err) == a["err"]
    assert np.array_equal(f.perm.cpu().numpy()[:n], a["perm"])
    assert np.array_equal(to_numpy_bits(f.y[:nv]), to_numpy_bits(s.y[:nv])), "FFN rows differ without a plan"
