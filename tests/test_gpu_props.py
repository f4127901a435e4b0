"""Property tests (seeded, fixed example budget) of the HIP path against the oracle on tiny
shapes: random queues through moe_assemble, and random arrival streams split over several
moe_combine_release calls.  Integer parts must match bit for bit; the combine runs on
integer-toy rows with power-of-two weights, whose sums are exact in any order, so the
released rows must match bit for bit too ([NOTES] numerical contract: bitwise results may
depend on arrival order only through rounding)."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import asynchronous_moe_expert_amd as M
import oracle as O
from gpu_helpers import dev, sync_err

pytestmark = pytest.mark.gpu

SETTINGS = dict(max_examples=40, derandomize=True, deadline=None, database=None,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()


@settings(**SETTINGS)
@given(n=st.integers(0, 2100), E=st.integers(1, 12), base=st.integers(0, 20), P=st.integers(1, 64),
       bad=st.floats(0.0, 0.3), seed=st.integers(0, 2 ** 31 - 1))
def test_assemble_property(n, E, base, P, bad, seed):
    rng = np.random.default_rng(seed)
    slot = rng.integers(0, P, n).astype(np.int32)
    expert = (base + rng.integers(0, E, n)).astype(np.int32)
    k = int(bad * n)
    if k:
        idx = rng.choice(n, k, replace=False)
        slot[idx[: k // 2]] = P + 1
        expert[idx[k // 2:]] = base - 1
    H = 8
    pool = dev(rng.standard_normal((P, H)).astype(np.float32))
    m = max(n, 1)
    perm, pos, rs = (torch.full((m,), -9, dtype=torch.int32, device="cuda") for _ in range(3))
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    M.moe_assemble(dev(slot), dev(expert), base, E, pool, perm, pos, counts, offsets, None, err, n=n, row_slot=rs)
    e = sync_err(err)
    a = O.assemble(slot, expert, base, E, P)
    assert e == a["err"]
    assert np.array_equal(counts.cpu().numpy(), a["counts"])
    assert np.array_equal(offsets.cpu().numpy(), a["offsets"])
    if n:
        assert np.array_equal(perm.cpu().numpy()[:n], a["perm"])
        assert np.array_equal(pos.cpu().numpy()[:n], a["pos"])
        nv = int(a["offsets"][-1])
        assert np.array_equal(rs.cpu().numpy()[:nv], slot[a["perm"][:nv]])


@settings(**SETTINGS)
@given(K=st.integers(1, 5), T=st.integers(1, 24), calls=st.integers(1, 3), extra=st.integers(0, 40),
       seed=st.integers(0, 2 ** 31 - 1), big_state=st.booleans())
def test_combine_property(K, T, calls, extra, seed, big_state):
    """Every (token, position) result once, in a random order, split over `calls` calls, plus
    `extra` retries, stale and out-of-range arrivals; the same stream on a small state (plan
    path) or on a 2^20-token state (linked-list path)."""
    rng = np.random.default_rng(seed)
    H = 16
    arr = [(t, j) for t in range(T) for j in range(K)]
    arr = [arr[i] for i in rng.permutation(len(arr))]
    n_rows = len(arr) + extra
    rows = rng.integers(-64, 64, size=(n_rows, H)).astype(np.float32)
    w = (2.0 ** -rng.integers(0, 6, size=n_rows)).astype(np.float32)
    stream = [(i, t, j, 0) for i, (t, j) in enumerate(arr)]
    for x in range(extra):  # retries of delivered positions, stale generations, bad indices
        kind = int(rng.integers(0, 3))
        t, j = arr[int(rng.integers(0, len(arr)))]
        if kind == 0:
            stream.insert(int(rng.integers(0, len(stream) + 1)), (len(arr) + x, t, j, 0))
        elif kind == 1:
            stream.insert(int(rng.integers(0, len(stream) + 1)), (len(arr) + x, t, j, 7))
        else:
            stream.insert(int(rng.integers(0, len(stream) + 1)), (len(arr) + x, T + 3, j, 0))
    cuts = sorted(rng.choice(np.arange(1, len(stream)), min(calls - 1, len(stream) - 1), replace=False)) \
        if len(stream) > 1 else []
    parts = np.split(np.arange(len(stream)), cuts)
    T_cap = (1 << 20) if big_state else T
    stp = M.ExpertStep(1, H, 64, K, M.MOE_F32, M.MOE_F32, 1, T_cap)
    ocs = O.CombineState(T_cap, K)
    rows_t = dev(rows)
    for part in parts:
        sel = [stream[i] for i in part]
        ri = np.array([x[0] for x in sel], np.int32)
        tok = np.array([x[1] for x in sel], np.int32)
        ks = np.array([x[2] for x in sel], np.int32)
        gen = np.array([x[3] for x in sel], np.uint32)
        # generations of the live arrivals follow the token's current one (tokens do not repeat
        # a generation here: each is released at most once)
        stp.err.zero_()
        stp.combine(rows_t, dev(ri), dev(tok), dev(ks), dev(w[ri]), dev(gen), m=len(sel), n_rows=n_rows)
        e = sync_err(stp.err)
        out, rel, oerr = O.combine_release(ocs, rows.astype(np.float64), ri, tok, ks, w[ri], gen)
        assert e == oerr
        n_rel = int(stp.rel_count.item())
        assert np.array_equal(stp.rel_list[:n_rel].cpu().numpy(), rel)
        if n_rel:
            g = stp.out[torch.as_tensor(rel, device="cuda").long()].cpu().numpy()
            assert np.array_equal(g, np.array([out[t] for t in rel], np.float32))
    assert np.array_equal(stp.state.mask[:T].cpu().numpy().view(np.uint32), ocs.mask[:T])
    assert np.array_equal(stp.state.tgen[:T].cpu().numpy().view(np.uint32), ocs.tgen[:T])
