"""The allocation-free combine entry point (moe_combine_release_noalloc: the library's static
scratch instead of the caller's workspace) against moe_combine_release with a workspace, on
two calls in a row, the second smaller: the first takes the linked-list path (more than 1024
arrivals), the second the plan path.  Error words, release lists, released rows, partial sums
and token state must agree bit for bit.  The call rejects more arrivals than its scratch holds."""
import numpy as np
import pytest
import torch

import asynchronous_moe_expert_amd as M
from gpu_helpers import dev, sync_err
from workloads.device import to_numpy_bits

pytestmark = pytest.mark.gpu


def _calls(rng, K, T, n_rows):
    out = []
    for m in (9000, 600):
        tok = rng.integers(0, T, m)
        ks = rng.integers(0, K, m)
        stale = rng.random(m) < 0.03
        row = rng.integers(0, n_rows, m)
        row[rng.random(m) < 0.01] = n_rows + 7     # row out of range
        ks[rng.random(m) < 0.01] = K + 1           # position out of range
        out.append((row.astype(np.int32), tok.astype(np.int32), ks.astype(np.int32),
                    rng.random(m).astype(np.float32), stale))
    return out


def test_noalloc_combine_matches_workspace_combine():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    print("no-alloc combine vs workspace combine", flush=True)
    rng = np.random.default_rng(31)
    K, H, T, n_rows = 4, 256, 3000, 12000
    rows = dev(rng.standard_normal((n_rows, H)).astype(np.float32)).to(torch.bfloat16)
    sts = [M.ExpertStep(1, H, 64, K, M.MOE_BF16, M.MOE_BF16, 1, T) for _ in range(2)]
    calls = _calls(rng, K, T, n_rows)
    res = [[], []]
    for c, (row, tok, ks, w, stale) in enumerate(calls):
        for k, (st, part) in enumerate(zip(sts, ("release", "noalloc"))):
            tg = st.state.tgen.cpu().numpy().view(np.uint32)
            g = np.where(stale, tg[tok] + 3, tg[tok]).astype(np.uint32)
            st.err.zero_()
            st.rel_count.fill_(-1)
            st._combine_room(len(tok))
            M.moe_combine_release(rows, dev(row), dev(tok), dev(ks), dev(w), dev(g), K, st.state, st.out,
                                  st.rel_list, st.rel_count, st.err, st.cmb_ws if part == "release" else None,
                                  m=len(tok), n_rows=n_rows, part=part)
            e = sync_err(st.err)
            n = int(st.rel_count.item())
            rel = st.rel_list[:n].cpu().numpy().copy()
            o = to_numpy_bits(st.out[torch.as_tensor(rel, device="cuda").long()]) if n else np.zeros((0, H))
            res[k].append((e, rel, o))
        (ea, ra, oa), (eb, rb, ob) = res[0][c], res[1][c]
        print(f"  call {c}: {len(tok)} arrivals, {len(ra)} released, err {ea:#x}", flush=True)
        assert ea == eb and ea != 0
        assert np.array_equal(ra, rb) and len(ra) > 0
        assert np.array_equal(oa, ob)
    sa, sb = sts[0].state, sts[1].state
    assert np.array_equal(sa.mask.cpu().numpy(), sb.mask.cpu().numpy())
    assert np.array_equal(sa.tgen.cpu().numpy(), sb.tgen.cpu().numpy())
    held = np.flatnonzero(sa.mask.cpu().numpy())
    assert len(held) > 0
    hi = torch.as_tensor(held, device="cuda").long()
    assert np.array_equal(sa.acc[hi].cpu().numpy().view(np.uint32), sb.acc[hi].cpu().numpy().view(np.uint32))
    # more arrivals than the static scratch holds: rejected on the host, nothing enqueued
    big = M.moe_combine_noalloc_max_arrivals() + 1
    z = torch.zeros(big, dtype=torch.int32, device="cuda")
    with pytest.raises(M.MoeError, match="static scratch"):
        M.moe_combine_release(rows, z, z, z, z.float(), z, K, sb, sts[1].out, sts[1].rel_list, sts[1].rel_count,
                              sts[1].err, None, m=big, n_rows=n_rows, part="noalloc")
