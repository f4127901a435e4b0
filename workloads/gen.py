"""Seeded synthetic workloads shaped like the pages' expert-parallel MoE layers.

The layer shapes come from the StreamEP write-up (marsggbo, "SOSP'26 | StreamEP", §3 and
§7: GPT-OSS-120B, 128 experts, top-4, hidden 2880, 36 layers) and from the CascadeEP /
ASAP prefill setting (uneven waves of ready tokens from attention replicas).  The
distributions (N(0, sigma) activations and weights, softmax-renormalised top-k router
weights, Zipf expert skew, uneven prefill waves) are synthetic stand-ins for the pages'
datasets and routing traces, which are not available.

Storage formats produced here:
  * "f32":  float32 arrays
  * "bf16": uint16 arrays holding bfloat16 bit patterns (round-to-nearest-even from fp32)
  * "fp8":  uint8 arrays holding OCP fp8 e4m3 ("e4m3fn") codes, plus one fp32 scale per
            weight row (scale = row amax / 448, codes = RNE(w / scale), saturating)

Every generator is a pure function of its arguments: the same call gives the same arrays.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

BASE_SEED = 20261202


def _rng(cfg: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED + cfg, *key])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (RNE), as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes (RNE), saturating at +-448, as uint8."""
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def zipf_probs(s: float, n: int) -> np.ndarray:
    """P(rank k) proportional to k^-s for k = 1..n; rank k is local expert k-1."""
    p = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


ZIPF_P = {1.2: zipf_probs(1.2, 8), 1.0: zipf_probs(1.0, 32)}


def _softmax64(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


@dataclass
class LayerWeights:
    """One layer's local experts.  wg, wu: [E][I][H]; wd: [E][H][I] (output-major rows).

    For dtype "fp8" the s* arrays hold one fp32 scale per stored row:
    sg, su: [E][I]; sd: [E][H].  The represented weight is code_value * scale.
    """

    dtype: str
    E: int
    H: int
    I: int
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    sg: Optional[np.ndarray] = None
    su: Optional[np.ndarray] = None
    sd: Optional[np.ndarray] = None


def _quant_rows(w: np.ndarray):
    amax = np.abs(w).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = to_e4m3_codes(w / scale[..., None])
    return codes, scale


def make_layer_weights(rng: np.random.Generator, E: int, H: int, I: int, sigma: float,
                       dtype: str) -> LayerWeights:
    """Draw E experts' SwiGLU weights ~ N(0, sigma) (sigma = standard deviation)."""
    sd_ = np.float32(sigma)
    if dtype in ("f32", "bf16"):
        wg = np.empty((E, I, H), np.float32 if dtype == "f32" else np.uint16)
        wu = np.empty_like(wg)
        wd = np.empty((E, H, I), wg.dtype)
        for e in range(E):
            wg[e] = _store(rng.standard_normal((I, H), dtype=np.float32) * sd_, dtype)
            wu[e] = _store(rng.standard_normal((I, H), dtype=np.float32) * sd_, dtype)
            wd[e] = _store(rng.standard_normal((H, I), dtype=np.float32) * sd_, dtype)
        return LayerWeights(dtype, E, H, I, wg, wu, wd)
    if dtype == "fp8":
        wg = np.empty((E, I, H), np.uint8)
        wu = np.empty_like(wg)
        wd = np.empty((E, H, I), np.uint8)
        sg = np.empty((E, I), np.float32)
        su = np.empty_like(sg)
        sdd = np.empty((E, H), np.float32)
        for e in range(E):
            wg[e], sg[e] = _quant_rows(rng.standard_normal((I, H), dtype=np.float32) * sd_)
            wu[e], su[e] = _quant_rows(rng.standard_normal((I, H), dtype=np.float32) * sd_)
            wd[e], sdd[e] = _quant_rows(rng.standard_normal((H, I), dtype=np.float32) * sd_)
        return LayerWeights(dtype, E, H, I, wg, wu, wd, sg, su, sdd)
    raise ValueError(dtype)


@dataclass
class Arrivals:
    """Expert results arriving at the home rank's combine: one row per arrival."""

    dtype: str
    rows: np.ndarray      # [m_rows][H] storage
    row_idx: np.ndarray   # [m] int32 row of `rows` carrying arrival i
    tok: np.ndarray       # [m] int32 combine-state token index
    kslot: np.ndarray     # [m] int32 position j in the token's top-k list
    w: np.ndarray         # [m] float32 router weight w_j
    gen: np.ndarray       # [m] uint32 token generation the result belongs to

    @property
    def m(self) -> int:
        return int(self.tok.shape[0])


@dataclass
class Batch:
    """One ready expert batch: the pool, the queue of (token, expert) pairs, and the
    results for the same tokens computed on other ranks (delivered before the step)."""

    act: str
    H: int
    K: int
    E_loc: int
    expert_base: int
    P: int
    pool: np.ndarray      # [P][H] storage
    slot: np.ndarray      # [n] int32 pool slot of the pair's token vector
    expert: np.ndarray    # [n] int32 global expert id
    tok: np.ndarray       # [n] int32 combine-state token index
    kslot: np.ndarray     # [n] int32 j of this pair in the token's top-k list
    w: np.ndarray         # [n] float32 router weight
    gen: np.ndarray       # [n] uint32 generation
    T: int                # tokens covered; token indices are 0..T-1
    remote: Optional[Arrivals] = None

    @property
    def n(self) -> int:
        return int(self.slot.shape[0])


def _topk(logits: np.ndarray, K: int) -> np.ndarray:
    # highest logits first; ties go to the lower expert id (stable order)
    return np.argsort(-logits, kind="stable")[:K]


def _remote_arrivals(rng, act: str, H: int, items) -> Arrivals:
    """items: list of (tok, j, w) for results computed elsewhere; rows ~ N(0,1)."""
    m = len(items)
    rows = _store(rng.standard_normal((max(m, 1), H), dtype=np.float32), act)[:m]
    tok = np.array([it[0] for it in items], np.int32)
    ks = np.array([it[1] for it in items], np.int32)
    w = np.array([it[2] for it in items], np.float32)
    return Arrivals(act, rows, np.arange(m, dtype=np.int32), tok, ks, w, np.zeros(m, np.uint32))


# ---------------------------------------------------------------- C0: tiny fp32 layer
def c0_tiny():
    """8 experts all local, top-2, hidden 64, intermediate 128, 128 pool slots, a queue
    of 32 ready tokens at random slots; everything fp32; all results arrive in one step."""
    rng = _rng(0)
    E, K, H, I, P, T = 8, 2, 64, 128, 128, 32
    pool = rng.standard_normal((P, H), dtype=np.float32)
    slots = rng.permutation(P)[:T].astype(np.int32)
    logits = rng.standard_normal((T, E))
    rows = []
    for t in range(T):
        top = _topk(logits[t], K)
        w = _softmax64(logits[t][top]).astype(np.float32)
        for j in range(K):
            rows.append((slots[t], int(top[j]), t, j, w[j]))
    order = rng.permutation(len(rows))
    rows = [rows[i] for i in order]
    weights = make_layer_weights(rng, E, H, I, 0.05, "f32")
    b = Batch("f32", H, K, E, 0, P, pool,
              np.array([r[0] for r in rows], np.int32), np.array([r[1] for r in rows], np.int32),
              np.array([r[2] for r in rows], np.int32), np.array([r[3] for r in rows], np.int32),
              np.array([r[4] for r in rows], np.float32), np.zeros(len(rows), np.uint32), T, None)
    return b, weights


# ------------------------------------------------------- C1: decode-shaped rank share
C1 = dict(E_total=128, E_loc=8, K=4, H=2880, I=2880, P=4096, n=256)


def c1_decode(rank: int = 0, with_weights: bool = True):
    """256 token-expert pairs for one of 16 ranks (8 local experts of 128, top-4).

    Tokens draw 128 N(0,1) logits; the expert set is the top-4 (a uniform 4-subset) and
    the router weights are the softmax of those 4 logits.  Tokens with no local expert are
    redrawn, as are tokens whose local pairs would overflow 256.  Results for the token's
    non-local experts are N(0,1) bf16 rows."""
    c = C1
    rng = _rng(1, rank)
    E_loc, K, H, n = c["E_loc"], c["K"], c["H"], c["n"]
    base = rank * E_loc
    toks = []
    npairs = 0
    while npairs < n:
        lg = rng.standard_normal(c["E_total"])
        top = _topk(lg, K)
        nl = int(((top >= base) & (top < base + E_loc)).sum())
        if nl == 0 or npairs + nl > n:
            continue
        toks.append((top, _softmax64(lg[top]).astype(np.float32)))
        npairs += nl
    T = len(toks)
    slots = rng.permutation(c["P"])[:T].astype(np.int32)
    pool = to_bf16_bits(rng.standard_normal((c["P"], H), dtype=np.float32))
    pairs, remote = [], []
    for t, (top, w) in enumerate(toks):
        for j in range(K):
            e = int(top[j])
            if base <= e < base + E_loc:
                pairs.append((slots[t], e, t, j, w[j]))
            else:
                remote.append((t, j, w[j]))
    order = rng.permutation(len(pairs))
    pairs = [pairs[i] for i in order]
    rem = _remote_arrivals(rng, "bf16", H, remote)
    b = Batch("bf16", H, K, E_loc, base, c["P"], pool,
              np.array([p[0] for p in pairs], np.int32), np.array([p[1] for p in pairs], np.int32),
              np.array([p[2] for p in pairs], np.int32), np.array([p[3] for p in pairs], np.int32),
              np.array([p[4] for p in pairs], np.float32), np.zeros(len(pairs), np.uint32), T, rem)
    wts = make_layer_weights(_rng(1, 1000 + rank), E_loc, H, c["I"], 0.02, "bf16") if with_weights else None
    return b, wts


# ------------------------------------------------------ C2: skewed ragged micro-queues
C2 = dict(E_loc=8, K=4, H=2880, I=2880, P=4096, batches=200, s=1.2)


def c2_weights() -> LayerWeights:
    return make_layer_weights(_rng(2, 1), 8, 2880, 2880, 0.02, "bf16")


def c2_pool() -> np.ndarray:
    return to_bf16_bits(_rng(2, 2).standard_normal((C2["P"], C2["H"]), dtype=np.float32))


def c2_skewed_batch(b: int, pool: np.ndarray) -> Batch:
    """Batch b (0-based) of 200: n ~ U{8..512} pairs, one local pair per token at a fresh
    random permutation of the pool slots, expert ~ Zipf(1.2) over the 8 local experts, the
    local pair at j ~ U{0..3} of a softmax over 4 N(0,1) logits; 3 remote results each."""
    c = C2
    rng = _rng(2, 0, b)
    n = int(rng.integers(8, 513))
    slots = rng.permutation(c["P"])[:n].astype(np.int32)
    experts = rng.choice(c["E_loc"], size=n, p=ZIPF_P[1.2]).astype(np.int32)
    w = _softmax64(rng.standard_normal((n, c["K"]))).astype(np.float32)
    jl = rng.integers(0, c["K"], size=n).astype(np.int32)
    remote = [(t, j, w[t, j]) for t in range(n) for j in range(c["K"]) if j != jl[t]]
    rem = _remote_arrivals(rng, "bf16", c["H"], remote)
    t = np.arange(n, dtype=np.int32)
    return Batch("bf16", c["H"], c["K"], c["E_loc"], 0, c["P"], pool, slots, experts, t, jl,
                 w[t, jl].astype(np.float32), np.zeros(n, np.uint32), n, rem)


# ------------------------------------------------------------- C4: prefill, fp8 weights
C4 = dict(E_total=256, E_loc=32, K=8, H=4096, I=2048, P=16384, waves=(6554, 4915, 3277, 1638), s=1.0)


@dataclass
class C4Setup:
    pool: np.ndarray
    expert: np.ndarray   # [16384] local expert of each token's one local pair
    w: np.ndarray        # [16384][8] router weights
    jl: np.ndarray       # [16384] j of the local pair
    order: np.ndarray    # [16384] token order; waves are consecutive slices
    weights: Optional[LayerWeights]


def c4_prefill_setup(with_weights: bool = True) -> C4Setup:
    """16384 tokens at slots 0..16383, one local pair each, expert ~ Zipf(1.0) over 32
    local experts, top-8 softmax weights, weights N(0,0.02) stored as fp8 e4m3 + row scales."""
    c = C4
    rng = _rng(4)
    P = c["P"]
    pool = np.empty((P, c["H"]), np.uint16)
    for r0 in range(0, P, 2048):
        pool[r0:r0 + 2048] = to_bf16_bits(rng.standard_normal((2048, c["H"]), dtype=np.float32))
    expert = rng.choice(c["E_loc"], size=P, p=ZIPF_P[1.0]).astype(np.int32)
    w = _softmax64(rng.standard_normal((P, c["K"]))).astype(np.float32)
    jl = rng.integers(0, c["K"], size=P).astype(np.int32)
    order = rng.permutation(P).astype(np.int32)
    wts = make_layer_weights(_rng(4, 1), c["E_loc"], c["H"], c["I"], 0.02, "fp8") if with_weights else None
    return C4Setup(pool, expert, w, jl, order, wts)


def c4_wave(setup: C4Setup, wave: int, with_remote: bool = True) -> Batch:
    """Wave `wave` (0..3) as its own ready batch; token index = pool slot."""
    c = C4
    lo = int(sum(c["waves"][:wave]))
    toks = setup.order[lo:lo + c["waves"][wave]]
    rem = None
    if with_remote:
        rng = _rng(4, 2, wave)
        items = [(int(t), j, setup.w[t, j]) for t in toks for j in range(c["K"]) if j != setup.jl[t]]
        rem = _remote_arrivals(rng, "bf16", c["H"], items)
    n = toks.shape[0]
    return Batch("bf16", c["H"], c["K"], c["E_loc"], 0, c["P"], setup.pool, toks.copy(),
                 setup.expert[toks].copy(), toks.copy(), setup.jl[toks].copy(),
                 setup.w[toks, setup.jl[toks]].astype(np.float32), np.zeros(n, np.uint32), c["P"], rem)


def merge_batches(batches: list) -> Batch:
    """Ready batches over one pool, concatenated in order into one batch (their queues back
    to back, remote results renumbered into one row block).  A single batch is returned as is."""
    if len(batches) == 1:
        return batches[0]
    b0 = batches[0]
    cat = lambda f: np.concatenate([getattr(b, f) for b in batches])  # noqa: E731
    rem = None
    if all(b.remote is not None for b in batches):
        offs = np.cumsum([0] + [b.remote.rows.shape[0] for b in batches[:-1]])
        rcat = lambda f: np.concatenate([getattr(b.remote, f) for b in batches])  # noqa: E731
        rem = Arrivals(b0.remote.dtype, rcat("rows"),
                       np.concatenate([b.remote.row_idx + o for b, o in zip(batches, offs)]).astype(np.int32),
                       rcat("tok"), rcat("kslot"), rcat("w"), rcat("gen"))
    return Batch(b0.act, b0.H, b0.K, b0.E_loc, b0.expert_base, b0.P, b0.pool, cat("slot"), cat("expert"),
                 cat("tok"), cat("kslot"), cat("w"), cat("gen"), b0.T, rem)


def subset_batch(b: Batch, keep) -> Batch:
    """The queue entries `keep` of a batch (in that order), with its pool, token range and remote
    results unchanged: tokens whose local pairs are dropped stay incomplete."""
    keep = np.asarray(keep)
    return Batch(b.act, b.H, b.K, b.E_loc, b.expert_base, b.P, b.pool, b.slot[keep].copy(), b.expert[keep].copy(),
                 b.tok[keep].copy(), b.kslot[keep].copy(), b.w[keep].copy(), b.gen[keep].copy(), b.T, b.remote)
