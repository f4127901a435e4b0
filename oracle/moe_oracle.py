"""CPU oracle for one expert-parallel rank's asynchronous MoE expert step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module: only the
test-suite, the package entry point's smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library (no kernels, headers, helpers or
constants); the error-flag values below are the documented contract, restated here.

What it computes, and where the pages define it
-----------------------------------------------
Sources (web pages, cited by title and section):
  [SEP]  marsggbo, "SOSP'26 | StreamEP" blog post (sections numbered as on the page)
  [NOTES] Steven He, "asynchronous MoE serving: StreamEP, buffering, and progress"
          (section "inferred obligations for a concrete protocol")
  [CEP]  "CascadeEP: Asynchronous Expert Execution for MoE Prefill under Attention
          Imbalance" (abstract: readiness tracked per generation, asynchronous expert start)

  * assemble  -- [SEP] §3 steps 1-4: ready token vectors sit in a GPU token pool, tracked
    by (request, layer, expert, top-k weight) metadata; the executor turns the scattered
    inputs of one expert micro-queue into one contiguous batch.  Reading: rows are grouped
    by local expert (ascending) and, within an expert, kept in queue order.
  * expert_ffn -- [SEP] §3 step 4 ("run the expert computation on the batch").  The pages
    do not give the FFN form; the plainest reading consistent with the GPT-OSS-style
    layer is a bias-free SwiGLU:  E(x) = Wd (silu(Wg x) * (Wu x)),  silu(z) = z/(1+e^-z).
  * combine_release -- [SEP] §3, combine equation  y = sum_{j=1..K} w_j E_j(x), and the
    rule that the first K-1 results of a token are buffered and the K-th makes it
    eligible for the next layer.  [NOTES] "inferred obligations": accept exactly the
    selected contributions once (retries must not double-count), tag contributions with a
    reuse generation, never release a token with a result missing.  [CEP]: readiness is
    tracked per generation; a slot is reset only after release.

Everything floating point is done in float64 on the stored input values (bf16 bit
patterns and fp8 codes are decoded exactly; an fp8 weight is code_value * row_scale).
Pins: tests/test_oracle.py checks every function here against closed forms, brute force
on tiny inputs, exact rational arithmetic and the pages' worked examples.
"""
from __future__ import annotations

import numpy as np

# Error flags (a bit mask; each call ORs in the flags of every entry it rejected).
ERR_SLOT_RANGE = 1 << 0       # pair's pool slot outside [0, P)
ERR_EXPERT_NONLOCAL = 1 << 1  # pair's expert not among this rank's experts
ERR_TOKEN_RANGE = 1 << 2      # arrival's token index outside [0, T_cap)
ERR_KSLOT_RANGE = 1 << 3      # arrival's top-k position outside [0, K)
ERR_ROW_RANGE = 1 << 4        # arrival's row index outside the row source
ERR_STALE_GEN = 1 << 5        # arrival's generation is not the token's current one
ERR_DUPLICATE = 1 << 6        # the token already holds a result for this top-k position


# ------------------------------------------------------------------ storage decoding
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (bf16 is the top half of an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 (no infinities, exponent bias 7, S.1111.111 is NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    v = sign * np.where(e > 0, normal, subnormal)
    return np.where((e == 0xF) & (c & 0x7 == 0x7), np.nan, v)


def decode(storage: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(storage, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(storage)
    if dtype == "fp8":
        return decode_e4m3(storage)
    raise ValueError(dtype)


# ------------------------------------------------------------------------- assemble
def assemble(slot, expert, expert_base: int, E_loc: int, P: int) -> dict:
    """Group a micro-queue's (slot, expert) pairs into a contiguous expert-major batch.

    Returns counts[E_loc], offsets[E_loc+1] (exclusive prefix sums, offsets[E_loc] = number
    of accepted pairs), perm[n] (perm[r] = queue index of the pair at assembled row r, -1
    past the accepted rows), pos[n] (assembled row of queue entry i, -1 if rejected) and
    the error mask.  A pair is rejected if its slot is outside the pool or its expert is
    not local; rejected pairs take no row.
    """
    n = len(slot)
    err = 0
    local = [-1] * n
    for i in range(n):
        s, e = int(slot[i]), int(expert[i])
        ok = True
        if not (0 <= s < P):
            err |= ERR_SLOT_RANGE
            ok = False
        if not (expert_base <= e < expert_base + E_loc):
            err |= ERR_EXPERT_NONLOCAL
            ok = False
        if ok:
            local[i] = e - expert_base
    counts = [0] * E_loc
    for i in range(n):
        if local[i] >= 0:
            counts[local[i]] += 1
    offsets = [0] * (E_loc + 1)
    for e in range(E_loc):
        offsets[e + 1] = offsets[e] + counts[e]
    next_row = list(offsets[:E_loc])
    perm = [-1] * n
    pos = [-1] * n
    for i in range(n):  # queue order: stable within an expert
        e = local[i]
        if e >= 0:
            r = next_row[e]
            next_row[e] += 1
            perm[r] = i
            pos[i] = r
    return dict(counts=np.array(counts, np.int32), offsets=np.array(offsets, np.int32),
                perm=np.array(perm, np.int32), pos=np.array(pos, np.int32), err=err)


def gather_rows(pool: np.ndarray, slot, perm, n_rows: int) -> np.ndarray:
    """Xb[r] = pool[slot[perm[r]]] for r < n_rows: a byte-exact copy of the stored rows."""
    out = np.empty((n_rows,) + pool.shape[1:], pool.dtype)
    for r in range(n_rows):
        out[r] = pool[int(slot[int(perm[r])])]
    return out


# ----------------------------------------------------------------------- expert FFN
def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """E(x) = Wd (silu(Wg x) * (Wu x)) for each row x of `x` ([m][H]); wg, wu: [I][H];
    wd: [H][I].  float64 throughout."""
    g = x @ wg.T
    u = x @ wu.T
    return (silu(g) * u) @ wd.T


def expert_weights(weights, e: int):
    """float64 (Wg, Wu, Wd) of local expert e; fp8 rows are code_value * row_scale."""
    dt = weights.dtype
    wg = decode(weights.wg[e], dt)
    wu = decode(weights.wu[e], dt)
    wd = decode(weights.wd[e], dt)
    if dt == "fp8":
        wg = wg * weights.sg[e].astype(np.float64)[:, None]
        wu = wu * weights.su[e].astype(np.float64)[:, None]
        wd = wd * weights.sd[e].astype(np.float64)[:, None]
    return wg, wu, wd


def expert_ffn(xb: np.ndarray, offsets, weights) -> np.ndarray:
    """Y[r] = E_e(Xb[r]) for the rows offsets[e] <= r < offsets[e+1] of each expert e."""
    n = int(offsets[-1])
    y = np.zeros((n, xb.shape[1]), np.float64)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = swiglu(xb[a:b], *expert_weights(weights, e))
    return y


def ffn_rows(x: np.ndarray, local_expert, weights) -> np.ndarray:
    """E_{e_r}(x_r) for a sample of rows (each with its own local expert)."""
    y = np.zeros((x.shape[0], x.shape[1]), np.float64)
    le = np.asarray(local_expert)
    for e in np.unique(le):
        idx = np.nonzero(le == e)[0]
        y[idx] = swiglu(x[idx], *expert_weights(weights, int(e)))
    return y


# ------------------------------------------------------------------ combine/release
class CombineState:
    """Per-token combine state of the home rank.

    mask[t]  bit j set once the result for top-k position j of token t was accepted
    tgen[t]  generation the token's next results must carry
    parts[t] accepted contributions w_j * E_j(x) by position j (float64)
    """

    def __init__(self, T_cap: int, K: int):
        self.T_cap, self.K = T_cap, K
        self.mask = np.zeros(T_cap, np.uint32)
        self.tgen = np.zeros(T_cap, np.uint32)
        self.parts: dict[int, dict[int, np.ndarray]] = {}


def combine_release(state: CombineState, rows: np.ndarray, row_idx, tok, kslot, w, gen):
    """Accept one call's arrivals in list order, then release every completed token.

    rows: float64 [n_rows][H] row source.  Arrival i carries rows[row_idx[i]] for
    (token tok[i], position kslot[i], weight w[i], generation gen[i]).

    An arrival is rejected (and its flag raised) if an index is out of range, if its
    generation is not the token's current one, or if the token already holds a result
    for that position (from an earlier call or earlier in this call).  After the call,
    each token holding all K positions is released: y_t = sum_j w_j E_j(x) summed in j
    order, its state is cleared and its generation advances.

    Returns (out: {t: y_t}, rel_list: ascending released tokens, err).
    """
    K, T_cap = state.K, state.T_cap
    n_rows = rows.shape[0]
    err = 0
    for i in range(len(tok)):
        t, j, r = int(tok[i]), int(kslot[i]), int(row_idx[i])
        bad = 0
        if not (0 <= t < T_cap):
            bad |= ERR_TOKEN_RANGE
        if not (0 <= j < K):
            bad |= ERR_KSLOT_RANGE
        if not (0 <= r < n_rows):
            bad |= ERR_ROW_RANGE
        if bad:
            err |= bad
            continue
        if int(gen[i]) != int(state.tgen[t]):
            err |= ERR_STALE_GEN
            continue
        if (int(state.mask[t]) >> j) & 1:
            err |= ERR_DUPLICATE
            continue
        state.mask[t] = np.uint32(int(state.mask[t]) | (1 << j))
        state.parts.setdefault(t, {})[j] = float(np.float32(w[i])) * rows[r]
    full = (1 << K) - 1
    out = {}
    rel = []
    for t in sorted(state.parts):
        if int(state.mask[t]) == full:
            acc = np.zeros_like(state.parts[t][0])
            for j in range(K):
                acc = acc + state.parts[t][j]
            out[t] = acc
            rel.append(t)
    for t in rel:
        del state.parts[t]
        state.mask[t] = 0
        state.tgen[t] = np.uint32(int(state.tgen[t]) + 1)
    return out, np.array(rel, np.int32), err


def combine_token(parts) -> np.ndarray:
    """y = sum_j w_j * row_j for one token, parts given in j order as (w, row64)."""
    acc = None
    for wj, row in parts:
        c = float(np.float32(wj)) * row
        acc = c if acc is None else acc + c
    return acc
