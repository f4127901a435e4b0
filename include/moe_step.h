/*
 * moe_step.h -- C ABI of libmoestep.so: one expert-parallel rank's asynchronous MoE
 * expert step on an AMD Instinct MI355X (gfx950).
 *
 * The step has three calls, in stream order:
 *
 *   moe_assemble            ready (token, expert) pairs scattered over an HBM token pool
 *                           -> one contiguous, expert-grouped batch
 *   moe_expert_ffn_grouped  per-expert SwiGLU FFN over the ragged per-expert row groups
 *   moe_combine_release     weighted combine y_t = sum_j w_j E_j(x_t) with per-token
 *                           arrival tracking; a token is released once all K results are in
 *
 * Sources for what each call computes (web pages, cited by title and section):
 *   [SEP]   marsggbo, "SOSP'26 | StreamEP" blog post: section 3 (token pool, metadata of
 *           request / layer / expert / top-k weight, per-layer micro-queues, assembly of a
 *           contiguous batch, buffering of partial top-k results, combine equation),
 *           section 6 (gather fused with the weighted merge during batch regrouping)
 *   [NOTES] Steven He, "asynchronous MoE serving: StreamEP, buffering, and progress",
 *           section "inferred obligations for a concrete protocol" (accept each selected
 *           contribution exactly once, tag reuse generations, never drop an expert result)
 *   [CEP]   "CascadeEP: Asynchronous Expert Execution for MoE Prefill under Attention
 *           Imbalance", abstract (expert FFN starts on whatever inputs are ready)
 *
 * Conventions shared by every call
 *   - Memory: the caller allocates every buffer (device memory unless stated).  The
 *     library never allocates, frees or synchronises.  Between calls it keeps only read-only
 *     device properties (compute-unit count, kernel occupancy), cached per device on first
 *     use with atomic stores, so concurrent calls from several host threads are safe; the one
 *     exception is moe_combine_release_noalloc, whose scratch is a static device array per GPU
 *     (its declaration below gives the limits and the races of overlapping calls).
 *   - Ordering: all work is enqueued on `stream` in call order.  Calls return as soon as
 *     the work is enqueued.
 *   - Host-side errors: a call validates its arguments first and, on failure, returns a
 *     negative moe_status and enqueues nothing.
 *   - Data-dependent errors: an entry whose index or tag is invalid is skipped and its
 *     MOE_ERR_* bit is OR-ed into the caller's device word *err (never cleared by the
 *     library).  Nothing is silently dropped: every skipped entry raises a bit.
 *   - Integer outputs (perm, pos, counts, offsets, release lists, state masks) are
 *     deterministic.  Floating-point outputs are within tolerance of an fp64 evaluation.
 */
#ifndef MOE_STEP_H
#define MOE_STEP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_STEP_VERSION 2  /* 2: moe_ffn_args.index */

/* Element storage types.  MOE_BF16 is bfloat16; MOE_FP8_E4M3 is OCP 8-bit float E4M3
 * (bias 7, max 448, no infinities), used for weights only, with one fp32 scale per
 * weight row (represented value = code value * row scale). */
typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Host-side return codes. */
typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL_NULL = -1,    /* a required pointer is NULL */
  MOE_EINVAL_SIZE = -2,    /* a size is negative or over a documented limit */
  MOE_EINVAL_DTYPE = -3,   /* unsupported dtype or dtype combination */
  MOE_EINVAL_ALIGN = -4,   /* a pointer or pitch is not 16-byte aligned */
  MOE_EINVAL_SHAPE = -5,   /* H or I is not a multiple of the required granule */
  MOE_EWORKSPACE = -6,     /* workspace pointer missing or too small */
  MOE_ELAUNCH = -7,        /* the HIP runtime refused a kernel launch */
  MOE_ESCRATCH = -8        /* more work than the library's static scratch holds */
} moe_status;

/* Device error flags (bits OR-ed into *err). */
#define MOE_ERR_SLOT_RANGE      (1u << 0) /* pair's pool slot outside [0, P) */
#define MOE_ERR_EXPERT_NONLOCAL (1u << 1) /* pair's expert outside [expert_base, +E_loc) */
#define MOE_ERR_TOKEN_RANGE     (1u << 2) /* arrival's token outside [0, T_cap) */
#define MOE_ERR_KSLOT_RANGE     (1u << 3) /* arrival's top-k position outside [0, K) */
#define MOE_ERR_ROW_RANGE       (1u << 4) /* arrival's row index outside [0, n_rows) */
#define MOE_ERR_STALE_GEN       (1u << 5) /* arrival's generation != token's current one */
#define MOE_ERR_DUPLICATE       (1u << 6) /* token already holds a result for that position */

/* ------------------------------------------------------------------ moe_assemble --
 * Builds the contiguous batch of one expert micro-queue ([SEP] section 3: the receptor
 * puts each token vector into the pool; the metadata names request, layer, expert and
 * top-k weight; the executor turns the queue's scattered inputs into one contiguous
 * batch).  The queue is the array order of the n pairs.
 *
 * Output rows are grouped by local expert (ascending) and, inside an expert, kept in
 * queue order:
 *   counts[e]   = number of accepted pairs of local expert e           (int32 [E_loc])
 *   offsets[e]  = sum of counts[0..e-1]; offsets[E_loc] = accepted pairs (int32 [E_loc+1])
 *   perm[r]     = queue index of the pair at batch row r; -1 for r >= offsets[E_loc] (int32 [n])
 *   pos[i]      = batch row of queue entry i, or -1 if it was rejected (int32 [n]; may be NULL)
 *   xb[r][:]    = byte copy of pool row slot[perm[r]]                  ([n][H] act_dtype, pitch H)
 * xb may be NULL: then no rows are copied and moe_expert_ffn_grouped reads them from the
 * pool itself (gather-on-load, see moe_ffn_args.perm).
 * A pair is rejected (no row, flag raised) if slot is outside [0, P) or
 * expert - expert_base is outside [0, E_loc).
 * Limits: 0 <= n <= 2^24, 1 <= E_loc <= 256, act_dtype F32 or BF16, H * element size a
 * multiple of 16 bytes, pool and xb 16-byte aligned, pool_pitch (elements) >= H with
 * pool_pitch * element size a multiple of 16. */
typedef struct moe_assemble_args {
  int32_t n;               /* pairs in the queue */
  const int32_t* slot;     /* [n] pool slot of the pair's token vector */
  const int32_t* expert;   /* [n] global expert id */
  int32_t expert_base;     /* first global expert id held by this rank */
  int32_t E_loc;           /* experts held by this rank */
  const void* pool;        /* [P][pool_pitch] token pool */
  int64_t P;               /* pool slots */
  int64_t pool_pitch;      /* elements between consecutive pool rows */
  int32_t H;               /* hidden size (elements per row) */
  int32_t act_dtype;       /* MOE_F32 or MOE_BF16 */
  int32_t* perm;           /* out [n] */
  int32_t* pos;            /* out [n], optional */
  int32_t* counts;         /* out [E_loc] */
  int32_t* offsets;        /* out [E_loc + 1] */
  void* xb;                /* out [n][H], optional */
  uint32_t* err;           /* device error word (OR-ed) */
  int32_t* row_slot;       /* out [n], optional: pool slot of batch row r (slot[perm[r]]), -1 past the
                              accepted pairs; the FFN's gather-on-load reads it in one step */
} moe_assemble_args;

int moe_assemble(const moe_assemble_args* args, hipStream_t stream);

/* ---------------------------------------------------------- weight packing (setup) --
 * The FFN reads weights in a tile-major "packed" layout so that every 64-lane load of a
 * weight tile is one contiguous 1 KiB run.  The layout, for one matrix M[N][Kd] (N output
 * rows, Kd contraction length; N % 16 == 0, Kd % 64 == 0):
 *   block (nb, kb) = rows 16nb..16nb+15, columns 64kb..64kb+63, stored at block index
 *   nb * (Kd / 64) + kb, 1024 elements per block.  Element (r, c) of a block, with
 *   g = c / 16, h = (c / 8) % 2, q = c % 8, lane = 16 g + r, sits at
 *     bf16, f32 :  h * 512 + lane * 8 + q
 *     fp8       :  lane * 16 + h * 8 + q
 * The gate/up matrix of expert e is the 2I x H matrix whose packed row strip s (16 rows)
 * holds gate rows 16(s/2).. if s is even and up rows 16(s/2).. if s is odd.  The down
 * matrix is Wd[e] (H x I).  Experts follow each other (expert stride = matrix size).
 * Inputs are the usual row-major, output-major arrays; fp8 row scales are not packed. */
typedef struct moe_pack_args {
  int32_t E_loc, H, I;
  int32_t w_dtype;         /* MOE_F32, MOE_BF16 or MOE_FP8_E4M3 */
  const void* wg;          /* [E_loc][I][H] gate weights */
  const void* wu;          /* [E_loc][I][H] up weights */
  const void* wd;          /* [E_loc][H][I] down weights */
  void* w_gu;              /* out: packed gate/up, E_loc * 2I * H elements */
  void* w_d;               /* out: packed down, E_loc * H * I elements */
} moe_pack_args;

int moe_pack_ffn_weights(const moe_pack_args* args, hipStream_t stream);

/* ---------------------------------------------------------- moe_expert_ffn_grouped --
 * For each local expert e and each batch row r in [offsets[e], offsets[e+1]):
 *   g = Wg_e x_r,  u = Wu_e x_r,  h = silu(g) * u  (silu(z) = z / (1 + exp(-z))),
 *   y_r = Wd_e h.
 * The pages name "the expert computation" on the assembled batch ([SEP] section 3) but not
 * its form; a bias-free SwiGLU is used.  Accumulation is fp32; h is stored in act_dtype
 * in the workspace; y is stored in act_dtype.  offsets is read on the device (it may come
 * straight from moe_assemble); n is only an upper bound on offsets[E_loc].
 * Supported (act, weight) pairs: (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).  For fp8 the
 * three scale arrays are required: s_gate, s_up [E_loc][I], s_down [E_loc][H].
 * Limits: 1 <= E_loc <= 256, H % 64 == 0, I % 64 == 0, 0 <= n <= 2^24; 16-byte aligned
 * buffers.  The workspace must hold moe_ffn_workspace_size(...) bytes: h ([n][I] in
 * act_dtype, rounded up to 256 bytes) and, for batches that can take the tiled path for
 * many rows per expert (bf16 activations, n_max >= 96 E_loc), 64 MiB of fp32 partial tiles
 * for the k-split of each XCD's last partial round of work units.  With a workspace sized
 * for h alone the call still runs, with those units computed whole (same values up to
 * rounding order).  Results are deterministic for a given device and workspace size.
 * ev_mid: optional hipEvent_t recorded on the stream between the gate/up kernel and
 * the down kernel (for timing); pass NULL otherwise.
 * ev_gu_start, ev_gu_stop: optional hipEvent_t pair (both or neither) that the gate/up
 * projection's own dispatches record: at the start of its kernel and at the end of its last
 * launch (the tiled GEMM path's finalize, when it runs one), so that hipEventElapsedTime
 * gives the projection's kernel time alone (for roofline figures); not recorded by the fp32
 * kernels.
 *
 * Gather-on-load ([SEP] section 6 fuses the gather of scattered token vectors into the
 * computation that consumes them): when perm != NULL the gate/up projection reads batch
 * row r straight from the token pool, row slot[perm[r]] (P rows, pitch pool_pitch
 * elements), and xb is not read (it may be NULL).  perm and slot are those of the
 * moe_assemble call for the same queue (which may then skip its copy, xb = NULL); a slot
 * outside [0, P) is clamped into range (moe_assemble gives such pairs no batch row).
 * With row_slot != NULL (moe_assemble's row_slot output) batch row r is pool row
 * row_slot[r]: the same rows, one dependent load fewer; perm and slot are then not read.
 * The pool must be 16-byte aligned with pool_pitch * element size a multiple of 16, and
 * for bf16 activations P * pool_pitch * 2 < 2^31 (MOE_EINVAL_SIZE otherwise).
 *
 * plan: optional (NULL: none).  The arguments of a moe_combine_plan call to enqueue with
 * this FFN; the call then does the work of moe_combine_plan(plan, stream) as well, with the
 * same results and validation (an invalid plan returns its error and enqueues nothing).
 * For an arrival list of at most 256 entries taking the plan path, on batches that take
 * the weight-streaming kernels (bf16 activations, fewer than 96 E_loc rows), the plan runs
 * in one extra workgroup of the gate/up launch, beside the FFN's work units (a decode-sized
 * batch leaves compute units free), so it costs no launch and no time of its own;
 * otherwise it is launched on the stream before the FFN.  Either way it reads only the
 * arrival metadata (including row_idx, so moe_assemble's pos must already be enqueued) and
 * the token state, and it is complete when the down projection starts; follow it with
 * moe_combine_apply(plan, ...) ordered after this call.
 *
 * index: optional (NULL: none).  The arguments of a moe_assemble call for this batch (index
 * only: its xb must be NULL; n, E_loc, H and act_dtype equal to this call's, MOE_EINVAL_SIZE
 * otherwise); the call then does that moe_assemble's work as well, with the same outputs and
 * validation (invalid index arguments return moe_assemble's status and enqueue nothing).
 * offsets, perm, slot, pool, P, pool_pitch and row_slot of this struct are then ignored: the
 * FFN uses the index's offsets and gathers batch rows from its pool (the ABI's
 * gather-on-load above, through its row_slot when given).  For queues of at most 256 pairs on
 * the weight-streaming path (bf16 activations, fewer than 96 E_loc rows) every gate/up
 * workgroup derives the index itself from slot and expert, in its local memory, before its
 * work units, and one extra workgroup writes the moe_assemble outputs (perm, pos, counts,
 * offsets, row_slot, err), so the index costs no launch of its own ([SEP] section 6 counts the
 * regrouping among the costs that asynchrony adds); a plan given with it then runs in that
 * workgroup on the batch rows it derived (or, when the plan cannot join the launch, is
 * launched right after the gate/up kernel, as it reads pos).  Otherwise moe_assemble is
 * launched on the stream before the FFN.  When that queue is longer than 1024 pairs and a plan
 * for the same batch is given (its row_idx is the index's pos and its m the queue length, so the
 * combine takes its linked-list path), the same launch also does the plan's link step (range
 * and generation checks, then each arrival pushed onto its token's list once its batch row is
 * known), with the same results, and the apply then runs only the merge and the release.
 * Either way the outputs are complete when the down projection starts. */
struct moe_combine_args;
typedef struct moe_ffn_args {
  int32_t n, E_loc, H, I;
  int32_t act_dtype, w_dtype;
  const void* xb;          /* [n][H] batch rows */
  const int32_t* offsets;  /* [E_loc + 1] device */
  const void* w_gu;        /* packed gate/up */
  const void* w_d;         /* packed down */
  const float* s_gate;     /* fp8 only */
  const float* s_up;       /* fp8 only */
  const float* s_down;     /* fp8 only */
  void* y;                 /* out [n][H] */
  void* workspace;
  size_t workspace_bytes;
  hipEvent_t ev_mid;       /* optional */
  const int32_t* perm;     /* optional gather-on-load: [n] batch row -> queue index */
  const int32_t* slot;     /* [n_queue] pool slot of each queue entry */
  const void* pool;        /* [P][pool_pitch] token pool (act_dtype) */
  int64_t P;               /* pool rows */
  int64_t pool_pitch;      /* elements between pool rows */
  const int32_t* row_slot; /* optional gather-on-load index: pool row of batch row r (moe_assemble's
                              row_slot); when set it replaces perm and slot (which may be NULL) */
  const struct moe_combine_args* plan; /* optional combine plan to run with the FFN (above) */
  hipEvent_t ev_gu_start;  /* optional, with ev_gu_stop: gate/up kernel duration (above) */
  hipEvent_t ev_gu_stop;
  const struct moe_assemble_args* index; /* optional queue index to derive with the FFN (above) */
} moe_ffn_args;

size_t moe_ffn_workspace_size(int32_t n_max, int32_t E_loc, int32_t H, int32_t I, int32_t act_dtype);
int moe_expert_ffn_grouped(const moe_ffn_args* args, hipStream_t stream);

/* ------------------------------------------------------------- moe_combine_release --
 * Per-token combine state of the home rank (all device memory, caller-owned):
 *   acc[t][H]  fp32 running sum of the accepted w_j * E_j(x); meaningful only while
 *              mask[t] != 0 (a token with no held result starts from zero)
 *   mask[t]    bit j set once the result for top-k position j was accepted
 *   tgen[t]    generation that the token's next results must carry
 *   head[t]    internal (arrival list of the running call), -1 between calls
 *   rflag[]    internal release flags, one byte per token, (T_cap + 15) / 16 * 16 bytes,
 *              16-byte aligned, all zero between calls
 * moe_state_reset() puts every token in generation `gen0` with nothing accepted. */
typedef struct moe_combine_state {
  float* acc;
  uint32_t* mask;
  int32_t* head;
  uint32_t* tgen;
  uint8_t* rflag;
  int32_t T_cap;           /* tokens the state can hold */
  int32_t H;
} moe_combine_state;

int moe_state_reset(const moe_combine_state* st, uint32_t gen0, hipStream_t stream);

/* Accepts m arriving expert results and releases every token that became complete.
 * ([SEP] section 3: a token's K results come back separately; the first K-1 are buffered
 * and the K-th makes it eligible for the next layer; combine is y = sum_j w_j E_j(x).
 * [SEP] section 6: the gather of scattered result rows is fused with the weighted merge.
 * [NOTES] obligations: each selected contribution is accepted once, with its own weight,
 * tagged by generation; weights are not renormalised.)
 * Arrival i carries row rows[row_idx[i]] (pitch row_pitch elements) as the result of
 * top-k position kslot[i] for token tok[i] in generation gen[i], with router weight w[i].
 * It is rejected (flag raised, no effect) if tok, kslot or row_idx is out of range, if
 * gen[i] != tgen[tok[i]], or if the token already holds position kslot[i] (from an earlier
 * call, or from an arrival of the same call with a lower index: the lowest index wins).
 * After the call every token holding all K positions is released:
 *   out[t][:]   = round-to-nearest-even(acc_t) in out_dtype, where acc_t is the fp32 sum
 *                 of the held partial sum and this call's w_a * row_a in arrival-index order
 *                 (the same inputs give the same bits)
 *   rel_list    = released tokens in ascending order, *rel_count of them (device int32)
 *   state       : mask[t] = 0, tgen[t] += 1
 * Tokens still missing results keep their partial sums.  The per-token arrival count of a
 * token still waiting is popcount(mask[t]) (the results it holds, each position once); the
 * mask is that count's output, finer than a count since it also names the positions held.
 * Limits: 1 <= K <= 32, 0 <= m <= 2^24, H % 8 == 0, rows/out dtypes F32 or BF16,
 * rel_list holds at least min(m, T_cap) entries; the workspace (device memory, 16-byte
 * aligned) holds moe_combine_workspace_size(m) bytes (16 + 24 m, rounded up to 16).
 * Calls of at most 1024 arrivals on a state of fewer than 2^20 tokens are planned by
 * one workgroup (sort by token and arrival index, then one workgroup per token); others
 * link per-token arrival lists.  Both give the same bits. */
typedef struct moe_combine_args {
  int32_t m;               /* arrivals */
  int32_t K;               /* results per token (top-k) */
  const void* rows;        /* row source (e.g. the FFN output y) */
  int32_t row_dtype;       /* MOE_F32 or MOE_BF16 */
  int64_t row_pitch;       /* elements between rows */
  int64_t n_rows;          /* rows available in `rows` */
  const int32_t* row_idx;  /* [m] */
  const int32_t* tok;      /* [m] */
  const int32_t* kslot;    /* [m] */
  const float* w;          /* [m] */
  const uint32_t* gen;     /* [m] */
  moe_combine_state state;
  void* out;               /* [T_cap][out_pitch] released rows */
  int32_t out_dtype;       /* MOE_F32 or MOE_BF16 */
  int64_t out_pitch;       /* elements */
  int32_t* rel_list;       /* out */
  int32_t* rel_count;      /* out, device int32 */
  uint32_t* err;           /* device error word (OR-ed) */
  void* workspace;         /* scratch for the call */
  size_t workspace_bytes;
} moe_combine_args;

size_t moe_combine_workspace_size(int32_t m_max);

int moe_combine_release(const moe_combine_args* args, hipStream_t stream);

/* moe_combine_release in two halves, for a caller that overlaps the first with other work
 * on another stream (the arrivals of an expert step are known before its FFN runs):
 *   moe_combine_plan   reads the arrival metadata and the token state only (validation,
 *                      per-token acceptance, state update, release list);
 *   moe_combine_apply  reads the result rows and writes the combined rows.
 * Call both with the same arguments, apply ordered after plan (same stream, or an event),
 * and change neither the arguments, the state nor the workspace in between; rel_list,
 * rel_count and err are final only after apply.  moe_combine_release(args, s) is
 * moe_combine_plan(args, s) followed by moe_combine_apply(args, s).  Both validate the
 * arguments as moe_combine_release does. */
int moe_combine_plan(const moe_combine_args* args, hipStream_t stream);
int moe_combine_apply(const moe_combine_args* args, hipStream_t stream);

/* moe_combine_release for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the same work and results bit
 * for bit, but the call's scratch lives in a device array owned by the library instead of
 * args->workspace (workspace and workspace_bytes are ignored and may be NULL / 0).  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   - Limit: at most moe_combine_noalloc_max_arrivals() arrivals (2^17) per call; a larger
 *     m returns MOE_ESCRATCH and enqueues nothing.  Other arguments are validated as by
 *     moe_combine_release.
 *   - Each GPU the library runs on holds one copy of the array (about 3 MiB) until the
 *     process ends; its address is looked up once per device, on the first call made with
 *     that device current (a failure returns MOE_ELAUNCH).
 *   - Every call on one GPU shares that GPU's array, and the array keeps the last call's
 *     contents (nothing in it needs clearing: a call reads only what it wrote earlier).
 *     Calls that overlap on one GPU (on different streams, or from several host threads
 *     without ordering) race on it; order them on one stream or with events. */
int moe_combine_release_noalloc(const moe_combine_args* args, hipStream_t stream);
size_t moe_combine_noalloc_max_arrivals(void);

/* ---------------------------------------------------------------------- helpers -- */
const char* moe_strerror(int status);
int moe_version(void);
/* sizeof of the argument structs as compiled into the library (which: 0 assemble,
 * 1 pack, 2 ffn, 3 combine state, 4 combine args), so that bindings can check their
 * own struct layout; 0 for an unknown id. */
size_t moe_struct_size(int which);

#ifdef __cplusplus
}
#endif

#endif /* MOE_STEP_H */
