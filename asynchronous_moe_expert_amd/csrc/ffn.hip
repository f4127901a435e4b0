// moe_expert_ffn_grouped: per-expert SwiGLU FFN over ragged, expert-grouped batch rows.
//
// What is computed ([SEP] section 3, "run the expert computation on the assembled batch";
// the pages leave the FFN form open, a bias-free SwiGLU is used):
//     y_r = Wd_e ( silu(Wg_e x_r) * (Wu_e x_r) )   for rows r of expert e
//
// Design (gfx950):
//   * Two launches: gate/up GEMM with the SwiGLU epilogue (writes h), then the down GEMM.
//   * Decode-sized batches (streaming kernel below): work unit = (row chunk of <= 48 rows of
//     one expert, WV waves x NS weight strips of 16 output columns).  Prefill-sized batches
//     (>= 96 rows per expert on average; the fp8 down projection from 48) take a tiled GEMM
//     further down: units of 256 rows x 256 columns, one workgroup per CU, for fp8 weights;
//     128-row chunks x 256 columns for bf16 weights.  The chunk list is derived on the device
//     from `offsets`, so ragged and empty experts need no host round trip.  The streaming
//     kernel's grid is what the device holds at once (CUs x occupancy) and strides over the
//     active units only: a decode batch's units all start in the first round and no
//     workgroup slot is spent on an idle unit.
//   * At decode sizes (tens of rows per expert) the step is bound by streaming the expert
//     weights once from HBM.  Each wave owns its strips over the whole contraction and
//     keeps R-1 k-steps of weight loads in flight in a register ring (packed layout: one
//     contiguous 1 KiB run per wave load); there is no split-k reduction.  The activation
//     k-tile is loaded once per workgroup, a quarter per wave issued together with the
//     weights of the same k-step (loads retire in order, so a shallower activation ring
//     would drain the weight ring), and shared through a double-buffered LDS tile whose
//     layout is the MFMA operand order (conflict-free 16-byte reads).
//   * MFMA v_mfma_f32_16x16x32_bf16 does the math.  The contraction order inside a 64-wide
//     k-step is permuted (lane group g takes 16 consecutive k, split over two MFMAs); the
//     packed weight layout and the activation tile apply the same permutation, so the
//     sums are exact dot products over all k.
//   * fp8 e4m3 weights are widened to bf16 in registers (exact: every e4m3 value is a
//     bf16 value) and the per-row scale is applied to the fp32 result in the epilogue.
//   * Units are spread XCD-aware: each XCD gets an equal contiguous range of unit ids,
//     numbered chunk-major, so a chunk's column blocks run on one XCD and read its rows
//     through that XCD's L2.
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "combine_plan.hpp"
#include "common.hpp"

namespace moe {

constexpr int kBK = 64;        // contraction per k-step
#ifndef MOE_FFN_STAGES
#define MOE_FFN_STAGES 2
#endif
constexpr int kStages = MOE_FFN_STAGES;  // register-ring depth of the weight/activation stream

// ------------------------------------------------------------------------- packing
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T* __restrict__ src, T* __restrict__ dst, int E, int rows,
                                                   int cols, int mode, int64_t dst_stride) {
  const int64_t per = (int64_t)rows * cols;
  const int64_t total = per * E;
  const int esz = (int)sizeof(T);
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t e = idx / per;
    const int64_t rem = idx - e * per;
    const int64_t row = rem / cols;
    const int64_t col = rem - row * cols;
    const int64_t prow = mode == 0 ? row : gu_packed_row(row, mode == 2);
    dst[e * dst_stride + packed_index(prow, col, cols, esz)] = src[idx];
  }
}

// ------------------------------------------------------------- gather-on-load rows
// Where batch row r's activations live.  Without a gather (perm == nullptr) they are row r
// of the batch matrix A ([n][Kd]).  With one, A is the token pool and row r is pool row
// row_slot[r] when that index is given, else slot[perm[r]] (clamped into [0, P): a pair
// moe_assemble rejected has no batch row, so the clamps only guard against inconsistent
// inputs), pitch `pitch` elements.  perm marks the gather; with row_slot it is not read.
struct GatherRows {
  const int32_t* perm;
  const int32_t* slot;
  int64_t pitch;
  int64_t P;
  const int32_t* row_slot;
  __device__ __forceinline__ int64_t row_offset(int r, int Kd) const {
    if (perm == nullptr) return (int64_t)r * Kd;
    int64_t s;
    if (row_slot != nullptr) {
      s = row_slot[r];
    } else {
      const int q = perm[r];
      s = slot[q < 0 ? 0 : q];
    }
    s = s < 0 ? 0 : (s >= P ? P - 1 : s);
    return s * pitch;
  }
  // row_offset of N rows at once: every row's index load is issued before the first is used
  // (one at a time, each row's lookup waited for the one before: up to 2N load latencies
  // between two units of a GEMM instead of two)
  template <int N>
  __device__ __forceinline__ void row_offsets(const int (&r)[N], int Kd, int64_t (&off)[N]) const {
    if (perm == nullptr) {
#pragma unroll
      for (int i = 0; i < N; ++i) off[i] = (int64_t)r[i] * Kd;
      return;
    }
    int s[N];
    if (row_slot != nullptr) {
#pragma unroll
      for (int i = 0; i < N; ++i) s[i] = row_slot[r[i]];
    } else {
      int q[N];
#pragma unroll
      for (int i = 0; i < N; ++i) q[i] = perm[r[i]];
#pragma unroll
      for (int i = 0; i < N; ++i) s[i] = slot[q[i] < 0 ? 0 : q[i]];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int64_t c = s[i] < 0 ? 0 : (s[i] >= P ? P - 1 : (int64_t)s[i]);
      off[i] = c * pitch;
    }
  }
};

// The queue index of a moe_assemble call (index only) derived inside the gate/up launch of a
// decode-sized batch (at most kQueueFusedMax pairs): every workgroup computes it in LDS from
// the raw slot and expert ids of the queue, and one extra workgroup writes the call's outputs.
constexpr int kQueueFusedMax = 256;
constexpr int kQueueMaxE = 256;
struct QueueIdx {
  const int32_t* slot;    // nullptr: no fused index
  const int32_t* expert;
  int base;
  int n;
  int64_t P;
  int32_t* perm;
  int32_t* pos;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_slot;
  uint32_t* err;
};

// [SEP] (marsggbo, "SOSP'26 | StreamEP") section 3: the scattered ready inputs of the queue
// become one batch grouped by expert.  The same stable order as the index kernels of
// moe_assemble: per-expert counts, exclusive offsets, and within an expert queue order (a
// 9-bit ballot match ranks a pair among equal keys of lower lanes; the per-wave counts are
// scanned across the waves).  Pairs live in threads 0..n-1 (n <= 256: waves 0..3).  Outputs
// in LDS: s_off [E_loc + 1], s_rs (pool slot of each batch row), s_pos (batch row of each
// queue entry, -1 for a rejected one); with `writer`, the moe_assemble outputs as well.  Every
// thread of the workgroup calls it (it has workgroup barriers).
template <int NT>
__device__ __forceinline__ void queue_index_lds(const QueueIdx& q, int E_loc, int* s_off, int* s_rs, int* s_pos,
                                                int (*s_wc)[kQueueMaxE + 1], unsigned* s_err, bool writer) {
  static_assert(NT >= kQueueFusedMax, "one pair per thread");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = q.n;
  for (int x = tid; x < 4 * E_loc; x += NT) s_wc[x / E_loc][x % E_loc] = 0;
  if (tid == 0) *s_err = 0u;
  int key = kQueueMaxE, sv = 0;
  unsigned bad = 0u;
  if (tid < n) {
    sv = q.slot[tid];
    const int e = q.expert[tid] - q.base;
    bool ok = true;
    if (sv < 0 || (int64_t)sv >= q.P) { bad |= MOE_ERR_SLOT_RANGE; ok = false; }
    if (e < 0 || e >= E_loc) { bad |= MOE_ERR_EXPERT_NONLOCAL; ok = false; }
    if (ok) key = e;
  }
  __syncthreads();
  uint64_t peers = ~0ull;
#pragma unroll
  for (int b = 0; b < 9; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  const int rank = __popcll(peers & ((1ull << lane) - 1ull));
  if (key < kQueueMaxE && rank == 0) s_wc[wv][key] = __popcll(peers);  // (key < 256 only on waves 0..3)
  if (bad) atomicOr(s_err, bad);
  __syncthreads();
  if (wv == 0) {  // exclusive scan over the experts (4 per lane), then each wave's first row per expert
    int c[4][4], v[4], sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = lane * 4 + k;
      v[k] = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        c[k][w] = e < E_loc ? s_wc[w][e] : 0;
        v[k] += c[k][w];
      }
      sum += v[k];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    int run = incl - sum;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = lane * 4 + k;
      if (e < E_loc) {
        s_off[e] = run;
        if (writer) {
          q.counts[e] = v[k];
          q.offsets[e] = run;
        }
        int r = run;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          s_wc[w][e] = r;
          r += c[k][w];
        }
      }
      run += v[k];
    }
    if (lane == 63) {
      s_off[E_loc] = incl;
      if (writer) q.offsets[E_loc] = incl;
    }
  }
  __syncthreads();
  if (key < kQueueMaxE) {
    const int r = s_wc[wv][key] + rank;
    s_rs[r] = sv;
    s_pos[tid] = r;
    if (writer) {
      q.perm[r] = tid;
      if (q.pos) q.pos[tid] = r;
      if (q.row_slot) q.row_slot[r] = sv;
    }
  } else if (tid < n) {
    s_pos[tid] = -1;
    if (writer && q.pos) q.pos[tid] = -1;
  }
  if (writer) {
    const int total = s_off[E_loc];
    if (tid < n && tid >= total) {  // batch rows past the accepted pairs
      q.perm[tid] = -1;
      if (q.row_slot) q.row_slot[tid] = -1;
    }
    if (tid == 0 && *s_err) atomicOr(q.err, *s_err);
  }
  __syncthreads();
}

// --------------------------------------------------------------- expert lookup helpers
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int E_loc, int r) {
  for (int e = 0; e < E_loc; ++e)
    if (r >= offsets[e] && r < offsets[e + 1]) return e;
  return -1;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }
// the same with a hardware reciprocal (about 1 ulp), for results rounded to bf16
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ------------------------------------------------------------------------- fp32 path
// Small-shape path (fp32 activations and weights): one thread per output element.
__global__ __launch_bounds__(256) void gateup_f32_kernel(const float* __restrict__ xb, const int32_t* __restrict__ offsets,
                                                         int E_loc, int n, int H, int I, const float* __restrict__ wgu,
                                                         float* __restrict__ h, GatherRows gr) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int r = (int)(idx / I), i = (int)(idx - (int64_t)r * I);
  if (r >= n || r >= offsets[E_loc]) return;
  const int e = expert_of_row(offsets, E_loc, r);
  if (e < 0) return;
  const float* w = wgu + (int64_t)e * 2 * I * H;
  const int64_t rg = gu_packed_row(i, false), ru = gu_packed_row(i, true);
  const float* xr = xb + gr.row_offset(r, H);
  float g = 0.f, u = 0.f;
  for (int k = 0; k < H; ++k) {
    const float x = xr[k];
    g = fmaf(x, w[packed_index(rg, k, H, 4)], g);
    u = fmaf(x, w[packed_index(ru, k, H, 4)], u);
  }
  h[(int64_t)r * I + i] = silu_mul(g, u);
}

__global__ __launch_bounds__(256) void down_f32_kernel(const float* __restrict__ h, const int32_t* __restrict__ offsets,
                                                       int E_loc, int n, int H, int I, const float* __restrict__ wd,
                                                       float* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int r = (int)(idx / H), o = (int)(idx - (int64_t)r * H);
  if (r >= n || r >= offsets[E_loc]) return;
  const int e = expert_of_row(offsets, E_loc, r);
  if (e < 0) return;
  const float* w = wd + (int64_t)e * H * I;
  float acc = 0.f;
  for (int i = 0; i < I; ++i) acc = fmaf(h[(int64_t)r * I + i], w[packed_index(o, i, I, 4)], acc);
  y[(int64_t)r * H + o] = acc;
}

// -------------------------------------------------------------- bf16 / fp8 MFMA path
// Widen 8 e4m3 codes (two dwords) to 8 bf16 values (exact: every e4m3 value is a bf16
// value); one v_cvt_scalef32_pk_bf16_fp8 per pair of codes, scale 1.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 16-byte weight load; NT marks it non-temporal (for weights read once per launch, so that
// they neither displace reused lines nor wait for allocation in the caches)
template <bool NT>
__device__ __forceinline__ uint4 wload(const uint4* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

template <int WDT, int NS>
struct WTile;  // one k-step of NS weight strips, as loaded (16 bytes per lane per run)

template <int NS>
struct WTile<MOE_BF16, NS> {
  uint4 raw[NS][2];
  template <bool NT>
  __device__ __forceinline__ void load(const char* __restrict__ p, int64_t strip_stride) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      raw[s][0] = wload<NT>(reinterpret_cast<const uint4*>(p + s * strip_stride));
      raw[s][1] = wload<NT>(reinterpret_cast<const uint4*>(p + s * strip_stride + 1024));
    }
  }
  __device__ __forceinline__ bf16x8 frag(int s, int h) const {
    bf16x8 r;
    __builtin_memcpy(&r, &raw[s][h], 16);
    return r;
  }
};

template <int NS>
struct WTile<MOE_FP8_E4M3, NS> {
  uint4 raw[NS];
  template <bool NT>
  __device__ __forceinline__ void load(const char* __restrict__ p, int64_t strip_stride) {
#pragma unroll
    for (int s = 0; s < NS; ++s) raw[s] = wload<NT>(reinterpret_cast<const uint4*>(p + s * strip_stride));
  }
  __device__ __forceinline__ bf16x8 frag(int s, int h) const {
    return h == 0 ? e4m3x8_to_bf16(raw[s].x, raw[s].y) : e4m3x8_to_bf16(raw[s].z, raw[s].w);
  }
};

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// This thread's share of one k-step activation tile (MT*16 rows x 64 k) staged through LDS.
// Tile piece t (16 bytes) is the MFMA A-operand run of lane t%64 for row tile t/128 and
// k-half (t/64)%2, so piece t sits at LDS byte 16t and a lane's operand read is one
// conflict-free 16-byte access at 16*((2mt + h)*64 + lane).
template <int MT, int NT>
struct APart {
  static constexpr int kPieces = MT * 128;
  static constexpr int J = (kPieces + NT - 1) / NT;  // pieces per thread (NT threads)
  u32x4 raw[J];
  __device__ __forceinline__ void load(const uint16_t* const* ap, int k0) {
    static_for<J>([&](auto j) { raw[j()] = *reinterpret_cast<const u32x4*>(ap[j()] + k0); });
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
    static_for<J>([&](auto j) {
      if (j() * NT + tid < kPieces) lds[j() * NT + tid] = raw[j()];
    });
  }
};

// Active work units of a ragged batch, found on the device from `offsets` (no host round
// trip).  A unit is (column block nb, row chunk c) where the chunks are the BM-row pieces of
// the non-empty expert groups, numbered in expert order; units are ordered nb-major, so the
// chunks that share a weight tile are neighbours.  Every wave of a workgroup builds the same
// table: lane j covers experts j, j+64, j+128, j+192.
struct ChunkTable {
  int a0[4], a1[4], start[4], nc[4];
  int total;  // number of row chunks (wave-uniform)

  __device__ __forceinline__ void build(const int32_t* __restrict__ offsets, int E_loc, int n_rows, int BM, int lane) {
    int base = 0;
    static_for<4>([&](auto jc) {
      constexpr int j = jc();
      a0[j] = a1[j] = nc[j] = 0;
      start[j] = base;
      if (j > 0 && 64 * j >= E_loc) return;  // (no expert in this group of 64)
      const int e = lane + 64 * j;
      int lo = 0, hi = 0;
      if (e < E_loc) {
        // clamp to [0, n_rows] so that inconsistent offsets can never address past the batch
        lo = min(max(offsets[e], 0), n_rows);
        hi = min(max(offsets[e + 1], lo), n_rows);
      }
      a0[j] = lo;
      a1[j] = hi;
      nc[j] = (hi - lo + BM - 1) / BM;
      int incl = nc[j];  // inclusive scan over the wave
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
      }
      start[j] = base + incl - nc[j];
      base += __shfl(incl, 63, 64);
    });
    total = __builtin_amdgcn_readfirstlane(base);
  }

  // expert, first row and end row of chunk c (0 <= c < total; e = -1 otherwise), and the
  // number of chunks of that expert
  __device__ __forceinline__ void find(int c, int BM, int& e, int& m0, int& mend, int& nce) const {
    e = -1;
    m0 = mend = nce = 0;
    static_for<4>([&](auto jc) {
      constexpr int j = jc();
      const uint64_t hit = __ballot(c >= start[j] && c < start[j] + nc[j]);
      if (hit && e < 0) {
        const int l = __builtin_ctzll(hit);
        e = l + 64 * j;
        m0 = __shfl(a0[j], l, 64) + (c - __shfl(start[j], l, 64)) * BM;
        mend = min(__shfl(a1[j], l, 64), m0 + BM);
        nce = __shfl(nc[j], l, 64);
      }
    });
  }
  __device__ __forceinline__ void find(int c, int BM, int& e, int& m0, int& mend) const {
    int nce;
    find(c, BM, e, m0, mend, nce);
  }
};

__device__ __forceinline__ void wg_barrier() {
  // LDS writes of every wave are complete and visible; global loads stay in flight
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

constexpr int kFfnWaves = 4;

// expert (or -1), column block and rows of unit u of the batch, when u < u_end.  Units are
// numbered chunk-major (u = chunk * n_blocks_N + nb).
__device__ __forceinline__ int next_unit(const int32_t* __restrict__ offsets, int E_loc, int n_rows, int BM, int lane,
                                         int u, int u_end, int n_blocks_N, int& nb, int& m0, int& mend, int& nce) {
  int e = -1;
  if (u < u_end) {
    ChunkTable tab;
    tab.build(offsets, E_loc, n_rows, BM, lane);
    const int c = u / n_blocks_N;
    nb = u - c * n_blocks_N;
    tab.find(c, BM, e, m0, mend, nce);
  }
  return e;
}


// MODE 0: gate/up GEMM + SwiGLU epilogue -> h [n][I];  MODE 1: down GEMM -> y [n][H].
// A unit is MT*16 rows of one expert x 4*NS weight strips (16 output columns each).  Each
// of the 4 waves owns NS strips over the whole contraction and streams them from HBM into a
// ring of R register sets (R-1 k-steps in flight), so no split-k reduction is needed; the
// activation k-tile is loaded once per workgroup (a quarter per wave, issued with the
// weights of the same k-step) and shared through a double-buffered LDS tile.  The grid is
// at most what the device holds at once and strides over the units, so every unit of a
// decode-sized batch starts in the first round and no workgroup slot goes to an idle unit.
// FQ (gate/up only): the queue index is derived in the launch itself (queue_index_lds): every
// workgroup reads its chunk table and batch rows from its own LDS copy, and the last workgroup
// writes moe_assemble's outputs and then runs the combine plan, if any, on the batch rows it
// derived.
template <int MODE, int WDT, int NS, int MT, int R, int WV, bool FQ>
__global__ __launch_bounds__(64 * WV) void ffn_mfma_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets_g,
                                                    int E_loc, const char* __restrict__ W,
                                                    const float* __restrict__ s0, const float* __restrict__ s1,
                                                    uint16_t* __restrict__ out, int Kd, int Nw, int out_ld,
                                                    int n_blocks_N, int n_rows, GatherRows gr_g, PlanJob plan,
                                                    QueueIdx qi) {
  constexpr int BM = MT * 16;
  static_assert(MODE == 1 || NS % 2 == 0, "gate/up waves own (gate, up) strip pairs");
  using AP = APart<MT, 64 * WV>;
  __shared__ u32x4 a_lds[2][AP::kPieces];
  constexpr int esz = WDT == MOE_FP8_E4M3 ? 1 : 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KS = Kd / kBK;
  const int n_strips = Nw / 16;
  const int64_t blk_bytes = 1024 * esz;
  const int64_t strip_stride = (int64_t)KS * blk_bytes;

  // With a combine plan (gate/up only, m <= 256) or a fused queue index the grid has one
  // workgroup more than the FFN needs; that last workgroup runs the plan (and writes the
  // index) beside the units (a decode-sized batch has fewer units than compute units).
  const bool with_plan = MODE == 0 && plan.m > 0;
  const int32_t* offsets = offsets_g;
  GatherRows gr = gr_g;
  if constexpr (MODE == 0 && !FQ) {
    if (with_plan && (int)blockIdx.x == (int)gridDim.x - 1) {
      combine_plan_body<64 * WV>(plan);
      return;
    }
  }
  if constexpr (MODE == 0 && FQ) {
    __shared__ int s_qoff[kQueueMaxE + 1], s_qrs[kQueueFusedMax], s_qpos[kQueueFusedMax];
    __shared__ int s_qwc[4][kQueueMaxE + 1];
    __shared__ unsigned s_qerr;
    const bool writer = (int)blockIdx.x == (int)gridDim.x - 1;
    queue_index_lds<64 * WV>(qi, E_loc, s_qoff, s_qrs, s_qpos, s_qwc, &s_qerr, writer);
    if (writer) {
      if (with_plan) {
        PlanJob pj = plan;
        pj.row_idx = s_qpos;  // moe_assemble's pos, as derived here
        combine_plan_body<64 * WV>(pj);
      }
      return;
    }
    offsets = s_qoff;
    gr.perm = s_qrs;  // (batch row r reads pool row s_qrs[r])
    gr.row_slot = s_qrs;
  }

  // XCD-aware order: physical workgroup b runs on XCD b % 8.  Each XCD gets an equal,
  // contiguous range of unit ids, numbered chunk-major, and its G/8 workgroups stride through
  // that range: a chunk's column blocks share its activation rows in the XCD's L2.  (Numbered
  // column-block-major instead, so that an expert's chunks shared each weight strip, the
  // prefill wave of 1638 pairs ran its gate/up 10 us slower: the rows are re-read by every
  // column block, the strips only by a big expert's few chunks, and the strips of single-chunk
  // experts are loaded non-temporally.)  The chunk table is built once for the first unit and
  // again for each later one, so that it holds no registers across the contraction.
  const int G = (int)gridDim.x - (with_plan || FQ ? 1 : 0), b = blockIdx.x, xcd = b & 7;
  int total, u, u_end, nb = 0, e = -1, m0 = 0, mend = 0, nce = 0;
  {
    ChunkTable tab;
    tab.build(offsets, E_loc, n_rows, BM, lane);
    total = tab.total;
    const int U = total * n_blocks_N;
    u = (int)((int64_t)U * xcd / 8) + (b >> 3);
    u_end = (int)((int64_t)U * (xcd + 1) / 8);
    if (u < u_end) {
      const int c = u / n_blocks_N;
      nb = u - c * n_blocks_N;
      tab.find(c, BM, e, m0, mend, nce);
    }
  }
  for (; u < u_end;
       u += G >> 3, e = next_unit(offsets, E_loc, n_rows, BM, lane, u, u_end, n_blocks_N, nb, m0, mend, nce)) {
    if (e < 0) break;  // not reachable: the table is the same on every build
    const int strip0 = (nb * WV + wv) * NS;  // this wave's first strip
    const bool wact = strip0 < n_strips;            // (the last block may be partial)
    const char* wlane = W + (int64_t)e * Nw * Kd * esz + (int64_t)(wact ? strip0 : 0) * strip_stride + lane * 16;
    // activation pieces of this thread (rows past the chunk read a copy of its last row;
    // their results are never stored)
    const uint16_t* ap[AP::J];
#pragma unroll
    for (int j = 0; j < AP::J; ++j) {
      const int t = min(j * 64 * WV + tid, AP::kPieces - 1), l = t & 63;
      int r = m0 + (t >> 7) * 16 + (l & 15);
      r = r < mend ? r : mend - 1;
      ap[j] = A + gr.row_offset(r, Kd) + (l >> 4) * 16 + ((t >> 6) & 1) * 8;
    }

    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const WTile<WDT, NS>& wt, const u32x4* tile) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 bf[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) bf[s] = wt.frag(s, h);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const u32x4 araw = tile[(mt * 2 + h) * 64 + lane];
          bf16x8 af;
          __builtin_memcpy(&af, &araw, 16);
#pragma unroll
          for (int s = 0; s < NS; ++s)
            acc[mt][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[s], acc[mt][s], 0, 0, 0);
        }
      }
    };

    // k-step i: issue the loads of step i+R-1 (clamped to the last step: valid memory,
    // result unused), park this thread's activation piece of step i in LDS, barrier, MFMAs.
    // Ring slots are compile-time indices so that every slot lives in registers.  The whole
    // pipeline is instantiated for both weight-load policies: non-temporal when the unit's
    // expert is a single row chunk (its weight strips are read once in this launch), cached
    // otherwise (the expert's other chunks re-read them through L2).
    auto pipeline = [&](auto nt) {
      WTile<WDT, NS> wr[R];
      AP ar[R];
      // Every load is unconditional (an idle wave streams valid strip-0 weights and its
      // results are never stored): a load under a branch makes the compiler's wait counts
      // assume the branch was not taken, which drains the ring at every k-step.
      auto issue = [&](auto slot, int ks) {
        ks = min(ks, KS - 1);
        wr[slot()].template load<nt()>(wlane + ks * blk_bytes, strip_stride);
        ar[slot()].load(ap, ks * kBK);
      };
      auto step = [&](auto slot, int i) {
        ar[slot()].store(a_lds[i & 1], tid);
        wg_barrier();
        compute(wr[slot()], a_lds[i & 1]);
      };
      static_for<R - 1>([&](auto v) { issue(v, v()); });
      int it = 0;
#pragma clang loop unroll(disable)
      for (; it + R <= KS; it += R) {
        static_for<R>([&](auto v) {
          issue(std::integral_constant<int, (v() + R - 1) % R>{}, it + v() + R - 1);
          __builtin_amdgcn_sched_barrier(0);
          step(v, it + v());
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // the remaining KS - it < R steps sit in slots 0, 1, ...
      static_for<R - 1>([&](auto v) {
        if (it + v() < KS) step(v, it + v());
      });
    };
    if (nce == 1)
      pipeline(std::true_type{});
    else
      pipeline(std::false_type{});
    wg_barrier();  // the next unit's first LDS writes wait for this unit's last reads
    if (!wact) continue;

    // epilogue; the accumulator of lane l holds column l%16 of a strip and rows 4(l/16)+q
    const int col16 = lane & 15, rq = (lane >> 4) * 4;
    if (MODE == 0) {
      const int I = out_ld;
#pragma unroll
      for (int p = 0; p < NS / 2; ++p) {
        const int i = (strip0 / 2 + p) * 16 + col16;
        float sg = 1.f, su = 1.f;
        if (WDT == MOE_FP8_E4M3) {
          sg = s0[(int64_t)e * I + i];
          su = s1[(int64_t)e * I + i];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = m0 + mt * 16 + rq + q;
            if (row < mend) {
              const float g = acc[mt][2 * p][q] * sg, uu = acc[mt][2 * p + 1][q] * su;
              out[(int64_t)row * I + i] = f32_to_bf16(silu_mul_fast(g, uu));
            }
          }
        }
      }
    } else {
      const int H = out_ld;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int col = (strip0 + s) * 16 + col16;
        const float sc = WDT == MOE_FP8_E4M3 ? s0[(int64_t)e * H + col] : 1.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = m0 + mt * 16 + rq + q;
            if (row < mend) out[(int64_t)row * H + col] = f32_to_bf16(acc[mt][s][q] * sc);
          }
        }
      }
    }
  }
}

// Workgroups of one kernel that the device holds at once (its CU count times the kernel's
// occupancy), cached per device for each kernel (the template argument is the kernel).  The
// cache holds read-only device properties: concurrent first calls compute the same value and
// store it with an atomic.
template <auto Kernel>
static int resident_workgroups(int threads) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];  // 0 = not yet known
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = -1;
  if (dev >= 0) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess) cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Kernel, threads, 0) != hipSuccess) per_cu = 0;
  const int r = cus > 0 && per_cu > 0 ? cus * per_cu : 1024;
  if (dev >= 0) cache[dev].store(r, std::memory_order_relaxed);
  return r;
}

template <int MODE, int WDT, int NS, int MT, int R, int WV, bool FQ>
static void launch_mfma_t(const void* A, const int32_t* offsets, int E_loc, const void* W, const float* s0,
                          const float* s1, void* out, int Kd, int Nw, int out_ld, int n, GatherRows gr,
                          const PlanJob& plan, const QueueIdx& qi, hipEvent_t ev0, hipEvent_t ev1,
                          hipStream_t stream) {
  constexpr int BM = MT * 16;
  constexpr auto kernel = ffn_mfma_kernel<MODE, WDT, NS, MT, R, WV, FQ>;
  static_assert(MODE == 1 || kPlanFusedMax <= 64 * WV, "a fused plan rounds m up to a power of two <= the threads");
  static_assert((kPlanFusedMax & (kPlanFusedMax - 1)) == 0, "kPlanFusedMax is a power of two");
  const int n_blocks_N = (Nw / 16 + WV * NS - 1) / (WV * NS);
  const int64_t chunks_max = (n + (int64_t)(BM - 1) * E_loc) / BM;  // ragged worst case
  int64_t grid = std::min<int64_t>(chunks_max * n_blocks_N, resident_workgroups<kernel>(64 * WV));
  grid = (grid + 7) / 8 * 8;  // the XCD-aware order needs a multiple of 8
  if (MODE == 0 && (plan.m > 0 || FQ)) grid += 1;  // the plan's (and index's) workgroup
  // (ev0, ev1: timestamps taken by the dispatch itself, or none)
  hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(64 * WV), 0, stream, ev0, ev1, 0, (const uint16_t*)A,
                        offsets, E_loc, (const char*)W, s0, s1, (uint16_t*)out, Kd, Nw, out_ld, n_blocks_N, n, gr,
                        plan, qi);
}

// ------------------------------------------------------------ prefill GEMM path
// For batches with many rows per expert the FFN is bound by the matrix cores, so the
// kernel is built around v_mfma_f32_32x32x16_bf16 (the shape that reaches the bf16 peak
// on gfx950) with every operand byte feeding as many MFMAs as registers allow:
//   * unit = (128-row chunk of one expert, 256 weight columns); each of the 4 waves owns
//     64 columns for all 128 rows (4 x 2 tiles of 32 x 32, 128 fp32 accumulators);
//   * the activation k-tile (128 rows x 64 k, bf16) is shared by the 4 waves through an
//     LDS ring: each wave copies its quarter straight from global memory into the stage
//     (buffer_load ... lds, 16 bytes per lane), several k-steps ahead; the 16-byte slots of
//     a tile row are XOR-swizzled so that the copies stay coalesced (8 rows x 128 B per
//     instruction) and the operand reads are free of bank conflicts;
//   * each wave loads its weight fragments several k-steps ahead straight from the packed
//     layout into a register ring (buffer loads: a per-lane offset fixed for the unit, the
//     k-step in a scalar register) and widens fp8 to bf16 in registers;
//   * software pipeline: the activation fragments are read from LDS one k-slice at a time
//     between the MFMAs of the previous slices, so LDS latency overlaps the math; one
//     workgroup per CU with a 4-stage ring for bf16 weights, two per CU with a 2-stage ring
//     and a 2-slice fragment ring for fp8 weights (one computes while the other waits);
//   * gate/up: a wave's 64 packed rows are 2 gate and 2 up strips; its column tile 0 takes
//     the gate strips and tile 1 the matching up strips, so the SwiGLU epilogue pairs values
//     within a lane (no cross-lane exchange);
//   * k-permutation: in MFMA s (0..3) of a 64-wide k-step, lane half hf uses
//     k = 32hf + 8s + q for both operands, so a lane's weight fragment for 32 columns is
//     two 16-byte runs of the packed fp8 block (four of the bf16 block) and the sums are
//     exact dot products over all k.
constexpr int kGemmBM = 128;
constexpr int kGemmWaveN = 64;
constexpr int kGemmBN = kGemmWaveN * kFfnWaves;
// ring depth (k-steps of loads in flight + 1; LDS stages and weight register slots).  With
// fp8 weights 6 and 8 stages fit (456 and 504 VGPRs, 96 and 128 KiB LDS) but measured
// 2-7% slower than 4
#ifndef MOE_FFN_GEMM_STAGES_FP8
#define MOE_FFN_GEMM_STAGES_FP8 4
#endif
// Workgroups per CU the tiled kernel is built for.  Two (fp8 weights only: bf16 weight
// fragments do not fit the 256-register budget) let one workgroup's MFMAs run while the other
// waits, with a 2-stage ring and a 2-slice fragment ring per wave.
#ifndef MOE_FFN_GEMM_OCC_FP8
#define MOE_FFN_GEMM_OCC_FP8 2
#endif
template <int WDT>
constexpr int gemm_occ() { return WDT == MOE_FP8_E4M3 ? MOE_FFN_GEMM_OCC_FP8 : 1; }
template <int WDT>
constexpr int gemm_stages() { return gemm_occ<WDT>() == 2 ? 2 : (WDT == MOE_FP8_E4M3 ? MOE_FFN_GEMM_STAGES_FP8 : 4); }

// s_waitcnt vmcnt(N) alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// at their no-wait maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// weight fragments of one k-step for a wave's 2 column tiles (as loaded)
template <int WDT>
struct GemmW;
template <>
struct GemmW<MOE_FP8_E4M3> {
  static constexpr int kLoads = 4;
  u32x4 raw[2][2];  // [tile][piece]: piece p holds k = 32hf + 16p + 0..15 of the lane's column
  // AUX: the loads' cache policy (2: non-temporal, for weights read once per launch)
  template <int AUX = 0>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t w, const int* voff, int soff) {
    static_for<2>([&](auto t) {
      raw[t()][0] = __builtin_amdgcn_raw_buffer_load_b128(w, voff[t()], soff, AUX);
      raw[t()][1] = __builtin_amdgcn_raw_buffer_load_b128(w, voff[t()] + 256, soff, AUX);
    });
  }
  __device__ __forceinline__ bf16x8 frag(int t, int s) const {
    const u32x4& p = raw[t][s >> 1];
    return (s & 1) ? e4m3x8_to_bf16(p[2], p[3]) : e4m3x8_to_bf16(p[0], p[1]);
  }
};
template <>
struct GemmW<MOE_BF16> {
  static constexpr int kLoads = 8;
  u32x4 raw[2][4];  // [tile][s]
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t w, const int* voff, int soff) {
    static_for<2>([&](auto t) {
      static_for<4>([&](auto s) {
        // g = 2hf + s/2 and h = s%2 of the packed bf16 block; the lane's hf part is in voff
        raw[t()][s()] = __builtin_amdgcn_raw_buffer_load_b128(w, voff[t()] + (s() & 1) * 1024 + (s() >> 1) * 256, soff, 0);
      });
    });
  }
  __device__ __forceinline__ bf16x8 frag(int t, int s) const {
    bf16x8 r;
    __builtin_memcpy(&r, &raw[t][s], 16);
    return r;
  }
};

// buffer resource over `bytes` bytes at p (gfx9 resource word 3); loads past the end read 0
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int64_t bytes) {
  const int n = (int)std::min<int64_t>(bytes, 0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
}

// Balancing the last round.  Each XCD takes a contiguous range of n units and runs them on
// its Gx = G/8 workgroups, R = n / Gx full rounds and a tail of T = n % Gx units.  A tail
// of at most Gx/2 units would leave most CUs idle for a whole unit time, so each tail unit
// is split along the contraction into S = min(Gx / T, 8, KS / 4) pieces of whole k-steps:
// workgroup j of the XCD takes piece j % S of tail unit j / S and writes its raw fp32
// accumulators to partial slot b = 8 j + xcd (one 128 KiB tile per workgroup); a finalize
// launch then sums each tail unit's S partial tiles in piece order and applies the
// epilogue.  With no partial area (or S < 2) the tail units run whole.
constexpr int kGemmAccRegs = 4 * 2 * 16;                         // fp32 accumulators per thread
constexpr int64_t kGemmPartFloats = (int64_t)kGemmAccRegs * 256;  // one partial tile
constexpr int kGemmSplitSlots = 512;  // partial tiles in the workspace (2 workgroups x 256 CUs)
constexpr int kGemmMaxSplit = 8;

struct GemmSplit {
  int u0, Gx, R, T, S;
  __device__ __forceinline__ void init(int U, int G, int xcd, int KS, bool enabled) {
    Gx = G >> 3;
    u0 = (int)((int64_t)U * xcd / 8);
    const int n = (int)((int64_t)U * (xcd + 1) / 8) - u0;
    R = n / Gx;
    T = n - R * Gx;
    S = 1;
    if (enabled && T > 0) S = min(min(Gx / T, kGemmMaxSplit), KS / 4);
    if (S < 2) S = 1;
  }
};

// chunk and column block of unit u (chunk-major: the column blocks of a chunk are
// neighbours, so an XCD's concurrent workgroups share the chunk's activation tile).  Tiles of
// 4 chunks x 8 blocks per expert, which also share each weight tile among 4 chunks, measured
// no faster.
__device__ __forceinline__ void gemm_unit_coords(int u, int n_blocks_N, int& c, int& nb) {
  c = u / n_blocks_N;
  nb = u - c * n_blocks_N;
}

// Epilogue of a 128 x 256 unit; accumulator v of lane l holds column l%32 and row
// 8(v/4) + 4(l/32) + v%4 of a tile.  gemm_store_group writes accumulators 4g .. 4g+3 of row
// tile mt of both column tiles (t = 0: a[], t = 1: b[]); for gate/up these are the gate and
// the up value of one h column.  sc0, sc1: the fp8 row scales of the lane's columns.
template <int MODE>
__device__ __forceinline__ void gemm_store_group(const float (&a)[4], const float (&b)[4], int mt, int g, int m0,
                                                 int mend, int col0, int hf, int l32, float sc0, float sc1,
                                                 uint16_t* __restrict__ out, int out_ld) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = m0 + mt * 32 + 8 * g + 4 * hf + k;
    if (row >= mend) continue;
    if (MODE == 0) {
      out[(int64_t)row * out_ld + col0 / 2 + l32] = f32_to_bf16(silu_mul_fast(a[k] * sc0, b[k] * sc1));
    } else {
      out[(int64_t)row * out_ld + col0 + l32] = f32_to_bf16(a[k] * sc0);
      out[(int64_t)row * out_ld + col0 + 32 + l32] = f32_to_bf16(b[k] * sc1);
    }
  }
}

// the lane's two fp8 row scales (1 for bf16 weights): gate/up: gate and up scale of h
// column col0/2 + l32; down: output columns col0 + l32 and col0 + 32 + l32
template <int MODE, int WDT>
__device__ __forceinline__ void gemm_scales(int e, int col0, int l32, const float* __restrict__ s0,
                                            const float* __restrict__ s1, int out_ld, float& sc0, float& sc1) {
  sc0 = sc1 = 1.f;
  if (WDT != MOE_FP8_E4M3) return;
  if (MODE == 0) {
    sc0 = s0[(int64_t)e * out_ld + col0 / 2 + l32];
    sc1 = s1[(int64_t)e * out_ld + col0 / 2 + l32];
  } else {
    sc0 = s0[(int64_t)e * out_ld + col0 + l32];
    sc1 = s0[(int64_t)e * out_ld + col0 + 32 + l32];
  }
}

template <int MODE, int WDT>
__device__ __forceinline__ void gemm_epilogue(const f32x16 (&acc)[4][2], int e, int m0, int mend, int col0, int hf,
                                              int l32, const float* __restrict__ s0, const float* __restrict__ s1,
                                              uint16_t* __restrict__ out, int out_ld) {
  float sc0, sc1;
  gemm_scales<MODE, WDT>(e, col0, l32, s0, s1, out_ld, sc0, sc1);
  static_for<4>([&](auto mt) {
    static_for<4>([&](auto g) {
      float a[4], b[4];
      static_for<4>([&](auto k) {
        a[k()] = acc[mt()][0][4 * g() + k()];
        b[k()] = acc[mt()][1][4 * g() + k()];
      });
      gemm_store_group<MODE>(a, b, mt(), g(), m0, mend, col0, hf, l32, sc0, sc1, out, out_ld);
    });
  });
}

// Partial tile layout: accumulator group q = 4 (2 mt + t) + v/4 of thread tid at
// part[1024 q + 4 tid .. + 3] (each wave stores and loads 1 KiB runs).  Buffer stores with the
// group offset in a scalar register, so no per-group 64-bit address stays live.
__device__ __forceinline__ void store_partial(const f32x16 (&acc)[4][2], float* __restrict__ part, int tid) {
  const __amdgpu_buffer_rsrc_t r = buffer_rsrc(part, kGemmPartFloats * 4);
  static_for<4>([&](auto mt) {
    static_for<2>([&](auto t) {
      static_for<4>([&](auto g) {
        constexpr int q = 4 * (2 * mt() + t()) + g();
        u32x4 v;
        static_for<4>([&](auto k) { v[k()] = __float_as_uint(acc[mt()][t()][4 * g() + k()]); });
        __builtin_amdgcn_raw_buffer_store_b128(v, r, 16 * tid, 4096 * q, 0);
      });
    });
  });
}

template <int MODE, int WDT>
__global__ __launch_bounds__(256, gemm_occ<WDT>()) void ffn_gemm_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                       int E_loc, const char* __restrict__ W,
                                                       const float* __restrict__ s0, const float* __restrict__ s1,
                                                       uint16_t* __restrict__ out, int Kd, int Nw, int out_ld,
                                                       int n_blocks_N, int n_rows, GatherRows gr,
                                                       float* __restrict__ parts) {
  constexpr int S = gemm_stages<WDT>();
  constexpr int esz = WDT == MOE_FP8_E4M3 ? 1 : 2;
  // activation k-tiles, S stages of 16 KiB.  One array per stage: the compiler then tells
  // the stages apart and makes an LDS read wait only for the copy into its own stage (with
  // a single array it waits for every copy in flight, draining the load pipeline each step)
  static_assert(S <= 4, "four stage arrays");
  __shared__ u32x4 a_lds0[kGemmBM * 8], a_lds1[kGemmBM * 8], a_lds2[kGemmBM * 8], a_lds3[kGemmBM * 8];
  auto stage = [&](auto st) -> u32x4* {
    if constexpr (st() == 0) return a_lds0;
    else if constexpr (st() == 1) return a_lds1;
    else if constexpr (st() == 2) return a_lds2;
    else return a_lds3;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KS = Kd / kBK;
  const int64_t strip_stride = (int64_t)KS * 1024 * esz;
  const int l32 = lane & 31, hf = lane >> 5;

  const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
  ChunkTable tab;
  tab.build(offsets, E_loc, n_rows, kGemmBM, lane);
  const int total = tab.total;
  GemmSplit sp;
  sp.init(total * n_blocks_N, gridDim.x, xcd, KS, parts != nullptr);
  // this workgroup's items: R full units (one more if the tail runs whole), then its piece
  const int n_full = sp.R + (sp.S == 1 && j < sp.T ? 1 : 0);
  const int n_items = n_full + (sp.S > 1 && j < sp.T * sp.S ? 1 : 0);
#pragma clang loop unroll(disable)
  for (int item = 0; item < n_items; ++item) {
    int u, k0 = 0, k1 = KS;
    const bool piece = item >= n_full;
    if (!piece) {
      u = sp.u0 + item * sp.Gx + j;
    } else {
      u = sp.u0 + sp.R * sp.Gx + j / sp.S;
      const int pc = j % sp.S;
      k0 = pc * KS / sp.S;
      k1 = (pc + 1) * KS / sp.S;
    }
    int c, nb, e, m0, mend;
    gemm_unit_coords(u, n_blocks_N, c, nb);
    tab.find(c, kGemmBM, e, m0, mend);
    if (e < 0) break;  // not reachable: every unit id below U names a chunk
    const int col0 = nb * kGemmBN + wv * kGemmWaveN;
    const bool wact = col0 < Nw;        // the last column block may be partial
    const int colw = wact ? col0 : 0;   // idle waves stream valid weights (results unused)
    // weight lane offsets (bytes into expert e's packed matrix).  The wave's 4 strips are
    // colw/16 + 0..3.  Gate/up: tile 0 takes the gate strips (+0, +2) and tile 1 the matching
    // up strips (+1, +3), so a lane holds the gate and up value of one h column in its two
    // tiles.  Down: tile t takes strips +2t, +2t+1 (32 consecutive output columns).
    const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(W + (int64_t)e * Nw * Kd * esz, (int64_t)Nw * Kd * esz);
    int wvo[2];
    static_for<2>([&](auto t) {
      const int half = l32 >> 4, r = l32 & 15;
      const int strip = colw / 16 + (MODE == 0 ? 2 * half + t() : 2 * t() + half);
      wvo[t()] = (int)(strip * strip_stride) + (32 * hf + r) * 16;
    });
    // activation copies: instruction d of this wave fills the 16-byte slots (4wv + d)*64 + lane
    // of a stage; slot P holds row P/8, 16-byte piece (P%8) ^ ((P/8 >> 1) & 7) of the row
    // (byte offset per lane, k-step in a scalar register).
    // (with a gather, A is the pool: the host checks that it spans under 2 GiB)
    const __amdgpu_buffer_rsrc_t ars =
        buffer_rsrc(A, gr.perm ? gr.P * gr.pitch * 2 : (int64_t)n_rows * Kd * 2);
    int avo[4];
    static_for<4>([&](auto d) {
      const int P = (wv * 4 + d()) * 64 + lane, row = P >> 3, kq = (P & 7) ^ ((row >> 1) & 7);
      const int r = min(m0 + row, mend - 1);
      avo[d()] = (int)((gr.row_offset(r, Kd) + kq * 8) * 2);
    });

    f32x16 acc[4][2];
    static_for<4>([&](auto i) { static_for<2>([&](auto jj) { acc[i()][jj()] = f32x16{}; }); });

    GemmW<WDT> wr[S];   // weight fragments of steps i .. i+S-1
    // activations of step ks go straight from global memory into LDS stage slot (16 bytes
    // per lane at the instruction's base + 16 lane, i.e. exactly the slot order above)
    auto issue_a = [&](auto slot, int ks) {
      ks = min(ks, k1 - 1);
      static_for<4>([&](auto d) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ars, (__attribute__((address_space(3))) void*)(stage(slot) + (wv * 4 + d()) * 64), 16, avo[d()],
            ks * kBK * 2, 0, 0);
      });
    };
    auto issue_w = [&](auto slot, int ks) { wr[slot()].load(wrs, wvo, min(ks, k1 - 1) * 1024 * esz); };
    // Workgroup barrier for the copy pipeline.  Before it this wave's LDS reads are complete
    // (so after it no wave still reads a stage a copy may refill) and the caller has waited
    // for its own copies with an explicit vmcnt; a release fence here would also wait for
    // every copy still in flight, draining the pipeline.  The acquire fence keeps the LDS
    // reads after the barrier.
    auto barrier = [&]() {
      __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // Software pipeline over k-steps i = k0, k0+1, ... (weight slot and LDS stage (i - k0) % S).
    // Step i: MFMAs of slice 0 of step i; wait until this wave's activation copy of step i+1
    // has landed in LDS, barrier (then every wave's has, and every wave has finished
    // reading the stage of step i); copy the activations of step i+S into that stage; then
    // for s = 0..3 read slice s of step i+1 and run the MFMAs of slice s+1 of step i, so each
    // LDS read has three slices of MFMAs to land in; finally load the weights of step i+S
    // into the slot step i's MFMAs have released.  Loads are issued in the order they are
    // needed.  The waits for the copies are explicit vmcnt counts (behind the copy of step
    // i+1 are the weights of i+1 and the S-2 later batches).  An item runs a whole number of
    // S-step groups: steps past k1 load clamped (valid) data and zero their activation
    // fragments, so every step has the same branch-free body.
    static_assert(S >= 2, "a ring of at least two stages");
    constexpr int kA = 4, kW = GemmW<WDT>::kLoads;
    auto issue = [&](auto slot, int ks) {
      issue_a(slot, ks);
      issue_w(slot, ks);
    };
    if constexpr (gemm_occ<WDT>() == 2) {
      // Two workgroups per CU: 2-stage ring, fragments of two k-slices at a time.  Step i:
      // slices 1-3 of step i are read from its stage one slice ahead of their MFMAs; after the
      // barrier (copy of step i+1 landed everywhere, stage of step i read by everyone) the
      // copy of step i+2 goes into that stage and slice 0 of step i+1 is read; the weights of
      // step i+2 load into the slot step i has released.  Behind the copy of step i+1 there
      // are only the weights of step i+1.  Steps past k1 zero their weight fragments.
      static_assert(S == 2, "two-workgroup variant: 2-stage ring");
      u32x4 fr[2][4];
      auto read2 = [&](auto stg, auto ss, auto dst) {
        const u32x4* tile = stage(stg);
        static_for<4>([&](auto mt) {
          const int row = mt() * 32 + l32, kq = 4 * hf + ss();
          fr[dst()][mt()] = tile[row * 8 + (kq ^ ((row >> 1) & 7))];
        });
      };
      // 32-row tiles that hold rows of the unit: the MFMAs of the rest (padding of an
      // expert's last chunk) are skipped; their accumulators stay zero and are never stored.
      // (With two workgroups per CU the freed matrix-core cycles go to the other one.)
      const int mt_act = __builtin_amdgcn_readfirstlane((mend - m0 + 31) / 32);
      auto mfma2 = [&](auto slot, auto ss, auto src, bool dead) {
        bf16x8 bw[2];
        static_for<2>([&](auto t) { bw[t()] = dead ? bf16x8{} : wr[slot()].frag(t(), ss()); });
        static_for<4>([&](auto mt) {
          if (mt() == 0 || mt() < mt_act) {
            bf16x8 a;
            __builtin_memcpy(&a, &fr[src()][mt()], 16);
            static_for<2>([&](auto t) {
              acc[mt()][t()] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw[t()], acc[mt()][t()], 0, 0, 0);
            });
          }
        });
      };
      __builtin_amdgcn_sched_barrier(0);
      issue(I0{}, k0);
      __builtin_amdgcn_sched_barrier(0);
      issue(I1{}, k0 + 1);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<kW + kA + kW>();  // the copy of step k0
      barrier();
      __builtin_amdgcn_sched_barrier(0);
      read2(I0{}, I0{}, I0{});
      const int n_steps = (k1 - k0 + 1) / 2 * 2;
#pragma clang loop unroll(disable)
      for (int it = 0; it < n_steps; it += 2) {
        static_for<2>([&](auto v) {
          using SL = std::integral_constant<int, v()>;
          using NX = std::integral_constant<int, 1 - v()>;
          const int i = k0 + it + v();
          const bool dead = i >= k1;
          read2(SL{}, I1{}, I1{});
          mfma2(SL{}, I0{}, I0{}, dead);
          __builtin_amdgcn_sched_barrier(0);
          read2(SL{}, I2{}, I0{});
          mfma2(SL{}, I1{}, I1{}, dead);
          __builtin_amdgcn_sched_barrier(0);
          read2(SL{}, I3{}, I1{});
          mfma2(SL{}, I2{}, I0{}, dead);
          __builtin_amdgcn_sched_barrier(0);
          wait_vmcnt<kW>();  // the copy of step i+1
          barrier();
          __builtin_amdgcn_sched_barrier(0);
          issue_a(SL{}, i + 2);  // the stage of step i is free now
          __builtin_amdgcn_sched_barrier(0);
          read2(NX{}, I0{}, I0{});
          mfma2(SL{}, I3{}, I1{}, dead);
          __builtin_amdgcn_sched_barrier(0);
          issue_w(SL{}, i + 2);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
    } else {
    u32x4 af[4][4];     // activation fragments [k-slice s][mt] of the step being computed
    auto read1 = [&](auto stg, auto ss) {  // fragments of k-slice ss
      const u32x4* tile = stage(stg);
      static_for<4>([&](auto mt) {
        const int row = mt() * 32 + l32, kq = 4 * hf + ss();
        af[ss()][mt()] = tile[row * 8 + (kq ^ ((row >> 1) & 7))];
      });
    };
    auto mfma1 = [&](auto slot, auto ss) {  // MFMAs of k-slice ss
      bf16x8 bw[2];
      static_for<2>([&](auto t) { bw[t()] = wr[slot()].frag(t(), ss()); });
      static_for<4>([&](auto mt) {
        bf16x8 a;
        __builtin_memcpy(&a, &af[ss()][mt()], 16);
        static_for<2>([&](auto t) {
          acc[mt()][t()] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw[t()], acc[mt()][t()], 0, 0, 0);
        });
      });
    };
    static_for<S>([&](auto v) {  // same batch order as the loop, so every wait matches the steady state
      __builtin_amdgcn_sched_barrier(0);
      issue(v, k0 + v());
    });
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kW + (S - 1) * (kA + kW)>();  // the copy of step k0
    barrier();
    __builtin_amdgcn_sched_barrier(0);
    read1(I0{}, I0{});
    read1(I0{}, I1{});
    read1(I0{}, I2{});
    read1(I0{}, I3{});
    const int n_steps = (k1 - k0 + S - 1) / S * S;
#pragma clang loop unroll(disable)
    for (int it = 0; it < n_steps; it += S) {
      static_for<S>([&](auto v) {
        constexpr int slot = v();
        using SL = std::integral_constant<int, slot>;
        using NX = std::integral_constant<int, (slot + 1) % S>;
        const int i = k0 + it + v();
        if (i >= k1) static_for<4>([&](auto ss) { static_for<4>([&](auto mt) { af[ss()][mt()] = u32x4{}; }); });
        mfma1(SL{}, I0{});
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kW + (S - 2) * (kA + kW)>();  // the copy of step i+1
        barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue_a(SL{}, i + S);  // the stage of step i is free now (no LDS reads pending)
        __builtin_amdgcn_sched_barrier(0);
        read1(NX{}, I0{});
        mfma1(SL{}, I1{});
        __builtin_amdgcn_sched_barrier(0);
        read1(NX{}, I1{});
        mfma1(SL{}, I2{});
        __builtin_amdgcn_sched_barrier(0);
        read1(NX{}, I2{});
        mfma1(SL{}, I3{});
        __builtin_amdgcn_sched_barrier(0);
        read1(NX{}, I3{});
        __builtin_amdgcn_sched_barrier(0);
        issue_w(SL{}, i + S);  // weight slot of step i is free after its last MFMAs
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    }
    // no copy may still be in flight into a stage the next item's prologue fills, and the
    // next item's copies wait for this item's last LDS reads
    wait_vmcnt<0>();
    barrier();
    if (!wact) continue;
    if (piece)
      store_partial(acc, parts + (int64_t)b * kGemmPartFloats, tid);
    else
      gemm_epilogue<MODE, WDT>(acc, e, m0, mend, col0, hf, l32, s0, s1, out, out_ld);
  }
}

// Sums each split tail unit's partial tiles in piece order and applies the epilogue.  One
// workgroup per (XCD, tail unit t, row tile mt, accumulator group g): its threads load the
// two float4 groups q = 8 mt + g (column tile 0) and 8 mt + 4 + g (tile 1) of all S pieces
// at once, so the whole pass is about one memory round trip.  Workgroup b: XCD b & 7,
// t = b >> 7, (mt, g) = (b >> 3) & 15 (a split needs T <= Gx/2, so 8 G workgroups cover
// every tail unit); the bookkeeping is the GEMM launch's with the same grid G.
template <int MODE, int WDT>
__global__ __launch_bounds__(256) void ffn_gemm_finalize_kernel(const int32_t* __restrict__ offsets, int E_loc,
                                                                int n_rows, int n_blocks_N, int KS, int G,
                                                                const float* __restrict__ parts,
                                                                const float* __restrict__ s0,
                                                                const float* __restrict__ s1,
                                                                uint16_t* __restrict__ out, int Nw, int out_ld) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int b = blockIdx.x, xcd = b & 7, t = b >> 7, mt = (b >> 5) & 3, g = (b >> 3) & 3;
  ChunkTable tab;
  tab.build(offsets, E_loc, n_rows, kGemmBM, lane);
  GemmSplit sp;
  sp.init(tab.total * n_blocks_N, G, xcd, KS, true);
  if (sp.S < 2 || t >= sp.T) return;
  int c, nb, e, m0, mend;
  gemm_unit_coords(sp.u0 + sp.R * sp.Gx + t, n_blocks_N, c, nb);
  tab.find(c, kGemmBM, e, m0, mend);
  const int col0 = nb * kGemmBN + wv * kGemmWaveN;
  if (e < 0 || col0 >= Nw || m0 + mt * 32 >= mend) return;  // (no barriers: waves leave independently)
  float4 v[kGemmMaxSplit][2];
#pragma unroll
  for (int pc = 0; pc < kGemmMaxSplit; ++pc) {
    if (pc < sp.S) {
      const float* part = parts + (int64_t)(((t * sp.S + pc) << 3) | xcd) * kGemmPartFloats + 4 * tid;
      v[pc][0] = *reinterpret_cast<const float4*>(part + 1024 * (8 * mt + g));
      v[pc][1] = *reinterpret_cast<const float4*>(part + 1024 * (8 * mt + 4 + g));
    }
  }
  float a[4] = {0.f, 0.f, 0.f, 0.f}, bb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int pc = 0; pc < kGemmMaxSplit; ++pc) {
    if (pc < sp.S) {
      a[0] += v[pc][0].x; a[1] += v[pc][0].y; a[2] += v[pc][0].z; a[3] += v[pc][0].w;
      bb[0] += v[pc][1].x; bb[1] += v[pc][1].y; bb[2] += v[pc][1].z; bb[3] += v[pc][1].w;
    }
  }
  float sc0, sc1;
  gemm_scales<MODE, WDT>(e, col0, l32, s0, s1, out_ld, sc0, sc1);
  gemm_store_group<MODE>(a, bb, mt, g, m0, mend, col0, hf, l32, sc0, sc1, out, out_ld);
}

// ------------------------------------------------ prefill GEMM with 256-row units (fp8 weights)
// One workgroup per CU, 4 waves; a unit is (chunk of up to 256 rows of one expert, 256 packed
// weight columns), each wave computing all 256 rows x its 64 columns (8 x 2 tiles of
// v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators).  Per 64-wide k-step a unit moves 32 KiB of
// activations (through a 4-stage LDS ring, buffer_load ... lds) and 16 KiB of fp8 weights (a
// 4-deep register ring per wave) for 8.4 MFLOP: twice the weight reuse of a 128-row unit, and
// twice the matrix-core work per k-step to cover each load's latency.  Activation fragments are
// read from LDS one k-slice ahead (two register sets), weights widened to bf16 in registers.
// 32-row tiles past a chunk's last row skip their LDS reads and MFMAs, so a unit costs in
// proportion to its rows (32-row granularity) and the tail chunks of small experts stay cheap.
//
// Work order: each workgroup's work is fixed on the device from `offsets` (no host round trip,
// no atomics).  The chunks are sorted by cost: every full 256-row chunk first (expert order),
// then each expert's partial last chunk by its 32-row tile count, descending (ties: expert
// order); a chunk's 256-column blocks are consecutive units.  Round 0 gives unit j to workgroup
// j, and workgroup j is the j % Gx-th of XCD j / Gx, so a chunk's column blocks run side by side
// on one XCD and share its activations in L2.  The later rounds go, in the same order, to the
// workgroups whose round-0 unit leaves room for another under the mean load (all of them on
// large batches) as a snake (reversed in alternate rounds, so that a workgroup that drew a
// large unit in one round draws a small one in the next), the last, partial round ranked by
// load (in the kernel below).
constexpr int kG2BM = 256;
constexpr int kG2MT = kG2BM / 32;
constexpr int kG2RankRounds = 8;
#ifndef MOE_G2_STAGES
#define MOE_G2_STAGES 4
#endif
constexpr int kG2S = MOE_G2_STAGES;
static_assert(kG2S == 4, "four LDS stages (the epilogue takes one per wave)");

// Chunks of 256 rows in cost order (above), kept in LDS so that no register holds the table
// across a unit's contraction: per expert its first and end row, full-chunk count and the
// sorted position of its first full chunk (non-decreasing in expert order), and for each
// partial chunk's sorted position past the full ones, its expert and 32-row tile count.
// Built by wave 0.
struct G2Table {
  int a0[256], a1[256], nf[256], fs[256], pe[256], pt[256];
  int E, F, total, psum;  // psum: the partial chunks' 32-row tiles, summed
};

__device__ __forceinline__ void g2_table_build(G2Table& tb, const int32_t* __restrict__ offsets, int E_loc,
                                               int n_rows, int lane) {
  int base = 0, pt[4] = {0, 0, 0, 0};
  static_for<4>([&](auto jc) {
    constexpr int j = jc();
    if (j > 0 && 64 * j >= E_loc) return;  // (no expert in this group of 64)
    const int e = lane + 64 * j;
    int lo = 0, hi = 0;
    if (e < E_loc) {  // clamped to [0, n_rows]: inconsistent offsets never address past the batch
      lo = min(max(offsets[e], 0), n_rows);
      hi = min(max(offsets[e + 1], lo), n_rows);
    }
    const int nf = (hi - lo) / kG2BM;
    pt[j] = ((hi - lo) % kG2BM + 31) / 32;
    int incl = nf;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (e < E_loc) {
      tb.a0[e] = lo;
      tb.a1[e] = hi;
      tb.nf[e] = nf;
      tb.fs[e] = base + incl - nf;
    }
    base += __shfl(incl, 63, 64);
  });
  int pos = 0, psum = 0;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int t = kG2MT; t >= 1; --t) {
    static_for<4>([&](auto jc) {
      constexpr int j = jc();
      if (j > 0 && 64 * j >= E_loc) return;
      const uint64_t bal = __ballot(pt[j] == t);
      if (pt[j] == t) {
        tb.pe[pos + __popcll(bal & below)] = lane + 64 * j;
        tb.pt[pos + __popcll(bal & below)] = t;
      }
      pos += __popcll(bal);
      psum += t * __popcll(bal);
    });
  }
  if (lane == 0) {
    tb.E = E_loc;
    tb.F = base;
    tb.total = base + pos;
    tb.psum = psum;
  }
}

// expert, first row and end row of sorted chunk q (0 <= q < total)
__device__ __forceinline__ void g2_find(const G2Table& tb, int q, int& e, int& m0, int& mend) {
  if (q < tb.F) {
    // the last expert whose first full chunk is at or before q (it has q among its full chunks)
    int lo = 0, hi = tb.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tb.fs[mid] <= q) lo = mid;
      else hi = mid - 1;
    }
    e = lo;
    m0 = tb.a0[e] + (q - tb.fs[e]) * kG2BM;
    mend = m0 + kG2BM;
  } else {
    e = tb.pe[q - tb.F];
    m0 = tb.a0[e] + tb.nf[e] * kG2BM;
    mend = tb.a1[e];
  }
}

// Epilogue of a 256-row unit through LDS.  Each wave converts its tile (down: 256 rows x 64
// output columns; gate/up: 256 x 32 h values) to bf16 in its own activation stage, free once
// the k-loop's last barrier has passed, reads it back row by row and stores 16 bytes per lane
// (down: 8 rows of 128 B per instruction, gate/up: 16 rows of 64 B) through a buffer resource
// that ends at the chunk's last row, so the stores of rows past it are dropped without a
// branch.  sc0, sc1: the lane's fp8 row scales (loaded ahead of the contraction).  Every
// per-lane address is derived here: left to the compiler, the row addresses were computed
// ahead of the contraction and kept in scratch across it, and each reload's wait for the
// memory counter then also waited for the stores issued before it (2-byte stores straight
// from the MFMA layout took ~2 us per 32-row tile this way, 13-17 us of an 8-tile unit).  The
// barrier after the read-back keeps the next unit's copies out of the stages until every wave
// has read its tile.
template <int MODE, int MTA>
__device__ __forceinline__ void g2_epilogue(const f32x16 (&acc)[MTA][2], u32x4* st, bool wact, int m0, int mend,
                                           int col0, int lane_in, float sc0, float sc1,
                                           uint16_t* __restrict__ out, int out_ld) {
  constexpr int CW = MODE == 0 ? 32 : 64;  // output columns of a wave
  constexpr int LPR = CW * 2 / 16;         // lanes per row on the read-back (16 bytes each)
  constexpr int RPI = 64 / LPR;            // rows per read-back instruction
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, hf = lane >> 5;
  if (wact) {
    uint16_t* t16 = reinterpret_cast<uint16_t*>(st) + 4 * hf * CW + l32;
    static_for<MTA>([&](auto mt) {
      static_for<4>([&](auto g) {
        static_for<4>([&](auto k) {
          constexpr int row = mt() * 32 + 8 * g() + k();  // + 4 hf (in t16)
          const float a = acc[mt()][0][4 * g() + k()], b = acc[mt()][1][4 * g() + k()];
          if constexpr (MODE == 0) {
            t16[row * CW] = f32_to_bf16(silu_mul_fast(a * sc0, b * sc1));
          } else {
            t16[row * CW] = f32_to_bf16(a * sc0);
            t16[row * CW + 32] = f32_to_bf16(b * sc1);
          }
        });
      });
    });
  }
  __syncthreads();
  if (wact) {
    const int rr = lane / LPR, cq = lane - rr * LPR;
    const __amdgpu_buffer_rsrc_t ors =
        buffer_rsrc(out + (int64_t)m0 * out_ld + (MODE == 0 ? col0 / 2 : col0), (int64_t)(mend - m0) * out_ld * 2);
    const int voff = (rr * out_ld + cq * 8) * 2;
    const u32x4* src = st + rr * LPR + cq;
    constexpr int NI = MTA * 32 / RPI;  // read-backs, in groups of up to 8 (reads, then stores)
    static_for<(NI + 7) / 8>([&](auto gi) {
      constexpr int i0 = gi() * 8, NG = NI - i0 < 8 ? NI - i0 : 8;
      u32x4 v[NG];
      static_for<NG>([&](auto j) { v[j()] = src[(i0 + j()) * RPI * LPR]; });
      static_for<NG>([&](auto j) {
        __builtin_amdgcn_raw_buffer_store_b128(v[j()], ors, voff, (i0 + j()) * RPI * out_ld * 2, 0);
      });
    });
  }
  __syncthreads();
}

template <int MODE>
__global__ __launch_bounds__(256, 1) void ffn_gemm256_kernel(const uint16_t* __restrict__ A,
                                                            const int32_t* __restrict__ offsets, int E_loc,
                                                            const char* __restrict__ W,
                                                            const float* __restrict__ s0,
                                                            const float* __restrict__ s1,
                                                            uint16_t* __restrict__ out, int Kd, int Nw, int out_ld,
                                                            int n_blocks_N, int n_rows, GatherRows gr) {
  constexpr int S = kG2S;
  constexpr int WDT = MOE_FP8_E4M3;
  // activation k-tiles, one array per stage (so that an LDS read waits only for the copy into
  // its own stage): 256 rows x 64 k bf16 = 32 KiB each
  __shared__ u32x4 g2_lds0[kG2BM * 8], g2_lds1[kG2BM * 8], g2_lds2[S > 2 ? kG2BM * 8 : 1],
      g2_lds3[S > 3 ? kG2BM * 8 : 1];
  auto stage = [&](auto st) -> u32x4* {
    if constexpr (st() == 0) return g2_lds0;
    else if constexpr (st() == 1) return g2_lds1;
    else if constexpr (st() == 2) return g2_lds2;
    else return g2_lds3;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KS = Kd / kBK;
  const int64_t strip_stride = (int64_t)KS * 1024;
  const int l32 = lane & 31, hf = lane >> 5;

  __shared__ G2Table tab;
  if (wv == 0) g2_table_build(tab, offsets, E_loc, n_rows, lane);
  __syncthreads();
  const int U = tab.total * n_blocks_N;
  const int G = gridDim.x, Gx = G >> 3, b = blockIdx.x;
  const int jw = (b & 7) * Gx + (b >> 3);  // logical workgroup: XCD-major
  // A unit of t row tiles costs t + 1 (measured unit times on prefill waves: 13 + 12.4 t us for
  // gate/up, 6 + 7.6 t for down).  Round 0 gives unit jw to logical workgroup jw.  The later units
  // go to the workgroups whose round-0 unit leaves room for at least the cheapest unit under the
  // target (the largest unit or the mean load, whichever is larger); a workgroup that drew one of
  // the largest units stops there when that is not so (prefill wave of 1638 pairs: the busiest
  // workgroup's model cost 11 -> 9, its down launch 76 -> 68 us).  Over those workgroups (their logical
  // order kept) the later rounds run as a snake (the first of them reversed: a workgroup that drew
  // a large unit draws a small one), and the last, partial round goes to the least loaded: its unit
  // i to the workgroup of rank i in (model cost, index) order (the snake alone hands it to the
  // workgroups that drew the largest units, up to 30 us longer).  For more than kG2RankRounds full
  // rounds the snake order is kept.
  auto ucost = [&](int uu) {
    const int q = uu / n_blocks_N;
    return (q < tab.F ? kG2MT : tab.pt[q - tab.F]) + 1;
  };
  __shared__ unsigned long long s_kept[4];
  __shared__ int s_below[4];
  int Gp = G, jk = jw;  // workgroups taking later units, this one's index among them
  bool later = true;
  const int total_cost = (tab.F * (kG2MT + 1) + tab.psum + (tab.total - tab.F)) * n_blocks_N;
  const int target = max(ucost(0), (total_cost + G - 1) / G), min_later = U > G ? ucost(U - 1) : 0;
  // (no workgroup is left out when even the largest unit leaves room for the cheapest)
  if (U > G && G <= 256 && ucost(0) + min_later > target) {
    const int w = wv * 64 + lane;
    const uint64_t bal = __ballot(w < G && ucost(w) + min_later <= target);
    if (lane == 0) s_kept[wv] = bal;
    __syncthreads();
    int cnt = 0, before = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint64_t x = s_kept[v];
      cnt += __popcll(x);
      before += v < (jw >> 6) ? __popcll(x) : v == (jw >> 6) ? __popcll(x & ((1ull << (jw & 63)) - 1ull)) : 0;
    }
    if (cnt > 0 && cnt < G) {
      Gp = __builtin_amdgcn_readfirstlane(cnt);
      jk = __builtin_amdgcn_readfirstlane(before);
      later = __builtin_amdgcn_readfirstlane((int)((s_kept[jw >> 6] >> (jw & 63)) & 1ull));
    }
  }
  const int U2 = U - G, R2 = U2 > 0 ? U2 / Gp : 0;
  const bool ranked = U2 > R2 * Gp && R2 + 1 <= kG2RankRounds && G <= 256;
  int tail_u = -1;  // this workgroup's unit of the last, partial round, if any
  if (ranked) {
    // model cost of kept workgroup (logical w, kept index k) over round 0 and the full later rounds
    auto cost_of = [&](int w, int k) {
      int c = ucost(w);
      for (int r = 0; r < R2; ++r) c += ucost(G + r * Gp + ((r & 1) ? k : Gp - 1 - k));
      return c;
    };
    // each wave ranks 64 workgroups (one per lane) against this one, among the kept ones
    const int w = wv * 64 + lane;
    int ahead = 0;
    if (later && w < G) {
      int k = w;
      bool kw = true;
      if (Gp < G) {
        const uint64_t x = s_kept[wv];
        kw = (x >> lane) & 1ull;
        k = __popcll(x & ((1ull << lane) - 1ull));
#pragma unroll
        for (int v = 0; v < 4; ++v) k += v < wv ? __popcll(s_kept[v]) : 0;
      }
      if (kw) {
        const int c = cost_of(w, k), mine = cost_of(jw, jk);
        ahead = c < mine || (c == mine && k < jk);
      }
    }
    const int cnt = __popcll(__ballot(ahead));
    if (lane == 0) s_below[wv] = cnt;
    __syncthreads();
    const int rank = s_below[0] + s_below[1] + s_below[2] + s_below[3];
    if (later && rank < U2 - R2 * Gp) tail_u = G + R2 * Gp + rank;
    tail_u = __builtin_amdgcn_readfirstlane(tail_u);
  }
#pragma clang loop unroll(disable)
  for (int r = 0;; ++r) {
    int u = jw;
    if (r > 0) {
      if (!later) break;
      const int r2 = r - 1;
      u = G + r2 * Gp + ((r2 & 1) ? jk : Gp - 1 - jk);
      if (r2 == R2 && ranked) u = tail_u < 0 ? U : tail_u;
    }
    if (u >= U) break;
    const int q = u / n_blocks_N, nb = u - q * n_blocks_N;
    int e, m0, mend;
    g2_find(tab, q, e, m0, mend);
    e = __builtin_amdgcn_readfirstlane(e);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    mend = __builtin_amdgcn_readfirstlane(mend);
    const int mt_act = __builtin_amdgcn_readfirstlane((mend - m0 + 31) / 32);
    const int col0 = nb * kGemmBN + wv * kGemmWaveN;
    const bool wact = col0 < Nw;       // the last column block may be partial
    const int colw = wact ? col0 : 0;  // idle waves stream valid weights (results unused)
    // the epilogue's fp8 row scales, loaded ahead of the contraction (idle waves: valid ones)
    float sc0, sc1;
    gemm_scales<MODE, WDT>(e, colw, l32, s0, s1, out_ld, sc0, sc1);
    const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(W + (int64_t)e * Nw * Kd, (int64_t)Nw * Kd);
    const int w_end = Nw * Kd;  // (the host keeps an expert's matrix under 2^30 bytes)
    int wvo[2];
    static_for<2>([&](auto t) {
      const int half = l32 >> 4, rr = l32 & 15;
      const int strip = colw / 16 + (MODE == 0 ? 2 * half + t() : 2 * t() + half);
      wvo[t()] = (int)(strip * strip_stride) + (32 * hf + rr) * 16;
    });
    const __amdgpu_buffer_rsrc_t ars =
        buffer_rsrc(A, gr.perm ? gr.P * gr.pitch * 2 : (int64_t)n_rows * Kd * 2);
    // LDS slot of this lane's fragment of k-slice ss in row tile 0 (tile mt adds 256 slots:
    // rows 32 mt + l32 keep the swizzle term of rows l32)
    int lds_off[4];
    static_for<4>([&](auto ss) { lds_off[ss()] = l32 * 8 + ((4 * hf + ss()) ^ ((l32 >> 1) & 7)); });

    // The unit with MTA row tiles of 32 rows (the chunk's rows rounded up to 32): the k-loop is
    // instantiated for MTA = 1..8, so that a chunk of few rows copies, reads and multiplies only
    // its tiles, without per-tile branches inside the loop (rounding to 64 rows instead executed
    // 6-11% more rows on prefill waves of 3277-6554 pairs: gate/up 2-5% slower).
    auto unit = [&](auto mta, auto nt) {
      constexpr int MTA = mta();
      // activation copies: instruction d of this wave fills the 16-byte slots (4 d + wv) * 64 +
      // lane of a stage; slot P holds row P / 8, piece (P % 8) ^ ((P / 8 >> 1) & 7) of that row
      // (rows past the chunk copy its last row; their results are never stored)
      int avo[MTA];
      {
        int rd[MTA];
        int64_t od[MTA];
        static_for<MTA>([&](auto d) {
          const int P = (4 * d() + wv) * 64 + lane;
          rd[d()] = min(m0 + (P >> 3), mend - 1);
        });
        gr.row_offsets(rd, Kd, od);
        static_for<MTA>([&](auto d) {
          const int P = (4 * d() + wv) * 64 + lane, row = P >> 3, kq = (P & 7) ^ ((row >> 1) & 7);
          avo[d()] = (int)((od[d()] + kq * 8) * 2);
        });
      }
      f32x16 acc[MTA][2];
      static_for<MTA>([&](auto i) { static_for<2>([&](auto jj) { acc[i()][jj()] = f32x16{}; }); });
      GemmW<WDT> wr[S];
      u32x4 af[2][MTA];
      auto issue_a = [&](auto slot, int ks) {
        ks = min(ks, KS - 1);
        static_for<MTA>([&](auto d) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              ars, (__attribute__((address_space(3))) void*)(stage(slot) + (4 * d() + wv) * 64), 16, avo[d()],
              ks * kBK * 2, 0, 0);
        });
      };
      // weights of k-step ks; past the contraction the offset lies beyond the expert's matrix,
      // where buffer loads return zeros, so those steps' MFMAs add nothing
      auto issue_w = [&](auto slot, int ks) {
        wr[slot()].template load<nt() ? 2 : 0>(wrs, wvo, ks < KS ? ks * 1024 : w_end);
      };
      auto read = [&](auto stg, auto ss, auto buf) {  // fragments of k-slice ss
        const u32x4* tile = stage(stg);
        static_for<MTA>([&](auto mt) { af[buf()][mt()] = tile[mt() * 256 + lds_off[ss()]]; });
      };
      bf16x8 bwb[2][2];  // widened weight fragments of two k-slices (this one and the next)
      auto cvt = [&](auto slot, auto ss, auto dst) {
        static_for<2>([&](auto t) { bwb[dst()][t()] = wr[slot()].frag(t(), ss()); });
      };
      auto mfma = [&](auto buf, auto wbuf) {
        static_for<MTA>([&](auto mt) {
          bf16x8 a;
          __builtin_memcpy(&a, &af[buf()][mt()], 16);
          static_for<2>([&](auto t) {
            acc[mt()][t()] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bwb[wbuf()][t()], acc[mt()][t()], 0, 0, 0);
          });
        });
      };
      // One wave per SIMD issues in order, so an instruction between two MFMAs costs matrix-core
      // time unless it fits in the shadow of the MFMA before it: the next slice's LDS reads,
      // weight widening and (at the step boundary) the copies are spread one or two per MFMA.
      auto interleave = [&]() {
        static_for<2 * MTA>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x122, 2, 0);  // up to two LDS reads / VALU / VMEM reads
        });
      };
      auto barrier = [&]() {
        __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      };
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      constexpr int kA = MTA, kW = GemmW<WDT>::kLoads;
      // Step i (stage and weight slot i % S): while the MFMAs of slice s run, slice s+1's
      // activation fragments are read and its weight fragments widened.  After slice 2 this wave
      // waits for its copy of step i+1 and the workgroup meets at a barrier (then every wave's
      // copy of step i+1 has landed and every wave has read the stage of step i); slice 3's MFMAs
      // then cover the copy of step i+S into that stage, slice 0 of step i+1 and the weights of
      // step i+S, loaded into the slot step i has released.  Behind the copy of step i+1 are its
      // weights and S-2 later (copy, weights) batches.  Steps past the contraction (when S does
      // not divide it) copy clamped activations and multiply them by zero weights.
      static_for<S>([&](auto v) {
        __builtin_amdgcn_sched_barrier(0);
        issue_a(v, v());
        issue_w(v, v());
      });
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<kW + (S - 1) * (kA + kW)>();  // the copy of step 0
      barrier();
      __builtin_amdgcn_sched_barrier(0);
      read(I0{}, I0{}, I0{});
      cvt(I0{}, I0{}, I0{});
      const int n_steps = (KS + S - 1) / S * S;
#pragma clang loop unroll(disable)
      for (int it = 0; it < n_steps; it += S) {
        static_for<S>([&](auto v) {
          using SL = std::integral_constant<int, v()>;
          using NX = std::integral_constant<int, (v() + 1) % S>;
          const int i = it + v();
          __builtin_amdgcn_sched_barrier(0);
          read(SL{}, I1{}, I1{});
          cvt(SL{}, I1{}, I1{});
          mfma(I0{}, I0{});
          interleave();
          __builtin_amdgcn_sched_barrier(0);
          read(SL{}, I2{}, I0{});
          cvt(SL{}, I2{}, I0{});
          mfma(I1{}, I1{});
          interleave();
          __builtin_amdgcn_sched_barrier(0);
          read(SL{}, I3{}, I1{});
          cvt(SL{}, I3{}, I1{});
          mfma(I0{}, I0{});
          interleave();
          __builtin_amdgcn_sched_barrier(0);
          wait_vmcnt<kW + (S - 2) * (kA + kW)>();  // the copy of step i+1
          barrier();
          __builtin_amdgcn_sched_barrier(0);
          issue_a(SL{}, i + S);  // the stage of step i is free now
          read(NX{}, I0{}, I0{});
          cvt(NX{}, I0{}, I0{});
          mfma(I1{}, I1{});
          issue_w(SL{}, i + S);  // (slot SL's raw weights were all widened above)
          interleave();
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // no copy may still be in flight into a stage the next unit's prologue fills, and the
      // next unit's copies wait for this unit's last LDS reads
      wait_vmcnt<0>();
      barrier();
      u32x4* est = wv == 0 ? g2_lds0 : wv == 1 ? g2_lds1 : wv == 2 ? g2_lds2 : g2_lds3;
      g2_epilogue<MODE, MTA>(acc, est, wact, m0, mend, col0, lane, sc0, sc1, out, out_ld);
    };
    // an expert of a single chunk has its weight tiles read by one unit each in this launch:
    // they are loaded non-temporally, so that they do not displace the activation rows the
    // chunk's other column blocks read through the same L2
    const bool once = q >= tab.F && tab.nf[e] == 0;
    auto run = [&](auto nt) {
      switch (mt_act) {
        case 1: unit(std::integral_constant<int, 1>{}, nt); break;
        case 2: unit(std::integral_constant<int, 2>{}, nt); break;
        case 3: unit(std::integral_constant<int, 3>{}, nt); break;
        case 4: unit(std::integral_constant<int, 4>{}, nt); break;
        case 5: unit(std::integral_constant<int, 5>{}, nt); break;
        case 6: unit(std::integral_constant<int, 6>{}, nt); break;
        case 7: unit(std::integral_constant<int, 7>{}, nt); break;
        default: unit(std::integral_constant<int, 8>{}, nt); break;
      }
    };
    if (once) run(std::true_type{});
    else run(std::false_type{});
  }
}

// parts: kGemmSplitSlots partial tiles of workspace, or nullptr (tail units run whole).
// ev0, ev1: optional timestamps taken by the dispatches themselves, at the start of the GEMM
// and at the end of the last launch of the projection (the finalize, if any).
#ifndef MOE_FFN_GEMM256
#define MOE_FFN_GEMM256 1  // fp8 weights: 256-row units (0: the 128-row two-workgroup kernel)
#endif
template <int MODE, int WDT>
static void launch_gemm(const void* A, const int32_t* offsets, int E_loc, const void* W, const float* s0,
                        const float* s1, void* out, int Kd, int Nw, int out_ld, int n, GatherRows gr, float* parts,
                        hipEvent_t ev0, hipEvent_t ev1, hipStream_t stream) {
  if constexpr (WDT == MOE_FP8_E4M3 && MOE_FFN_GEMM256) {
    // (takes_gemm keeps each expert's fp8 matrix under 2^30 bytes: 32-bit weight offsets)
    constexpr auto k256 = ffn_gemm256_kernel<MODE>;
    const int n_blocks_N = (Nw + kGemmBN - 1) / kGemmBN;
    const int64_t chunks_max = (n + (int64_t)(kG2BM - 1) * E_loc) / kG2BM;
    int64_t grid = std::min<int64_t>(chunks_max * n_blocks_N, resident_workgroups<k256>(256));
    grid = (grid + 7) / 8 * 8;  // the XCD-major order needs a multiple of 8
    (void)parts;
    hipExtLaunchKernelGGL(k256, dim3((unsigned)grid), dim3(256), 0, stream, ev0, ev1, 0, (const uint16_t*)A, offsets,
                          E_loc, (const char*)W, s0, s1, (uint16_t*)out, Kd, Nw, out_ld, n_blocks_N, n, gr);
    return;
  }
  constexpr auto kernel = ffn_gemm_kernel<MODE, WDT>;
  const int n_blocks_N = (Nw + kGemmBN - 1) / kGemmBN;
  const int64_t chunks_max = (n + (int64_t)(kGemmBM - 1) * E_loc) / kGemmBM;
  int64_t grid = std::min<int64_t>(chunks_max * n_blocks_N, resident_workgroups<kernel>(256));
  grid = (grid + 7) / 8 * 8;
  if (grid > kGemmSplitSlots) parts = nullptr;
  // The down projection's units are half as long (K = I), so a split tail saves less than the
  // finalize launch and the partial tiles cost; it runs whole tail units (prefill waves of
  // 6554 / 4915 / 3277 pairs: down 4-7, 6-8 and 16-20 us faster than with the split).
  if (MODE == 1) parts = nullptr;
  hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), 0, stream, ev0, parts ? nullptr : ev1, 0,
                        (const uint16_t*)A, offsets, E_loc, (const char*)W, s0, s1, (uint16_t*)out, Kd, Nw, out_ld,
                        n_blocks_N, n, gr, parts);
  if (parts)
    hipExtLaunchKernelGGL((ffn_gemm_finalize_kernel<MODE, WDT>), dim3((unsigned)(8 * grid)), dim3(256), 0, stream,
                          nullptr, ev1, 0, offsets, E_loc, n, n_blocks_N, Kd / kBK, (int)grid, (const float*)parts, s0,
                          s1, (uint16_t*)out, Nw, out_ld);
}

// Row-chunk height: tall enough that an average expert group fits one chunk with room for
// the spread of a ragged batch (1.5x the mean group), so each weight tile is read once.
#ifndef MOE_FFN_MT
#define MOE_FFN_MT 0  // 0: choose from the batch shape
#endif
#ifndef MOE_FFN_NS_GU
#define MOE_FFN_NS_GU 2
#endif
#ifndef MOE_FFN_NS_D
#define MOE_FFN_NS_D 2
#endif
#ifndef MOE_FFN_R_GU
#define MOE_FFN_R_GU 3
#endif
#ifndef MOE_FFN_R_D
#define MOE_FFN_R_D 4
#endif
// Waves per workgroup.  A CU streams at most ~27 GB/s (its outstanding L1 misses over the
// HBM latency), so the kernel time is set by the busiest CU: at the decode shape (8 experts,
// 2880 x 2880) 6 waves x 2 strips (gate/up) and 3 waves x 2 strips (down) make 240 units,
// at most one per CU, where 4-wave units made 360 (two on some CUs) and 184.
#ifndef MOE_FFN_WV_GU
#define MOE_FFN_WV_GU 6
#endif
#ifndef MOE_FFN_WV_D
#define MOE_FFN_WV_D 3
#endif

static int pick_mt(int n, int E_loc) {
  if (MOE_FFN_MT > 0) return MOE_FFN_MT;
  const int want = (3 * n + 2 * E_loc - 1) / (2 * E_loc);
  const int mt = (want + 15) / 16;
  return mt < 2 ? 2 : (mt > 3 ? 3 : mt);
}

// Prefill-sized batches (many rows per expert) go to the MFMA-bound GEMM kernel.
#ifndef MOE_FFN_GEMM_ROWS
#define MOE_FFN_GEMM_ROWS 96  // mean rows per expert from which the GEMM kernel is used
#endif
// The fp8 down projection (K = I) takes the 256-row GEMM from fewer rows per expert: on the
// prefill wave of 1638 pairs over 32 experts (51 per expert) it runs in 90 us there against 100
// on the weight-streaming kernel, where the gate/up projection (K = H, twice the columns) is
// 8-11 us slower on the GEMM.
#ifndef MOE_FFN_GEMM_ROWS_FP8_DOWN
#define MOE_FFN_GEMM_ROWS_FP8_DOWN 48
#endif

// whether a projection over n rows takes the tiled GEMM kernel (the GEMM kernel addresses its
// activation operand with 32-bit byte offsets)
// (the tiled kernels address activations with 32-bit byte offsets, and the 256-row kernel
// an expert's weight matrix too, with zero-returning loads just past its end)
static bool takes_gemm(int n, int E_loc, int Kd, int Nw, int w_esz, const GatherRows& gr,
                       int min_rows = MOE_FFN_GEMM_ROWS) {
  const int64_t a_bytes = gr.perm ? gr.P * gr.pitch * 2 : (int64_t)n * Kd * 2;
  const int64_t w_bytes = (int64_t)Nw * Kd * w_esz;
  return MOE_FFN_MT == 0 && (int64_t)n >= (int64_t)min_rows * E_loc && a_bytes < ((int64_t)1 << 31) &&
         w_bytes < ((int64_t)1 << 30);
}

// plan: a combine plan for the streaming gate/up launch's spare workgroup (m = 0: none;
// the caller passes one only when takes_gemm is false)
template <int MODE, int WDT>
static void launch_mfma(const void* A, const int32_t* offsets, int E_loc, const void* W, const float* s0,
                        const float* s1, void* out, int Kd, int Nw, int out_ld, int n, GatherRows gr, float* parts,
                        const PlanJob& plan, const QueueIdx& qi, hipEvent_t ev0, hipEvent_t ev1,
                        hipStream_t stream) {
  constexpr int NS = MODE == 0 ? MOE_FFN_NS_GU : MOE_FFN_NS_D;
  constexpr int R = MODE == 0 ? MOE_FFN_R_GU : MOE_FFN_R_D;
  constexpr int WV = MODE == 0 ? MOE_FFN_WV_GU : MOE_FFN_WV_D;
  constexpr int min_rows = MODE == 1 && WDT == MOE_FP8_E4M3 ? MOE_FFN_GEMM_ROWS_FP8_DOWN : MOE_FFN_GEMM_ROWS;
  if (takes_gemm(n, E_loc, Kd, Nw, WDT == MOE_FP8_E4M3 ? 1 : 2, gr, min_rows)) {
    launch_gemm<MODE, WDT>(A, offsets, E_loc, W, s0, s1, out, Kd, Nw, out_ld, n, gr, parts, ev0, ev1, stream);
    return;
  }
  // (the caller passes a fused queue index only for the gate/up projection of a batch that
  // takes the weight-streaming kernel)
  const bool fq = MODE == 0 && qi.slot != nullptr;
  switch (pick_mt(n, E_loc) * 2 + (fq ? 1 : 0)) {
    case 4:
      launch_mfma_t<MODE, WDT, NS, 2, R, WV, false>(A, offsets, E_loc, W, s0, s1, out, Kd, Nw, out_ld, n, gr, plan, qi,
                                                    ev0, ev1, stream);
      break;
    case 5:
      launch_mfma_t<MODE, WDT, NS, 2, R, WV, MODE == 0>(A, offsets, E_loc, W, s0, s1, out, Kd, Nw, out_ld, n, gr, plan,
                                                        qi, ev0, ev1, stream);
      break;
    case 7:
      launch_mfma_t<MODE, WDT, NS, 3, R, WV, MODE == 0>(A, offsets, E_loc, W, s0, s1, out, Kd, Nw, out_ld, n, gr, plan,
                                                        qi, ev0, ev1, stream);
      break;
    default:
      launch_mfma_t<MODE, WDT, NS, 3, R, WV, false>(A, offsets, E_loc, W, s0, s1, out, Kd, Nw, out_ld, n, gr, plan, qi,
                                                    ev0, ev1, stream);
      break;
  }
}

}  // namespace moe

using namespace moe;

static size_t h_bytes(int64_t n, int I, int esz) { return ((size_t)n * (size_t)I * esz + 255) / 256 * 256; }
static constexpr size_t kPartAreaBytes = (size_t)kGemmSplitSlots * kGemmPartFloats * sizeof(float);

// h [n_max][I], then (for batches that can take the GEMM path) the partial tiles of its
// split tail units
extern "C" size_t moe_ffn_workspace_size(int32_t n_max, int32_t E_loc, int32_t H, int32_t I, int32_t act_dtype) {
  (void)H;
  const int esz = dtype_size(act_dtype);
  if (n_max < 0 || I < 0 || esz == 0) return 0;
  const bool gemm = act_dtype == MOE_BF16 && E_loc >= 1 && (int64_t)n_max >= (int64_t)MOE_FFN_GEMM_ROWS * E_loc;
  return h_bytes(n_max, I, esz) + (gemm ? kPartAreaBytes : 0);
}

extern "C" int moe_pack_ffn_weights(const moe_pack_args* a, hipStream_t stream) {
  if (!a) return MOE_EINVAL_NULL;
  if (a->E_loc < 1 || a->E_loc > 256 || a->H < 64 || a->I < 64) return MOE_EINVAL_SIZE;
  if (a->H % 64 || a->I % 64) return MOE_EINVAL_SHAPE;
  const int esz = dtype_size(a->w_dtype);
  if (esz == 0) return MOE_EINVAL_DTYPE;
  if (!a->wg || !a->wu || !a->wd || !a->w_gu || !a->w_d) return MOE_EINVAL_NULL;
  const int64_t per = (int64_t)a->I * a->H;
  const int64_t total = per * a->E_loc;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 g((unsigned)blocks), t(256);
#define MOE_PACK(T)                                                                                                 \
  hipLaunchKernelGGL(pack_kernel<T>, g, t, 0, stream, (const T*)a->wg, (T*)a->w_gu, a->E_loc, a->I, a->H, 1, 2 * per); \
  hipLaunchKernelGGL(pack_kernel<T>, g, t, 0, stream, (const T*)a->wu, (T*)a->w_gu, a->E_loc, a->I, a->H, 2, 2 * per); \
  hipLaunchKernelGGL(pack_kernel<T>, g, t, 0, stream, (const T*)a->wd, (T*)a->w_d, a->E_loc, a->H, a->I, 0, per);
  if (esz == 4) {
    MOE_PACK(float)
  } else if (esz == 2) {
    MOE_PACK(uint16_t)
  } else {
    MOE_PACK(uint8_t)
  }
#undef MOE_PACK
  return launch_status();
}

extern "C" int moe_expert_ffn_grouped(const moe_ffn_args* a, hipStream_t stream) {
  if (!a) return MOE_EINVAL_NULL;
  if (a->n < 0 || a->n > (1 << 24) || a->E_loc < 1 || a->E_loc > 256 || a->H < 64 || a->I < 64)
    return MOE_EINVAL_SIZE;
  if (a->H % 64 || a->I % 64) return MOE_EINVAL_SHAPE;
  const bool f32 = a->act_dtype == MOE_F32 && a->w_dtype == MOE_F32;
  const bool bf = a->act_dtype == MOE_BF16 && a->w_dtype == MOE_BF16;
  const bool f8 = a->act_dtype == MOE_BF16 && a->w_dtype == MOE_FP8_E4M3;
  if (!f32 && !bf && !f8) return MOE_EINVAL_DTYPE;
  // the queue index to enqueue with the FFN (a moe_assemble call, index only): validated like
  // moe_assemble, so that an invalid one enqueues nothing; its buffers then replace offsets
  // and the gather fields of a
  const moe_assemble_args* ix = a->index;
  if (ix) {
    const int rc = check_assemble_args(ix);
    if (rc != MOE_OK) return rc;
    if (ix->xb || ix->n != a->n || ix->E_loc != a->E_loc || ix->H != a->H || ix->act_dtype != a->act_dtype)
      return MOE_EINVAL_SIZE;
  }
  const int32_t* offsets = ix ? ix->offsets : a->offsets;
  if (!offsets) return MOE_EINVAL_NULL;
  // the combine plan to enqueue with the FFN: validated here, so that an invalid one
  // enqueues nothing; job.m > 0 when it may run inside the gate/up launch
  PlanJob job{};
  if (a->plan) {
    const int rc = combine_plan_job(a->plan, &job);
    if (rc != MOE_OK) return rc;
  }
  if (a->n == 0) {
    if (ix) {
      const int rc = moe_assemble(ix, stream);
      if (rc != MOE_OK) return rc;
    }
    if (a->plan) {
      const int rc = moe_combine_plan(a->plan, stream);
      if (rc != MOE_OK) return rc;
    }
    if (a->ev_mid) (void)hipEventRecord(a->ev_mid, stream);
    return MOE_OK;
  }
  // the rows the gate/up projection reads: the batch xb, or pool rows through the queue
  GatherRows gr{nullptr, nullptr, 0, 0, nullptr};
  const void* x_src = a->xb;
  const int32_t* g_perm = ix ? ix->perm : a->perm;
  const int32_t* g_slot = ix ? ix->slot : a->slot;
  const int32_t* g_row_slot = ix ? ix->row_slot : a->row_slot;
  const void* g_pool = ix ? ix->pool : a->pool;
  const int64_t g_P = ix ? ix->P : a->P, g_pitch = ix ? ix->pool_pitch : a->pool_pitch;
  if (g_perm || g_row_slot) {
    const int esz = dtype_size(a->act_dtype);
    if ((!g_row_slot && !g_slot) || !g_pool) return MOE_EINVAL_NULL;
    if (g_P < 1 || g_pitch < a->H) return MOE_EINVAL_SIZE;
    if (!f32 && (double)g_P * (double)g_pitch * esz >= 2147483648.0) return MOE_EINVAL_SIZE;
    if (!aligned16(g_pool) || (g_pitch * esz) % 16) return MOE_EINVAL_ALIGN;
    // (perm only marks the gather when row_slot is given; it is then never read)
    gr = GatherRows{g_perm ? g_perm : g_row_slot, g_slot, g_pitch, g_P, g_row_slot};
    x_src = g_pool;
  }
  if (!x_src || !a->w_gu || !a->w_d || !a->y) return MOE_EINVAL_NULL;
  if (f8 && (!a->s_gate || !a->s_up || !a->s_down)) return MOE_EINVAL_NULL;
  if (!aligned16(x_src) || !aligned16(a->w_gu) || !aligned16(a->w_d) || !aligned16(a->y)) return MOE_EINVAL_ALIGN;
  const GatherRows none{nullptr, nullptr, 0, 0, nullptr};
  // h is required; the partial area after it is optional (see below)
  if (!a->workspace || a->workspace_bytes < h_bytes(a->n, a->I, dtype_size(a->act_dtype))) return MOE_EWORKSPACE;
  if (!aligned16(a->workspace)) return MOE_EINVAL_ALIGN;
  const int n = a->n, H = a->H, I = a->I, E = a->E_loc;
  // partial tiles for the GEMM path's split tail, when the workspace has room for them
  // (it does when sized by moe_ffn_workspace_size for a batch of at least n rows)
  float* parts = nullptr;
  {
    const size_t off = h_bytes(n, I, dtype_size(a->act_dtype));
    if (a->workspace_bytes >= off + kPartAreaBytes) parts = (float*)((char*)a->workspace + off);
  }
  // the queue index joins the gate/up launch of the streaming kernel for queues of up to
  // kQueueFusedMax pairs, else moe_assemble runs first; the plan joins the same launch, else
  // it runs before the FFN (after the gate/up launch when that launch derives the index, since
  // the plan reads its pos)
  const bool streaming = !f32 && !takes_gemm(n, E, H, 2 * I, f8 ? 1 : 2, gr);
  QueueIdx qi{};
  bool linked = false;  // the plan's link step ran in the index launch
  if (ix && streaming && n <= kQueueFusedMax) {
    qi = QueueIdx{ix->slot, ix->expert, ix->expert_base, n, ix->P, ix->perm, ix->pos,
                  ix->counts, ix->offsets, ix->row_slot, ix->err};
  } else if (ix) {
    // the index kernel of a longer queue also links the arrivals of a list-path plan over its
    // own batch rows (the combine's link step), instead of a launch of their own
    LinkJob lj{};
    if (a->plan && a->plan->row_idx == ix->pos && a->plan->m == ix->n && assemble_links(ix->n)) {
      const int rc = combine_link_job(a->plan, &lj);
      if (rc != MOE_OK) return rc;
    }
    linked = lj.m > 0;
    const int rc = linked ? assemble_with_link(ix, lj, stream) : moe_assemble(ix, stream);
    if (rc != MOE_OK) return rc;
  }
  if (!streaming) job.m = 0;
  // (a plan that runs in the launch deriving the index reads the batch rows derived there, so
  // only a plan over the index's own pos joins it)
  if (qi.slot && a->plan && a->plan->row_idx != ix->pos) job.m = 0;
  const bool plan_after_gu = a->plan && qi.slot && job.m == 0;
  if (a->plan && job.m == 0 && !plan_after_gu && !linked) {
    const int rc = moe_combine_plan(a->plan, stream);
    if (rc != MOE_OK) return rc;
  }
  const PlanJob no_plan{};
  // the gate/up kernel's own start/stop timestamps, when asked for as a pair
  const bool ev_pair = a->ev_gu_start && a->ev_gu_stop;
  const hipEvent_t ev0 = ev_pair ? a->ev_gu_start : nullptr, ev1 = ev_pair ? a->ev_gu_stop : nullptr;
  if (f32) {
    const int64_t t1 = (int64_t)n * I, t2 = (int64_t)n * H;
    hipLaunchKernelGGL(gateup_f32_kernel, dim3((unsigned)((t1 + 255) / 256)), dim3(256), 0, stream,
                       (const float*)x_src, offsets, E, n, H, I, (const float*)a->w_gu, (float*)a->workspace, gr);
    if (a->ev_mid) (void)hipEventRecord(a->ev_mid, stream);
    hipLaunchKernelGGL(down_f32_kernel, dim3((unsigned)((t2 + 255) / 256)), dim3(256), 0, stream,
                       (const float*)a->workspace, offsets, E, n, H, I, (const float*)a->w_d, (float*)a->y);
    return launch_status();
  }
  const QueueIdx no_q{};
  if (bf) {
    launch_mfma<0, MOE_BF16>(x_src, offsets, E, a->w_gu, nullptr, nullptr, a->workspace, H, 2 * I, I, n, gr, parts, job,
                             qi, ev0, ev1, stream);
  } else {
    launch_mfma<0, MOE_FP8_E4M3>(x_src, offsets, E, a->w_gu, a->s_gate, a->s_up, a->workspace, H, 2 * I, I, n, gr,
                                 parts, job, qi, ev0, ev1, stream);
  }
  if (plan_after_gu) {
    const int rc = moe_combine_plan(a->plan, stream);
    if (rc != MOE_OK) return rc;
  }
  if (a->ev_mid) (void)hipEventRecord(a->ev_mid, stream);
  if (bf)
    launch_mfma<1, MOE_BF16>(a->workspace, offsets, E, a->w_d, nullptr, nullptr, a->y, I, H, H, n, none, parts, no_plan,
                             no_q, nullptr, nullptr, stream);
  else
    launch_mfma<1, MOE_FP8_E4M3>(a->workspace, offsets, E, a->w_d, a->s_down, nullptr, a->y, I, H, H, n, none, parts,
                                 no_plan, no_q, nullptr, nullptr, stream);
  return launch_status();
}
