// Planning half of the combine for calls of up to kPlanMax arrivals, shared by the planning
// kernel (combine.hip) and the weight-streaming gate/up kernel (ffn.hip), which runs it in
// one extra workgroup beside its work units, so that the plan costs no launch of its own.
//
// [SEP] (marsggbo, "SOSP'26 | StreamEP") section 3: the first K-1 results of a token are
// held and the K-th releases it; [NOTES] (Steven He, inferred obligations): each top-k
// position is accepted once, tagged with the token's generation.
#pragma once

#include "common.hpp"
#include "combine_link.hpp"

namespace moe {

constexpr int kPlanThreads = 1024;
// Arrivals a single planning workgroup takes: up to 1024 the one-pass rank sort applies;
// above that a bitonic network over 2048-4096 keys costs more (30-50 us on prefill waves)
// than the linked-list path it replaces.
constexpr int kPlanMax = 1024;
constexpr int kPlanTokLimit = 1 << 20;    // states under 2^20 tokens: key = token << 12 | arrival
constexpr uint32_t kNoTok = 0xfffffu;     // token field of a rejected arrival's key
// workspace of the plan path (int32): [0] segment count, [4 + 4s ...] segment s =
// (token, first list entry, accepted arrivals, flags: 1 complete, 2 held a partial sum),
// then list[m] of (row index, weight bits): each segment's accepted arrivals in
// arrival-index order.
__host__ __device__ constexpr int64_t plan_list_offset(int m) { return 4 + 4 * (int64_t)m; }

// exclusive prefix sum over the workgroup (T threads); *total gets the sum
template <int T>
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wsum, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int x = __shfl_up(incl, d);
    if (lane >= d) incl += x;
  }
  __syncthreads();  // s_wsum is free (earlier users are done)
  if (lane == 63) s_wsum[wv] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < T / 64; ++w) {
    const int c = s_wsum[w];
    before += w < wv ? c : 0;
    total += c;
  }
  return before + incl - v;
}

// arguments of one planning pass (one moe_combine_plan call)
struct PlanJob {
  int m, K, T_cap;
  int64_t n_rows;
  const int32_t* row_idx;
  const int32_t* tok;
  const int32_t* kslot;
  const float* wgt;
  const uint32_t* gen;
  uint32_t* tgen;
  uint32_t* mask;
  int32_t* ws;
  int32_t* rel_list;
  int32_t* rel_count;
  uint32_t* err;
};

// T threads: kPlanThreads, or 256 for calls of at most 256 arrivals (every decode step), where a
// quarter of the waves makes each workgroup barrier cheaper; or the 384 threads of the decode
// gate/up launch, which runs the plan in a spare workgroup.  Takes m arrivals whose next
// power of two is at most T (m <= 256 for the 384-thread case); every thread of the
// workgroup calls it (it has workgroup barriers).
template <int T>
__device__ __forceinline__ void combine_plan_body(const PlanJob& job) {
  const int m = job.m, K = job.K, T_cap = job.T_cap;
  const int64_t n_rows = job.n_rows;
  const int32_t* __restrict__ row_idx = job.row_idx;
  const int32_t* __restrict__ tok = job.tok;
  const int32_t* __restrict__ kslot = job.kslot;
  const float* __restrict__ wgt = job.wgt;
  const uint32_t* __restrict__ gen = job.gen;
  uint32_t* __restrict__ tgen = job.tgen;
  uint32_t* __restrict__ mask = job.mask;
  int32_t* __restrict__ ws = job.ws;
  int32_t* __restrict__ rel_list = job.rel_list;
  int32_t* __restrict__ rel_count = job.rel_count;
  uint32_t* __restrict__ err = job.err;
  static_assert(T <= kPlanMax, "arrival index fits the key's 12 bits");
  __shared__ uint32_t key[T];
  __shared__ int2 s_rw[T];      // (row index, weight bits) of each arrival
  __shared__ uint32_t s_mask[T];  // mask of the arrival's token before the call
  __shared__ uint8_t s_j[T];
  __shared__ int s_wsum[T / 64];
  __shared__ unsigned s_err;
  const int tid = threadIdx.x;
  int N = 1;
  while (N < m) N <<= 1;
  if (tid == 0) s_err = 0u;
  // 1. validation, with the token's generation and mask fetched in the same round trip;
  //    key = token << 12 | arrival for an accepted candidate, kNoTok << 12 | arrival for a
  //    rejected one or padding: every key is distinct and the rejected ones sort last
  unsigned flags = 0u;
  for (int i = tid; i < N; i += T) {
    uint32_t k = (kNoTok << 12) | (uint32_t)i;
    if (i < m) {
      const int t = tok[i], j = kslot[i];
      const int64_t r = row_idx[i];
      const float w = wgt[i];
      const uint32_t g = gen[i];
      unsigned f = 0u;
      if (t < 0 || t >= T_cap) f |= MOE_ERR_TOKEN_RANGE;
      if (j < 0 || j >= K) f |= MOE_ERR_KSLOT_RANGE;
      if (r < 0 || r >= n_rows) f |= MOE_ERR_ROW_RANGE;
      if (!f) {
        const uint32_t tg = tgen[t], mk = mask[t];
        if (g != tg) f |= MOE_ERR_STALE_GEN;
        s_mask[i] = mk;
      }
      if (!f) {
        k = ((uint32_t)t << 12) | (uint32_t)i;
        s_j[i] = (uint8_t)j;
        s_rw[i] = make_int2((int)r, __float_as_int(w));
      }
      flags |= f;
    }
    key[i] = k;
  }
  __syncthreads();
  // 2. sort key[0, N) ascending (by token, then arrival index).  Keys are distinct, so each
  //    key's place is the number of smaller keys: one pass over LDS per thread.
  {
    const uint32_t k = tid < N ? key[tid] : 0u;
    int rank = 0;
    if (tid < N) {
      if (N >= 4) {  // N is a power of two
        const uint4* k4 = reinterpret_cast<const uint4*>(key);
        for (int x = 0; x < N / 4; ++x) {
          const uint4 v = k4[x];
          rank += (v.x < k) + (v.y < k) + (v.z < k) + (v.w < k);
        }
      } else {
        for (int x = 0; x < N; ++x) rank += key[x] < k;
      }
    }
    __syncthreads();
    if (tid < N) key[rank] = k;
  }
  __syncthreads();
  // 3.-5. segments, in rounds of T sorted positions (one per thread, so that
  // every segment's state load is in flight at once): a position whose token differs from
  // its predecessor's heads a segment; its thread accepts the segment's positions in
  // arrival order, updates the token's state and writes the segment record; completed
  // tokens go to the release list in segment (= ascending token) order.
  const uint32_t full = K >= 32 ? 0xffffffffu : ((1u << K) - 1u);
  int32_t* seg_rec = ws + 4;
  int2* list2 = reinterpret_cast<int2*>(ws + plan_list_offset(m));
  int n_seg = 0, n_rel = 0;
  for (int p0 = 0; p0 < N; p0 += T) {
    const int p = p0 + tid;
    bool head = false;
    uint32_t t = 0u;
    if (p < N && (key[p] >> 12) != kNoTok) {
      t = key[p] >> 12;
      head = p == 0 || (key[p - 1] >> 12) != t;
    }
    uint32_t mk = head ? s_mask[key[p] & 4095u] : 0u;
    int round_seg = 0, round_rel = 0;
    const int seg = n_seg + block_exclusive_scan<T>(head ? 1 : 0, s_wsum, round_seg);
    bool complete = false;
    if (head) {
      const bool started = mk != 0u;
      int na = 0;
      for (int x = p; x < N && (key[x] >> 12) == t; ++x) {
        const int a = (int)(key[x] & 4095u);
        const uint32_t bit = 1u << s_j[a];
        if (mk & bit) {
          flags |= MOE_ERR_DUPLICATE;
        } else {
          mk |= bit;
          list2[p + na++] = s_rw[a];
        }
      }
      complete = mk == full;
      reinterpret_cast<int4*>(seg_rec)[seg] = make_int4((int)t, p, na, (complete ? 1 : 0) | (started ? 2 : 0));
      if (complete) {
        mask[t] = 0u;
        tgen[t] = tgen[t] + 1u;
      } else {
        mask[t] = mk;
      }
    }
    const int o = n_rel + block_exclusive_scan<T>(complete ? 1 : 0, s_wsum, round_rel);
    if (complete) rel_list[o] = (int)t;
    n_seg += round_seg;
    n_rel += round_rel;
  }
  if (flags) atomicOr(&s_err, flags);
  __syncthreads();
  if (tid == 0) {
    ws[0] = n_seg;
    *rel_count = n_rel;
    if (s_err) atomicOr(err, s_err);
  }
}

// Host side (combine.hip).  Validates a combine call like moe_combine_plan; on MOE_OK,
// *job is that call's plan when it can run inside the decode gate/up launch (plan path and
// m <= kPlanFusedMax), and job->m = 0 otherwise (then the caller launches moe_combine_plan).
constexpr int kPlanFusedMax = 256;
int combine_plan_job(const moe_combine_args* a, PlanJob* job);

}  // namespace moe
