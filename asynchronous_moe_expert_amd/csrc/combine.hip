// moe_combine_release: router-weighted combine with per-token arrival tracking.
//
// [SEP] (marsggbo, "SOSP'26 | StreamEP") section 3: a token's K expert results come back
// separately; the first K-1 are held, the K-th makes the token eligible for the next
// layer; the merge is y = sum_j w_j E_j(x).  Section 6: the gather of the scattered
// result vectors is fused with the weighted merge.  [NOTES] (Steven He, "asynchronous MoE
// serving", inferred obligations): each selected contribution is accepted exactly once,
// with its weight, tagged with a reuse generation; no result may be dropped.  [CEP]
// (CascadeEP abstract / readiness tracking): state is reset only after release.
//
// Three kernels per call; none needs another workgroup's float results within a launch,
// so there are no device-scope fences (on this GPU a fence writes back and invalidates the
// XCD's whole L2) and no float atomics:
//   1. link: one thread per arrival.  Index/generation checks, then a lock-free push onto
//      the token's arrival list (head[t], next[i]); it also copies the token's mask (the
//      held positions before this call) next to the arrival.
//   2. merge: one workgroup per arrival; the workgroup of the token's first pushed arrival
//      (the list's tail) owns the token for the call.  It sorts the token's arrivals by
//      index, accepts top-k positions in that order (a position already held is a
//      duplicate), and computes
//      acc + sum w_a * row_a in fp32 in the same order (bit-reproducible).  If the token is
//      complete it writes out[t] = RNE(sum), clears mask[t], advances tgen[t] and sets its
//      release flag; otherwise it stores the partial sum back into acc[t].
//   3. release: one workgroup compacts the release flags into rel_list in ascending token
//      order (16 flags per thread per pass) and clears them.
//
// Calls of up to kPlanMax (1024) arrivals (every decode step) take a two-kernel path instead,
// with the same results bit for bit:
//   1. plan: one workgroup validates the arrivals, sorts them by (token, arrival index) in
//      LDS (rank sort), accepts top-k positions in index order per token, updates mask and
//      generation, and writes the release list (the sorted segments are already in token
//      order) and one segment record per touched token;
//   2. apply: one workgroup per segment sums held partial + w_a * row_a in index order and
//      writes the released row or the new partial sum.
// No linked lists, no per-token flag scan over the whole state, one launch fewer.
#include <algorithm>
#include <atomic>

#include "combine_plan.hpp"
#include "common.hpp"

namespace moe {

template <typename T>
struct RowIO;

template <>
struct RowIO<float> {
  static __device__ __forceinline__ void load8(const float* p, float v[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store8(float* p, const float v[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

template <>
struct RowIO<uint16_t> {
  static __device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store8(uint16_t* p, const float v[8]) {
    uint4 a;
    a.x = pack_bf16x2(v[0], v[1]);
    a.y = pack_bf16x2(v[2], v[3]);
    a.z = pack_bf16x2(v[4], v[5]);
    a.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = a;
  }
};

// apply workgroup: 384 threads cover a 2880-wide bf16 row (360 vectors of 8) in one pass
// (256 threads took two for 104 of them: decode combine 7.5 -> 6.7 us)
constexpr int kCmbThreads = 384;
#ifndef MOE_MERGE_THREADS
#define MOE_MERGE_THREADS 256
#endif
constexpr int kMergeThreads = MOE_MERGE_THREADS;  // merge workgroup (one per arrival)
constexpr int kMaxChain = 64;  // arrivals of one token handled per pass of the merge
constexpr int kMergeVec = 4;   // 8-element vectors per thread loaded in one batch (rows up to 8192 wide)
constexpr int kRowBatch = 4;   // result rows of one token loaded before they are summed (list and plan paths)

// Kernel 1: one thread per arrival: the link step (combine_link.hpp) with the arrival's batch
// row from row_idx.
__global__ __launch_bounds__(256) void combine_link_kernel(LinkJob j, const int32_t* __restrict__ row_idx) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= j.m) return;
  LinkIn a = link_load_meta(j, i);
  const int64_t r = row_idx[i];
  link_load_state(j, a);
  link_push(j, i, r, a);
}

// Kernel 2: one workgroup per arrival; the workgroup of the token's first pushed arrival (the
// one whose list link is -1: exactly one per touched token) owns the token for this call, all
// others exit after their first round trip.  The owner sorts the token's arrivals by index,
// accepts top-k positions in that order (a repeat of a held position is a duplicate), and
// sums acc + w_a * row_a in the same order in fp32, so results do not depend on scheduling.
// acc[t] is only read while the token holds earlier results (mask != 0): a fresh token starts
// from zero.  The owner loads the list head together with its own result row and the held
// sum, so a token's only arrival of the call (every token of a prefill wave) costs two
// dependent round trips (its metadata, then head and rows) instead of three.
// Empty asm statements that read values: every load those values come from is then issued, and
// waited for, at that point.  Without them the compiler sinks loads past the branches that
// follow (each value is used on one side only), and the merge's one round trip for an
// arrival's metadata became four dependent ones, its rows one per 256 vectors.
template <int VPT>
__device__ __forceinline__ void hold_rows(const float (&s)[VPT][8], const float (&x)[VPT][8], int h) {
  if constexpr (VPT == 1) {
    asm volatile("" ::"v"(s[0][0]), "v"(s[0][4]), "v"(x[0][0]), "s"(h));
  } else if constexpr (VPT == 2) {
    asm volatile("" ::"v"(s[0][0]), "v"(s[0][4]), "v"(x[0][0]), "v"(s[1][0]), "v"(s[1][4]), "v"(x[1][0]), "s"(h));
  } else {
    static_assert(VPT == 4, "1, 2 or 4 vectors per thread");
    asm volatile("" ::"v"(s[0][0]), "v"(s[0][4]), "v"(x[0][0]), "v"(s[1][0]), "v"(s[1][4]), "v"(x[1][0]),
                 "v"(s[2][0]), "v"(s[2][4]), "v"(x[2][0]), "v"(s[3][0]), "v"(s[3][4]), "v"(x[3][0]), "s"(h));
  }
}

// VPT: 8-element vectors per thread of a row when the whole row fits one batch of loads (1, 2
// or 4: the host picks the smallest that covers H / 8 vectors), else 0.  Vector indices past the
// row are clamped to its last vector, so that every load of a batch is issued, unconditionally,
// before the first is used; their values are never stored.
template <typename TR, typename TO, int VPT>
__global__ __launch_bounds__(kMergeThreads) void combine_merge_kernel(
    int K, int H, const TR* __restrict__ rows, int64_t row_pitch, const int32_t* __restrict__ row_idx,
    const int32_t* __restrict__ tok, const int32_t* __restrict__ kslot, const float* __restrict__ wgt,
    float* __restrict__ acc, uint32_t* __restrict__ mask, uint32_t* __restrict__ tgen,
    uint8_t* __restrict__ rflag, int32_t* __restrict__ head, const int32_t* __restrict__ next,
    const uint32_t* __restrict__ mpre, TO* __restrict__ out, int64_t out_pitch, uint32_t* __restrict__ err) {
  __shared__ int s_list[kMaxChain];
  __shared__ int s_buf[kMaxChain];
  __shared__ int s_n, s_more, s_first;
  __shared__ uint32_t s_mask1;
  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  // everything indexed by the arrival in one round trip (all in range: i < m)
  int nx = next[i];
  const int t = tok[i];
  const int j_i = kslot[i];
  const float w_i = wgt[i];
  const int r32 = row_idx[i];
  const uint32_t m_t = mpre[i];
  // (the kernel arguments the owner needs next are fetched in the same round trip; nx is an
  // in/out operand so that the test below cannot be scheduled between these loads)
  asm volatile("" : "+s"(nx) : "s"(t), "s"(j_i), "s"(w_i), "s"(r32), "s"(m_t), "s"(rows), "s"(acc), "s"(head),
               "s"(out), "s"(row_pitch), "s"(out_pitch), "s"(H), "s"(K));
  const int64_t r_i = r32;
  if (nx != -1) return;  // rejected by the range/generation checks (-2), or not the tail
  const uint32_t full = K >= 32 ? 0xffffffffu : ((1u << K) - 1u);
  float* a = acc + (int64_t)t * H;
  TO* o = out + (int64_t)t * out_pitch;
  const int nv = H >> 3;
  const bool started = m_t != 0u;  // acc[t] holds earlier results
  if constexpr (VPT > 0) {
    // the held sum and this arrival's row are loaded with the list head, before it is known
    // whether other arrivals joined the list
    const TR* x_row = rows + r_i * row_pitch;
    int vq[VPT];
#pragma unroll
    for (int q = 0; q < VPT; ++q) vq[q] = min(tid + q * kMergeThreads, nv - 1);
    float sum[VPT][8], x[VPT][8];
    if (started) {
#pragma unroll
      for (int q = 0; q < VPT; ++q) RowIO<float>::load8(a + vq[q] * 8, sum[q]);
    } else {
#pragma unroll
      for (int q = 0; q < VPT; ++q)
#pragma unroll
        for (int k = 0; k < 8; ++k) sum[q][k] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < VPT; ++q) RowIO<TR>::load8(x_row + vq[q] * 8, x[q]);
    const int h_t = head[t];
    hold_rows<VPT>(sum, x, h_t);
    if (h_t == i) {
      // the token's only arrival of this call: no list to walk or sort, the same accept rule
      // and the same fp32 operations as below
      const uint32_t bit = 1u << j_i;
      const bool dup = (m_t & bit) != 0u;
      const uint32_t m_new = m_t | bit;
      const bool complete = !dup && m_new == full;
      if (!dup) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
          if (tid + q * kMergeThreads < nv) {
#pragma unroll
            for (int k = 0; k < 8; ++k) sum[q][k] = fmaf(w_i, x[q][k], sum[q][k]);
            if (complete) RowIO<TO>::store8(o + vq[q] * 8, sum[q]);
            else RowIO<float>::store8(a + vq[q] * 8, sum[q]);
          }
        }
      }
      // every wave has read head[t] (its branch above needed the value) before thread 0 resets
      // it: a wave that read the reset value would take the list path below alone
      __syncthreads();
      if (tid == 0) {
        if (dup) atomicOr(err, MOE_ERR_DUPLICATE);
        head[t] = -1;
        if (complete) {
          mask[t] = 0u;
          tgen[t] = tgen[t] + 1u;
          rflag[t] = 1;
        } else {
          mask[t] = m_new;
        }
      }
      return;
    }
  }
  const int cursor = head[t];  // list head (the newest arrival)
  int lo = -1;      // arrivals with index <= lo are already merged
  bool have = false;  // acc values of this call live in `a` (not yet in registers)
  uint32_t m_now = m_t;
  while (true) {
    // collect the next batch of up to kMaxChain arrivals with the smallest indices > lo
    if (tid == 0) {
      int n = 0, more = 0, c = cursor;
      // the list is in push order; walk all of it, keep the kMaxChain smallest above lo
      int* buf = s_buf;
      while (c >= 0) {
        if (c > lo) {
          if (n < kMaxChain) {
            buf[n++] = c;
          } else {
            int mx = 0;
            for (int q = 1; q < n; ++q) mx = buf[q] > buf[mx] ? q : mx;
            if (c < buf[mx]) buf[mx] = c;
            more = 1;
          }
        }
        c = next[c];
      }
      for (int q = 1; q < n; ++q) {  // insertion sort, ascending arrival index
        const int v = buf[q];
        int p = q - 1;
        while (p >= 0 && buf[p] > v) {
          buf[p + 1] = buf[p];
          --p;
        }
        buf[p + 1] = v;
      }
      // accept in index order; duplicates of held positions are rejected
      uint32_t mk = m_now;
      unsigned flag = 0u;
      int na = 0;
      for (int q = 0; q < n; ++q) {
        const uint32_t bit = 1u << kslot[buf[q]];
        if (mk & bit) {
          flag |= MOE_ERR_DUPLICATE;
        } else {
          mk |= bit;
          s_list[na++] = buf[q];
        }
      }
      if (flag) atomicOr(err, flag);
      s_n = na;
      s_more = more;
      s_first = n ? buf[n - 1] : lo;
      s_mask1 = mk;
    }
    __syncthreads();
    const int na = s_n;
    const bool more = s_more;
    const uint32_t m_new = s_mask1;
    const bool complete = !more && m_new == full;
    for (int v = tid; v < nv; v += kMergeThreads) {
      float sum[8];
      if (started || have) {
        RowIO<float>::load8(a + v * 8, sum);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) sum[k] = 0.f;
      }
      // kRowBatch rows in flight at a time (the batch's last slots repeat its last row and are
      // not added), summed in arrival-index order
      for (int q0 = 0; q0 < na; q0 += kRowBatch) {
        float x[kRowBatch][8], w[kRowBatch];
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
          const int arr = s_list[min(q0 + u, na - 1)];
          w[u] = wgt[arr];
          RowIO<TR>::load8(rows + (int64_t)row_idx[arr] * row_pitch + v * 8, x[u]);
        }
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
          if (q0 + u < na) {
#pragma unroll
            for (int k = 0; k < 8; ++k) sum[k] = fmaf(w[u], x[u][k], sum[k]);
          }
        }
      }
      if (complete) RowIO<TO>::store8(o + v * 8, sum);
      else RowIO<float>::store8(a + v * 8, sum);
    }
    have = have || na > 0;
    m_now = m_new;
    lo = s_first;
    __syncthreads();
    if (!more) break;
  }
  if (tid == 0) {
    head[t] = -1;
    if (m_now == full) {
      mask[t] = 0u;
      tgen[t] = tgen[t] + 1u;
      rflag[t] = 1;
    } else {
      mask[t] = m_now;
    }
  }
}

constexpr int kRelThreads = 1024;

// Kernel 3: ascending compaction of the tokens whose release flag is set: 16 flags per
// thread per pass (one 16-byte load), a workgroup-wide exclusive scan of the per-thread
// counts, then each thread writes its tokens in order and clears their flags.
// Only tokens that this call's arrivals name can hold a flag, so the scan covers the 16-token
// groups from the smallest to the largest such token (clamped into the state) rather than
// the whole state.
__global__ __launch_bounds__(kRelThreads) void combine_release_kernel(int T_cap, int m, const int32_t* __restrict__ tok,
                                                                      uint8_t* __restrict__ rflag,
                                                                      int32_t* __restrict__ rel_list,
                                                                      int32_t* __restrict__ rel_count) {
  __shared__ int s_wtot[kRelThreads / 64];
  __shared__ int s_lo[kRelThreads / 64], s_hi[kRelThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int lo = T_cap, hi = -1;
  // (eight loads in flight per thread: one round trip per 8192 arrivals; m >= 1 here, as the
  // loop does not run for m = 0)
  for (int x0 = 0; x0 < m; x0 += 8 * kRelThreads) {
    int tv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      tv[u] = tok[min(x0 + u * kRelThreads + tid, m - 1)];  // (unconditional: no wait between the loads)
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (x0 + u * kRelThreads + tid < m) {
        const int t = min(max(tv[u], 0), T_cap - 1);
        lo = min(lo, t);
        hi = max(hi, t);
      }
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    lo = min(lo, __shfl_xor(lo, d));
    hi = max(hi, __shfl_xor(hi, d));
  }
  if (lane == 0) {
    s_lo[wv] = lo;
    s_hi[wv] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kRelThreads / 64; ++w) {
    lo = min(lo, s_lo[w]);
    hi = max(hi, s_hi[w]);
  }
  const int vlo = hi < 0 ? 0 : lo >> 4;
  const int nvec = hi < 0 ? 0 : (hi >> 4) + 1;
  int base = 0;
  for (int v0 = vlo; v0 < nvec; v0 += kRelThreads) {
    const int v = v0 + tid;
    uint4 f = make_uint4(0u, 0u, 0u, 0u);
    if (v < nvec) f = reinterpret_cast<const uint4*>(rflag)[v];
    const uint32_t fw[4] = {f.x, f.y, f.z, f.w};
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) cnt += __popc(fw[k] & 0x01010101u);
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int x = __shfl_up(incl, d);
      if (lane >= d) incl += x;
    }
    if (lane == 63) s_wtot[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kRelThreads / 64; ++w) {
      const int c = s_wtot[w];
      before += w < wv ? c : 0;
      total += c;
    }
    if (cnt) {
      int o = base + before + incl - cnt;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if ((fw[k >> 2] >> (8 * (k & 3))) & 1u) {
          const int t = v * 16 + k;
          rel_list[o++] = t;
        }
      }
      reinterpret_cast<uint4*>(rflag)[v] = make_uint4(0u, 0u, 0u, 0u);
    }
    base += total;
    __syncthreads();
  }
  if (tid == 0) *rel_count = base;
}

__global__ __launch_bounds__(256) void state_reset_kernel(float* __restrict__ acc, int64_t n_acc,
                                                          uint32_t* __restrict__ mask, int32_t* __restrict__ head,
                                                          uint32_t* __restrict__ tgen, uint8_t* __restrict__ rflag,
                                                          int T_cap, uint32_t gen0) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n_acc; x += stride) acc[x] = 0.f;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < T_cap; x += stride) {
    mask[x] = 0u;
    head[x] = -1;
    tgen[x] = gen0;
  }
  const int64_t nf = ((int64_t)T_cap + 15) / 16 * 16;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < nf; x += stride) rflag[x] = 0;
}


// ------------------------------------------------------------------ two-kernel path
// T threads: kPlanThreads, or 256 for calls of at most 256 arrivals (every decode step).
template <int T>
__global__ __launch_bounds__(T) void combine_plan_kernel(PlanJob job) {
  combine_plan_body<T>(job);
}

// One workgroup per segment of the plan: held partial sum (if any) plus the accepted
// arrivals' w_a * row_a in arrival-index order, fp32 (the same order and operations as the
// merge kernel, so both paths give the same bits).
template <typename TR, typename TO>
__global__ __launch_bounds__(kCmbThreads) void combine_apply_kernel(int H, const TR* __restrict__ rows,
                                                                    int64_t row_pitch, float* __restrict__ acc,
                                                                    const int32_t* __restrict__ ws, int m,
                                                                    TO* __restrict__ out, int64_t out_pitch) {
  __shared__ float s_w[32];
  __shared__ int64_t s_row[32];
  const int sidx = blockIdx.x, tid = threadIdx.x;
  // the segment count and this workgroup's record in one round trip (the record slot exists for
  // every workgroup: the grid is at most m); cnt is an in/out asm operand so that the test below
  // cannot be scheduled between the two loads
  int cnt = ws[0];
  const int4 sg = reinterpret_cast<const int4*>(ws + 4)[sidx];
  asm volatile("" : "+s"(cnt) : "s"(sg.x), "s"(sg.y), "s"(sg.z), "s"(sg.w), "s"(H), "s"(m), "s"(acc), "s"(rows),
               "s"(row_pitch), "s"(out), "s"(out_pitch));
  if (sidx >= cnt) return;
  const int t = sg.x, na = sg.z;
  const bool complete = sg.w & 1, started = sg.w & 2;
  float* at = acc + (int64_t)t * H;
  TO* o = out + (int64_t)t * out_pitch;
  const int nv = H >> 3;
  // this thread's first vector of the held sum is loaded with the list entries (the barrier
  // below waits for both)
  float sum0[8];
  if (started && tid < nv) {
    RowIO<float>::load8(at + tid * 8, sum0);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) sum0[k] = 0.f;
  }
  if (tid < na) {
    const int2 rw = reinterpret_cast<const int2*>(ws + plan_list_offset(m))[sg.y + tid];
    s_row[tid] = rw.x;
    s_w[tid] = __int_as_float(rw.y);
  }
  __syncthreads();
  for (int v = tid; v < nv; v += kCmbThreads) {
    float sum[8];
    if (v == tid) {
#pragma unroll
      for (int k = 0; k < 8; ++k) sum[k] = sum0[k];
    } else if (started) {
      RowIO<float>::load8(at + v * 8, sum);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) sum[k] = 0.f;
    }
    // kRowBatch rows in flight at a time (the batch's last slots repeat its last row and are not
    // added), summed in arrival-index order
    for (int q0 = 0; q0 < na; q0 += kRowBatch) {
      float x[kRowBatch][8];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) RowIO<TR>::load8(rows + s_row[min(q0 + u, na - 1)] * row_pitch + v * 8, x[u]);
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        if (q0 + u < na) {
          const float w = s_w[q0 + u];
#pragma unroll
          for (int k = 0; k < 8; ++k) sum[k] = fmaf(w, x[u][k], sum[k]);
        }
      }
    }
    if (complete) RowIO<TO>::store8(o + v * 8, sum);
    else RowIO<float>::store8(at + v * 8, sum);
  }
}

template <typename TR, typename TO>
static void launch_apply(const moe_combine_args* a, hipStream_t stream) {
  const moe_combine_state& s = a->state;
  const int grid = std::min(a->m, s.T_cap);
  hipLaunchKernelGGL((combine_apply_kernel<TR, TO>), dim3((unsigned)grid), dim3(kCmbThreads), 0, stream, s.H,
                     (const TR*)a->rows, a->row_pitch, s.acc, (const int32_t*)a->workspace, a->m,
                     (TO*)a->out, a->out_pitch);
}

template <typename TR, typename TO, int VPT>
static void launch_merge_vpt(const moe_combine_args* a, hipStream_t stream) {
  const moe_combine_state& s = a->state;
  hipLaunchKernelGGL((combine_merge_kernel<TR, TO, VPT>), dim3((unsigned)a->m), dim3(kMergeThreads), 0, stream, a->K,
                     s.H, (const TR*)a->rows, a->row_pitch, a->row_idx, a->tok, a->kslot, a->w, s.acc, s.mask, s.tgen,
                     s.rflag, s.head, (const int32_t*)a->workspace, (const uint32_t*)a->workspace + a->m, (TO*)a->out,
                     a->out_pitch, a->err);
}

template <typename TR, typename TO>
static void launch_merge(const moe_combine_args* a, hipStream_t stream) {
  const int vpt = (a->state.H / 8 + kMergeThreads - 1) / kMergeThreads;
  if (vpt <= 1) launch_merge_vpt<TR, TO, 1>(a, stream);
  else if (vpt <= 2) launch_merge_vpt<TR, TO, 2>(a, stream);
  else if (vpt <= kMergeVec) launch_merge_vpt<TR, TO, kMergeVec>(a, stream);
  else launch_merge_vpt<TR, TO, 0>(a, stream);
}

static int check_state(const moe_combine_state* s) {
  if (s->T_cap < 1 || s->T_cap > (1 << 30) || s->H < 8) return MOE_EINVAL_SIZE;
  if (s->H % 8) return MOE_EINVAL_SHAPE;
  if (!s->acc || !s->mask || !s->head || !s->tgen || !s->rflag) return MOE_EINVAL_NULL;
  if (!aligned16(s->acc) || !aligned16(s->rflag)) return MOE_EINVAL_ALIGN;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_combine_workspace_size(int32_t m_max) {
  // the larger of the two paths' needs: next[m] and the tokens' masks before the call (list
  // path), and the plan records
  if (m_max <= 0) return 16;
  const size_t plan = (size_t)plan_list_offset(m_max) * 4 + (size_t)m_max * 8;
  return (std::max(plan, (size_t)m_max * 8) + 15) / 16 * 16;
}

extern "C" int moe_state_reset(const moe_combine_state* st, uint32_t gen0, hipStream_t stream) {
  if (!st) return MOE_EINVAL_NULL;
  const int rc = check_state(st);
  if (rc != MOE_OK) return rc;
  const int64_t n_acc = (int64_t)st->T_cap * st->H;
  int64_t blocks = (n_acc + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(state_reset_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, st->acc, n_acc, st->mask,
                     st->head, st->tgen, st->rflag, st->T_cap, gen0);
  return launch_status();
}

// Argument checks shared by the combine entry points (host side, before any launch).
static int check_combine(const moe_combine_args* a) {
  if (!a) return MOE_EINVAL_NULL;
  const int rc = check_state(&a->state);
  if (rc != MOE_OK) return rc;
  if (a->m < 0 || a->m > (1 << 24) || a->K < 1 || a->K > 32 || a->n_rows < 0) return MOE_EINVAL_SIZE;
  if ((a->row_dtype != MOE_F32 && a->row_dtype != MOE_BF16) || (a->out_dtype != MOE_F32 && a->out_dtype != MOE_BF16))
    return MOE_EINVAL_DTYPE;
  if (!a->rel_list || !a->rel_count || !a->err) return MOE_EINVAL_NULL;
  if (a->m > 0) {
    if (!a->row_idx || !a->tok || !a->kslot || !a->w || !a->gen || !a->out) return MOE_EINVAL_NULL;
    if (a->n_rows > 0 && !a->rows) return MOE_EINVAL_NULL;
    const int rs = dtype_size(a->row_dtype), os = dtype_size(a->out_dtype);
    if (a->row_pitch < a->state.H || a->out_pitch < a->state.H) return MOE_EINVAL_SIZE;
    if ((a->row_pitch * rs) % 16 || (a->out_pitch * os) % 16 || !aligned16(a->out) ||
        (a->rows && !aligned16(a->rows)))
      return MOE_EINVAL_ALIGN;
    if (!a->workspace || a->workspace_bytes < moe_combine_workspace_size(a->m)) return MOE_EWORKSPACE;
    if (!aligned16(a->workspace)) return MOE_EINVAL_ALIGN;
  }
  return MOE_OK;
}

static bool plan_path(const moe_combine_args* a) {
  return a->m > 0 && a->m <= kPlanMax && a->state.T_cap < kPlanTokLimit;
}

static PlanJob make_plan_job(const moe_combine_args* a) {
  const moe_combine_state& s = a->state;
  PlanJob j;
  j.m = a->m;
  j.K = a->K;
  j.T_cap = s.T_cap;
  j.n_rows = a->n_rows;
  j.row_idx = a->row_idx;
  j.tok = a->tok;
  j.kslot = a->kslot;
  j.wgt = a->w;
  j.gen = a->gen;
  j.tgen = s.tgen;
  j.mask = s.mask;
  j.ws = (int32_t*)a->workspace;
  j.rel_list = a->rel_list;
  j.rel_count = a->rel_count;
  j.err = a->err;
  return j;
}

// the list path's link step: next[m] and mpre[m] at the start of the workspace
static LinkJob make_link_job(const moe_combine_args* a) {
  const moe_combine_state& s = a->state;
  LinkJob j;
  j.m = a->m;
  j.K = a->K;
  j.T_cap = s.T_cap;
  j.n_rows = a->n_rows;
  j.tok = a->tok;
  j.kslot = a->kslot;
  j.gen = a->gen;
  j.tgen = s.tgen;
  j.mask = s.mask;
  j.head = s.head;
  j.next = (int32_t*)a->workspace;
  j.mpre = (uint32_t*)a->workspace + a->m;
  j.err = a->err;
  return j;
}

int moe::combine_link_job(const moe_combine_args* a, LinkJob* job) {
  const int rc = check_combine(a);
  if (rc != MOE_OK) return rc;
  *job = LinkJob{};
  if (a->m > 0 && !plan_path(a)) *job = make_link_job(a);
  return MOE_OK;
}

int moe::combine_plan_job(const moe_combine_args* a, PlanJob* job) {
  const int rc = check_combine(a);
  if (rc != MOE_OK) return rc;
  *job = make_plan_job(a);
  if (!plan_path(a) || a->m > kPlanFusedMax) job->m = 0;
  return MOE_OK;
}

extern "C" int moe_combine_plan(const moe_combine_args* a, hipStream_t stream) {
  const int rc = check_combine(a);
  if (rc != MOE_OK) return rc;
  const moe_combine_state& s = a->state;
  if (plan_path(a)) {
    const PlanJob job = make_plan_job(a);
    if (a->m <= 256)
      hipLaunchKernelGGL(combine_plan_kernel<256>, dim3(1), dim3(256), 0, stream, job);
    else
      hipLaunchKernelGGL(combine_plan_kernel<kPlanThreads>, dim3(1), dim3(kPlanThreads), 0, stream, job);
  } else if (a->m > 0) {
    hipLaunchKernelGGL(combine_link_kernel, dim3((unsigned)((a->m + 255) / 256)), dim3(256), 0, stream,
                       make_link_job(a), a->row_idx);
  }
  return launch_status();
}

extern "C" int moe_combine_apply(const moe_combine_args* a, hipStream_t stream) {
  const int rc = check_combine(a);
  if (rc != MOE_OK) return rc;
  const bool rb = a->row_dtype == MOE_BF16, ob = a->out_dtype == MOE_BF16;
  if (plan_path(a)) {
    if (rb && ob) launch_apply<uint16_t, uint16_t>(a, stream);
    else if (rb) launch_apply<uint16_t, float>(a, stream);
    else if (ob) launch_apply<float, uint16_t>(a, stream);
    else launch_apply<float, float>(a, stream);
    return launch_status();
  }
  if (a->m > 0) {
    if (rb && ob) launch_merge<uint16_t, uint16_t>(a, stream);
    else if (rb) launch_merge<uint16_t, float>(a, stream);
    else if (ob) launch_merge<float, uint16_t>(a, stream);
    else launch_merge<float, float>(a, stream);
  }
  hipLaunchKernelGGL(combine_release_kernel, dim3(1), dim3(kRelThreads), 0, stream, a->state.T_cap, a->m, a->tok,
                     a->state.rflag, a->rel_list, a->rel_count);
  return launch_status();
}

extern "C" int moe_combine_release(const moe_combine_args* a, hipStream_t stream) {
  const int rc = moe_combine_plan(a, stream);
  if (rc != MOE_OK) return rc;
  return moe_combine_apply(a, stream);
}

// ------------------------------------------------------------ allocation-free variant
// For callers that cannot allocate (code under graph capture, serving loops that forbid
// hipMalloc): moe_combine_release with the scratch in a library-owned device array instead of
// the caller's workspace.  The array is sized for kStaticMaxArrivals arrivals; each device
// holds its own copy, at an address taken once per device with hipGetSymbolAddress (the
// array's name is only a host-side stand-in and is never passed to a kernel).
constexpr int kStaticMaxArrivals = 1 << 17;
constexpr size_t kStaticScratchBytes = (16 + 24 * (size_t)kStaticMaxArrivals + 15) / 16 * 16;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDev = 64;
std::atomic<void*> g_scratch[kMaxScratchDev];  // per device: the address of its copy of `scratch`

// The device address of the current device's scratch array (looked up on first use with that
// device current); nullptr with *rc set on failure.
void* device_scratch(int* rc) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDev) {
    *rc = MOE_ELAUNCH;
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
    *rc = MOE_ELAUNCH;
    return nullptr;
  }
  g_scratch[dev].store(q, std::memory_order_release);  // racing first calls store the same address
  return q;
}
}  // namespace

extern "C" size_t moe_combine_noalloc_max_arrivals(void) { return (size_t)kStaticMaxArrivals; }

extern "C" int moe_combine_release_noalloc(const moe_combine_args* a, hipStream_t stream) {
  if (!a) return MOE_EINVAL_NULL;
  if (a->m > kStaticMaxArrivals) return MOE_ESCRATCH;
  int rc = MOE_OK;
  void* ws = device_scratch(&rc);
  if (!ws) return rc;
  static_assert(kStaticScratchBytes >= 16 + 24 * (size_t)kStaticMaxArrivals, "scratch holds the plan path's records");
  moe_combine_args b = *a;
  b.workspace = ws;  // every word of it that a call reads was written earlier in the same call
  b.workspace_bytes = kStaticScratchBytes;
  return moe_combine_release(&b, stream);
}
