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
// Two kernels:
//   1. arrive: one wave per arrival.  Lane 0 validates the indices and the generation and
//      claims bit j of mask[t] with an atomic OR (a second claim of the same bit, in this
//      call or an earlier one, is a duplicate).  The row is gathered with 16-byte loads,
//      scaled by w and
//        - if this arrival completes the token and every other accepted result has
//          finished accumulating (done[t] == K-1), written straight out:
//          out[t] = RNE(acc[t] + w * row), acc[t] = 0  (the common decode case: one
//          atomic-free pass over the row);
//        - otherwise added to acc[t] with fp32 atomics; after a release fence the wave
//          bumps done[t], and the wave that brings done[t] to K finalises the token.
//   2. release: one workgroup scans the token range touched by the call (tracked in
//      span[]) in ascending order, compacts the tokens whose mask is full into rel_list
//      (deterministic order), clears their mask and advances their generation.
#include "common.hpp"

namespace moe {

constexpr int kCmbWavesPerBlock = 4;

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

template <typename TR, typename TO>
__global__ __launch_bounds__(256) void combine_arrive_kernel(
    int m, int K, int H, const TR* __restrict__ rows, int64_t row_pitch, int64_t n_rows,
    const int32_t* __restrict__ row_idx, const int32_t* __restrict__ tok, const int32_t* __restrict__ kslot,
    const float* __restrict__ wgt, const uint32_t* __restrict__ gen, float* __restrict__ acc,
    uint32_t* __restrict__ mask, uint32_t* __restrict__ done, const uint32_t* __restrict__ tgen,
    int32_t* __restrict__ span, int T_cap, TO* __restrict__ out, int64_t out_pitch, uint32_t* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kCmbWavesPerBlock + (threadIdx.x >> 6);
  if (i >= m) return;
  const int t = tok[i], j = kslot[i];
  const int64_t r = row_idx[i];
  unsigned flag = 0u;
  if (t < 0 || t >= T_cap) flag |= MOE_ERR_TOKEN_RANGE;
  if (j < 0 || j >= K) flag |= MOE_ERR_KSLOT_RANGE;
  if (r < 0 || r >= n_rows) flag |= MOE_ERR_ROW_RANGE;
  if (!flag && gen[i] != tgen[t]) flag |= MOE_ERR_STALE_GEN;
  int path = 0;  // 1: accumulate with atomics, 2: direct finalise
  if (!flag) {
    const uint32_t bit = 1u << j;
    uint32_t old = 0u;
    uint32_t d = 0u;
    if (lane == 0) {
      old = atomicOr(&mask[t], bit);
      if (!(old & bit) && __popc(old | bit) == K) d = __hip_atomic_load(&done[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    old = __shfl(old, 0);
    d = __shfl(d, 0);
    if (old & bit) {
      flag |= MOE_ERR_DUPLICATE;
    } else {
      path = (__popc(old | bit) == K && d == (uint32_t)(K - 1)) ? 2 : 1;
      if (lane == 0) {
        atomicMin(&span[0], t);
        atomicMax(&span[1], t);
      }
    }
  }
  if (flag) {
    if (lane == 0) atomicOr(err, flag);
    return;
  }
  const float w = wgt[i];
  const TR* src = rows + r * row_pitch;
  float* a = acc + (int64_t)t * H;
  TO* o = out + (int64_t)t * out_pitch;
  const int nv = H >> 3;
  if (path == 2) {
    __threadfence();  // acquire: the other K-1 results are complete in acc[t]
    for (int v = lane; v < nv; v += 64) {
      float x[8], s[8];
      RowIO<TR>::load8(src + v * 8, x);
      RowIO<float>::load8(a + v * 8, s);
#pragma unroll
      for (int k = 0; k < 8; ++k) s[k] = fmaf(w, x[k], s[k]);
      RowIO<TO>::store8(o + v * 8, s);
      const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      RowIO<float>::store8(a + v * 8, z);
    }
    if (lane == 0) __hip_atomic_store(&done[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  for (int v = lane; v < nv; v += 64) {
    float x[8];
    RowIO<TR>::load8(src + v * 8, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) unsafeAtomicAdd(a + v * 8 + k, w * x[k]);
  }
  __threadfence();  // release: this result's additions are visible before done[t] moves
  uint32_t prev = 0u;
  if (lane == 0) prev = atomicAdd(&done[t], 1u);
  prev = __shfl(prev, 0);
  if (prev != (uint32_t)(K - 1)) return;
  __threadfence();  // acquire: all K results are in acc[t]
  for (int v = lane; v < nv; v += 64) {
    float s[8];
    RowIO<float>::load8(a + v * 8, s);
    RowIO<TO>::store8(o + v * 8, s);
    const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    RowIO<float>::store8(a + v * 8, z);
  }
  if (lane == 0) __hip_atomic_store(&done[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kRelThreads = 1024;

__global__ __launch_bounds__(kRelThreads) void combine_release_kernel(int K, uint32_t* __restrict__ mask,
                                                                      uint32_t* __restrict__ tgen,
                                                                      int32_t* __restrict__ span,
                                                                      int32_t* __restrict__ rel_list,
                                                                      int32_t* __restrict__ rel_count) {
  __shared__ int s_wtot[kRelThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lo = span[0], hi = span[1];
  const uint32_t full = K >= 32 ? 0xffffffffu : ((1u << K) - 1u);
  int base = 0;
  for (int t0 = lo; t0 <= hi; t0 += kRelThreads) {  // empty when nothing was accepted
    const int t = t0 + tid;
    const bool rel = t <= hi && mask[t] == full;
    const uint64_t bal = __ballot(rel);
    if (lane == 0) s_wtot[wv] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kRelThreads / 64; ++w) {
      const int c = s_wtot[w];
      before += w < wv ? c : 0;
      total += c;
    }
    if (rel) {
      rel_list[base + before + __popcll(bal & ((1ull << lane) - 1ull))] = t;
      mask[t] = 0u;
      tgen[t] = tgen[t] + 1u;
    }
    base += total;
    __syncthreads();
  }
  if (tid == 0) {
    *rel_count = base;
    span[0] = 0x7fffffff;
    span[1] = -1;
  }
}

__global__ __launch_bounds__(256) void state_reset_kernel(float* __restrict__ acc, int64_t n_acc,
                                                          uint32_t* __restrict__ mask, uint32_t* __restrict__ done,
                                                          uint32_t* __restrict__ tgen, int32_t* __restrict__ span,
                                                          int T_cap, uint32_t gen0) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n_acc; x += stride) acc[x] = 0.f;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < T_cap; x += stride) {
    mask[x] = 0u;
    done[x] = 0u;
    tgen[x] = gen0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    span[0] = 0x7fffffff;
    span[1] = -1;
  }
}

template <typename TR, typename TO>
static void launch_arrive(const moe_combine_args* a, hipStream_t stream) {
  const moe_combine_state& s = a->state;
  const unsigned blocks = (unsigned)((a->m + kCmbWavesPerBlock - 1) / kCmbWavesPerBlock);
  hipLaunchKernelGGL((combine_arrive_kernel<TR, TO>), dim3(blocks), dim3(64 * kCmbWavesPerBlock), 0, stream, a->m,
                     a->K, s.H, (const TR*)a->rows, a->row_pitch, a->n_rows, a->row_idx, a->tok, a->kslot, a->w,
                     a->gen, s.acc, s.mask, s.done, s.tgen, s.span, s.T_cap, (TO*)a->out, a->out_pitch, a->err);
}

static int check_state(const moe_combine_state* s) {
  if (s->T_cap < 1 || s->T_cap > (1 << 30) || s->H < 8) return MOE_EINVAL_SIZE;
  if (s->H % 8) return MOE_EINVAL_SHAPE;
  if (!s->acc || !s->mask || !s->done || !s->tgen || !s->span) return MOE_EINVAL_NULL;
  if (!aligned16(s->acc)) return MOE_EINVAL_ALIGN;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_state_reset(const moe_combine_state* st, uint32_t gen0, hipStream_t stream) {
  if (!st) return MOE_EINVAL_NULL;
  const int rc = check_state(st);
  if (rc != MOE_OK) return rc;
  const int64_t n_acc = (int64_t)st->T_cap * st->H;
  int64_t blocks = (n_acc + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(state_reset_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, st->acc, n_acc, st->mask,
                     st->done, st->tgen, st->span, st->T_cap, gen0);
  return launch_status();
}

extern "C" int moe_combine_release(const moe_combine_args* a, hipStream_t stream) {
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
    const bool rb = a->row_dtype == MOE_BF16, ob = a->out_dtype == MOE_BF16;
    if (rb && ob) launch_arrive<uint16_t, uint16_t>(a, stream);
    else if (rb) launch_arrive<uint16_t, float>(a, stream);
    else if (ob) launch_arrive<float, uint16_t>(a, stream);
    else launch_arrive<float, float>(a, stream);
  }
  hipLaunchKernelGGL(combine_release_kernel, dim3(1), dim3(kRelThreads), 0, stream, a->K, a->state.mask,
                     a->state.tgen, a->state.span, a->rel_list, a->rel_count);
  return launch_status();
}
