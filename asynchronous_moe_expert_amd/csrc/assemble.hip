// moe_assemble: expert-grouped batch assembly from a scattered token pool.
//
// [SEP] (marsggbo, "SOSP'26 | StreamEP", section 3): tokens wait in a GPU pool, the expert
// micro-queue lists them with their metadata, and the executor turns the queue's scattered
// inputs into one contiguous batch.  Here the batch is grouped by local expert so that the
// grouped FFN sees one contiguous row range per expert.
//
// Two kernels:
//   1. index kernel (one workgroup of 1024 threads, 256 for small queues; one workgroup per
//      1024-pair segment for longer queues, see assemble_index_multi_kernel): per-expert histogram in LDS, a wave scan
//      for the exclusive offsets, then a stable scatter of queue indices.  Stability
//      inside each chunk of one pair per thread comes from a 9-bit wave "match" (ballot per
//      key bit) giving each pair its rank among equal keys of lower lanes, plus per-wave
//      counts scanned across the waves.  Integer-only, so the result is deterministic.
//   2. row gather: one 16-byte vector per thread, flattened over rows x 16-byte chunks so
//      that consecutive lanes copy consecutive bytes of a row (fully coalesced reads of each
//      pool row and writes of each batch row).
#include "common.hpp"
#include "combine_link.hpp"

namespace moe {

constexpr int kMaxElocAsm = 256;

// kAsmThreads threads: 1024, or 256 for queues of at most 256 pairs (every decode step),
// where a quarter of the waves makes each workgroup barrier cheaper.
template <int kAsmThreads>
__global__ __launch_bounds__(kAsmThreads) void assemble_index_kernel(
    int n, const int32_t* __restrict__ slot, const int32_t* __restrict__ expert, int base, int E_loc, int64_t P,
    int32_t* __restrict__ perm, int32_t* __restrict__ pos, int32_t* __restrict__ row_slot,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, uint32_t* __restrict__ err) {
  constexpr int kAsmWaves = kAsmThreads / kWave;
  __shared__ int s_run[kMaxElocAsm];
  __shared__ int s_wcnt[kAsmWaves][kMaxElocAsm + 1];
  __shared__ int s_total;
  __shared__ unsigned s_err;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  for (int e = tid; e < E_loc; e += kAsmThreads) s_run[e] = 0;
  if (tid == 0) s_err = 0u;
  __syncthreads();

  // pass 1: validate and count.  key = local expert, or kMaxElocAsm for a rejected pair or
  // past the end; the keys (and slots) of the first kCached chunks stay in registers for
  // pass 2 (one global round trip per chunk fewer)
  constexpr int kCached = 8;
  unsigned myerr = 0u;
  auto key_of = [&](int i, int& sv) {
    int key = kMaxElocAsm;
    sv = 0;
    if (i < n) {
      const int64_t s = slot[i];
      sv = (int)s;
      const int e = expert[i] - base;
      bool ok = true;
      if (s < 0 || s >= P) { myerr |= MOE_ERR_SLOT_RANGE; ok = false; }
      if (e < 0 || e >= E_loc) { myerr |= MOE_ERR_EXPERT_NONLOCAL; ok = false; }
      if (ok) key = e;
    }
    return key;
  };
  int kc[kCached], ks[kCached];
#pragma unroll
  for (int c = 0; c < kCached; ++c) {
    kc[c] = key_of(c * kAsmThreads + tid, ks[c]);
    if (kc[c] < kMaxElocAsm) atomicAdd(&s_run[kc[c]], 1);
  }
  for (int i = kCached * kAsmThreads + tid; i < n; i += kAsmThreads) {
    int sv;
    const int key = key_of(i, sv);
    if (key < kMaxElocAsm) atomicAdd(&s_run[key], 1);
  }
  if (myerr) atomicOr(&s_err, myerr);
  __syncthreads();

  // exclusive scan of the counts (wave 0; 4 experts per lane covers E_loc <= 256)
  if (wv == 0) {
    int v[4], sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = lane * 4 + k;
      v[k] = e < E_loc ? s_run[e] : 0;
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
        counts[e] = v[k];
        offsets[e] = run;
        s_run[e] = run;  // running output row of expert e
      }
      run += v[k];
    }
    if (lane == 63) {
      offsets[E_loc] = incl;
      s_total = incl;
    }
  }
  __syncthreads();

  // pass 2: stable scatter, one chunk of kAsmThreads queue entries at a time
  auto scatter = [&](int i, int key, int sv) {
    for (int x = tid; x < kAsmWaves * E_loc; x += kAsmThreads) s_wcnt[x / E_loc][x % E_loc] = 0;
    __syncthreads();
    uint64_t peers = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    if (key < kMaxElocAsm && rank == 0) s_wcnt[wv][key] = __popcll(peers);
    __syncthreads();
    if (tid < E_loc) {
      int run = s_run[tid];
#pragma unroll
      for (int w = 0; w < kAsmWaves; ++w) {
        const int cnt = s_wcnt[w][tid];
        s_wcnt[w][tid] = run;
        run += cnt;
      }
      s_run[tid] = run;
    }
    __syncthreads();
    if (key < kMaxElocAsm) {
      const int r = s_wcnt[wv][key] + rank;
      perm[r] = i;
      if (pos) pos[i] = r;
      if (row_slot) row_slot[r] = sv;
    } else if (i < n && pos) {
      pos[i] = -1;
    }
    __syncthreads();
  };
#pragma unroll
  for (int c = 0; c < kCached; ++c)
    if (c * kAsmThreads < n) scatter(c * kAsmThreads + tid, kc[c], ks[c]);
  for (int c0 = kCached * kAsmThreads; c0 < n; c0 += kAsmThreads) {
    const int i = c0 + tid;
    int key = kMaxElocAsm;  // "rejected / past the end" key
    int sv = 0;
    if (i < n) {
      const int64_t s = slot[i];
      const int e = expert[i] - base;
      sv = (int)s;
      if (s >= 0 && s < P && e >= 0 && e < E_loc) key = e;
    }
    scatter(i, key, sv);
  }
  for (int r = s_total + tid; r < n; r += kAsmThreads) {
    perm[r] = -1;
    if (row_slot) row_slot[r] = -1;
  }
  if (tid == 0 && s_err) atomicOr(err, s_err);
}

// Queues of more than one chunk: one workgroup of 1024 threads per 1024-pair segment of the
// queue.  Every workgroup counts all n keys (a few KiB of L2-resident ids per workgroup), so each
// one derives the same per-expert counts and offsets, and it also counts the keys before its own
// segment; it then scatters only its segment, stably, from running positions offsets[e] + (keys
// of expert e before the segment).  No workgroup waits for another and no scratch is needed.
// Workgroup 0 writes counts, offsets and the error bits (it sees every key).
// Each key is counted by one LDS atomic into one of kIdxCopies counters of its expert (chosen by
// lane): a Zipf-skewed queue puts a quarter of all pairs on one expert, and lanes of a wave that
// add to one address are served one after another (one counter per expert, and a second atomic
// for the keys before the segment, made this kernel 7.2 instead of 5.5 us at 6554 pairs and 11.9
// instead of 7.4 us at 16384).
constexpr int kIdxT = 1024;    // threads per workgroup = pairs per segment
constexpr int kIdxCopies = 4;  // LDS counters per expert
// link (m > 0): the combine's link step for the queue's own arrivals (arrival i = pair i, its
// batch row the pos[i] derived here): the arrival's metadata is loaded with the first keys, its
// token's state after the count, and the push made once the row is known.
__global__ __launch_bounds__(kIdxT) void assemble_index_multi_kernel(
    int n, const int32_t* __restrict__ slot, const int32_t* __restrict__ expert, int base, int E_loc, int64_t P,
    int32_t* __restrict__ perm, int32_t* __restrict__ pos, int32_t* __restrict__ row_slot,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, uint32_t* __restrict__ err, LinkJob link) {
  constexpr int kT = kIdxT, kWaves = kT / kWave, kC = kIdxCopies, kCS = kC + 1;
  __shared__ int s_bef[kMaxElocAsm * kCS];  // keys before this segment: expert e, copy c at e * kCS + c
  __shared__ int s_aft[kMaxElocAsm * kCS];  // keys from this segment on
  __shared__ int s_run[kMaxElocAsm];
  __shared__ int s_wcnt[kWaves][kMaxElocAsm + 1];
  __shared__ int s_total;
  __shared__ unsigned s_err;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seg0 = blockIdx.x * kT;
  for (int x = tid; x < E_loc * kCS; x += kT) {
    s_bef[x] = 0;
    s_aft[x] = 0;
  }
  for (int x = tid; x < kWaves * E_loc; x += kT) s_wcnt[x / E_loc][x % E_loc] = 0;
  if (tid == 0) s_err = 0u;
  __syncthreads();
  const bool linking = link.m > 0 && seg0 + tid < link.m;
  LinkIn la;
  if (linking) la = link_load_meta(link, seg0 + tid);
  // every key (validated) in batches of kU chunks whose ids are loaded before any is counted
  constexpr int kU = 8;
  const int cp = lane % kC;
  unsigned myerr = 0u;
  int my_key = kMaxElocAsm, my_slot = 0;
  for (int i0 = 0; i0 < n; i0 += kU * kT) {
    int sv[kU], ev[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * kT + tid;
      sv[u] = i < n ? slot[i] : 0;
      ev[u] = i < n ? expert[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c0 = i0 + u * kT;  // first pair of this chunk (uniform)
      if (c0 + tid < n) {
        const int e = ev[u] - base;
        bool ok = true;
        if (sv[u] < 0 || (int64_t)sv[u] >= P) { myerr |= MOE_ERR_SLOT_RANGE; ok = false; }
        if ((unsigned)e >= (unsigned)E_loc) { myerr |= MOE_ERR_EXPERT_NONLOCAL; ok = false; }
        if (ok) atomicAdd(&(c0 < seg0 ? s_bef : s_aft)[e * kCS + cp], 1);
        if (c0 == seg0) {  // this thread's own pair of the segment
          my_key = ok ? e : kMaxElocAsm;
          my_slot = sv[u];
        }
      }
    }
  }
  if (blockIdx.x == 0 && myerr) atomicOr(&s_err, myerr);
  if (linking) link_load_state(link, la);
  __syncthreads();
  // wave 0: exclusive scan of the counts (4 experts per lane covers E_loc <= 256)
  if (wv == 0) {
    int v[4], bf[4], sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = lane * 4 + k;
      v[k] = 0;
      bf[k] = 0;
      if (e < E_loc) {
#pragma unroll
        for (int c = 0; c < kC; ++c) {
          bf[k] += s_bef[e * kCS + c];
          v[k] += s_aft[e * kCS + c];
        }
        v[k] += bf[k];
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
        if (blockIdx.x == 0) {
          counts[e] = v[k];
          offsets[e] = run;
        }
        s_run[e] = run + bf[k];  // this segment's first row of expert e
      }
      run += v[k];
    }
    if (lane == 63) {
      if (blockIdx.x == 0) offsets[E_loc] = incl;
      s_total = incl;
    }
  }
  // meanwhile the other waves: this segment's stable order, i.e. each pair's rank among equal
  // keys of lower lanes from a 9-bit ballot match, and each wave's count per expert (rejected
  // pairs and lanes past n carry kMaxElocAsm)
  const int i = seg0 + tid;
  uint64_t peers = ~0ull;
#pragma unroll
  for (int b = 0; b < 9; ++b) {
    const bool bit = (my_key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  const int rank = __popcll(peers & ((1ull << lane) - 1ull));
  if (my_key < kMaxElocAsm && rank == 0) s_wcnt[wv][my_key] = __popcll(peers);
  __syncthreads();
  if (tid < E_loc) {  // each expert's first row for each wave of this segment
    int run = s_run[tid];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int cnt = s_wcnt[w][tid];
      s_wcnt[w][tid] = run;
      run += cnt;
    }
  }
  __syncthreads();
  int my_row = -1;
  if (my_key < kMaxElocAsm) {
    const int r = s_wcnt[wv][my_key] + rank;
    my_row = r;
    perm[r] = i;
    if (pos) pos[i] = r;
    if (row_slot) row_slot[r] = my_slot;
  } else if (i < n && pos) {
    pos[i] = -1;
  }
  if (linking) link_push(link, i, my_row, la);
  // rows past the accepted pairs, split over the workgroups by segment
  const int total = s_total;
  if (i < n && i >= total) {
    perm[i] = -1;
    if (row_slot) row_slot[i] = -1;
  }
  if (blockIdx.x == 0 && tid == 0 && s_err) atomicOr(err, s_err);
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const int32_t* __restrict__ perm,
                                                           const int32_t* __restrict__ slot,
                                                           const int32_t* __restrict__ n_valid_ptr,
                                                           const char* __restrict__ pool, int64_t pitch_bytes,
                                                           char* __restrict__ xb, int row_bytes, int cpr) {
  const int64_t lim = (int64_t)(*n_valid_ptr) * cpr;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < lim; g += (int64_t)gridDim.x * 256) {
    const int r = (int)(g / cpr);
    const int c = (int)(g - (int64_t)r * cpr);
    const int64_t s = slot[perm[r]];
    const uint4 v = *reinterpret_cast<const uint4*>(pool + s * pitch_bytes + (int64_t)c * 16);
    *reinterpret_cast<uint4*>(xb + (int64_t)r * row_bytes + (int64_t)c * 16) = v;
  }
}

}  // namespace moe

using namespace moe;

int moe::check_assemble_args(const moe_assemble_args* a) {
  if (!a) return MOE_EINVAL_NULL;
  if (a->n < 0 || a->n > (1 << 24) || a->E_loc < 1 || a->E_loc > kMaxElocAsm || a->H < 1 || a->P < 0 ||
      a->pool_pitch < a->H)
    return MOE_EINVAL_SIZE;
  if (a->act_dtype != MOE_F32 && a->act_dtype != MOE_BF16) return MOE_EINVAL_DTYPE;
  if (!a->counts || !a->offsets || !a->err) return MOE_EINVAL_NULL;
  const int esz = dtype_size(a->act_dtype);
  if ((a->H * esz) % 16 || (a->pool_pitch * esz) % 16) return MOE_EINVAL_ALIGN;
  if (a->n > 0) {
    if (!a->slot || !a->expert || !a->perm || !a->pool) return MOE_EINVAL_NULL;
    if (!aligned16(a->pool) || (a->xb && !aligned16(a->xb))) return MOE_EINVAL_ALIGN;
  }
  return MOE_OK;
}

// moe_assemble's launches (arguments already checked); link.m > 0 only with the multi-segment
// index kernel (n > kIdxT)
static int assemble_launch(const moe_assemble_args* a, const LinkJob& link, hipStream_t stream) {
  const int esz = dtype_size(a->act_dtype);
  const int row_bytes = a->H * esz;
  const int64_t pitch_bytes = a->pool_pitch * esz;
  if (a->n <= 256)
    hipLaunchKernelGGL(assemble_index_kernel<256>, dim3(1), dim3(256), 0, stream, a->n, a->slot, a->expert,
                       a->expert_base, a->E_loc, a->P, a->perm, a->pos, a->row_slot, a->counts, a->offsets, a->err);
  else if (a->n <= 1024)
    hipLaunchKernelGGL(assemble_index_kernel<1024>, dim3(1), dim3(1024), 0, stream, a->n, a->slot, a->expert,
                       a->expert_base, a->E_loc, a->P, a->perm, a->pos, a->row_slot, a->counts, a->offsets, a->err);
  else
    hipLaunchKernelGGL(assemble_index_multi_kernel, dim3((unsigned)((a->n + kIdxT - 1) / kIdxT)), dim3(kIdxT), 0, stream,
                       a->n, a->slot, a->expert, a->expert_base, a->E_loc, a->P, a->perm, a->pos, a->row_slot,
                       a->counts, a->offsets, a->err, link);
  if (a->n == 0 || !a->xb) return launch_status();  // no xb: the FFN gathers on load
  const int cpr = row_bytes / 16;
  const int64_t work = (int64_t)a->n * cpr;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a->perm, a->slot,
                     a->offsets + a->E_loc, (const char*)a->pool, pitch_bytes, (char*)a->xb, row_bytes, cpr);
  return launch_status();
}

extern "C" int moe_assemble(const moe_assemble_args* a, hipStream_t stream) {
  const int rc = check_assemble_args(a);
  if (rc != MOE_OK) return rc;
  return assemble_launch(a, LinkJob{}, stream);
}

bool moe::assemble_links(int n) { return n > kIdxT; }

int moe::assemble_with_link(const moe_assemble_args* a, const LinkJob& link, hipStream_t stream) {
  const int rc = check_assemble_args(a);
  if (rc != MOE_OK) return rc;
  if (!assemble_links(a->n) || link.m != a->n || !a->pos) return MOE_EINVAL_SIZE;
  return assemble_launch(a, link, stream);
}
