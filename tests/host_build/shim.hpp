// Host build of device code from the HIP sources, for CPU tests only (never linked into the
// library): each workgroup's threads run as host threads and __syncthreads is a barrier over
// them, so a kernel that relies on a thread or wave reaching a point it does not reach, or on
// ordering the GPU does not give, shows up here (with AddressSanitizer, as the first bad
// access).  Only what the combine's link, merge and apply kernels use is provided.
#pragma once
#include <algorithm>
#include <condition_variable>
#include <mutex>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <cmath>
#include <thread>
#include <vector>

#include "moe_step.h"  // (the error bits; its HIP runtime header compiles on the host)

// after the HIP headers, which define these qualifiers for host code their own way (there
// __shared__ would make every thread's "local memory" a private stack array)
#undef __global__
#undef __device__
#undef __host__
#undef __forceinline__
#undef __launch_bounds__
#undef __shared__
#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static

struct HostDim { int x, y, z; };
inline thread_local HostDim threadIdx, blockIdx;
inline HostDim blockDim, gridDim;

// The barrier of the running workgroup.  Every arrival records where it came from (a
// __syncthreads line, or the end of the workgroup), and each phase checks that all threads
// came from the same place: on the GPU a workgroup whose threads reach different barriers (or
// some the end of the kernel while others wait) has no defined behaviour, and a host thread
// that ran ahead would otherwise pair with the wrong phase and read local memory early.
struct HostBarrier {
  std::vector<int> site;
  std::mutex mu;
  std::condition_variable cv;
  int n, arrived = 0;
  long gen = 0;
  explicit HostBarrier(int threads) : site(threads, 0), n(threads) {}
  void arrive_and_wait() {
    std::unique_lock<std::mutex> lk(mu);
    const long g = gen;
    if (++arrived == n) {
      for (int t = 1; t < n; ++t)
        if (site[t] != site[0]) {
          std::fprintf(stderr, "workgroup %d: thread 0 at barrier site %d, thread %d at %d\n", blockIdx.x, site[0], t,
                       site[t]);
          std::abort();
        }
      arrived = 0;
      ++gen;
      cv.notify_all();
    } else {
      cv.wait(lk, [&] { return gen != g; });
    }
  }
};
inline HostBarrier* g_host_barrier = nullptr;
inline void host_syncthreads(int line) {
  g_host_barrier->site[threadIdx.x] = line;
  g_host_barrier->arrive_and_wait();
}
#define __syncthreads() host_syncthreads(__LINE__)
inline float __uint_as_float(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
inline uint32_t __float_as_uint(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
inline float __int_as_float(int u) { float f; std::memcpy(&f, &u, 4); return f; }
inline int atomicExch(int* p, int v) { return __atomic_exchange_n(p, v, __ATOMIC_SEQ_CST); }
inline unsigned atomicOr(unsigned* p, unsigned v) { return __atomic_fetch_or(p, v, __ATOMIC_SEQ_CST); }
using std::max;
using std::min;
// (uint4, float4, int4, int2 and make_float4: the HIP vector types, from the runtime header)

namespace moe {
inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
inline uint32_t pack_bf16x2(float lo, float hi) { return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16); }
constexpr int64_t plan_list_offset(int m) { return 4 + 4 * (int64_t)m; }
}  // namespace moe

// Runs f() as a grid of `grid` workgroups of `block` threads, one workgroup at a time (its
// __shared__ statics are the workgroup's local memory).  Every thread of a workgroup must
// leave the kernel at the same point, as the device kernels here do.
template <typename F>
inline void run_grid(int grid, int block, F f) {
  blockDim = {block, 1, 1};
  gridDim = {grid, 1, 1};
  HostBarrier hb(block);
  g_host_barrier = &hb;
  std::vector<std::thread> th;
  for (int t = 0; t < block; ++t)
    th.emplace_back([&, t] {
      threadIdx = {t, 0, 0};
      for (int b = 0; b < grid; ++b) {
        blockIdx = {b, 0, 0};
        f();
        host_syncthreads(-1);  // (the end of the workgroup)
      }
    });
  for (auto& x : th) x.join();
}
