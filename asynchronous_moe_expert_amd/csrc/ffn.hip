// moe_expert_ffn_grouped: per-expert SwiGLU FFN over ragged, expert-grouped batch rows.
//
// What is computed ([SEP] section 3, "run the expert computation on the assembled batch";
// the pages leave the FFN form open, a bias-free SwiGLU is used):
//     y_r = Wd_e ( silu(Wg_e x_r) * (Wu_e x_r) )   for rows r of expert e
//
// Design (gfx950):
//   * Two launches: gate/up GEMM with the SwiGLU epilogue (writes h), then the down GEMM.
//   * Work unit = (row chunk of <= 64 rows of one expert, 64 packed output columns).  The
//     chunk list is derived on the device from `offsets`, so ragged and empty experts need
//     no host round trip; the grid is sized for the worst case and surplus workgroups exit.
//   * Each workgroup (4 waves) splits the contraction over its waves (k-steps w, w+4, ...),
//     streams the 64-column weight tile exactly once from HBM straight into registers
//     (packed layout: one contiguous 1 KiB run per wave load), and reduces the four partial
//     tiles through LDS.  At decode sizes (tens of rows per expert) the step is bound by
//     streaming the expert weights, so the design goal is all CUs reading disjoint weight
//     bytes with deep load queues; MFMA v_mfma_f32_16x16x32_bf16 does the math.
//   * The contraction order inside a 64-wide k-step is permuted (lane group g takes 16
//     consecutive k, split over two MFMAs) so that an activation row is read as 32-byte
//     runs; the packed weight layout applies the same permutation, so the sums are exact
//     dot products over all k.
//   * fp8 e4m3 weights are widened to bf16 in registers (exact: every e4m3 value is a
//     bf16 value) and the per-row scale is applied to the fp32 result in the epilogue.
//   * Workgroup ids are remapped so that each XCD gets a contiguous range of work units:
//     chunks sharing a weight tile run on one XCD, back to back (L2 reuse for big experts).
#include "common.hpp"

namespace moe {

constexpr int kBK = 64;        // contraction per k-step
constexpr int kFfnWaves = 4;
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

// --------------------------------------------------------------- expert lookup helpers
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int E_loc, int r) {
  for (int e = 0; e < E_loc; ++e)
    if (r >= offsets[e] && r < offsets[e + 1]) return e;
  return -1;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ------------------------------------------------------------------------- fp32 path
// Small-shape path (fp32 activations and weights): one thread per output element.
__global__ __launch_bounds__(256) void gateup_f32_kernel(const float* __restrict__ xb, const int32_t* __restrict__ offsets,
                                                         int E_loc, int n, int H, int I, const float* __restrict__ wgu,
                                                         float* __restrict__ h) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int r = (int)(idx / I), i = (int)(idx - (int64_t)r * I);
  if (r >= n || r >= offsets[E_loc]) return;
  const int e = expert_of_row(offsets, E_loc, r);
  if (e < 0) return;
  const float* w = wgu + (int64_t)e * 2 * I * H;
  const int64_t rg = gu_packed_row(i, false), ru = gu_packed_row(i, true);
  float g = 0.f, u = 0.f;
  for (int k = 0; k < H; ++k) {
    const float x = xb[(int64_t)r * H + k];
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
// Widen 8 e4m3 codes (two dwords) to 8 bf16 values (exact).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  uint32_t p[4];
  // values are exact in bf16, so truncating the low half of the fp32 pattern is exact
  p[0] = (__float_as_uint(a.x) >> 16) | (__float_as_uint(a.y) & 0xffff0000u);
  p[1] = (__float_as_uint(b.x) >> 16) | (__float_as_uint(b.y) & 0xffff0000u);
  p[2] = (__float_as_uint(c.x) >> 16) | (__float_as_uint(c.y) & 0xffff0000u);
  p[3] = (__float_as_uint(d.x) >> 16) | (__float_as_uint(d.y) & 0xffff0000u);
  bf16x8 r;
  __builtin_memcpy(&r, p, 16);
  return r;
}

template <int WDT, int NS>
struct WTile;  // one k-step of NS weight strips, as loaded (16 bytes per lane per run)

template <int NS>
struct WTile<MOE_BF16, NS> {
  uint4 raw[NS][2];
  __device__ __forceinline__ void load(const char* __restrict__ p, int64_t strip_stride) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      raw[s][0] = *reinterpret_cast<const uint4*>(p + s * strip_stride);
      raw[s][1] = *reinterpret_cast<const uint4*>(p + s * strip_stride + 1024);
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
  __device__ __forceinline__ void load(const char* __restrict__ p, int64_t strip_stride) {
#pragma unroll
    for (int s = 0; s < NS; ++s) raw[s] = *reinterpret_cast<const uint4*>(p + s * strip_stride);
  }
  __device__ __forceinline__ bf16x8 frag(int s, int h) const {
    return h == 0 ? e4m3x8_to_bf16(raw[s].x, raw[s].y) : e4m3x8_to_bf16(raw[s].z, raw[s].w);
  }
};

template <int MT>
struct ATile {
  uint4 raw[MT][2];
  __device__ __forceinline__ void load(const uint16_t* const* arow, int k0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4* p = reinterpret_cast<const uint4*>(arow[mt] + k0);
      raw[mt][0] = p[0];
      raw[mt][1] = p[1];
    }
  }
};

// MODE 0: gate/up GEMM + SwiGLU epilogue -> h [n][I];  MODE 1: down GEMM -> y [n][H].
// A work unit is MT*16 rows of one expert x NS*16 packed output columns.
template <int MODE, int WDT, int NS, int MT>
#ifndef MOE_FFN_WPE
#define MOE_FFN_WPE 0  // > 0: ask the compiler for this many waves per SIMD
#endif
#if MOE_FFN_WPE > 0
#define MOE_FFN_OCC __attribute__((amdgpu_waves_per_eu(MOE_FFN_WPE, MOE_FFN_WPE)))
#else
#define MOE_FFN_OCC
#endif
__global__ __launch_bounds__(256) MOE_FFN_OCC void ffn_mfma_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                       int E_loc, const char* __restrict__ W,
                                                       const float* __restrict__ s0, const float* __restrict__ s1,
                                                       uint16_t* __restrict__ out, int Kd, int Nw, int out_ld,
                                                       int n_blocks_N, int chunks_max, int n_rows) {
  constexpr int BM = MT * 16;
  static_assert(MODE == 1 || NS % 2 == 0, "gate/up tiles pair gate and up strips");
  __shared__ f32x4 red[kFfnWaves - 1][MT][NS][64];
  constexpr int esz = WDT == MOE_FP8_E4M3 ? 1 : 2;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;

  // XCD-aware remap: physical workgroup b runs on XCD b % 8; give each XCD a contiguous
  // range of logical ids, ordered (column block, chunk) so chunks sharing weights are adjacent.
  const int G = gridDim.x, b = blockIdx.x;
  const int L = (b & 7) * (G >> 3) + (b >> 3);
  const int nb = L / chunks_max;
  int c = L - nb * chunks_max;
  if (nb >= n_blocks_N) return;
  int e = 0, m0 = 0, mend = 0;
  bool found = false;
  for (e = 0; e < E_loc; ++e) {
    // clamp to [0, n_rows] so that inconsistent offsets can never address past the batch
    const int a0 = min(max(offsets[e], 0), n_rows), a1 = min(max(offsets[e + 1], a0), n_rows);
    const int nc = (a1 - a0 + BM - 1) / BM;
    if (c < nc) {
      m0 = a0 + c * BM;
      mend = min(a1, m0 + BM);
      found = true;
      break;
    }
    c -= nc;
  }
  if (!found) return;
  const int KS = Kd / kBK;

  // weight strips NS*nb .. NS*nb+NS-1 of expert e; block (strip, ks) at (strip*KS + ks) blocks
  const int64_t blk_bytes = 1024 * esz;
  const int64_t strip_stride = (int64_t)KS * blk_bytes;
  const char* wlane = W + (int64_t)e * Nw * Kd * esz + (int64_t)(nb * NS) * strip_stride + lane * 16;

  // activation rows: lane -> row m0 + 16mt + lane%16 (clamped into the chunk; rows past the
  // chunk are computed on a copy of its last row and never stored), 32 bytes at
  // k = 64ks + 16*(lane/16)
  const uint16_t* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = m0 + mt * 16 + (lane & 15);
    r = r < mend ? r : mend - 1;
    arow[mt] = A + (int64_t)r * Kd + (lane >> 4) * 16;
  }

  f32x4 acc[MT][NS];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const WTile<WDT, NS>& wt, const ATile<MT>& at) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 bf[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) bf[s] = wt.frag(s, h);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bf16x8 af;
        __builtin_memcpy(&af, &at.raw[mt][h], 16);
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[mt][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[s], acc[mt][s], 0, 0, 0);
      }
    }
  };

  // this wave's k-steps are wv, wv+4, ...; a ring of kStages register sets keeps the loads
  // of the next kStages-1 steps in flight while the current step feeds the MFMAs.  Loads
  // past the end are clamped to the last step (valid memory, result unused), so no load is
  // conditional; the scheduling barriers keep each prefetch batch ahead of the MFMAs.
  const int nsteps = KS > wv ? (KS - wv + kFfnWaves - 1) / kFfnWaves : 0;
  auto kstep = [&](int i) { return min(wv + kFfnWaves * i, KS - 1); };
  if (nsteps > 0) {
    WTile<WDT, NS> wr[kStages];
    ATile<MT> ar[kStages];
#pragma unroll
    for (int u = 0; u < kStages - 1; ++u) {
      wr[u].load(wlane + kstep(u) * blk_bytes, strip_stride);
      ar[u].load(arow, kstep(u) * kBK);
    }
    int it = 0;
#pragma clang loop unroll(disable)
    for (; it + kStages <= nsteps; it += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        const int ld = (u + kStages - 1) % kStages;
        wr[ld].load(wlane + kstep(it + u + kStages - 1) * blk_bytes, strip_stride);
        ar[ld].load(arow, kstep(it + u + kStages - 1) * kBK);
        __builtin_amdgcn_sched_barrier(0);
        compute(wr[u], ar[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int rest = nsteps - it;  // < kStages; those steps sit in ring slots 0..rest-1
#pragma unroll
    for (int u = 0; u < kStages - 1; ++u)
      if (u < rest) compute(wr[u], ar[u]);
  }

  // split-k reduction: waves 1..3 park their partial tiles in LDS, wave 0 sums
  if (wv > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < NS; ++s) red[wv - 1][mt][s][lane] = acc[mt][s];
  }
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int w = 0; w < kFfnWaves - 1; ++w) acc[mt][s] += red[w][mt][s][lane];

  // epilogue; the accumulator of lane l holds column l%16 of a strip and rows 4(l/16)+q
  const int col16 = lane & 15, rq = (lane >> 4) * 4;
  if (MODE == 0) {
    const int I = out_ld;
#pragma unroll
    for (int p = 0; p < NS / 2; ++p) {
      const int i = (nb * (NS / 2) + p) * 16 + col16;
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
            const float g = acc[mt][2 * p][q] * sg, u = acc[mt][2 * p + 1][q] * su;
            out[(int64_t)row * I + i] = f32_to_bf16(silu_mul(g, u));
          }
        }
      }
    }
  } else {
    const int H = out_ld;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int col = (nb * NS + s) * 16 + col16;
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

template <int MODE, int WDT, int NS, int MT>
static void launch_mfma_t(const void* A, const int32_t* offsets, int E_loc, const void* W, const float* s0,
                          const float* s1, void* out, int Kd, int Nw, int out_ld, int n, hipStream_t stream) {
  constexpr int BM = MT * 16;
  const int n_blocks_N = Nw / (16 * NS);
  const int chunks_max = (n + (BM - 1) * E_loc) / BM;
  int64_t grid = (int64_t)chunks_max * n_blocks_N;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((ffn_mfma_kernel<MODE, WDT, NS, MT>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const uint16_t*)A, offsets, E_loc, (const char*)W, s0, s1, (uint16_t*)out, Kd, Nw, out_ld,
                     n_blocks_N, chunks_max, n);
}

// Row-chunk height: tall enough that an average expert group fits one chunk with room for
// the spread of a ragged batch (1.5x the mean group), so each weight tile is read once.
#ifndef MOE_FFN_MT
#define MOE_FFN_MT 0  // 0: choose from the batch shape
#endif
#ifndef MOE_FFN_NS_GU
#define MOE_FFN_NS_GU 4
#endif
#ifndef MOE_FFN_NS_D
#define MOE_FFN_NS_D 4
#endif

static int pick_mt(int n, int E_loc) {
  if (MOE_FFN_MT > 0) return MOE_FFN_MT;
  const int want = (3 * n + 2 * E_loc - 1) / (2 * E_loc);
  const int mt = (want + 15) / 16;
  return mt < 2 ? 2 : (mt > 3 ? 3 : mt);  // taller chunks measured slower at decode sizes
}

template <int MODE, int WDT>
static void launch_mfma(const void* A, const int32_t* offsets, int E_loc, const void* W, const float* s0,
                        const float* s1, void* out, int Kd, int Nw, int out_ld, int n, hipStream_t stream) {
  // gate/up: 4 strips (32 gate + 32 up columns) per workgroup; down: 4 strips
  constexpr int NS = MODE == 0 ? MOE_FFN_NS_GU : MOE_FFN_NS_D;
  switch (pick_mt(n, E_loc)) {
    case 2: launch_mfma_t<MODE, WDT, NS, 2>(A, offsets, E_loc, W, s0, s1, out, Kd, Nw, out_ld, n, stream); break;
    case 3: launch_mfma_t<MODE, WDT, NS, 3>(A, offsets, E_loc, W, s0, s1, out, Kd, Nw, out_ld, n, stream); break;
    default: launch_mfma_t<MODE, WDT, NS, 4>(A, offsets, E_loc, W, s0, s1, out, Kd, Nw, out_ld, n, stream); break;
  }
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_ffn_workspace_size(int32_t n_max, int32_t E_loc, int32_t H, int32_t I, int32_t act_dtype) {
  (void)E_loc;
  (void)H;
  const int esz = dtype_size(act_dtype);
  if (n_max < 0 || I < 0 || esz == 0) return 0;
  return ((size_t)n_max * (size_t)I * esz + 255) / 256 * 256;
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
  if (!a->offsets) return MOE_EINVAL_NULL;
  if (a->n == 0) {
    if (a->ev_mid) (void)hipEventRecord(a->ev_mid, stream);
    return MOE_OK;
  }
  if (!a->xb || !a->w_gu || !a->w_d || !a->y) return MOE_EINVAL_NULL;
  if (f8 && (!a->s_gate || !a->s_up || !a->s_down)) return MOE_EINVAL_NULL;
  if (!aligned16(a->xb) || !aligned16(a->w_gu) || !aligned16(a->w_d) || !aligned16(a->y)) return MOE_EINVAL_ALIGN;
  const size_t ws = moe_ffn_workspace_size(a->n, a->E_loc, a->H, a->I, a->act_dtype);
  if (!a->workspace || a->workspace_bytes < ws) return MOE_EWORKSPACE;
  if (!aligned16(a->workspace)) return MOE_EINVAL_ALIGN;
  const int n = a->n, H = a->H, I = a->I, E = a->E_loc;
  if (f32) {
    const int64_t t1 = (int64_t)n * I, t2 = (int64_t)n * H;
    hipLaunchKernelGGL(gateup_f32_kernel, dim3((unsigned)((t1 + 255) / 256)), dim3(256), 0, stream,
                       (const float*)a->xb, a->offsets, E, n, H, I, (const float*)a->w_gu, (float*)a->workspace);
    if (a->ev_mid) (void)hipEventRecord(a->ev_mid, stream);
    hipLaunchKernelGGL(down_f32_kernel, dim3((unsigned)((t2 + 255) / 256)), dim3(256), 0, stream,
                       (const float*)a->workspace, a->offsets, E, n, H, I, (const float*)a->w_d, (float*)a->y);
    return launch_status();
  }
  if (bf) {
    launch_mfma<0, MOE_BF16>(a->xb, a->offsets, E, a->w_gu, nullptr, nullptr, a->workspace, H, 2 * I, I, n, stream);
    if (a->ev_mid) (void)hipEventRecord(a->ev_mid, stream);
    launch_mfma<1, MOE_BF16>(a->workspace, a->offsets, E, a->w_d, nullptr, nullptr, a->y, I, H, H, n, stream);
  } else {
    launch_mfma<0, MOE_FP8_E4M3>(a->xb, a->offsets, E, a->w_gu, a->s_gate, a->s_up, a->workspace, H, 2 * I, I, n,
                                 stream);
    if (a->ev_mid) (void)hipEventRecord(a->ev_mid, stream);
    launch_mfma<1, MOE_FP8_E4M3>(a->workspace, a->offsets, E, a->w_d, a->s_down, nullptr, a->y, I, H, H, n, stream);
  }
  return launch_status();
}
