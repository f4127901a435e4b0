// Shared device/host helpers for libmoestep (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_step.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a NaN (gfx950's v_cvt_pk_bf16_f32; the
// integer rounding sequence with its NaN branch cost a dozen instructions per value)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const __bf16 h = (__bf16)f;
  uint16_t r;
  __builtin_memcpy(&r, &h, 2);
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Index of element (n, k) of an [N][Kd] matrix in the packed tile-major layout documented
// in moe_step.h (blocks of 16 rows x 64 columns; within a block, lane = 16*(k%64/16) + n%16
// and h = (k/8)%2 select a 16-byte run that one MFMA operand register group reads).
__host__ __device__ __forceinline__ int64_t packed_index(int64_t n, int64_t k, int64_t Kd, int esz) {
  const int64_t nb = n >> 4, r = n & 15, kb = k >> 6, c = k & 63;
  const int64_t g = c >> 4, h = (c >> 3) & 1, q = c & 7, lane = g * 16 + r;
  const int64_t blk = (nb * (Kd >> 6) + kb) << 10;
  return blk + (esz == 1 ? lane * 16 + h * 8 + q : h * 512 + lane * 8 + q);
}

// Packed gate/up row of gate row i (up = false) or up row i (up = true): strips of 16 rows
// alternate gate, up, gate, up, ... so that one 64-row tile holds 32 matching (g, u) pairs.
__host__ __device__ __forceinline__ int64_t gu_packed_row(int64_t i, bool up) {
  return (i >> 4) * 32 + (up ? 16 : 0) + (i & 15);
}

inline int dtype_size(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : dt == MOE_FP8_E4M3 ? 1 : 0; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline int launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

// Host-side argument checks of moe_assemble (MOE_OK or the status it returns); also used by
// moe_expert_ffn_grouped for a queue index it enqueues itself.
int check_assemble_args(const moe_assemble_args* a);

}  // namespace moe
