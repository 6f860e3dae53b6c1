// Internal helpers shared by the libdsa HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "dsa.h"

namespace dsa {

// ---------------------------------------------------------------------------
// Host-side error reporting
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

#define DSA_REQUIRE(cond, status, ...)      \
  do {                                      \
    if (!(cond)) {                          \
      ::dsa::set_error(__VA_ARGS__);        \
      return (status);                      \
    }                                       \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks the launch that was just enqueued.
dsa_status launch_status(const char* what);

__host__ __device__ constexpr inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over aligned groups of N lanes (N in {4, 8, 16}) with DPP row moves
// (no LDS traffic): quad swaps, then the half-row and row mirrors.  Every
// lane of a group ends with the group sum.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

template <int N>
__device__ __forceinline__ float group_sum_dpp(float v) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  v += dpp_mov<0xB1>(v);                 // quad_perm 1,0,3,2
  v += dpp_mov<0x4E>(v);                 // quad_perm 2,3,0,1
  if (N >= 8) v += dpp_mov<0x141>(v);    // row_half_mirror: lane i <-> 7-i within 8
  if (N >= 16) v += dpp_mov<0x140>(v);   // row_mirror: lane i <-> 15-i within 16
  return v;
}

// Wave-wide inclusive prefix sum with DPP (no LDS): row shifts by 1, 2, 4, 8
// (lanes shifted in from outside the row read 0), then the row-15 and row-31
// broadcasts carry row totals into the following rows.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_shift_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xf, true);
}

__device__ __forceinline__ float wave_incl_scan_dpp(float v) {
  v += __int_as_float(dpp_shift_i<0x111, 0xf>(__float_as_int(v)));   // row_shr:1
  v += __int_as_float(dpp_shift_i<0x112, 0xf>(__float_as_int(v)));   // row_shr:2
  v += __int_as_float(dpp_shift_i<0x114, 0xf>(__float_as_int(v)));   // row_shr:4
  v += __int_as_float(dpp_shift_i<0x118, 0xf>(__float_as_int(v)));   // row_shr:8
  v += __int_as_float(dpp_shift_i<0x142, 0xa>(__float_as_int(v)));   // row_bcast:15 into rows 1, 3
  v += __int_as_float(dpp_shift_i<0x143, 0xc>(__float_as_int(v)));   // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += (uint32_t)dpp_shift_i<0x111, 0xf>((int)v);
  v += (uint32_t)dpp_shift_i<0x112, 0xf>((int)v);
  v += (uint32_t)dpp_shift_i<0x114, 0xf>((int)v);
  v += (uint32_t)dpp_shift_i<0x118, 0xf>((int)v);
  v += (uint32_t)dpp_shift_i<0x142, 0xa>((int)v);
  v += (uint32_t)dpp_shift_i<0x143, 0xc>((int)v);
  return v;
}

// 2^x on the hardware exp unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace dsa
