// Device-side helpers shared by the gfx950 kernels of libmsa.
//
// MFMA operand conventions used throughout (CDNA4, wave64):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l supplies row (l % 32), eight k-slots 8*(l/32) .. 8*(l/32)+7
//     B: lane l supplies column (l % 32), the same eight k-slots
//     D: lane l holds column (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4), i = 0..15
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l supplies row (l % 16), k-slots 8*(l/16) .. +7
//     B: lane l supplies column (l % 16), the same k-slots
//     D: lane l holds column (l % 16), rows 4*(l/16) + i, i = 0..3
// Only the row/column placement and the output layout matter: A and B are
// always loaded with the same k-slot -> k assignment, so the hardware's own
// ordering of the reduction index cannot change the product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native vector types for register arrays: arrays of HIP's uint4/float4
// structs are not promoted to registers by the compiler and end in scratch.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // raw bfloat16 bits in memory

constexpr int kWave = 64;
// Fourth word of a raw (unswizzled, stride 0) buffer resource on gfx9-family
// chips: 32-bit data format, no index stride; byte offsets >= the record count
// are out of range (loads return 0, stores are dropped).
constexpr int kBufferWord3 = 0x00020000;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 zero_bf16x8() {
  const u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}
// two 8-byte halves (keys {0..3} and {8..11} of a 16-key slice) -> one operand
__device__ __forceinline__ bf16x8 join_bf16x4(u32x2 lo, u32x2 hi) {
  const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// Transposing LDS read of gfx950 (ds_read_b64_tr_b16).  In each group of 16
// lanes, lane 4a + c receives element c of the 8-byte words addressed by
// lanes a, a + 4, a + 8 and a + 12 of the group, in that order.  tr_lane_off
// places those words so that lane l gets 4 consecutive rows of a row-major
// bf16 tile (row stride `stride`) at column l % 32, starting 4 (l / 32) rows
// down: the k-slot layout of an MFMA operand whose k-slots run over rows.
__device__ __forceinline__ int tr_lane_off(int lane, int stride) {
  return (4 * (lane >> 5) + ((lane >> 2) & 3)) * stride + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
}
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const bf16_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
// -0.0 is folded onto +0.0 first so that the two zeros tie.  Every non-NaN
// float maps to a key >= 1; key 0 is free to mean "no candidate".
__device__ __forceinline__ uint32_t order_key(float f) {
  f = (f == 0.0f) ? 0.0f : f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace msa
