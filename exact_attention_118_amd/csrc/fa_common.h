// Device-side building blocks shared by the libfa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand layout (lane l of 64):
//   A[m][k]: m = l % 32, k = (l / 32) * 8 + e      (e = vector element 0..7)
//   B[k][n]: n = l % 32, k = (l / 32) * 8 + e
//   C[m][n]: n = l % 32, m = (i / 4) * 8 + (l / 32) * 4 + i % 4   (i = 0..15)
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transposed read of 16-bit data.  Within each group of 16 lanes, lane s
// supplies the address of 4 consecutive elements; lane r receives element
// (r % 4) of the rows supplied by lanes r/4, r/4 + 4, r/4 + 8, r/4 + 12.
// When lane s points at row (k0 + s/4), column (n0 + (s%4)*4) of a row-major
// tile, lane r receives column n0 + r of rows k0 .. k0+3.
__device__ __forceinline__ bf16x4 lds_read_tr(const FA_LDS void* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)p);
  return __builtin_bit_cast(bf16x4, v);
}

template <typename T>
__device__ __forceinline__ const FA_LDS T* to_lds(const T* p) {
  return (const FA_LDS T*)p;
}

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, (uint4){0u, 0u, 0u, 0u});
}

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroups are dispatched round-robin over the XCDs (block b runs on XCD
// b % 8).  Map the hardware block index to a logical index so that each XCD
// receives one contiguous range of logical indices: neighbouring logical
// tiles (which share K/V rows) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int x = bid % kNumXcd, slot = bid / kNumXcd;
  const int q = nblocks / kNumXcd, r = nblocks % kNumXcd;
  const int start = (x < r) ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  return start + slot;
}

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace fa
