// Machine probes for bench.py's --probes mode (measurement only; no part of
// the attention path).  They answer two questions about the MI355X that the
// kernels' design rests on:
//  * what the bf16 matrix cores sustain, and at what shader clock, when their
//    operands are constant or random bits, and when each MFMA also carries
//    1 KB of LDS reads and/or the softmax's vector-ALU mix (one exponential and
//    four FMAs), the per-MFMA budget of the attention kernels;
//  * how fast device-scope fp32 atomic adds run against plain stores in the
//    access pattern a dQ accumulation by atomics would have (one 32 x 32 fp32
//    MFMA result tile per wave, rows of 128 floats).
// Built into libfa_probe.so next to libfa.so; exported as plain C symbols.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// 8 bf16 values with random signs and mantissas and exponents of 0.5 .. 1
// (RANDOM), or eight copies of 1.0.
template <bool RANDOM>
__device__ __forceinline__ bf16x8 operand(unsigned seed) {
  u32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = RANDOM ? ((mix(seed * 4 + e) & 0x807f807fu) | 0x3f003f00u) : 0x3f803f80u;
  return __builtin_bit_cast(bf16x8, u);
}

// A operand as the attention kernels read a transposed fragment: two
// ds_read_b64_tr_b16 (8 bytes per lane each), lane l supplying row l/4 (and
// row l/4 + 4 for the second) and 8-byte column group l%4 of a tile with
// 288-byte rows (a 32-byte pad per 256-byte row spreads the four rows of a
// 16-lane group over distinct banks).  `base` is a byte offset into the tile.
__device__ __forceinline__ bf16x8 tr_pair(const __attribute__((address_space(3))) char* tile,
                                          unsigned base) {
  const unsigned l = threadIdx.x & 63;
  const unsigned o = base + (l >> 2) * 288 + (l & 3) * 8;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(tile + o));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(tile + o + 4 * 288));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 8 waves per workgroup, one workgroup per CU (two waves per SIMD); with ONE,
// 4 waves and 96 KB of LDS per workgroup, so that one fits a CU (one wave per
// SIMD, up to 512 registers each).  Per loop step a wave issues 32 MFMAs
// (v_mfma_f32_32x32x16_bf16 into four accumulators) with A operands cycling
// through 8 registers (LDS = false) or read from LDS just before (LDS = true:
// 1 KB per wave, four steps ahead: one 16-byte read per lane, or with TR two
// 8-byte transposed reads per lane; with HALF only every other MFMA's A comes
// from LDS, 0.5 KB per MFMA), B from 8 registers; VALU adds one v_exp_f32 and
// four v_fma_f32 on independent registers after each MFMA.
template <bool RANDOM, bool LDS, bool VALU, bool TR, bool ONE, bool HALF>
__global__ __launch_bounds__(ONE ? 256 : 512, 1)
__attribute__((amdgpu_waves_per_eu(ONE ? 1 : 2, ONE ? 1 : 2)))
void mfma_probe(float* out, int iters) {
  constexpr int kTile = ONE ? 6144 : 4096;  // 96 or 64 KB
  __shared__ bf16x8 tile[kTile];
  for (int i = threadIdx.x; i < kTile; i += blockDim.x) tile[i] = operand<RANDOM>(i * 977u + blockIdx.x);
  __syncthreads();
  bf16x8 a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = operand<RANDOM>(threadIdx.x * 8u + k + blockIdx.x * 4096u);
    b[k] = operand<RANDOM>(threadIdx.x * 8u + k + 777777u + blockIdx.x * 4096u);
  }
  unsigned off[8];  // per-lane LDS element offsets, fixed for the kernel
#pragma unroll
  for (int k = 0; k < 8; ++k) off[k] = (threadIdx.x + 512u * k) & 4095u;  // in every tile size
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = (f32x16){};
  float e[16], f[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    e[i] = 1e-3f * (threadIdx.x + i);
    f[i] = 1.0f + 1e-3f * i;
  }
  for (int it = 0; it < iters; ++it) {
    bf16x8 ring[4];
    const __attribute__((address_space(3))) char* tl =
        (const __attribute__((address_space(3))) char*)tile;
    if (LDS) {
#pragma unroll
      for (int m = 0; m < 4; ++m) ring[m] = TR ? tr_pair(tl, m * 8192u) : tile[off[m]];
    }
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      bf16x8 x = a[m & 7];
      if (LDS && (!HALF || (m & 1) == 0)) {
        const int r = HALF ? (m >> 1) : m;
        x = ring[r & 3];
        ring[r & 3] = TR ? tr_pair(tl, ((r + 4) & 7) * 8192u) : tile[off[(r + 4) & 7]];
      }
      acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, b[(m * 3) & 7], acc[m & 3], 0, 0, 0);
      if (VALU) {
        asm volatile("v_exp_f32 %0, %0" : "+v"(e[m & 15]));
#pragma unroll
        for (int q = 0; q < 4; ++q)
          asm volatile("v_fma_f32 %0, %0, %1, %2"
                       : "+v"(f[(m + q) & 15])
                       : "v"(f[(m + q + 3) & 15]), "v"(f[(m + q + 5) & 15]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[k][i];
#pragma unroll
  for (int i = 0; i < 16; ++i) s += e[i] + f[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// fp32 adds into a [nrb * 32][128] buffer: per step a wave adds one 32 x 32
// tile (16 values per lane, each instruction covering two 128-byte row
// segments, the layout of an MFMA result with the head dim along lanes) at
// row block (block * 7 + step) mod nrb, column block `wave`.  ATOMIC: a
// relaxed device-scope atomic add (global_atomic_add_f32, no return); else a
// plain store of the same bytes.
template <bool ATOMIC>
__global__ __launch_bounds__(256) void add_probe(float* buf, int nrb, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int it = 0; it < iters; ++it) {
    const int rb = (int)(((long long)blockIdx.x * 7 + it) % nrb);
    float* base = buf + (size_t)rb * 32 * 128 + wave * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = (i / 4) * 8 + (lane >> 5) * 4 + (i & 3);
      if (ATOMIC)
        __hip_atomic_fetch_add(base + r * 128, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        base[r * 128] = 1.0f;
    }
  }
}

}  // namespace

extern "C" {

// mode bit 0: random operands; bit 1: 1 KB of LDS reads per MFMA; bit 2: one
// exponential and four FMAs per MFMA; bit 3 (with bit 1): the LDS reads as
// pairs of 8-byte transposed reads; bit 4: one wave per SIMD (2 * blocks
// workgroups of 4 waves, one per CU at a time); bit 5 (with bit 1): LDS reads
// for every other MFMA only (0.5 KB per MFMA).  `out` holds blocks * 512
// floats.  Each launch issues blocks * 8 * iters * 32 MFMAs of 32768 flop.
int fa_probe_mfma(int mode, int blocks, int iters, float* out, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
#define FA_PROBE_CASE(M)                                                                        \
  case M:                                                                                       \
    hipLaunchKernelGGL((mfma_probe<(M & 1) != 0, (M & 2) != 0, (M & 4) != 0, (M & 8) != 0,       \
                                   (M & 16) != 0, (M & 32) != 0>),                              \
                       dim3((M & 16) ? 2 * blocks : blocks), dim3((M & 16) ? 256 : 512), 0, s,  \
                       out, iters);                                                             \
    break;
  switch (mode) {
    FA_PROBE_CASE(0) FA_PROBE_CASE(1) FA_PROBE_CASE(2) FA_PROBE_CASE(3)
    FA_PROBE_CASE(4) FA_PROBE_CASE(5) FA_PROBE_CASE(6) FA_PROBE_CASE(7)
    FA_PROBE_CASE(10) FA_PROBE_CASE(11) FA_PROBE_CASE(14) FA_PROBE_CASE(15)
    FA_PROBE_CASE(17) FA_PROBE_CASE(23) FA_PROBE_CASE(39) FA_PROBE_CASE(55)
    default:
      return (int)hipErrorInvalidValue;  // combinations not built
  }
#undef FA_PROBE_CASE
  return (int)hipGetLastError();
}

// atomic != 0: atomic adds, else stores.  buf holds nrb * 32 * 128 floats;
// each launch adds (or stores) blocks * iters * 4096 values.
int fa_probe_adds(int atomic, float* buf, int nrb, int blocks, int iters, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!buf || nrb <= 0 || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  if (atomic)
    hipLaunchKernelGGL((add_probe<true>), dim3(blocks), dim3(256), 0, s, buf, nrb, iters);
  else
    hipLaunchKernelGGL((add_probe<false>), dim3(blocks), dim3(256), 0, s, buf, nrb, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
