// Device-side building blocks shared by the libfa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The MFMA kernels take 16-bit inputs, bf16 or fp16; Vec<T> names their
// 8- and 4-element vectors.
template <typename T> struct Vec;
template <> struct Vec<bf16> {
  typedef bf16x8 x8;
  typedef bf16x4 x4;
};
template <> struct Vec<f16> {
  typedef f16x8 x8;
  typedef f16x4 x4;
};

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;

// 32x32x16 bf16 / fp16 MFMA, fp32 accumulate.  Operand layout (lane l of 64):
//   A[m][k]: m = l % 32, k = (l / 32) * 8 + e      (e = vector element 0..7)
//   B[k][n]: n = l % 32, k = (l / 32) * 8 + e
//   C[m][n]: n = l % 32, m = (i / 4) * 8 + (l / 32) * 4 + i % 4   (i = 0..15)
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// LDS transposed read of 16-bit data.  Within each group of 16 lanes, lane s
// supplies the address of 4 consecutive elements; lane r receives element
// (r % 4) of the rows supplied by lanes r/4, r/4 + 4, r/4 + 8, r/4 + 12.
// When lane s points at row (k0 + s/4), column (n0 + (s%4)*4) of a row-major
// tile, lane r receives column n0 + r of rows k0 .. k0+3.
template <typename T = bf16>
__device__ __forceinline__ typename Vec<T>::x4 lds_read_tr(const FA_LDS void* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)p);
  return __builtin_bit_cast(typename Vec<T>::x4, v);
}

template <typename T>
__device__ __forceinline__ const FA_LDS T* to_lds(const T* p) {
  return (const FA_LDS T*)p;
}

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x8 concat(f16x4 a, f16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <typename V8>
__device__ __forceinline__ V8 zero8() {
  return __builtin_bit_cast(V8, (uint4){0u, 0u, 0u, 0u});
}
__device__ __forceinline__ bf16x8 zero_bf16x8() { return zero8<bf16x8>(); }

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

// Swizzled LDS tiles.  A [rows][D] bf16 tile is stored without padding, each
// row's 16-byte chunks permuted: logical chunk c of row r sits at physical
// chunk c ^ swz<D>(r).  The permutation makes both access patterns of the
// kernels free of LDS bank conflicts: 16 lanes reading 16 consecutive rows at
// one logical chunk (ds_read_b128), and 32 lanes reading 4 consecutive rows
// times 4 consecutive chunks (ds_read_b64_tr_b16).
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
}

// Byte offsets into swizzled tiles, in a form that costs one VALU XOR per LDS
// read: the row part, the swizzled chunk and the byte within the chunk occupy
// disjoint bit ranges, so the lane-dependent part is computed once and each
// read XORs in a compile-time constant.

// Row reads (ds_read_b128): the lane reads row rb + l32 (rb a multiple of 32)
// at logical chunk c.
// `chalf` (0 or 1) is a lane-dependent chunk added to every c (the lane half).
template <int D>
struct SwzRow {
  unsigned x;
  __device__ __forceinline__ SwzRow(int l32, int chalf)
      : x((unsigned)(l32 * 2 * D) ^ ((unsigned)(swz<D>(l32) ^ chalf) << 4)) {}
  __device__ __forceinline__ explicit SwzRow(unsigned x_) : x(x_) {}
  // The same lane offsets in the tile buffer `flip` bytes away, flip being a
  // power of two above every offset inside a tile.
  __device__ __forceinline__ SwzRow flipped(unsigned flip) const { return SwzRow(x ^ flip); }
  __device__ __forceinline__ unsigned off(int rb, int c) const {
    return (unsigned)(rb * 2 * D) + (x ^ ((unsigned)c << 4));
  }
};

// Transpose reads (ds_read_b64_tr_b16): the lane supplies row
// rb + tr_row + 8*hi (rb a multiple of 16) and column cb + tr_col (cb a
// multiple of 32), where tr_row < 8 and tr_col < 32 are its lane constants.
template <int D>
struct SwzTr {
  unsigned y[2];
  __device__ __forceinline__ SwzTr(int tr_row, int tr_col) {
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = tr_row + 8 * hi;
      y[hi] = (unsigned)(r * 2 * D) ^ ((unsigned)((tr_col >> 3) ^ swz<D>(r)) << 4) ^
              (unsigned)((tr_col & 7) * 2);
    }
  }
  __device__ __forceinline__ SwzTr() {}
  __device__ __forceinline__ SwzTr flipped(unsigned flip) const {
    SwzTr t;
    t.y[0] = y[0] ^ flip;
    t.y[1] = y[1] ^ flip;
    return t;
  }
  __device__ __forceinline__ unsigned off(int rb, int hi, int cb) const {
    return (unsigned)(rb * 2 * D) + (y[hi] ^ ((unsigned)(cb >> 3) << 4));
  }
};

template <typename T>
__device__ __forceinline__ const T* at_byte(const void* base, unsigned off) {
  return (const T*)((const char*)base + off);
}

// gfx9 buffer descriptor, word 3: 32-bit data format, so that raw (untyped)
// buffer loads are range-checked per dword against the record count.
constexpr int kRsrcWord3 = 0x00020000;

// Raw buffer resource over `bytes` bytes at base: a load at a byte offset at
// or past `bytes` returns zeros and touches no memory.  (The resource type
// exists only in the device pass; the host pass, which never runs these
// functions, sees an empty body, since clang otherwise drops the host launch
// stubs of some kernels that use it.)
#if __HIP_DEVICE_COMPILE__
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}
#endif

// Direct-to-LDS tile loads through a buffer resource (buffer_load_dwordx4 with
// the lds flag: lane i of a wave instruction writes 16 bytes at the
// instruction's LDS base + 16 i).  Rows [row0, row0 + ROWS) of a row-major
// [nvalid, D] matrix of 16-bit elements go into a tile swizzled as swz lays it out; rows at
// or past nvalid read as zeros.  A lane keeps the byte offsets of its PER
// chunks for the whole kernel; the row base, the row count and the LDS
// address are wave-uniform (scalar registers), so a load costs no vector-ALU
// instruction.  The data is in LDS once every wave has waited for vmcnt and
// passed a barrier.
template <int D, int ROWS, int THREADS>
struct BufTile {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int PER = ROWS * CPR / THREADS;   // loads per wave per tile
  static_assert(PER * THREADS == ROWS * CPR && THREADS % 64 == 0, "tile split");
  unsigned voff[PER];
  int wave;  // wave-uniform
  __device__ __forceinline__ BufTile(int wave_uniform, int lane) : wave(wave_uniform) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int slot = (wave * PER + u) * 64 + lane;
      const int r = slot / CPR, pch = slot % CPR;
      voff[u] = (unsigned)(r * D * 2 + ((pch ^ swz<D>(r)) << 4));
    }
  }
  // Load u (0 <= u < PER) of this wave for the tile at row0 into lds.
  template <typename T>
  __device__ __forceinline__ void part(const T* g, int row0, int nvalid, T* lds, int u) const {
    static_assert(sizeof(T) == 2, "16-bit elements");
    // (readfirstlane: the clamp compiles to a vector instruction, and a
    // resource in vector registers would need a loop over its distinct values)
#if __HIP_DEVICE_COMPILE__
    const int rows = __builtin_amdgcn_readfirstlane(min(max(nvalid - row0, 0), ROWS));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(g + (size_t)min(row0, nvalid) * D, rows * D * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(lds + (wave * PER + u) * 64 * 8),
                                             16, voff[u], 0, 0, 0);
#endif
  }
  template <typename T>
  __device__ __forceinline__ void tile(const T* g, int row0, int nvalid, T* lds) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) part(g, row0, nvalid, lds, u);
  }
};

// Additive bias as the kernels take it: element (b, h, i, j) of the bias at
// ptr[b*sb + h*sh + i*sq + j] (16-bit elements; sq a multiple of 8), folded
// into the raw scores as bias * inv_scale so that the exponent stays
// s * scale * log2(e) - m.
struct BiasDev {
  const void* ptr;
  long long sb, sh, sq;
  int H;
  float inv_scale;
};

// Reads of an additive bias through a buffer descriptor over one head's bias
// block of `nelem` 16-bit elements (element offsets below 2^30): loads past
// the block return zeros and touch no memory.  Lanes read different rows, so
// the offsets are per lane; the descriptor is wave-uniform.
template <typename T>
struct BiasReader {
  static_assert(sizeof(T) == 2, "16-bit elements");
#if __HIP_DEVICE_COMPILE__
  __amdgpu_buffer_rsrc_t rs;
#endif
  __device__ __forceinline__ BiasReader(const T* base, long long nelem) {
#if __HIP_DEVICE_COMPILE__
    // The range check of a buffer load works on whole dwords: a dword that
    // runs past the range reads as zero even where its first half is in it.
    // The range is therefore rounded up to the 16-byte block that holds the
    // last element; with a 16-byte aligned base that block lies in the page
    // of a valid byte, so reading it cannot fault.  Callers keep nelem <=
    // 2^30, so the range fits the 32-bit field.
    const unsigned long long bytes = ((unsigned long long)nelem * 2 + 15) & ~15ull;
    rs = make_rsrc(base, (int)(unsigned)(bytes < 0xfffffff0ull ? bytes : 0xfffffff0ull));
#endif
  }
  // Elements e .. e+3 (e a multiple of 4), packed as loaded.
  __device__ __forceinline__ typename Vec<T>::x4 load4(unsigned e) const {
    typename Vec<T>::x4 r = {};
#if __HIP_DEVICE_COMPILE__
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(e * 2), 0, 0);
    r = __builtin_bit_cast(typename Vec<T>::x4, v);
#endif
    return r;
  }
  // Element e, as fp32.
  __device__ __forceinline__ float load1(unsigned e) const {
    float r = 0.f;
#if __HIP_DEVICE_COMPILE__
    const unsigned short v = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(e * 2), 0, 0);
    r = (float)__builtin_bit_cast(T, v);
#endif
    return r;
  }
};

// Wait for this wave's outstanding vector-memory operations (including the
// direct-to-LDS loads above).
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Keeps the computation of v at this point of the instruction stream: the
// empty volatile asm reads and rewrites v, so whatever produces v must come
// before it, and the asm itself keeps its place among the other volatile
// statements and scheduling barriers.  Without it the compiler sinks pure
// arithmetic (exponentials, conversions) towards its first use, undoing an
// interleave of vector-ALU work with MFMAs.
template <typename T>
__device__ __forceinline__ void pin(T& v) { asm volatile("" : "+v"(v)); }

}  // namespace fa
