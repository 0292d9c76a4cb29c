// Device-side building blocks shared by the libfa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
constexpr int kNumCu = 256;  // compute units of an MI355X

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

// 16x16x32 bf16 / fp16 MFMA, fp32 accumulate.  Operand layout (lane l of 64):
//   A[m][k]: m = l % 16, k = (l / 16) * 8 + e      (e = vector element 0..7)
//   B[k][n]: n = l % 16, k = (l / 16) * 8 + e
//   C[m][n]: n = l % 16, m = (l / 16) * 4 + i      (i = 0..3)
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + a + b for two 16-bit values as they are rounded (one v_dot2c_f32_bf16
// or v_dot2c_f32_f16 against the pair (1, 1)): the sum of the probabilities
// that enter the P V product, so that the output's normaliser carries the
// same rounding as its numerator.
__device__ __forceinline__ float add_pair(bf16 a, bf16 b, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {a, b};
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  return __builtin_amdgcn_fdot2_f32_bf16(v, one, acc, false);
}
__device__ __forceinline__ float add_pair(f16 a, f16 b, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 v = {a, b};
  const f16x2 one = {(f16)1.f, (f16)1.f};
  return __builtin_amdgcn_fdot2(v, one, acc, false);
}

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

// Combine v with its value in lane l ^ 32 (the other half of the wave), for
// every lane l.  v_permlane32_swap exchanges the two halves of its operands,
// which leaves each lane holding v_l and v_{l^32}; the operations below are
// commutative, so both halves get the same result bit for bit.  A vector-ALU
// exchange, where __shfl_xor would go through the LDS crossbar.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// A 16-byte direct-to-LDS load (lane i writes at lds + 16 i) issued from
// inline assembly, with its buffer descriptor as four scalar words.  The
// compiler's wait-count tracking does not see it, so the caller waits for it
// explicitly (s_waitcnt vmcnt); in exchange its target does not join the
// LDS regions that the compiler tracks for its own direct-to-LDS loads,
// which would otherwise make it wait for those after each one.  The load
// takes its LDS address from m0, a register the compiler reserves for
// itself: the sequence saves m0, sets it, leaves the one wait state that an
// m0 write needs before a direct-to-LDS load reads it (the gfx9 hazard
// rule), issues the load and restores m0, so the compiler sees m0 unchanged.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void* base, unsigned bytes) {
  const unsigned long long a = (unsigned long long)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = (int)kRsrcWord3;
  return r;
}
// NT: the load is non-temporal (the nt cache-policy bit), for data that no
// other workgroup reads again.
template <bool NT>
__device__ __forceinline__ void lds_dma16_asm(i32x4 rsrc, unsigned voff, const FA_LDS void* lds) {
  unsigned saved;
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"((unsigned)(size_t)lds)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"((unsigned)(size_t)lds)
        : "memory");
  }
}

// Before direct-to-LDS loads overwrite a region that this wave has just
// read: the reads must have returned.  The compiler places its wait for a
// read just before the first use of the value, and plain arithmetic on the
// value may be scheduled after the loads' inline assembly, so the wait is
// made explicit.
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Cache-policy operand of a buffer load that marks it non-temporal (the nt
// bit of the gfx940-family policy: sc0 = 1, nt = 2, sc1 = 16): for streams
// that no other workgroup reads again, which then pass the caches by.
constexpr int kLoadNonTemporal = 2;

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
  // Load u (0 <= u < PER) of this wave for the tile at row0 into lds.  AUX
  // is the load's cache policy: 0, or kLoadNonTemporal for data that no other
  // workgroup reads again.
  template <int AUX = 0, typename T>
  __device__ __forceinline__ void part(const T* g, int row0, int nvalid, T* lds, int u) const {
    static_assert(sizeof(T) == 2, "16-bit elements");
    // (readfirstlane: the clamp compiles to a vector instruction, and a
    // resource in vector registers would need a loop over its distinct values)
#if __HIP_DEVICE_COMPILE__
    const int rows = __builtin_amdgcn_readfirstlane(min(max(nvalid - row0, 0), ROWS));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(g + (size_t)min(row0, nvalid) * D, rows * D * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(lds + (wave * PER + u) * 64 * 8),
                                             16, voff[u], 0, 0, AUX);
#endif
  }
  template <int AUX = 0, typename T>
  __device__ __forceinline__ void tile(const T* g, int row0, int nvalid, T* lds) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) part<AUX>(g, row0, nvalid, lds, u);
  }
};

// Additive bias as the kernels take it: element (b, h, i, j) of the bias at
// ptr[b*sb + h*sh + i*sq + j] (16-bit elements; sq a multiple of 8), folded
// into the raw scores as bias * inv_scale so that the exponent stays
// s * scale * log2(e) - m.
//
// Optional tile map of the bias (tmap != nullptr): one byte per 128-row x
// 64-key tile of each bias head, nonzero iff the tile holds an entry above
// -inf; tile (b, h, qt, kt) at tmap[b*tm_sb + h*tm_sh + qt*nkt4 + kt], rows
// padded with zeros to nkt4 (a multiple of 4) bytes.  The kernels visit only
// the tiles between the first and the last nonzero byte of their row (or
// column) of the map: all-masked tiles contribute exact zeros.
constexpr int kMapRows = 128;
constexpr int kMapKeys = 64;

struct BiasDev {
  const void* ptr;
  long long sb, sh, sq;
  int H;
  float inv_scale;
  const unsigned char* tmap;
  long long tm_sb, tm_sh;
  int nkt4;
  // Nonzero when every bias element is read by one head of one batch only
  // (no broadcast with a zero stride over more than one head or batch): its
  // loads are then non-temporal.  A broadcast bias is re-read by the other
  // heads and keeps cached loads.
  int stream;
};

// BiasDev of a bias with element strides sb (batch), sh (head), sq (row),
// for B batches of H heads.
inline BiasDev make_bias_dev(const void* ptr, long long sb, long long sh, long long sq, int B,
                             int H, float scale, const unsigned char* tmap, long long tm_sb,
                             long long tm_sh, int nkt4) {
  const bool reused = (sh == 0 && H > 1) || (sb == 0 && B > 1);
  return BiasDev{ptr, sb, sh, sq, H, 1.f / scale, tmap, tm_sb, tm_sh, nkt4, reused ? 0 : 1};
}

// First and last nonzero byte of row[0 .. n) (lo > hi when none), over the
// wave: lane i reads bytes i, i + 64, ...; the result is wave-uniform.
__device__ __forceinline__ void map_range(const unsigned char* row, int n, int lane, int& lo,
                                          int& hi) {
  lo = 0x7fffffff;
  hi = -1;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(i < n && row[i] != 0);
    if (m != 0ull) {
      lo = min(lo, base + (int)__builtin_ctzll(m));
      hi = base + 63 - (int)__builtin_clzll(m);
    }
  }
}

// First and last query tile qt in [0, nqt) whose NB bytes kt0 .. kt0+NB-1 of
// the map are not all zero (NB = 2 or 4, kt0 a multiple of NB: one aligned
// load per row, inside the row's padding to nkt4 bytes); lo > hi when none.
template <int NB>
__device__ __forceinline__ void map_range_cols(const unsigned char* head, int nqt, int nkt4,
                                               int kt0, int lane, int& lo, int& hi) {
  static_assert(NB == 2 || NB == 4, "two or four map bytes per workgroup");
  typedef typename std::conditional<NB == 4, unsigned, unsigned short>::type W;
  lo = 0x7fffffff;
  hi = -1;
  for (int base = 0; base < nqt; base += 64) {
    const int qt = base + lane;
    const unsigned w = qt < nqt ? (unsigned)*(const W*)(head + (size_t)qt * nkt4 + kt0) : 0u;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(w != 0u);
    if (m != 0ull) {
      lo = min(lo, base + (int)__builtin_ctzll(m));
      hi = base + 63 - (int)__builtin_clzll(m);
    }
  }
}

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
};

// Dropout on the normalised probabilities (the V1 algorithm in the 51CTO
// FlashAttention V1/V2 notes, "FlashAttention V2 相比 V1 有哪些改进", applies it
// inside the loop).  The bits come from Philox4x32-10 (Salmon, Moraes, Dror
// and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011, section
// 3.2), one call per block of 4 query rows x 4 keys: key (seed_lo, seed_hi),
// counter (key / 4, row / 4, b*H + h, offset); word row % 4 holds the block's
// row and byte key % 4 of that word the score.  A score is kept iff its byte
// is below thresh (1..255), and kept probabilities are scaled by inv_keep =
// 256 / thresh.
struct DropDev {
  unsigned seed_lo, seed_hi, offset, thresh;
  float inv_keep;
};

// Philox4x32-10 of counter x, in place.  Per round: the two products
// M0 * x0 and M1 * x2 (32 x 32 -> 64 bits); the new words are (hi1 ^ x1 ^ k0,
// lo1, hi0 ^ x3 ^ k1, lo0); the round key then advances by the Weyl
// constants W0, W1, so round r uses (seed_lo + r * W0, seed_hi + r * W1)
// mod 2^32.  The keys are wave-uniform (scalar work), and a call may be split
// into its rounds so that they run between other work.
__device__ __forceinline__ void philox_round(unsigned (&x)[4], unsigned k0, unsigned k1) {
  const unsigned long long p0 = (unsigned long long)0xD2511F53u * x[0];
  const unsigned long long p1 = (unsigned long long)0xCD9E8D57u * x[2];
  const unsigned hi0 = (unsigned)(p0 >> 32), lo0 = (unsigned)p0;
  const unsigned hi1 = (unsigned)(p1 >> 32), lo1 = (unsigned)p1;
  x[0] = hi1 ^ x[1] ^ k0;
  x[1] = lo1;
  x[2] = hi0 ^ x[3] ^ k1;
  x[3] = lo0;
}
constexpr unsigned kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

__device__ __forceinline__ void philox4x32_10(unsigned (&x)[4], unsigned k0, unsigned k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) philox_round(x, k0 + r * kPhiloxW0, k1 + r * kPhiloxW1);
}

// 4 x 4 transpose of dwords across the 4 lanes of a quad (lanes 4a .. 4a+3):
// on entry lane t holds x[0..3]; on exit x[c] of lane t is what x[t] of lane
// c held.  Two butterfly stages of quad-permute moves (DPP) and selects.
__device__ __forceinline__ unsigned quad_xor1(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
}
__device__ __forceinline__ unsigned quad_xor2(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
}
__device__ __forceinline__ void quad_transpose(unsigned (&x)[4], int lane) {
  const bool odd = lane & 1, upper = lane & 2;
  const unsigned a0 = quad_xor1(x[1]), a1 = quad_xor1(x[0]);
  const unsigned a2 = quad_xor1(x[3]), a3 = quad_xor1(x[2]);
  x[0] = odd ? a0 : x[0];
  x[1] = odd ? x[1] : a1;
  x[2] = odd ? a2 : x[2];
  x[3] = odd ? x[3] : a3;
  const unsigned b0 = quad_xor2(x[2]), b1 = quad_xor2(x[3]);
  const unsigned b2 = quad_xor2(x[0]), b3 = quad_xor2(x[1]);
  x[0] = upper ? b0 : x[0];
  x[1] = upper ? b1 : x[1];
  x[2] = upper ? x[2] : b2;
  x[3] = upper ? x[3] : b3;
}

// 4 x 4 transpose of the bytes of x[0..3] within a lane: byte r of x[e] on
// exit is byte e of x[r] on entry.
__device__ __forceinline__ void byte_transpose(unsigned (&x)[4]) {
  const unsigned a0 = __builtin_amdgcn_perm(x[1], x[0], 0x06020400u);
  const unsigned a1 = __builtin_amdgcn_perm(x[1], x[0], 0x07030501u);
  const unsigned a2 = __builtin_amdgcn_perm(x[3], x[2], 0x06020400u);
  const unsigned a3 = __builtin_amdgcn_perm(x[3], x[2], 0x07030501u);
  x[0] = __builtin_amdgcn_perm(a2, a0, 0x05040100u);
  x[1] = __builtin_amdgcn_perm(a3, a1, 0x05040100u);
  x[2] = __builtin_amdgcn_perm(a2, a0, 0x07060302u);
  x[3] = __builtin_amdgcn_perm(a3, a1, 0x07060302u);
}

// Random bytes for a lane that holds query row `row` and keys
// key0 + c*8 + e (c, e = 0..3; key0 a multiple of 4), the lanes of its quad
// holding rows 4a .. 4a+3 and the same keys: each lane makes one of the
// quad's four calls (key block (key0 + 8t) / 4 for quad lane t), then the quad
// exchanges words.  On exit byte e of x[c] belongs to (row, key0 + c*8 + e).
__device__ __forceinline__ void drop_counter_rows(unsigned (&x)[4], const DropDev& dr, int bh,
                                                  int row, int key0, int lane) {
  const int t = lane & 3;
  x[0] = (unsigned)(key0 + t * 8) >> 2;
  x[1] = (unsigned)row >> 2;
  x[2] = (unsigned)bh;
  x[3] = dr.offset;
}
__device__ __forceinline__ void drop_bytes_rows(unsigned (&x)[4], const DropDev& dr, int bh,
                                                int row, int key0, int lane) {
  drop_counter_rows(x, dr, bh, row, key0, lane);
  philox4x32_10(x, dr.seed_lo, dr.seed_hi);
  quad_transpose(x, lane);
}

// Random bytes for a lane that holds key `key` and query rows
// row0 + 8g + r (g, r = 0..3; row0 a multiple of 4), the lanes of its quad
// holding keys 4b .. 4b+3 and the same rows: each lane makes one of the
// quad's four calls, transposes its bytes, then the quad exchanges words.
// On exit byte r of x[g] belongs to (row0 + 8g + r, key).
__device__ __forceinline__ void drop_counter_keys(unsigned (&x)[4], const DropDev& dr, int bh,
                                                  int key, int row0, int lane) {
  const int t = lane & 3;
  x[0] = (unsigned)key >> 2;
  x[1] = (unsigned)(row0 + 8 * t) >> 2;
  x[2] = (unsigned)bh;
  x[3] = dr.offset;
}
__device__ __forceinline__ void drop_bytes_keys(unsigned (&x)[4], const DropDev& dr, int bh,
                                                int key, int row0, int lane) {
  drop_counter_keys(x, dr, bh, key, row0, lane);
  philox4x32_10(x, dr.seed_lo, dr.seed_hi);
  byte_transpose(x);
  quad_transpose(x, lane);
}

// The random byte of one score (row, key) of flat head bh, from its own call
// (the fp32 kernels, which hold one row or one key per thread).
__device__ __forceinline__ unsigned drop_byte(const DropDev& dr, int bh, int row, int key) {
  unsigned w[4] = {(unsigned)key >> 2, (unsigned)row >> 2, (unsigned)bh, dr.offset};
  philox4x32_10(w, dr.seed_lo, dr.seed_hi);
  const int r = row & 3;
  const unsigned word = r == 0 ? w[0] : r == 1 ? w[1] : r == 2 ? w[2] : w[3];
  return (word >> (8 * (key & 3))) & 0xFFu;
}

// Keep decision for byte b (0..3) of a word of random bytes.
__device__ __forceinline__ bool drop_keep(unsigned word, int b, unsigned thresh) {
  return ((word >> (8 * b)) & 0xFFu) < thresh;
}

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
