// Tile map of an additive bias: one byte per 128-row x 64-key tile of each
// bias head, nonzero iff the tile holds an entry above -inf.  The attention
// kernels that take the map visit only the tiles between the first and the
// last nonzero byte of their row (forward, dQ) or column (dK/dV) of it, so a
// block-sparse bias (a band, blocks along the diagonal, padding) skips its
// all-masked tiles: their probabilities are exact zeros, and leaving them out
// changes no result.  Customised masks are the reason the 51CTO FlashAttention
// V1/V2 notes give for writing one's own kernel; the "+ mask" term of the
// score formula (the CSDN post "Flash Attention1", section "Flash Attention")
// is the bias.
//
// One workgroup per tile: thread t reads row t/2, keys (t%2)*32 .. +31 with
// 8-byte buffer loads (rows past Nq and keys past Nk do not count); the
// workgroup ORs the findings.  The kernel reads the bias once and is bound by
// HBM bandwidth; the map is meant to be computed once per bias and reused.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void bias_tile_map_kernel(const T* __restrict__ bias,
                                                            long long sb, long long sh,
                                                            long long sq, int Hb, int Nq, int Nk,
                                                            int nqt, int nkt4,
                                                            unsigned char* __restrict__ tmap) {
  static_assert(kMapRows * 2 == 256 && kMapKeys == 64, "one thread per half row of a tile");
  const int kt = blockIdx.x % nkt4;
  const int rest = blockIdx.x / nkt4;
  const int qt = rest % nqt;
  const int hb = rest / nqt;  // bias head b' * Hb + h'
  const int b = hb / Hb, h = hb - b * Hb;
  const int row = qt * kMapRows + (threadIdx.x >> 1);
  const int key0 = kt * kMapKeys + (threadIdx.x & 1) * 32;
  const T* base = bias + b * sb + h * sh;
  const BiasReader<T> br(base, (long long)(Nq - 1) * sq + Nk);
  bool any = false;
  if (row < Nq && key0 < Nk) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const typename Vec<T>::x4 v = br.load4((unsigned)((long long)row * sq + key0 + 4 * q));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        any |= (key0 + 4 * q + e < Nk) && !((float)v[e] == -INFINITY);  // NaN counts as present
    }
  }
  const int found = __syncthreads_or(any ? 1 : 0);
  if (threadIdx.x == 0) tmap[blockIdx.x] = found ? 1 : 0;
}

}  // namespace

hipError_t launch_bias_tile_map(const BiasArgs& bias, int B, int H, int Nq, int Nk, bool fp16,
                                unsigned char* tmap, hipStream_t s) {
  const int Bb = bias.sb ? B : 1, Hb = bias.sh ? H : 1;
  const int nqt = (Nq + kMapRows - 1) / kMapRows;
  const int nkt4 = ((Nk + kMapKeys - 1) / kMapKeys + 3) / 4 * 4;
  const long long nblocks = (long long)Bb * Hb * nqt * nkt4;
  if (nblocks == 0) return hipSuccess;
  if (fp16)
    hipLaunchKernelGGL((bias_tile_map_kernel<f16>), dim3((unsigned)nblocks), dim3(256), 0, s,
                       (const f16*)bias.ptr, bias.sb, bias.sh, bias.sq, Hb, Nq, Nk, nqt, nkt4,
                       tmap);
  else
    hipLaunchKernelGGL((bias_tile_map_kernel<bf16>), dim3((unsigned)nblocks), dim3(256), 0, s,
                       (const bf16*)bias.ptr, bias.sb, bias.sh, bias.sq, Hb, Nq, Nk, nqt, nkt4,
                       tmap);
  return hipGetLastError();
}

}  // namespace fa
