// Host-side launchers of the libfa kernels (internal to the library).
// Each returns the hipError_t of its launch(es); shapes are validated by the
// caller (fa_api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Optional additive bias: element (b, h, i, j) at ptr[b*sb + h*sh + i*sq + j]
// (ptr == nullptr: none).  Same element type as Q.
// Optional tile map of that bias (tmap == nullptr: none): byte (b, h, qt, kt)
// at tmap[b*tm_sb + h*tm_sh + qt*nkt4 + kt], nonzero iff the 128-row x 64-key
// tile holds an entry above -inf.
struct BiasArgs {
  const void* ptr = nullptr;
  long long sb = 0, sh = 0, sq = 0;
  const unsigned char* tmap = nullptr;
  long long tm_sb = 0, tm_sh = 0;
  int nkt4 = 0;
};

// Optional dropout on the normalised probabilities (on == false: none).  A
// score is kept iff its Philox byte is below thresh (1..255); kept
// probabilities are scaled by inv_keep = 256 / thresh.
struct DropArgs {
  bool on = false;
  unsigned seed_lo = 0, seed_hi = 0, offset = 0, thresh = 256;
  float inv_keep = 1.f;
};

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* L;
  int B, H, Nq, Nk, d;
  float scale;
  bool causal;
  BiasArgs bias;
  DropArgs drop;
};

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const float* L;
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  int B, H, Nq, Nk, d;
  float scale;
  bool causal;
  float* LD;  // fp32 workspace: per head and block of 32 query rows, L * log2(e) and -D, D = rowsum(dO * O)
  BiasArgs bias;
  DropArgs drop;
  // 16-bit dtypes at d = 128: the dS buffer (bwd_ds_bytes) when the
  // backward stores dS in the dK/dV kernel and forms dQ from it; nullptr:
  // the dQ kernel recomputes S and dP instead.
  void* dS = nullptr;
};

// Bytes of the dS buffer of the stored-dS backward for B*H heads.
size_t bwd_ds_bytes(int BH, int Nq, int Nk);

// Tiled forward (Q-tile per workgroup, K/V streamed through LDS).
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);

// Split-key forward for one query row per head, then the logsumexp combine.
// part_o: [splits, B*H, d] fp32, part_l: [splits, B*H] fp32.
hipError_t launch_fwd_split_bf16(const FwdArgs& a, int splits, float* part_o, float* part_l,
                                 hipStream_t s);
hipError_t launch_fwd_split_f16(const FwdArgs& a, int splits, float* part_o, float* part_l,
                                hipStream_t s);

// Backward: D = rowsum(dO*O) and L*log2(e); dK and dV; dQ.
// `stages`: bit 1 the (L*log2 e, -D) blocks, bit 2 dK/dV kernel, bit 4 dQ kernel (2 and 4 read them).
hipError_t launch_bwd_bf16(const BwdArgs& a, int stages, hipStream_t s);
hipError_t launch_bwd_f16(const BwdArgs& a, int stages, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t s);

// Key splits for a few query rows (1 < Nq <= 128): the tiled forward kernel on
// (query tile, chunk of `chunk` keys), partials as above with B*H*Nq rows,
// then the combine of those partials into O and L.
hipError_t launch_fwd_rows_split_bf16(const FwdArgs& a, int splits, int chunk, float* part_o,
                                      float* part_l, hipStream_t s);
hipError_t launch_fwd_rows_split_f16(const FwdArgs& a, int splits, int chunk, float* part_o,
                                     float* part_l, hipStream_t s);
hipError_t launch_split_combine_bf16(const FwdArgs& a, int splits, const float* part_o,
                                     const float* part_l, hipStream_t s);
hipError_t launch_split_combine_f16(const FwdArgs& a, int splits, const float* part_o,
                                    const float* part_l, hipStream_t s);

// Tile map of a bias (16-bit dtypes): one byte per 128-row x 64-key tile of
// each bias head (Bb = sb ? B : 1, Hb = sh ? H : 1 heads), rows of nkt4 bytes.
hipError_t launch_bias_tile_map(const BiasArgs& bias, int B, int H, int Nq, int Nk, bool fp16,
                                unsigned char* tmap, hipStream_t s);

// Key-chunk length used by the split path for `splits` chunks of Nk keys.
int split_chunk(int Nk, int splits);

}  // namespace fa
