// libfa C ABI: argument checks, path selection and launches (declared in include/fa.h).
#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa_launch.h"

namespace {

constexpr int kVersion = 2 * 10000 + 0 * 100 + 0;
constexpr size_t kAlign = 16;
constexpr size_t kWsAlign = 256;
constexpr int kSplitTargetBlocks = 2048;  // aim for ~8 workgroups per CU on the split path
constexpr int kSplitMinKeys = 256;        // do not split below this many keys per chunk
// Key splits for a few query rows (1 < Nq <= kRowsSplitMaxNq: one 128-row
// query tile per head): the tiled kernel per (query tile, key chunk).
constexpr int kRowsSplitMaxNq = 128;
constexpr int kRowsSplitTarget = 1024;  // workgroups (4 waves each) to aim for
constexpr int kRowsSplitMinKeys = 512;  // keys per chunk at least (8 key tiles)
constexpr int kRowsSplitAlign = 128;    // chunks are whole pairs of 64-key tiles

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

bool dtype_ok(fa_dtype t) { return t == FA_BF16 || t == FA_FP16 || t == FA_FP32; }
bool is_mfma(fa_dtype t) { return t == FA_BF16 || t == FA_FP16; }

// Common shape checks.  Returns FA_OK when the sizes are usable; sets *empty
// when there is nothing to compute for the forward pass.
fa_status check_dims(int B, int H, int Nq, int Nk, int d, float scale, int causal, fa_dtype dtype) {
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // The kernels mask a score by setting it to -inf before it is multiplied by
  // scale, which needs a positive, finite multiplier.
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_UNSUPPORTED;
  const long long bh = (long long)B * H;
  if (bh > INT_MAX) return FA_ERR_SHAPE;
  // every workgroup count below is at most bh * ceil(N / 64) and must fit in int
  const long long nmax = (Nq > Nk ? Nq : Nk);
  if (bh * ((nmax + 63) / 64) > INT_MAX) return FA_ERR_SHAPE;
  if (bh > 0 && Nq > 0 && Nk == 0) return FA_ERR_SHAPE;
  if (causal && Nq > Nk && bh > 0 && Nq > 0) return FA_ERR_SHAPE;
  return FA_OK;
}

int auto_splits(int BH, int Nk) {
  int s = (kSplitTargetBlocks + BH - 1) / BH;
  const int by_keys = (Nk + kSplitMinKeys - 1) / kSplitMinKeys;
  if (s > by_keys) s = by_keys;
  return s < 1 ? 1 : s;
}

// Effective split count: chunks of ceil(Nk/s) keys, none empty.
int effective_splits(int Nk, int s) {
  if (s < 1) s = 1;
  if (s > Nk) s = Nk;
  const int chunk = fa::split_chunk(Nk, s);
  return (Nk + chunk - 1) / chunk;
}

// Chunk length of the row-split path: ceil(Nk / s) rounded up to whole tile pairs.
int rows_split_chunk(int Nk, int s) {
  const int c = (Nk + s - 1) / s;
  return (c + kRowsSplitAlign - 1) / kRowsSplitAlign * kRowsSplitAlign;
}

int rows_auto_splits(int BH, int Nk) {
  int s = (kRowsSplitTarget + BH - 1) / BH;
  const int by_keys = Nk / kRowsSplitMinKeys;
  if (s > by_keys) s = by_keys;
  return s < 1 ? 1 : s;
}

// 0: tiled path, >0: split path with that many splits, <0: unsupported combination.
int choose_splits(int B, int H, int Nq, int Nk, fa_dtype dtype, int num_splits) {
  if (num_splits < 0) return -1;
  if (Nq == 1 && is_mfma(dtype)) {
    const int s = num_splits == 0 ? auto_splits(B * H, Nk) : num_splits;
    return effective_splits(Nk, s);
  }
  if (Nq > 1 && Nq <= kRowsSplitMaxNq && is_mfma(dtype)) {
    int s = num_splits == 0 ? rows_auto_splits(B * H, Nk) : num_splits;
    if (s > Nk) s = Nk;
    if (s <= 1) return 0;  // one chunk: the tiled path
    const int chunk = rows_split_chunk(Nk, s);
    const int eff = (Nk + chunk - 1) / chunk;
    // partial rows (B*H*Nq per split) are indexed with 32-bit counts
    if ((long long)B * H * Nq * eff > INT_MAX / 128) return 0;
    return eff > 1 ? eff : 0;
  }
  if (num_splits > 1) return -1;
  return 0;
}

struct SplitWs {
  size_t o_bytes, l_off, total;
};

SplitWs split_ws(int BH, int d, int splits) {
  SplitWs w;
  w.o_bytes = (size_t)splits * BH * d * sizeof(float);
  w.l_off = round_up(w.o_bytes, kWsAlign);
  w.total = w.l_off + round_up((size_t)splits * BH * sizeof(float), kWsAlign);
  return w;
}

// Backward workspace: per head and block of 32 query rows, the rows' fp32
// L*log2(e) and then their -D (rows past Nq zero).
size_t bwd_ws_bytes(int BH, int Nq) {
  return round_up((size_t)BH * ((Nq + 31LL) / 32) * 64 * sizeof(float), kWsAlign);
}

// After it, the dS buffer of the stored-dS backward, where that path runs:
// the dK/dV kernel stores dS and dQ = dS K reads it, instead of a dQ kernel
// that recomputes S and dP (two of its three GEMMs).  The buffer holds 2
// bytes per (query, key) pair, padded to 32 x 32 blocks, so it grows with
// Nq * Nk.  The path runs for bf16 and fp16 at d = 128, with or without a
// bias, with Nq and Nk of at least kDsMinLen, a buffer of at most
// kDsMaxBytes, and a grid of at least kDsMinBlocks 128-key blocks over all
// heads (B*H*ceil(min(Nq, Nk)/128); twice that with a causal mask).
// Measured against recomputation (same process, steady state): 4-15% faster
// at d = 128 from 1024 such blocks (N = 1024-8192), and non-causal from 512;
// 6-12% with a dense bias (single calls: its dQ kernel no longer reads the
// bias).  Slower at d = 64, where the recomputed GEMMs cost half as much and
// the dS traffic the same, and on small grids (6-58% with 128-512 blocks
// causal, 40% with 128 non-causal), where the fused recomputing launch runs
// the dQ workgroups on the CUs that the key blocks' chains leave idle.
constexpr size_t kDsMaxBytes = size_t(8) << 30;
constexpr int kDsMinLen = 1024;
constexpr long long kDsMinBlocks = 512;
bool bwd_stores_ds(int BH, int Nq, int Nk, int d, bool causal, fa_dtype dtype) {
  if (dtype == FA_FP32 || d != 128 || BH <= 0 || Nq < kDsMinLen || Nk < kDsMinLen) return false;
  const long long blocks = (long long)BH * ((std::min(Nq, Nk) + 127LL) / 128);
  if (blocks < (causal ? 2 : 1) * kDsMinBlocks) return false;
  // The padded buffer holds at least 2 bytes per pair: past the bound by that
  // count (in 128-bit arithmetic), the call recomputes.  Below it Nq and Nk
  // are at most 2^22, far from overflowing fa::bwd_ds_bytes, which sizes the
  // padded buffer exactly (check_dims admits Nk near 2^31).
  if ((unsigned __int128)BH * (unsigned)Nq * (unsigned)Nk * 2 > kDsMaxBytes) return false;
  return fa::bwd_ds_bytes(BH, Nq, Nk) <= kDsMaxBytes;
}
// dS buffer bytes of a call with these sizes (0: it recomputes dQ).  The
// workspace query, which has no causal argument, asks for the non-causal
// rule, whose grid bound is the lower one.
size_t bwd_ds_ws_bytes(int BH, int Nq, int Nk, int d, bool causal, fa_dtype dtype) {
  return bwd_stores_ds(BH, Nq, Nk, d, causal, dtype) ? round_up(fa::bwd_ds_bytes(BH, Nq, Nk), kWsAlign)
                                                     : 0;
}

// Scratch of fa_bwd_noalloc: the per-row L*log2(e) and -D that fa_bwd keeps
// in the caller's workspace (8 bytes per query row, rows padded to 32 per head).  One copy per GPU, held until the process
// ends; every call on a GPU shares it.  In host code `scratch` names a
// host-side stand-in, never the device memory: the kernels get the device
// address that hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
fa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid or inconsistent sizes";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: dtype, head dim, scale or option not supported";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed";
  }
  return "unknown fa_status";
}

int fa_version(void) { return kVersion; }

int fa_fwd_num_splits(int B, int H, int Nq, int Nk, int d, fa_dtype dtype, int num_splits) {
  if (check_dims(B, H, Nq, Nk, d, 1.f, 0, dtype) != FA_OK) return 0;
  if ((long long)B * H * Nq == 0) return 0;
  const int s = choose_splits(B, H, Nq, Nk, dtype, num_splits);
  return s > 0 ? s : (s == 0 ? 1 : 0);
}

size_t fa_fwd_workspace_size(int B, int H, int Nq, int Nk, int d, fa_dtype dtype, int num_splits) {
  if (check_dims(B, H, Nq, Nk, d, 1.f, 0, dtype) != FA_OK) return 0;
  if ((long long)B * H * Nq == 0) return 0;
  const int s = choose_splits(B, H, Nq, Nk, dtype, num_splits);
  if (s <= 0) return 0;
  return split_ws(B * H * Nq, d, s).total;
}

size_t fa_bwd_workspace_size(int B, int H, int Nq, int Nk, int d, fa_dtype dtype) {
  if (check_dims(B, H, Nq, Nk, d, 1.f, 0, dtype) != FA_OK) return 0;
  return bwd_ws_bytes(B * H, Nq) + bwd_ds_ws_bytes(B * H, Nq, Nk, d, false, dtype);
}

int fa_bwd_stores_ds(int B, int H, int Nq, int Nk, int d, int causal, fa_dtype dtype) {
  if (check_dims(B, H, Nq, Nk, d, 1.f, causal, dtype) != FA_OK) return 0;
  return bwd_stores_ds(B * H, Nq, Nk, d, causal != 0, dtype) ? 1 : 0;
}

}  // extern "C"

namespace {

// Additive-bias checks (see fa_fwd_bias): rows of at least Nk elements, 16-byte
// aligned rows and head blocks, element offsets within a head below 2^30.
// Geometry of a bias tile map: Bb x Hb heads of nqt rows of nkt4 bytes.
struct MapGeom {
  long long Bb, Hb, nqt, nkt4;
  long long bytes() const { return Bb * Hb * nqt * nkt4; }
};
MapGeom map_geom(long long sb, long long sh, int B, int H, int Nq, int Nk) {
  MapGeom g;
  g.Bb = sb ? B : 1;
  g.Hb = sh ? H : 1;
  g.nqt = (Nq + 127LL) / 128;
  g.nkt4 = ((Nk + 63LL) / 64 + 3) / 4 * 4;
  return g;
}

// Attach a caller's tile map of map_bytes bytes to the bias arguments (bias
// already checked): the kernels read every byte of the geometry below, so a
// smaller buffer is refused.
fa_status attach_map(const unsigned char* map, size_t map_bytes, int B, int H, int Nq, int Nk,
                     fa_dtype dtype, fa::BiasArgs* b) {
  if (!map) return FA_OK;
  if (!b->ptr || dtype == FA_FP32) return FA_ERR_UNSUPPORTED;
  if (!aligned(map)) return FA_ERR_ALIGN;
  const MapGeom g = map_geom(b->sb, b->sh, B, H, Nq, Nk);
  if (g.bytes() > INT_MAX) return FA_ERR_SHAPE;
  if (map_bytes < (size_t)g.bytes()) return FA_ERR_WORKSPACE;
  b->tmap = map;
  b->nkt4 = (int)g.nkt4;
  b->tm_sh = b->sh ? g.nqt * g.nkt4 : 0;
  b->tm_sb = b->sb ? g.Hb * g.nqt * g.nkt4 : 0;
  return FA_OK;
}

fa_status check_bias(const void* bias, long long sb, long long sh, long long sq, int Nq, int Nk) {
  if (!bias) return FA_ERR_NULL;
  if (!aligned(bias)) return FA_ERR_ALIGN;
  if (sb < 0 || sh < 0 || sq < Nk || sq < 1) return FA_ERR_SHAPE;
  if (sq % 8 != 0 || sb % 8 != 0 || sh % 8 != 0) return FA_ERR_ALIGN;
  if (Nq > 0 && (long long)(Nq - 1) * sq + Nk > (1LL << 30)) return FA_ERR_SHAPE;
  return FA_OK;
}

// Dropout probability p -> keep threshold T = round((1 - p) * 256) (ties to
// even, in double): a score is kept iff its random byte is below T, and kept
// probabilities are scaled by 256 / T.  T = 256 (p below 1/512) keeps every
// score, which is the path without dropout.
fa_status make_dropout(float p, unsigned long long seed, unsigned offset, fa::DropArgs* out) {
  if (!(p >= 0.f && p < 1.f)) return FA_ERR_UNSUPPORTED;
  const int t = (int)std::nearbyint((1.0 - (double)p) * 256.0);
  if (t < 1) return FA_ERR_UNSUPPORTED;
  fa::DropArgs d;
  d.on = t < 256;
  d.seed_lo = (unsigned)(seed & 0xFFFFFFFFull);
  d.seed_hi = (unsigned)(seed >> 32);
  d.offset = offset;
  d.thresh = (unsigned)t;
  d.inv_keep = (float)(256.0 / t);
  *out = d;
  return FA_OK;
}

// The forward pass behind every forward entry point; num_splits as fa_fwd
// takes it, or -1 for the tiled path only (the bias and dropout entry points).
fa_status fwd_impl(const void* Q, const void* K, const void* V, const fa::BiasArgs& bias,
                   const fa::DropArgs& drop, void* O,
                   float* L, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   fa_dtype dtype, int num_splits, void* workspace, size_t workspace_bytes,
                   void* stream) {
  fa_status st = check_dims(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if ((long long)B * H * Nq == 0) return FA_OK;
  if (!Q || !K || !V || !O || !L) return FA_ERR_NULL;
  if (!aligned(Q) || !aligned(K) || !aligned(V) || !aligned(O) || !aligned(L)) return FA_ERR_ALIGN;
  // num_splits < 0 here: the tiled path only (the bias and dropout entry points)
  const int splits = (num_splits < 0 || bias.ptr || drop.on)
                         ? 0
                         : choose_splits(B, H, Nq, Nk, dtype, num_splits);
  if (splits < 0) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{Q, K, V, O, L, B, H, Nq, Nk, d, scale, causal != 0};
  a.bias = bias;
  a.drop = drop;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (splits > 0) {
    const SplitWs w = split_ws(B * H * Nq, d, splits);
    if (!workspace || workspace_bytes < w.total) return FA_ERR_WORKSPACE;
    if (!aligned(workspace)) return FA_ERR_ALIGN;
    float* part_o = static_cast<float*>(workspace);
    float* part_l = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.l_off);
    if (Nq == 1) {
      a.causal = false;  // one query row sees every key under bottom-right alignment
      e = (dtype == FA_BF16) ? fa::launch_fwd_split_bf16(a, splits, part_o, part_l, s)
                             : fa::launch_fwd_split_f16(a, splits, part_o, part_l, s);
    } else {
      const int chunk = rows_split_chunk(Nk, splits);
      e = (dtype == FA_BF16)
              ? fa::launch_fwd_rows_split_bf16(a, splits, chunk, part_o, part_l, s)
              : fa::launch_fwd_rows_split_f16(a, splits, chunk, part_o, part_l, s);
      if (e == hipSuccess)
        e = (dtype == FA_BF16) ? fa::launch_split_combine_bf16(a, splits, part_o, part_l, s)
                               : fa::launch_split_combine_f16(a, splits, part_o, part_l, s);
    }
  } else if (dtype == FA_BF16) {
    e = fa::launch_fwd_bf16(a, s);
  } else if (dtype == FA_FP16) {
    e = fa::launch_fwd_f16(a, s);
  } else {
    e = fa::launch_fwd_f32(a, s);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status bwd_impl(const void* Q, const void* K, const void* V, const fa::BiasArgs& bias,
                   const fa::DropArgs& drop, const void* O, const float* L, const void* dO, void* dQ, void* dK, void* dV,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal, fa_dtype dtype,
                   void* workspace, size_t workspace_bytes, void* stream, int stages,
                   bool allow_ds = true) {
  if (stages <= 0 || stages > FA_BWD_ALL) return FA_ERR_UNSUPPORTED;
  fa_status st = check_dims(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if ((long long)B * H == 0 || (Nq == 0 && Nk == 0)) return FA_OK;
  if (!K || !V || !dK || !dV) return FA_ERR_NULL;
  if (Nq > 0 && (!Q || !O || !L || !dO || !dQ)) return FA_ERR_NULL;
  if (!aligned(K) || !aligned(V) || !aligned(dK) || !aligned(dV)) return FA_ERR_ALIGN;
  if (Nq > 0 && (!aligned(Q) || !aligned(O) || !aligned(L) || !aligned(dO) || !aligned(dQ)))
    return FA_ERR_ALIGN;
  // stored dS, where it runs (not for fa_bwd_noalloc)
  const size_t ws_ld = bwd_ws_bytes(B * H, Nq);
  const size_t ws_ds = allow_ds ? bwd_ds_ws_bytes(B * H, Nq, Nk, d, causal != 0, dtype) : 0;
  if (Nq > 0 && (!workspace || workspace_bytes < ws_ld + ws_ds)) return FA_ERR_WORKSPACE;
  if (Nq > 0 && !aligned(workspace)) return FA_ERR_ALIGN;
  fa::BwdArgs a{Q, K, V, O, L, dO, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal != 0,
                nullptr};
  a.bias = bias;
  a.drop = drop;
  if (Nq > 0) a.LD = static_cast<float*>(workspace);
  if (ws_ds > 0) a.dS = static_cast<char*>(workspace) + ws_ld;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e =
      (dtype == FA_BF16)   ? fa::launch_bwd_bf16(a, stages, s)
      : (dtype == FA_FP16) ? fa::launch_bwd_f16(a, stages, s)
                           : fa::launch_bwd_f32(a, stages, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H,
                 int Nq, int Nk, int d, float scale, int causal, fa_dtype dtype, int num_splits,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (num_splits < 0) {
    const fa_status st = check_dims(B, H, Nq, Nk, d, scale, causal, dtype);
    return st != FA_OK ? st : FA_ERR_UNSUPPORTED;
  }
  return fwd_impl(Q, K, V, fa::BiasArgs{}, fa::DropArgs{}, O, L, B, H, Nq, Nk, d, scale, causal,
                  dtype, num_splits,
                  workspace, workspace_bytes, stream);
}

fa_status fa_fwd_bias(const void* Q, const void* K, const void* V, const void* bias,
                      long long bias_sb, long long bias_sh, long long bias_sq, void* O, float* L,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal, fa_dtype dtype,
                      void* stream) {
  fa_status st = check_dims(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if ((long long)B * H * Nq == 0) return FA_OK;
  st = check_bias(bias, bias_sb, bias_sh, bias_sq, Nq, Nk);
  if (st != FA_OK) return st;
  fa::BiasArgs b;
  b.ptr = bias;
  b.sb = bias_sb;
  b.sh = bias_sh;
  b.sq = bias_sq;
  return fwd_impl(Q, K, V, b, fa::DropArgs{}, O, L, B, H, Nq, Nk, d, scale, causal, dtype, -1,
                  nullptr, 0, stream);
}

fa_status fa_bwd_bias(const void* Q, const void* K, const void* V, const void* bias,
                      long long bias_sb, long long bias_sh, long long bias_sq, const void* O,
                      const float* L, const void* dO, void* dQ, void* dK, void* dV, int B, int H,
                      int Nq, int Nk, int d, float scale, int causal, fa_dtype dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = check_dims(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if ((long long)B * H == 0 || Nq == 0) {
    return bwd_impl(Q, K, V, fa::BiasArgs{}, fa::DropArgs{}, O, L, dO, dQ, dK, dV, B, H, Nq, Nk,
                    d, scale, causal, dtype, workspace, workspace_bytes, stream, FA_BWD_ALL);
  }
  st = check_bias(bias, bias_sb, bias_sh, bias_sq, Nq, Nk);
  if (st != FA_OK) return st;
  fa::BiasArgs b;
  b.ptr = bias;
  b.sb = bias_sb;
  b.sh = bias_sh;
  b.sq = bias_sq;
  return bwd_impl(Q, K, V, b, fa::DropArgs{}, O, L, dO, dQ, dK, dV, B, H, Nq, Nk, d, scale,
                  causal, dtype, workspace, workspace_bytes, stream, FA_BWD_ALL);
}

fa_status fa_fwd_ex(const void* Q, const void* K, const void* V, const void* bias,
                    long long bias_sb, long long bias_sh, long long bias_sq,
                    const unsigned char* bias_tile_map, size_t bias_tile_map_bytes,
                    float dropout_p, unsigned long long seed, unsigned int offset, void* O,
                    float* L, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                    fa_dtype dtype, void* stream) {
  fa_status st = check_dims(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  fa::DropArgs dr;
  st = make_dropout(dropout_p, seed, offset, &dr);
  if (st != FA_OK) return st;
  if ((long long)B * H * Nq == 0) return FA_OK;
  fa::BiasArgs b;
  if (bias) {
    st = check_bias(bias, bias_sb, bias_sh, bias_sq, Nq, Nk);
    if (st != FA_OK) return st;
    b.ptr = bias;
    b.sb = bias_sb;
    b.sh = bias_sh;
    b.sq = bias_sq;
  }
  st = attach_map(bias_tile_map, bias_tile_map_bytes, B, H, Nq, Nk, dtype, &b);
  if (st != FA_OK) return st;
  return fwd_impl(Q, K, V, b, dr, O, L, B, H, Nq, Nk, d, scale, causal, dtype, -1, nullptr, 0,
                  stream);
}

fa_status fa_bwd_ex(const void* Q, const void* K, const void* V, const void* bias,
                    long long bias_sb, long long bias_sh, long long bias_sq,
                    const unsigned char* bias_tile_map, size_t bias_tile_map_bytes,
                    float dropout_p, unsigned long long seed, unsigned int offset,
                    const void* O, const float* L,
                    const void* dO, void* dQ, void* dK, void* dV, int B, int H, int Nq, int Nk,
                    int d, float scale, int causal, fa_dtype dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  fa_status st = check_dims(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  fa::DropArgs dr;
  st = make_dropout(dropout_p, seed, offset, &dr);
  if (st != FA_OK) return st;
  fa::BiasArgs b;
  if (bias && (long long)B * H > 0 && Nq > 0) {
    st = check_bias(bias, bias_sb, bias_sh, bias_sq, Nq, Nk);
    if (st != FA_OK) return st;
    b.ptr = bias;
    b.sb = bias_sb;
    b.sh = bias_sh;
    b.sq = bias_sq;
    st = attach_map(bias_tile_map, bias_tile_map_bytes, B, H, Nq, Nk, dtype, &b);
    if (st != FA_OK) return st;
  } else if (bias_tile_map && !bias) {
    return FA_ERR_UNSUPPORTED;
  }
  return bwd_impl(Q, K, V, b, dr, O, L, dO, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal, dtype,
                  workspace, workspace_bytes, stream, FA_BWD_ALL);
}

size_t fa_bias_tile_map_size(long long bias_sb, long long bias_sh, int B, int H, int Nq,
                             int Nk) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return 0;
  return (size_t)map_geom(bias_sb, bias_sh, B, H, Nq, Nk).bytes();
}

fa_status fa_bias_tile_map(const void* bias, long long bias_sb, long long bias_sh,
                           long long bias_sq, int B, int H, int Nq, int Nk, fa_dtype dtype,
                           unsigned char* tile_map, size_t tile_map_bytes, void* stream) {
  if (!dtype_ok(dtype) || dtype == FA_FP32) return FA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
  const MapGeom g = map_geom(bias_sb, bias_sh, B, H, Nq, Nk);
  if (g.bytes() == 0) return FA_OK;
  if (g.bytes() > INT_MAX) return FA_ERR_SHAPE;
  fa_status st = check_bias(bias, bias_sb, bias_sh, bias_sq, Nq, Nk);
  if (st != FA_OK) return st;
  if (!tile_map) return FA_ERR_NULL;
  if (tile_map_bytes < (size_t)g.bytes()) return FA_ERR_WORKSPACE;
  fa::BiasArgs b;
  b.ptr = bias;
  b.sb = bias_sb;
  b.sh = bias_sh;
  b.sq = bias_sq;
  const hipError_t e = fa::launch_bias_tile_map(b, B, H, Nq, Nk, dtype == FA_FP16, tile_map,
                                                reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* L,
                 const void* dO, void* dQ, void* dK, void* dV, int B, int H, int Nq, int Nk, int d,
                 float scale, int causal, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return fa_bwd_stages(Q, K, V, O, L, dO, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal, dtype,
                       workspace, workspace_bytes, stream, FA_BWD_ALL);
}

fa_status fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                         const float* L, const void* dO, void* dQ, void* dK, void* dV, int B,
                         int H, int Nq, int Nk, int d, float scale, int causal, fa_dtype dtype,
                         void* stream) {
  const fa_status st = check_dims(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if ((long long)B * H == 0 || Nq == 0) {
    return bwd_impl(Q, K, V, fa::BiasArgs{}, fa::DropArgs{}, O, L, dO, dQ, dK, dV, B, H, Nq, Nk,
                    d, scale, causal, dtype, nullptr, 0, stream, FA_BWD_ALL);
  }
  if (bwd_ws_bytes(B * H, Nq) > kNoAllocScratchBytes) return FA_ERR_WORKSPACE;
  void* ws = nullptr;
  const fa_status sa = scratch_address(&ws);
  if (sa != FA_OK) return sa;
  return bwd_impl(Q, K, V, fa::BiasArgs{}, fa::DropArgs{}, O, L, dO, dQ, dK, dV, B, H, Nq, Nk, d,
                  scale, causal, dtype, ws, kNoAllocScratchBytes, stream, FA_BWD_ALL,
                  /*allow_ds=*/false);
}

size_t fa_bwd_noalloc_max_rows(void) { return kNoAllocScratchBytes / 8; }

fa_status fa_bwd_stages(const void* Q, const void* K, const void* V, const void* O,
                        const float* L, const void* dO, void* dQ, void* dK, void* dV, int B,
                        int H, int Nq, int Nk, int d, float scale, int causal, fa_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream, int stages) {
  return bwd_impl(Q, K, V, fa::BiasArgs{}, fa::DropArgs{}, O, L, dO, dQ, dK, dV, B, H, Nq, Nk, d,
                  scale, causal, dtype, workspace, workspace_bytes, stream, stages);
}

}  // extern "C"
