// Backward pass kernels: dQ, dK, dV of f = sum(dO * O).
//
// Method: the backward pass recomputes the probabilities from Q, K and the
// forward logsumexp L instead of storing them (the Huawei Cloud post
// "FlashAttention", section 3, Recomputation; the 51CTO FlashAttention V1/V2
// notes, "FlashAttention V2相比V1有哪些改进": the backward pass needs only L).
// It also takes the per-row auxiliary D, which the notes name and the softmax
// Jacobian fixes as D = rowsum(dO * O).  Per (query, key) pair:
//     S = Q K^T            P  = exp(S * scale - L)
//     dP = dO V^T          dS = P * (dP - D)
//     dV += P^T dO         dK += scale * dS^T Q         dQ += scale * dS K
//
// dK and dV are computed with the grid over key blocks (the notes, "Thread
// Block Level 并行": the backward pass splits the key sequence across thread
// blocks), each workgroup keeping its dK and dV block on chip while it loops
// over query blocks.  dQ needs a sum over every key block.  The notes
// ("Sequence Parallel") weigh global atomic adds, which are slow, against
// per-key-block dQ buffers reduced afterwards, whose size grows with N^2 / BC.
// On MI355X fp32 atomic adds run at about a fifth of the store bandwidth.
// This library forms dQ per query block instead, in registers, with no
// atomics and no fp32 accumulator (every output is deterministic), one of two
// ways:
//  * stored dS (bf16/fp16, d = 128, long sequences; the host picks it): the
//    dK/dV kernel also writes its dS blocks, 2 bytes per pair, and
//    bwd_dq_ds_kernel, gridded over query blocks, forms dQ = scale * dS K from
//    them: the five GEMMs of the notes, for 4 bytes of HBM traffic per pair;
//  * otherwise bwd_dq_kernel recomputes S and dP for its rows (two extra
//    GEMMs per pair, seven in all) and needs no workspace beyond D; it runs in
//    one launch with the dK/dV workgroups (bwd_fused_kernel below).
//
// gfx950 mapping:
//  * bwd_dkdv_kernel: 256 threads = 4 waves, two workgroups per CU (two
//    waves per SIMD), so one wave's MFMAs overlap the other's LDS reads,
//    exponentials and barrier waits, and the two workgroups' barriers are
//    independent.  A workgroup owns BC = 128 keys and each wave 32 of them
//    (64 KB of LDS: the K block and two Q and dO buffers; with a bias, 8
//    waves and 256 keys, one workgroup per CU), so dK and dV stay
//    wave-private (the notes, "Warp Level 并行": with keys split across warps,
//    dV, dS and dK need no cross-warp reduction).  Scores are laid out with the
//    key along lanes (S = Q K^T on the 32x32x16 bf16/fp16 MFMA): rounded to 16 bits,
//    the fp32 accumulators of P and dS are directly the B operands of
//    dV^T = dO^T P and dK^T = Q^T dS; dO^T and Q^T come from the row-major LDS
//    tiles through the transpose read ds_read_b64_tr_b16.  K stays in LDS, the
//    wave's 32 rows of V in registers; Q, dO, L, D of the next 32-row query
//    block are loaded into registers while the current one is processed and
//    are double-buffered in LDS, so one barrier per query block suffices.
//  * bwd_dq_kernel: the forward pass's layout.  4 waves own 32 query rows
//    each (the notes' "sliced-Q": no cross-wave reduction); scores are computed
//    transposed, S^T = K Q^T and dP^T = V dO^T, so each lane holds one query
//    row and its L and D are scalars; dS^T feeds dQ^T = K^T dS^T from
//    registers, with K^T read from the K tile by the transpose read.  K and V
//    tiles of 64 keys are loaded straight into LDS (swizzled, double-buffered).
//  * Grids: the key-block grid pins heads to XCDs when B*H is a multiple of 8
//    (a head's workgroups then share one L2 for their re-reads of Q and dO)
//    and dispatches key blocks in order of decreasing work, which already
//    balances the causal triangle; the query-block
//    grid uses the forward pass's mapping, causal query tiles in pairs
//    (t, nqt-1-t) of equal total work.
//  * bwd_dq_ds_kernel: the dQ kernel's grid and wave layout without its
//    softmax: per 64-key tile a wave stages its two 2 KB dS chunks in LDS and
//    issues 16 MFMAs (d = 128) reading K^T and dS^T by transpose reads; bound
//    by the HBM reads of dS (both the dS stores and these reads carry the
//    non-temporal hint: 5-7% faster than cached accesses on the long-sequence
//    backward, whose 2 GiB of dS would otherwise pass through the caches).
//  * bwd_fused_kernel (no bias): both grids in one launch, merged by expected
//    workgroup length (long key blocks, then the dQ workgroups, then the short
//    key blocks), so that the dQ workgroups fill the CUs the long key blocks
//    leave, and on short sequences, where a few long key-block chains set the
//    time, the two grids run side by side (B4 H16 N1024 d64 causal:
//    63.5 -> 52.4 us for the backward pass).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

BiasDev bias_dev(const BiasArgs& b, int B, int H, float scale) {
  return make_bias_dev(b.ptr, b.sb, b.sh, b.sq, B, H, scale, b.tmap, b.tm_sb, b.tm_sh, b.nkt4);
}


// The backward workspace LD holds, per head and block of kLdRows query
// rows (64 floats), the rows' L2 = L * log2(e) (the exponent base of the
// kernels below) and -D, D = sum_k dO_ik O_ik in fp32; rows past Nq hold
// zeros.  Without dropout the block is [L2 x 32 | -D x 32]: one 16-byte read
// of -D fills four elements of a dP accumulator, which dK/dV then starts
// from -D instead of zero (dS = P (dP - D)).  With dropout, whose dP is
// masked and scaled before -D is added, the rows are interleaved,
// (L2_r, -D_r) for r = 0..31, so that one 16-byte read brings both values of
// two rows.  ld_index gives a row's L2; its -D is ld_nd_off floats on.
constexpr int kLdRows = 32;
template <bool DROP>
__host__ __device__ __forceinline__ size_t ld_index(int bh, int row, int nblk) {
  const int r = row % kLdRows;
  return ((size_t)bh * nblk + row / kLdRows) * (2 * kLdRows) + (DROP ? 2 * r : r);
}
template <bool DROP>
constexpr int ld_nd_off() { return DROP ? 1 : kLdRows; }

// dS buffer of the stored-dS backward (dK/dV kernel writes, dQ kernel reads):
// per head and 32-row query block, one 2 KB chunk per group of 32 keys (the
// keys of one dK/dV wave), 8 groups per 256 keys (keys padded to 256, which
// covers both the 128-key and, with a bias, the 256-key dK/dV workgroups);
// the chunks of a query block are consecutive.  A chunk holds the 16-bit dS of its 32 x 32 block as
// 64 16-byte slots: slot (kc, h, k) has the dS of key k of the group for the
// rows kc*16 + (e/4)*8 + h*4 + e%4 of the block (e = 0..7, one element each),
// i.e. what lane h*32 + k of the dK/dV wave holds as the MFMA operand of row
// chunk kc.  The slot lies at byte kc*1024 + h*512 + (k ^ 4(2kc + h))*16:
// each dK/dV store fills 1 KB in one piece, and the XOR spreads the dQ
// kernel's transposed reads of a chunk over all LDS banks.
constexpr int kDsChunk = 1024;  // elements per chunk
__host__ __device__ __forceinline__ int ds_chunks_per_row(int Nk) { return ((Nk + 255) / 256) * 8; }
__host__ __device__ __forceinline__ unsigned ds_chunk_off(int kc, int h, int k) {
  return (unsigned)(kc * 1024 + h * 512 + ((k ^ (4 * (2 * kc + h))) * 16));
}

template <int D, typename T, bool DROP>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O,
                                                      const T* __restrict__ dO,
                                                      const float* __restrict__ L,
                                                      float* __restrict__ LD, int Nq, int nblk) {
  constexpr int TPR = D / 8;      // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;  // rows per workgroup, all in one block of a head
  static_assert(kLdRows % RPB == 0, "a workgroup's rows lie in one block");
  const int wph = nblk * (kLdRows / RPB);  // workgroups per head (the grid has B*H * wph)
  const int bh = blockIdx.x / wph;
  const int r = (blockIdx.x - bh * wph) * RPB + threadIdx.x / TPR;  // row, padded
  const bool valid = r < Nq;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (valid) {
    const size_t base = ((size_t)bh * Nq + r) * D + part * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)O[base + e], (float)dO[base + e], acc);
  }
#pragma unroll
  for (int msk = TPR / 2; msk >= 1; msk >>= 1) acc += __shfl_xor(acc, msk, 64);
  if (part == 0) {
    const size_t i = ld_index<DROP>(bh, r, nblk);
    LD[i] = valid ? L[(size_t)bh * Nq + r] * kLog2e : 0.f;
    LD[i + ld_nd_off<DROP>()] = valid ? -acc : 0.f;
  }
}

// ---------------------------------------------------------------------------
// dK and dV: one workgroup per (key block, batch*head), 32 keys per wave.
// Without a bias: 4 waves and 128 keys, 64 KB of LDS, two workgroups per CU.
// With a bias, whose double-buffered tiles would take a pair of such
// workgroups just past the 160 KB of a CU: 8 waves and 256 keys, one per CU.
template <bool BIAS>
struct KvShape {
  static constexpr int kWaves = BIAS ? 8 : 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBC = kWaves * 32;  // keys per workgroup
  static constexpr int kPerCU = BIAS ? 1 : 2;
};
constexpr int kKvBR = 32;  // query rows per inner iteration

// LDS of a dK/dV workgroup: [Q buffers 0,1 | dO buffers 0,1 | K block], all
// swizzled (see swz); the (L2, -D) block of the query block per buffer;
// the bias tiles (BIAS).
template <typename T, int D, bool BIAS>
struct DkdvLds {
  static constexpr int BC = KvShape<BIAS>::kBC, BR = kKvBR;
  __attribute__((aligned(1024))) T smem[4 * BR * D + BC * D];
  __attribute__((aligned(16))) float sLD[2][2 * BR];
  alignas(BIAS ? 1024 : 16) T sBias[BIAS ? 2 * BR * BC : 8];
};

// Block `bid` of the key-block grid (the kernel's blockIdx.x).  DS: each
// wave also stores the dS of every query block it runs, as a 2 KB chunk of
// the dS buffer (layout at ds_chunk_off; two 16-byte non-temporal stores per
// lane, chunk half kc as soon as its 16 rows are formed), for bwd_dq_ds_kernel.
template <typename T, int D, bool CAUSAL, bool BIAS, bool DROP, bool DS = false>
__device__ __forceinline__ void dkdv_body(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ LD, T* __restrict__ dK,
    T* __restrict__ dV, int Nq, int Nk, int nkt, int BH, int hpx, float c, float scale, int off,
    BiasDev bias, DropDev drop, DkdvLds<T, D, BIAS>& lds, int bid, T* __restrict__ dSg = nullptr) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  constexpr int kKvWaves = KvShape<BIAS>::kWaves, kKvThreads = KvShape<BIAS>::kThreads;
  constexpr int BC = KvShape<BIAS>::kBC, BR = kKvBR;
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int NKK = D / 16;    // MFMA k-steps over the head dim
  constexpr int NNT = D / 32;    // 32-wide tiles over the head dim
  constexpr int KTILE = BC * D;  // elements of the K block
  constexpr int QTILE = BR * D;  // elements of one Q or dO tile
  constexpr int NIQ = BR * CPR / 64;           // direct-to-LDS loads per Q (or dO) tile
  constexpr int IPW = 2 * NIQ / kKvWaves;      // ... per wave for both tiles
  static_assert(IPW * kKvWaves == 2 * NIQ && IPW >= 1, "query tile load split");
  static_assert(2 * BR == 64, "one dword load per lane carries the (L2, -D) block");
  static_assert(NIQ % IPW == 0, "a wave loads from one tile");

  // Query block it uses buffers it & 1; the loop is unrolled by two so that
  // their offsets are constants.  The query tiles come first: their many
  // reads then carry the buffer offset in the 16-bit offset field of the LDS
  // instruction, which offsets past the 64 KB K block would not fit (each
  // read would need an address add).
  static_assert(sizeof(lds.smem) == (4 * QTILE + KTILE) * sizeof(T), "LDS layout");
  T* const smem = lds.smem;
  float (&sLD)[2][2 * BR] = lds.sLD;
  T* const sQ0 = smem;
  T* const sdO0 = smem + 2 * QTILE;
  T* const sK = smem + 4 * QTILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, s16 = lane & 15;

  int bh, kt;
  if (hpx > 0) {  // B*H = 8 * hpx: head bh runs on XCD bh % 8
    const int x = bid % kNumXcd, slot = bid / kNumXcd;
    bh = x + kNumXcd * (slot % hpx);
    kt = slot / hpx;
  } else {
    kt = bid / BH;
    bh = bid - kt * BH;
  }
  const int k0 = kt * BC;
  const int kw0 = k0 + wave * 32;  // this wave's first key
  const int mykey = kw0 + l32;     // the key of this lane's accumulator column
  const size_t qbase = (size_t)bh * Nq * D;
  const size_t kbase = (size_t)bh * Nk * D;
  const int nqb_ld = (Nq + BR - 1) / BR;  // blocks per head of the (L2, -D) workspace
  static_assert(BR == kLdRows, "one (L2, -D) block per query block");
  // DS: this wave's chunk of query block 0 and this lane's two 16-byte slots
  // in a chunk (elements); query block qb adds qb * ds_row.
  [[maybe_unused]] T* ds_wave = nullptr;
  [[maybe_unused]] size_t ds_row = 0;
  [[maybe_unused]] unsigned ds_lane[2] = {0u, 0u};
  if constexpr (DS) {
    static_assert(BR == 32, "dS chunks: 32 x 32 blocks");
    ds_row = (size_t)ds_chunks_per_row(Nk) * kDsChunk;
    ds_wave = dSg + (size_t)bh * nqb_ld * ds_row + (size_t)(kw0 / 32) * kDsChunk;
    ds_lane[0] = ds_chunk_off(0, half, l32) / 2;
    ds_lane[1] = ds_chunk_off(1, half, l32) / 2;
  }

  // Additive bias (BIAS) of this head, staged per query block: a tile of
  // BR rows x BC keys per buffer, double-buffered like Q and dO and filled by
  // the same direct-to-LDS loads (rows past Nq read as zeros; keys past Nk
  // are masked).  Row r keeps its 16-byte chunk c at c ^ 2*(r & 3), so the
  // transposed reads below (4 rows x 16 keys per 16 lanes) hit distinct
  // banks.  Lane offsets are fixed; block offsets go into the descriptor.
  constexpr int BTILE = BR * BC;                 // elements of one bias tile
  constexpr int NIB = BTILE * 2 / 16 / 64;       // direct-to-LDS loads per bias tile
  constexpr int IPB = NIB / kKvWaves;            // ... per wave
  static_assert(IPB * kKvWaves == NIB, "bias tile load split");
  T* const sBias = lds.sBias;
  const T* bias_h = nullptr;
  unsigned boff[IPB];
  unsigned bread = 0;  // byte offset of this lane's transposed read of row group 0
  if constexpr (BIAS) {
    const int b = bh / bias.H, h = bh - b * bias.H;
    bias_h = (const T*)bias.ptr + b * bias.sb + h * bias.sh;
#pragma unroll
    for (int u = 0; u < IPB; ++u) {
      const int slot = (wave * IPB + u) * 64 + lane;
      const int r = slot / (BC / 8), pch = slot % (BC / 8);
      // wraps only for rows past Nq, whose reads fall outside the descriptor
      boff[u] = (unsigned)((long long)r * bias.sq * 2) + (unsigned)((pch ^ (2 * (r & 3))) << 4);
    }
    // Lane l receives key kw0 + l%32 of rows 8g + 4*half + 0..3 (g = 0..3)
    // when lane s of each 16-lane group m points at row 4*(m/2) + s/4 (+8g),
    // keys wave*32 + (m%2)*16 + (s%4)*4 .. +3 of the tile.
    const int m = lane >> 4;
    const int row = 4 * (m >> 1) + (s16 >> 2);
    const int col = wave * 32 + (m & 1) * 16 + (s16 & 3) * 4;
    bread = (unsigned)(row * BC * 2 + (((col >> 3) ^ (2 * (row & 3))) << 4) + (col & 7) * 2);
  }

  // Query blocks that can see any key of this workgroup.
  int nqb = (Nq + BR - 1) / BR;
  int qb_first = CAUSAL ? max(0, k0 - off) / BR : 0;
  // Bias tile map (BIAS): only the query blocks from the first to the last
  // 128-row tile that holds an entry above -inf for one of this workgroup's
  // two 64-key tiles.
  if constexpr (BIAS) {
    static_assert(BC % kMapKeys == 0 && kMapRows % BR == 0, "tile map granularity");
    if (bias.tmap) {
      const int b = bh / bias.H, h = bh - b * bias.H;
      int lo, hi;
      map_range_cols<BC / kMapKeys>(bias.tmap + b * bias.tm_sb + h * bias.tm_sh, (Nq + kMapRows - 1) / kMapRows,
                     bias.nkt4, k0 / kMapKeys, lane, lo, hi);
      if (lo > hi) {
        nqb = qb_first;
      } else {
        qb_first = max(qb_first, lo * (kMapRows / BR));
        nqb = min(nqb, (hi + 1) * (kMapRows / BR));
      }
    }
  }
  const int nloop = nqb - qb_first;

  // Direct-to-LDS loads of query block qb through buffer resources: this
  // wave's IPW chunks of the Q (waves 0 .. 8/2-1) or dO tile, and (last
  // wave) the (L2, -D) block; rows past Nq read as zeros.  Lane offsets
  // are fixed; the rest is wave-uniform.
  const int tsel = (wave * IPW) / NIQ;  // 0: Q, 1: dO
  const T* const qsrc = (tsel ? dO : Q) + qbase;
  T* const qdst0 = (tsel ? sdO0 : sQ0) + ((wave * IPW) % NIQ) * 64 * 8;
  unsigned qoff[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int slot = ((wave * IPW) % NIQ + u) * 64 + lane;
    const int r = slot / CPR, pch = slot % CPR;
    qoff[u] = (unsigned)(r * D * 2 + ((pch ^ swz<D>(r)) << 4));
  }
  auto load_block = [&](int qb, int buf) {
    const int qi0 = qb * BR;
#if __HIP_DEVICE_COMPILE__
    const int rows = __builtin_amdgcn_readfirstlane(min(Nq - qi0, BR));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qsrc + (size_t)qi0 * D, rows * D * 2);
#pragma unroll
    for (int u = 0; u < IPW; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (FA_LDS void*)(qdst0 + buf * QTILE + u * 64 * 8), 16, qoff[u], 0, 0, 0);
    if (wave == kKvWaves - 1) {
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(LD + ld_index<DROP>(bh, qi0, nqb_ld), 2 * BR * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (FA_LDS void*)&sLD[buf][0], 4, lane * 4, 0,
                                               0, 0);
    }
    if constexpr (BIAS) {
      // the block's bias from row qi0, key k0 on: (Nq-1-qi0)*sq + Nk-k0 elements,
      // the range rounded up to 16 bytes as in BiasReader
      const long long ext = (long long)(Nq - 1 - qi0) * bias.sq + (Nk - k0);
      const unsigned long long nb = ((unsigned long long)ext * 2 + 15) & ~15ull;
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(bias_h + (size_t)qi0 * bias.sq + k0,
                    (int)(unsigned)(nb < 0xfffffff0ull ? nb : 0xfffffff0ull));
      if (bias.stream) {
#pragma unroll
        for (int u = 0; u < IPB; ++u)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rb, (FA_LDS void*)(sBias + buf * BTILE + (wave * IPB + u) * 64 * 8), 16, boff[u],
              0, 0, kLoadNonTemporal);
      } else {
#pragma unroll
        for (int u = 0; u < IPB; ++u)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rb, (FA_LDS void*)(sBias + buf * BTILE + (wave * IPB + u) * 64 * 8), 16, boff[u],
              0, 0, 0);
      }
    }
#endif
  };

  // K block (rows past Nk read as zeros) and the first query block.
  {
    using KB = BufTile<D, BC, kKvThreads>;
    const KB kb(wave, lane);
    kb.tile(K + kbase, k0, Nk, sK);
  }
  if (nloop > 0) load_block(qb_first, 0);
  // This wave's V rows in registers (B operand of dP = dO V^T).
  T8 vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    vf[kk] = (mykey < Nk) ? *(const T8*)(V + kbase + (size_t)mykey * D + kk * 16 + half * 8)
                          : zero8<T8>();
  f32x16 dkacc[NNT], dvacc[NNT];
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) {
    dkacc[nt] = (f32x16){};
    dvacc[nt] = (f32x16){};
  }
  vm_wait_all();
  __syncthreads();

  // Byte offsets, within a tile, of this lane's LDS operand reads (buffers
  // and row blocks are instruction offsets): Q/dO rows l32 and K rows
  // kw0 - k0 + l32, 16-byte chunk 2*kk + half; transpose reads of dO^T / Q^T.
  unsigned qa[NKK], ka[NKK], ta[2 * NNT];
  {
    const SwzRow<D> qrow_sw(l32, half);
    const SwzRow<D> krow_sw(SwzRow<D>(l32, half).x + (unsigned)(wave * 64 * D));
    const int tr_row = (g >> 1) * 4 + (s16 >> 2);
    const int tr_col = (g & 1) * 16 + (s16 & 3) * 4;
    const SwzTr<D> tr_sw(tr_row, tr_col);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qa[kk] = qrow_sw.off(0, kk * 2);
      ka[kk] = krow_sw.off(0, kk * 2);
    }
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt) ta[hi * NNT + nt] = tr_sw.off(0, hi, nt * 32);
  }

  // One query block (P = buffer parity it & 1, a constant at both inlined
  // call sites).
  auto block_step = [&](const int P, int it) __attribute__((always_inline)) {
    const int qi0 = (qb_first + it) * BR;
    if (it + 1 < nloop) load_block(qb_first + it + 1, 1 - P);

    // Causal: a wave whose keys all lie after every row of the block has no
    // work.  (DS: it runs the block all the same, masked to zeros, so that
    // every wave stores two chunks per block, which the wait below counts.)
    const bool wave_idle = CAUSAL && !DS && (kw0 > qi0 + BR - 1 + off);
    if (!wave_idle) {
      const T* const tQ = sQ0 + P * QTILE;
      const T* const tdO = sdO0 + P * QTILE;
      const float* tLD = sLD[P];
      // S = Q K^T and dP = dO V^T: 32 rows x this wave's 32 keys.  Step kk
      // needs the Q, K and dO fragments of head-dim chunk kk; those of step
      // kk + 1 are read before step kk's MFMAs are issued.
      // dP starts from -D of its row (element i: row (i/4)*8 + half*4 + i%4),
      // so that dS = P (dP - D) needs no subtraction; with dropout, whose dP
      // is masked and scaled first, from zero.
      f32x16 sacc = (f32x16){}, dpacc;
      if constexpr (DROP) {
        dpacc = (f32x16){};
      } else {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x4 nd = *(const f32x4*)(tLD + kLdRows + gq * 8 + half * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) dpacc[gq * 4 + e] = nd[e];
        }
      }
      // Bias of rows qi0 + 8g + half*4 + 0..3, key mykey, from the staged
      // tile (rows past Nq read zeros, keys past Nk are masked below), read
      // before the MFMAs.
      typename Vec<T>::x4 bq[BIAS ? 4 : 1];
      if constexpr (BIAS) {
        const T* tb = sBias + P * BTILE;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          bq[gq] = lds_read_tr<T>(to_lds(at_byte<T>(tb, bread + gq * 8 * BC * 2)));
      }
      {
        auto ldstep = [&](int kk, T8* f) {
          f[0] = *at_byte<T8>(tQ, qa[kk]);
          f[1] = *at_byte<T8>(sK, ka[kk]);
          f[2] = *at_byte<T8>(tdO, qa[kk]);
        };
        T8 fa[3], fb[3];
        ldstep(0, fa);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          T8* cur = (kk & 1) ? fb : fa;
          T8* nxt = (kk & 1) ? fa : fb;
          if (kk + 1 < NKK) ldstep(kk + 1, nxt);
          sacc = mfma32(cur[0], cur[1], sacc);
          dpacc = mfma32(cur[2], vf[kk], dpacc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (BIAS) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sacc[i] = fmaf((float)bq[i >> 2][i & 3], bias.inv_scale, sacc[i]);
      }
      // Lane holds key mykey and rows (i/4)*8 + half*4 + i%4 of the block.
      // Rows past the end and, causal, rows before the key's diagonal get
      // score -inf, hence P = 0 and dS = 0 (only blocks that cross the
      // diagonal or an end need it).
      if ((qi0 + BR > Nq) || (kw0 + 32 > Nk) || (CAUSAL && (kw0 + 31 > qi0 + off))) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = qi0 + (i >> 2) * 8 + half * 4 + (i & 3);
          const bool vis = (q < Nq) && (mykey < Nk) && (!CAUSAL || mykey <= q + off);
          if (!vis) sacc[i] = -INFINITY;
        }
      }
      // P = exp2(S*c - L2) and dS = P * (dP - D) for the pair of rows of
      // elements i, i+1 (i even) of chunk kc = i / 8, in two halves: the
      // probabilities, then dS and both conversions to T.
      T8 pf[2], dsf[2];
      float pp[2];
      // Dropout (DROP): byte r of rbk[g] is the random byte of row
      // qi0 + 8g + half*4 + r and key mykey.  P times the mask goes into dV
      // (1 / keep-probability applied at the end); dP is masked and scaled
      // before dS = P (dP - D).
      unsigned rbk[4];
      if constexpr (DROP) drop_bytes_keys(rbk, drop, bh, mykey, qi0 + half * 4, lane);
      // (with dropout pds_p returns -D of the two rows, read with their L2)
      auto pds_p = [&](int i) {
        const int ql = (i >> 2) * 8 + half * 4 + (i & 3);  // rows ql, ql + 1 (ql even)
        float2 l2, nd = make_float2(0.f, 0.f);
        if constexpr (DROP) {
          const f32x4 v = *(const f32x4*)(tLD + 2 * ql);  // (L2, -D) of both rows
          l2 = make_float2(v[0], v[2]);
          nd = make_float2(v[1], v[3]);
        } else {
          l2 = *(const float2*)(tLD + ql);
        }
        pp[0] = fast_exp2(fmaf(sacc[i], c, -l2.x));
        pp[1] = fast_exp2(fmaf(sacc[i + 1], c, -l2.y));
        return nd;
      };
      auto pds_ds = [&](int i, float2 dd) {
        const int kc = i >> 3, e = i & 7;
        if constexpr (DROP) {
          const bool k0 = drop_keep(rbk[i >> 2], i & 3, drop.thresh);
          const bool k1 = drop_keep(rbk[i >> 2], (i + 1) & 3, drop.thresh);
          pf[kc][e] = (T)(k0 ? pp[0] : 0.f);
          pf[kc][e + 1] = (T)(k1 ? pp[1] : 0.f);
          dsf[kc][e] = (T)(pp[0] * ((k0 ? dpacc[i] * drop.inv_keep : 0.f) + dd.x));
          dsf[kc][e + 1] = (T)(pp[1] * ((k1 ? dpacc[i + 1] * drop.inv_keep : 0.f) + dd.y));
        } else {
          pf[kc][e] = (T)pp[0];
          pf[kc][e + 1] = (T)pp[1];
          dsf[kc][e] = (T)(pp[0] * dpacc[i]);  // dpacc = dP - D
          dsf[kc][e + 1] = (T)(pp[1] * dpacc[i + 1]);
        }
      };
      // dV^T += dO^T P and dK^T += Q^T dS over the 16 rows of chunk kc
      // (2 * NNT MFMAs, A operands by transpose reads); with `overlap`, the
      // probabilities of chunk kc + 1 are computed between them.
      auto dvdk = [&](int kc, bool overlap) {
        auto afrag = [&](int st) {  // st: (head-dim tile st/2, dO^T if even else Q^T)
          const T* base = (st & 1) ? tQ : tdO;
          const unsigned rb = kc * 16 * 2 * D;
          return concat(lds_read_tr<T>(to_lds(at_byte<T>(base, ta[st >> 1] + rb))),
                        lds_read_tr<T>(to_lds(at_byte<T>(base, ta[NNT + (st >> 1)] + rb))));
        };
        constexpr int NS = 2 * NNT, RING = 2;
        static_assert(NS == 4 || NS == 8, "two or four probability pairs per chunk step pair");
        T8 ring[RING];
        float2 dd;
#pragma unroll
        for (int st = 0; st < RING; ++st) ring[st] = afrag(st);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const T8 a = ring[st % RING];
          if (st + RING < NS) ring[st % RING] = afrag(st + RING);
          if (st & 1) dkacc[st >> 1] = mfma32(a, dsf[kc], dkacc[st >> 1]);
          else dvacc[st >> 1] = mfma32(a, pf[kc], dvacc[st >> 1]);
          if (overlap) {
            // NS steps carry the 4 pairs of chunk kc + 1: D = 128 takes a
            // pair per two steps (probabilities, then dS), D = 64 a pair per
            // step.
            if constexpr (NS == 8) {
              const int i = (kc + 1) * 8 + (st >> 1) * 2;
              if ((st & 1) == 0) {
                dd = pds_p(i);
                pin(pp[0]);
                pin(pp[1]);
              } else {
                pds_ds(i, dd);
                pin(pf[kc + 1]);
                pin(dsf[kc + 1]);
              }
            } else {
              const int i = (kc + 1) * 8 + st * 2;
              pds_ds(i, pds_p(i));
              pin(pf[kc + 1]);
              pin(dsf[kc + 1]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
#pragma unroll
      for (int i = 0; i < 8; i += 2) pds_ds(i, pds_p(i));
      T* const ds_blk = DS ? ds_wave + (size_t)(qi0 / BR) * ds_row : nullptr;
      if constexpr (DS) __builtin_nontemporal_store(dsf[0], (T8*)(ds_blk + ds_lane[0]));
      // The dV/dK MFMAs run at a raised issue priority, so that the two waves
      // of a SIMD (from the two workgroups of a CU) tend to alternate between
      // this phase and the other's S / dP loads and MFMAs (about 2% faster
      // than equal priorities on the long-sequence backward).
      __builtin_amdgcn_s_setprio(1);
      dvdk(0, true);   // probabilities of rows 16..31 overlap the MFMAs of rows 0..15
      if constexpr (DS) __builtin_nontemporal_store(dsf[1], (T8*)(ds_blk + ds_lane[1]));
      dvdk(1, false);
      __builtin_amdgcn_s_setprio(0);
    }
    // this wave's part of the next query block has landed (DS: the two dS
    // stores, issued after those loads, may still be in flight)
    if constexpr (DS) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else vm_wait_all();
    __syncthreads();
  };
  for (int it = 0; it < nloop; it += 2) {
    block_step(0, it);
    if (it + 1 < nloop) block_step(1, it + 1);
  }

  // Epilogue: dK = scale * dK_acc, dV = dV_acc (times 1 / keep-probability
  // with dropout); lane holds key mykey.
  const float vscale = DROP ? drop.inv_keep : 1.f;
  if (mykey < Nk) {
    T* dkrow = dK + kbase + (size_t)mykey * D;
    T* dvrow = dV + kbase + (size_t)mykey * D;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        T4 vk, vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vk[e] = (T)(dkacc[nt][gg * 4 + e] * scale);
          vv[e] = (T)(dvacc[nt][gg * 4 + e] * vscale);
        }
        *(T4*)(dkrow + nt * 32 + gg * 8 + half * 4) = vk;
        *(T4*)(dvrow + nt * 32 + gg * 8 + half * 4) = vv;
      }
  }
}

template <typename T, int D, bool CAUSAL, bool BIAS, bool DROP, bool DS>
__global__ __launch_bounds__(KvShape<BIAS>::kThreads, KvShape<BIAS>::kPerCU)
__attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                     const T* __restrict__ dO, const float* __restrict__ LD, T* __restrict__ dK,
                     T* __restrict__ dV, int Nq, int Nk, int nkt, int BH, int hpx, float c,
                     float scale, int off, BiasDev bias, DropDev drop, T* __restrict__ dSg) {
  __shared__ DkdvLds<T, D, BIAS> lds;
  dkdv_body<T, D, CAUSAL, BIAS, DROP, DS>(Q, K, V, dO, LD, dK, dV, Nq, Nk, nkt, BH, hpx, c,
                                          scale, off, bias, drop, lds, blockIdx.x, dSg);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (query tile of 128, batch*head), key tiles streamed.
constexpr int kDqBR = 128;  // query rows per workgroup
constexpr int kDqBC = 64;   // keys per K/V tile
constexpr int kDqThreads = 256;

// LDS of a dQ workgroup: K tiles (buffers 0/1), V tiles (buffers 2/3), then
// the bias staging (BIAS).
template <typename T, int D, bool BIAS>
struct DqLds {
  __attribute__((aligned(1024))) T smem[4 * kDqBC * D + (BIAS ? (kDqThreads / 64) * 32 * kDqBC : 0)];
};

// Block `bid` of a grid of `nblk` query-tile workgroups.
template <typename T, int D, bool CAUSAL, bool BIAS, bool DROP>
__device__ __forceinline__ void dq_body(const T* __restrict__ Q, const T* __restrict__ K,
                                        const T* __restrict__ V, const T* __restrict__ dO,
                                        const float* __restrict__ LD, T* __restrict__ dQ, int Nq,
                                        int Nk, int nqt, float c, float scale, int off,
                                        BiasDev bias, DropDev drop, DqLds<T, D, BIAS>& lds,
                                        int bid, int nblk) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  constexpr int BR = kDqBR, BC = kDqBC;
  constexpr int NKK = D / 16;
  constexpr int NNT = D / 32;
  constexpr int TILE = BC * D;

  // K tiles (buffers 0/1) and V tiles (buffers 2/3), swizzled (see swz) and
  // double-buffered: tile j+1 loads while tile j (buffers j & 1) is read.
  // The key loop is unrolled by two so that buffer offsets are constants.
  // Bias staging (BIAS), after the tiles: 32 rows x BC keys per wave, rows
  // of 8 chunks of 16 bytes, chunk c of row r at c ^ ((r / 2) % 8) (reads of
  // one chunk per row take the minimum two LDS passes).
  constexpr int BSTAGE = BIAS ? (kDqThreads / 64) * 32 * BC : 0;
  static_assert(sizeof(lds.smem) == (4 * TILE + BSTAGE) * sizeof(T), "LDS layout");
  T* const smem = lds.smem;
  T* const sK0 = smem;
  T* const sV0 = smem + 2 * TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T* const sBw = smem + 4 * TILE + wave * 32 * BC;  // this wave's bias region (BIAS)
  const int half = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, s16 = lane & 15;

  // Causal: one workgroup per pair of query tiles (t, nqt-1-t), taken in
  // turn, so that every workgroup carries the same number of key tiles.
  const int nwg = CAUSAL ? (nqt + 1) / 2 : nqt;  // workgroups per head
  const int logical = xcd_remap(bid, nblk);
  const int bh = logical / nwg;
  const int t = logical - bh * nwg;
  const size_t qbase = (size_t)bh * Nq * D;
  const T* Kh = K + (size_t)bh * Nk * D;
  const T* Vh = V + (size_t)bh * Nk * D;

  // Additive bias (BIAS) of this head: lane row qrow, keys along elements.
  const T* bias_h = nullptr;
  long long bias_n = 0;
  if constexpr (BIAS) {
    const int b = bh / bias.H, h = bh - b * bias.H;
    bias_h = (const T*)bias.ptr + b * bias.sb + h * bias.sh;
    bias_n = (long long)(Nq - 1) * bias.sq + Nk;
  }
  // the head's bias as buffer descriptor words, range rounded up to 16 bytes
  // as in BiasReader
  const i32x4 brw = rsrc_words(
      bias_h, (unsigned)min(((unsigned long long)bias_n * 2 + 15) & ~15ull, 0xfffffff0ull));
  typedef typename Vec<T>::x4 BT4;

  using KV = BufTile<D, BC, kDqThreads>;
  const KV kv(wave, lane);
  static_assert(2 * KV::PER <= 2 * NKK, "tile loads fit the first score half");

  // Byte offsets, within a tile, of this lane's LDS operand reads (row
  // blocks and buffers are instruction offsets).  S^T and dP^T: the A
  // fragment of step st is row mt*32 + l32 of K (even st) or V (odd st),
  // 16-byte chunk 2*(st>>1) + half.  dQ^T += K^T dS^T: step st reads K^T for
  // the 16 keys of chunk st / NNT of half mt and head-dim tile st % NNT.
  unsigned ra[NKK], ta[2 * NNT];
  {
    const SwzRow<D> rowsw(l32, half);
    const int tr_row = (g >> 1) * 4 + (s16 >> 2);
    const int tr_col = (g & 1) * 16 + (s16 & 3) * 4;
    const SwzTr<D> trsw(tr_row, tr_col);
#pragma unroll
    for (int i = 0; i < NKK; ++i) ra[i] = rowsw.off(0, 2 * i);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt) ta[hi * NNT + nt] = trsw.off(0, hi, nt * 32);
  }
  auto sfrag = [&](int buf, int mt, int st) {
    const T* base = ((st & 1) ? sV0 : sK0) + buf * TILE;
    return *at_byte<T8>(base, ra[st >> 1] + mt * 32 * 2 * D);
  };
  auto kt_frag = [&](int buf, int mt, int st) {
    const unsigned rb = (mt * 32 + (st / NNT) * 16) * 2 * D;
    const T* base = sK0 + buf * TILE;
    return concat(lds_read_tr<T>(to_lds(at_byte<T>(base, ta[st % NNT] + rb))),
                  lds_read_tr<T>(to_lds(at_byte<T>(base, ta[NNT + st % NNT] + rb))));
  };
  constexpr int SRING = 4, TRING = 3;

  for (int pass = 0; pass < (CAUSAL ? 2 : 1); ++pass) {
    const int qt = !CAUSAL ? t : (pass == 0 ? nqt - 1 - t : t);
    if (CAUSAL && pass == 1 && t == nqt - 1 - t) break;  // odd count: the middle tile once
    if (pass == 1) __syncthreads();  // the first tile's last LDS reads precede the new loads
    const int q0 = qt * BR;

    // This lane's query row: Q^T and dO^T fragments (B operands), L and D.
    const int qrow = q0 + wave * 32 + l32;
    T8 qf[NKK], dof[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const size_t o = qbase + (size_t)qrow * D + kk * 16 + half * 8;
      qf[kk] = (qrow < Nq) ? *(const T8*)(Q + o) : zero8<T8>();
      dof[kk] = (qrow < Nq) ? *(const T8*)(dO + o) : zero8<T8>();
    }
    const int nqb_ld = (Nq + kLdRows - 1) / kLdRows;
    const size_t li = ld_index<DROP>(bh, qrow, nqb_ld);
    const float l2 = (qrow < Nq) ? LD[li] : INFINITY;
    const float ndrow = (qrow < Nq) ? LD[li + ld_nd_off<DROP>()] : 0.f;  // -D

    const int kend = CAUSAL ? min(Nk, q0 + BR + off) : Nk;
    int ntiles = (kend + BC - 1) / BC;
    int jbeg = 0;
    // Bias tile map (BIAS): only the key tiles from the first to the last that
    // hold an entry above -inf for this query tile (jbeg stays even, so tile
    // j keeps buffers j & 1).
    if constexpr (BIAS) {
      static_assert(BR == kMapRows && BC == kMapKeys, "tile map granularity");
      if (bias.tmap) {
        const int b = bh / bias.H, h = bh - b * bias.H;
        int lo, hi;
        map_range(bias.tmap + b * bias.tm_sb + h * bias.tm_sh + (size_t)qt * bias.nkt4,
                  (Nk + BC - 1) / BC, lane, lo, hi);
        if (lo > hi) {
          ntiles = 0;
        } else {
          jbeg = lo & ~1;
          ntiles = min(ntiles, hi + 1);
        }
      }
    }
    const int wrow_lo = q0 + wave * 32;

    f32x16 dqacc[NNT];
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) dqacc[nt] = (f32x16){};

    kv.tile(Kh, jbeg * BC, Nk, sK0);
    kv.tile(Vh, jbeg * BC, Nk, sV0);
    vm_wait_all();
    __syncthreads();

    // Bias (BIAS): each wave stages its 32 rows x BC keys of a tile in its own
    // region with four direct-to-LDS loads of whole 128-byte rows, issued one
    // tile ahead (after the current tile's bias was read), and reads its
    // lanes' pieces back; rows past Nq read zeros, keys past Nk are masked.
    // Load u, lane l: row 8u + l/8 of the wave's 32, stored chunk l%8, which
    // holds chunk (l%8) ^ ((row / 2) % 8) of the row, i.e. c0 for even u and
    // c0 ^ 4 for odd u.  One per-lane base (wraps only for rows past Nq, whose
    // loads fall outside the descriptor); the row step is scalar.
    const unsigned bbase =
        BIAS ? (unsigned)((long long)(q0 + wave * 32 + (lane >> 3)) * bias.sq * 2) : 0u;
    const unsigned bstep = BIAS ? (unsigned)(bias.sq * 16) : 0u;  // 8 rows, in bytes
    const unsigned bc0 = (unsigned)(((lane & 7) ^ (lane >> 4)) << 4);
    auto bias_issue = [&](int k0b) {
      lds_reads_done();  // the region's previous contents have been read
      if (bias.stream) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          lds_dma16_asm<true>(brw, bbase + u * bstep + ((u & 1) ? (bc0 ^ 64u) : bc0) + (unsigned)k0b * 2,
                              (const FA_LDS void*)(sBw + u * 64 * 8));
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          lds_dma16_asm<false>(brw, bbase + u * bstep + ((u & 1) ? (bc0 ^ 64u) : bc0) + (unsigned)k0b * 2,
                               (const FA_LDS void*)(sBw + u * 64 * 8));
      }
    };
    // Chunks q0b .. q0b+3 (keys q*8 + half*4 .. +3 of this lane's row).
    auto bias_fetch = [&](BT4 (&bb)[8], int q0b) {
      const unsigned rowb = (unsigned)l32 * (BC * 2) + (unsigned)half * 8;
      const unsigned x = (unsigned)(l32 >> 1) & 7u;
#pragma unroll
      for (int q = q0b; q < q0b + 4; ++q)
        bb[q] = *at_byte<BT4>(sBw, rowb + (((unsigned)q ^ x) << 4));
    };
    if constexpr (BIAS) bias_issue(jbeg * BC);

    // One key tile j (P = buffer parity j & 1, a constant at both inlined
    // call sites).
    auto tile_step = [&](const int P, int j) __attribute__((always_inline)) {
      const int k0 = j * BC;
      // dS^T for the 16 keys of element e of half mt: lane holds row qrow and
      // keys k0 + mt*32 + (i/4)*8 + half*4 + i%4.
      f32x16 sacc[2], dpacc[2];
      T8 dsf[4];
      // Bias of this tile (BIAS): half mt, elements g*4 .. g*4+3 are keys
      // k0 + mt*32 + g*8 + half*4 + 0..3, read from the staged region before
      // half 0's scores are complete and added after each half's scores.
      BT4 bb[BIAS ? 8 : 1];
      auto bias_half = [&](int mt) {
        if constexpr (BIAS) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sacc[mt][g * 4 + e] = fmaf((float)bb[mt * 4 + g][e], bias.inv_scale, sacc[mt][g * 4 + e]);
        }
      };
      // Dropout (DROP): byte e of rb[mt][c] is the random byte of row qrow
      // and key k0 + mt*32 + c*8 + half*4 + e; dP is masked and scaled before
      // dS = P (dP - D).
      // Each half's bytes are made just before its dS elements.
      unsigned rb[2][4];
      auto ds_elem = [&](int mt, int i) {
        const float p = fast_exp2(fmaf(sacc[mt][i], c, -l2));
        float dp = dpacc[mt][i];
        if constexpr (DROP)
          dp = drop_keep(rb[mt][i >> 2], i & 3, drop.thresh) ? dp * drop.inv_keep : 0.f;
        dsf[mt * 2 + (i >> 3)][i & 7] = (T)(p * (dp + ndrow));
      };
      // Keys past the end and, causal, keys after the row's diagonal get
      // score -inf, hence P = 0 and dS = 0; only tiles that cross the
      // diagonal or the end need it.
      auto mask_half = [&](int mt) {
        if ((k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > wrow_lo + off))) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + mt * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            const bool vis = (key < Nk) && (!CAUSAL || key <= qrow + off);
            if (!vis) sacc[mt][i] = -INFINITY;
          }
        }
      };
      // S^T, dP^T of half mt (16 MFMAs); with `overlap`, the dS elements of
      // half mt - 1 are computed between them; half 0 also issues the
      // direct-to-LDS loads of K and V tile j+1 (rows past the end read as
      // zeros; the last tile loads nothing anybody reads).
      auto sdp_half = [&](int mt, bool overlap) {
        sacc[mt] = (f32x16){};
        dpacc[mt] = (f32x16){};
        T8 ring[SRING];
#pragma unroll
        for (int st = 0; st < SRING; ++st) ring[st] = sfrag(P, mt, st);
#pragma unroll
        for (int st = 0; st < 2 * NKK; ++st) {
          const T8 a = ring[st % SRING];
          if (st + SRING < 2 * NKK) ring[st % SRING] = sfrag(P, mt, st + SRING);
          if (st & 1) dpacc[mt] = mfma32(a, dof[st >> 1], dpacc[mt]);
          else sacc[mt] = mfma32(a, qf[st >> 1], sacc[mt]);
          if (mt == 0 && (st & 1) == 0 && (st >> 1) < 2 * KV::PER) {
            const int di = st >> 1;
            if (di < KV::PER)
              kv.part(Kh, k0 + BC, Nk, sK0 + (1 - P) * TILE, di);
            else
              kv.part(Vh, k0 + BC, Nk, sV0 + (1 - P) * TILE, di - KV::PER);
          }
          if (overlap) {
            // the 16 dS elements of half mt - 1 in pairs, so that each pair
            // takes one packed conversion: a pair per step (D = 64) or per
            // two steps (D = 128)
            constexpr int SPP = (2 * NKK) / 8;
            if ((st + 1) % SPP == 0) {
              const int i = (st / SPP) * 2;
              ds_elem(mt - 1, i);
              ds_elem(mt - 1, i + 1);
              pin(dsf[(mt - 1) * 2 + i / 8]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // dQ^T += K^T dS^T over half mt (2*NNT MFMAs), with the ne dS elements
      // e0 .. e0+ne-1 of half 1 computed between them, a pair at a time,
      // spread over the first `window` steps.
      auto dq_half = [&](int mt, int e0, int ne, int window) {
        T8 ring[TRING];
#pragma unroll
        for (int st = 0; st < TRING; ++st) ring[st] = kt_frag(P, mt, st);
#pragma unroll
        for (int st = 0; st < 2 * NNT; ++st) {
          const T8 a = ring[st % TRING];
          if (st + TRING < 2 * NNT) ring[st % TRING] = kt_frag(P, mt, st + TRING);
          dqacc[st % NNT] = mfma32(a, dsf[mt * 2 + st / NNT], dqacc[st % NNT]);
#pragma unroll
          for (int q = 0; q < ne / 2; ++q)
            if (q * window / (ne / 2) == st) {
              ds_elem(1, e0 + 2 * q);
              ds_elem(1, e0 + 2 * q + 1);
              pin(dsf[2 + (e0 + 2 * q) / 8]);
            }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      sdp_half(0, false);
      if constexpr (BIAS) {
        // the 2 * KV::PER tile loads of half 0 were issued after this tile's
        // bias loads and complete in order
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * KV::PER) : "memory");
        bias_fetch(bb, 0);
      }
      bias_half(0);
      mask_half(0);
      if constexpr (DROP) drop_bytes_rows(rb[0], drop, bh, qrow, k0 + half * 4, lane);
      sdp_half(1, true);   // dS of half 0 overlaps the MFMAs of half 1
      if constexpr (BIAS) bias_fetch(bb, 4);
      bias_half(1);
      if constexpr (BIAS) bias_issue(k0 + BC);  // the region is free: stage tile j+1
      mask_half(1);
      if constexpr (DROP) drop_bytes_rows(rb[1], drop, bh, qrow, k0 + 32 + half * 4, lane);
      if constexpr (D == 128) {
        dq_half(0, 0, 8, 2 * NNT);  // half 1's first chunk of dS overlaps dQ of half 0
        dq_half(1, 8, 8, NNT);      // its second chunk the steps that read the first
      } else {
        dq_half(0, 0, 16, 2 * NNT);
        dq_half(1, 0, 0, 1);
      }

      // this wave's part of tile j+1 has landed (with a bias, the 4 bias
      // loads of tile j+1, issued last, may still be in flight)
      if constexpr (BIAS) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else vm_wait_all();
      __syncthreads();
    };
    // Causal: tiles whose first key lies past the diagonal of this wave's
    // last row contribute nothing to its rows; after its last useful tile the
    // wave only takes its part in the loads and barriers of the rest.
    const int jact = (CAUSAL && !BIAS) ? min(ntiles, (wrow_lo + 31 + off) / BC + 1) : ntiles;
    for (int j = jbeg; j < jact; j += 2) {
      tile_step(0, j);
      if (j + 1 < jact) tile_step(1, j + 1);
    }
    for (int j = max(jact, jbeg); j < ntiles; ++j) {
      const int P = (j - jbeg) & 1;
#pragma unroll
      for (int di = 0; di < KV::PER; ++di) {
        kv.part(Kh, (j + 1) * BC, Nk, sK0 + (1 - P) * TILE, di);
        kv.part(Vh, (j + 1) * BC, Nk, sV0 + (1 - P) * TILE, di);
      }
      vm_wait_all();
      __syncthreads();
    }
    if constexpr (BIAS) vm_wait_all();  // the last, unused bias loads

    // Epilogue: dQ = scale * dQ_acc; lane holds row qrow.
    if (qrow < Nq) {
      T* out = dQ + qbase + (size_t)qrow * D;
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          T4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (T)(dqacc[nt][gg * 4 + e] * scale);
          *(T4*)(out + nt * 32 + gg * 8 + half * 4) = v;
        }
    }
  }
}

template <typename T, int D, bool CAUSAL, bool BIAS, bool DROP>
__global__ __launch_bounds__(kDqThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                   const T* __restrict__ dO, const float* __restrict__ LD, T* __restrict__ dQ,
                   int Nq, int Nk, int nqt, float c, float scale, int off, BiasDev bias,
                   DropDev drop) {
  __shared__ DqLds<T, D, BIAS> lds;
  dq_body<T, D, CAUSAL, BIAS, DROP>(Q, K, V, dO, LD, dQ, Nq, Nk, nqt, c, scale, off, bias, drop,
                                    lds, blockIdx.x, gridDim.x);
}

// dQ from the stored dS: dQ = scale * dS K, one workgroup per (query tile of
// 128, batch*head) as in bwd_dq_kernel (causal tiles paired), K tiles and
// each wave's dS chunks streamed through LDS.  No softmax work remains: per
// 64-key tile a wave issues 16 (D = 128) or 8 MFMAs, reading K^T and dS^T
// fragments with transposed LDS reads.
template <typename T, int D>
struct DqDsLds {
  static constexpr int kWaveDs = 2 * kDsChunk;  // elements of a wave's dS per tile
  __attribute__((aligned(1024))) T smem[2 * kDqBC * D + 2 * (kDqThreads / 64) * kWaveDs];
};

template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void dq_ds_body(const T* __restrict__ K, const T* __restrict__ dSg,
                                           T* __restrict__ dQ, int Nq, int Nk, int nqt,
                                           float scale, int off, BiasDev bias,
                                           DqDsLds<T, D>& lds) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  constexpr int BR = kDqBR, BC = kDqBC;
  constexpr int NNT = D / 32;
  constexpr int TILE = BC * D;
  constexpr int NW = kDqThreads / 64;
  constexpr int WDS = DqDsLds<T, D>::kWaveDs;
  static_assert(BC == 64 && BR == NW * 32, "two dS chunks per wave and key tile");
  T* const sK0 = lds.smem;             // K tiles, buffers 0/1
  T* const sD0 = lds.smem + 2 * TILE;  // dS, [buffer][wave][chunk 0/1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, s16 = lane & 15;

  const int nwg = CAUSAL ? (nqt + 1) / 2 : nqt;  // workgroups per head
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nwg;
  const int t = logical - bh * nwg;
  const T* Kh = K + (size_t)bh * Nk * D;
  const int nqb = (Nq + 31) / 32;
  const int cpr = ds_chunks_per_row(Nk);

  using KV = BufTile<D, BC, kDqThreads>;
  const KV kv(wave, lane);

  // K^T fragments (A operand): step st of half mt reads the 16 keys of chunk
  // st / NNT of half mt, head-dim tile st % NNT (as in bwd_dq_kernel).
  unsigned ta[2 * NNT];
  {
    const int tr_row = (g >> 1) * 4 + (s16 >> 2);
    const int tr_col = (g & 1) * 16 + (s16 & 3) * 4;
    const SwzTr<D> trsw(tr_row, tr_col);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt) ta[hi * NNT + nt] = trsw.off(0, hi, nt * 32);
  }
  auto kt_frag = [&](int buf, int mt, int st) {
    const unsigned rb = (mt * 32 + (st / NNT) * 16) * 2 * D;
    const T* base = sK0 + buf * TILE;
    return concat(lds_read_tr<T>(to_lds(at_byte<T>(base, ta[st % NNT] + rb))),
                  lds_read_tr<T>(to_lds(at_byte<T>(base, ta[NNT + st % NNT] + rb))));
  };
  // dS^T fragments (B operand): lane l takes row l%32 of the wave's block and
  // the keys 16h + (e/4)*8 + (l/32)*4 + e%4 of chunk mt.  Each transposed read
  // has lane 4r + cc of a 16-lane group point at key 4*(g/2) + r (+8 for the
  // second read) and rows 16*(g%2) + 4cc .. +3 of the chunk, which the slot
  // layout puts at ds_chunk_off(g%2, cc%2, key) + (cc/2)*8; keys +8 and +16
  // flip slot bit 3 (byte 128) and add 256 bytes.
  const int r4 = s16 >> 2, cc = s16 & 3;
  const unsigned dsa = ds_chunk_off(g & 1, cc & 1, (g >> 1) * 4 + r4) + (unsigned)(cc >> 1) * 8;
  const unsigned dsb = dsa ^ 128u;
  auto ds_frag = [&](int buf, int mt, int h) {
    const T* base = sD0 + (buf * NW + wave) * WDS;
    const unsigned o = (unsigned)(mt * 2048 + h * 256);
    return concat(lds_read_tr<T>(to_lds(at_byte<T>(base, dsa + o))),
                  lds_read_tr<T>(to_lds(at_byte<T>(base, dsb + o))));
  };
  constexpr int TRING = 3;

  for (int pass = 0; pass < (CAUSAL ? 2 : 1); ++pass) {
    const int qt = !CAUSAL ? t : (pass == 0 ? nqt - 1 - t : t);
    if (CAUSAL && pass == 1 && t == nqt - 1 - t) break;  // odd count: the middle tile once
    if (pass == 1) __syncthreads();  // the first tile's last LDS reads precede the new loads
    const int q0 = qt * BR;
    const int qb = qt * NW + wave;  // this wave's 32-row query block
    const int wrow_lo = q0 + wave * 32;
    const int qrow = wrow_lo + l32;
    // chunks 2j, 2j+1 (4 KB) of the wave's row of dS chunks into buffer buf
    // (a row past Nq reads as zeros).  The loads are issued from inline
    // assembly, which the compiler's wait tracking does not see (its own
    // direct-to-LDS loads made it wait for them before this tile's reads);
    // the wait at the end of the tile covers them.
    const i32x4 rdw = rsrc_words(dSg + ((size_t)bh * nqb + min(qb, nqb - 1)) * cpr * kDsChunk,
                                 qb < nqb ? (unsigned)cpr * kDsChunk * 2 : 0u);
    auto ds_load = [&](int j, int buf) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        lds_dma16_asm<true>(rdw, (unsigned)(j * 4096 + u * 1024 + lane * 16),
                             (const FA_LDS void*)(sD0 + (buf * NW + wave) * WDS + u * 512));
    };

    const int kend = CAUSAL ? min(Nk, q0 + BR + off) : Nk;
    int ntiles = kend > 0 ? (kend + BC - 1) / BC : 0;
    // Bias tile map: only the key tiles from the first to the last active one
    // of this query tile (jbeg even, so tile j keeps K buffer j & 1); an
    // inactive tile inside holds no stored dS and contributes zeros.
    int jbeg = 0;
    const unsigned char* mrow = nullptr;
    if (bias.tmap) {
      const int b = bh / bias.H, h = bh - b * bias.H;
      mrow = bias.tmap + b * bias.tm_sb + h * bias.tm_sh + (size_t)qt * bias.nkt4;
      int lo, hi;
      map_range(mrow, (Nk + BC - 1) / BC, lane, lo, hi);
      if (lo > hi) {
        ntiles = 0;
      } else {
        jbeg = lo & ~1;
        ntiles = min(ntiles, hi + 1);
      }
    }
    // Causal: key tiles past the diagonal of this wave's last row hold no
    // dS for it; after its last useful tile (and at once, for a wave whose
    // rows all lie past Nq) the wave only takes its part in the K loads and
    // barriers of the rest.  The dK/dV kernel stores every chunk with a key
    // visible to a row of its block; of this wave's tiles before jact only
    // the second chunk of the last may have none (and is then never read).
    const int jact = qb >= nqb ? 0
                     : CAUSAL ? min(ntiles, max(wrow_lo + 31 + off, -1) / BC + 1) : ntiles;
    const bool last_half_live = !CAUSAL || (2 * jact - 1) * 32 <= wrow_lo + 31 + off;

    f32x16 dqacc[NNT];
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) dqacc[nt] = (f32x16){};

    if (ntiles > jbeg) kv.tile(Kh, jbeg * BC, Nk, sK0);
    if (jact > jbeg) ds_load(jbeg, 0);
    vm_wait_all();
    __syncthreads();

    auto tile_step = [&](const int P, int j) __attribute__((always_inline)) {
      // K tile j+1 and this wave's dS chunks of tile j+1 (past the last
      // tile: data nobody reads)
#pragma unroll
      for (int u = 0; u < KV::PER; ++u) kv.part(Kh, (j + 1) * BC, Nk, sK0 + (1 - P) * TILE, u);
      ds_load(j + 1, 1 - P);
      const bool tile_on = !mrow || mrow[j] != 0;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        T8 d0 = ds_frag(P, mt, 0), d1 = ds_frag(P, mt, 1);
        if (!tile_on || (mt == 1 && j == jact - 1 && !last_half_live)) {
          d0 = zero8<T8>();
          d1 = zero8<T8>();
        }
        T8 ring[TRING];
#pragma unroll
        for (int st = 0; st < TRING; ++st) ring[st] = kt_frag(P, mt, st);
#pragma unroll
        for (int st = 0; st < 2 * NNT; ++st) {
          const T8 a = ring[st % TRING];
          if (st + TRING < 2 * NNT) ring[st % TRING] = kt_frag(P, mt, st + TRING);
          dqacc[st % NNT] = mfma32(a, st < NNT ? d0 : d1, dqacc[st % NNT]);
        }
      }
      vm_wait_all();  // this wave's part of tile j+1 has landed
      __syncthreads();
    };
    for (int j = jbeg; j < jact; j += 2) {
      tile_step(0, j);
      if (j + 1 < jact) tile_step(1, j + 1);
    }
    for (int j = max(jact, jbeg); j < ntiles; ++j) {
      const int P = j & 1;
#pragma unroll
      for (int u = 0; u < KV::PER; ++u) kv.part(Kh, (j + 1) * BC, Nk, sK0 + (1 - P) * TILE, u);
      vm_wait_all();
      __syncthreads();
    }

    // Epilogue: dQ = scale * dQ_acc; lane holds row qrow.
    if (qrow < Nq) {
      T* out = dQ + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          T4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (T)(dqacc[nt][gg * 4 + e] * scale);
          *(T4*)(out + nt * 32 + gg * 8 + half * 4) = v;
        }
    }
  }
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kDqThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_ds_kernel(const T* __restrict__ K, const T* __restrict__ dSg, T* __restrict__ dQ,
                      int Nq, int Nk, int nqt, float scale, int off, BiasDev bias) {
  __shared__ DqDsLds<T, D> lds;
  dq_ds_body<T, D, CAUSAL>(K, dSg, dQ, Nq, Nk, nqt, scale, off, bias, lds);
}

// dK/dV and dQ in one launch (no bias: both then run 256-thread workgroups,
// two per CU), sharing one LDS allocation.  Workgroups start in block order,
// and both grids already list their workgroups longest first, so the launch
// merges them by expected length: blocks 0 .. n1-1 are the first key blocks
// (those longer than a dQ workgroup), the next nqpad blocks the query-tile
// grid (nq workgroups; the few blocks past it return at once), the rest the
// remaining key blocks.  n1 and nqpad are multiples of 8, so that each grid's
// XCD mapping still sees block b on XCD b % 8.  The dQ workgroups thus fill
// CUs as the long key blocks finish and the short key blocks come last: on
// short sequences, where a few long chains set the time, the two grids run
// side by side, and two dependent launches become one.
template <typename T, int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kDqThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_fused_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                      const T* __restrict__ dO, const float* __restrict__ LD,
                      T* __restrict__ dQ, T* __restrict__ dK, T* __restrict__ dV, int Nq,
                      int Nk, int nkt, int BH, int hpx, int n1, int nqpad, int nq, int nqt,
                      float c, float scale,
                      int off, BiasDev bias, DropDev drop) {
  static_assert(KvShape<false>::kThreads == kDqThreads, "one workgroup size");
  __shared__ union {
    DkdvLds<T, D, false> kv;
    DqLds<T, D, false> q;
  } lds;
  const int b = blockIdx.x;
  if (b < n1 || b >= n1 + nqpad) {
    dkdv_body<T, D, CAUSAL, false, DROP>(Q, K, V, dO, LD, dK, dV, Nq, Nk, nkt, BH, hpx, c, scale,
                                         off, bias, drop, lds.kv, b < n1 ? b : b - nqpad);
  } else if (b - n1 < nq) {
    dq_body<T, D, CAUSAL, false, DROP>(Q, K, V, dO, LD, dQ, Nq, Nk, nqt, c, scale, off, bias,
                                       drop, lds.q, b - n1, nq);
  }
}

// ---------------------------------------------------------------------------
// fp32 backward (correctness path): one thread per key row for dK/dV, one
// thread per query row for dQ; plain fp32 FMAs and expf.
constexpr int kF32BT = 64;

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kF32BT) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ L, const float* __restrict__ dO, const float* __restrict__ LD,
    float* __restrict__ dK, float* __restrict__ dV, int Nq, int Nk, int nkt, float scale,
    int off, BiasDev bias, DropDev drop) {
  __shared__ float sq[D], sdo[D];
  const int bh = blockIdx.x / nkt;
  const int kt = blockIdx.x - bh * nkt;
  const int key = kt * kF32BT + threadIdx.x;
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
  const float* bias_h = nullptr;  // this head's additive bias, if any
  if (bias.ptr) {
    const int b = bh / bias.H, h = bh - b * bias.H;
    bias_h = (const float*)bias.ptr + b * bias.sb + h * bias.sh;
  }
  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    k[e] = (key < Nk) ? K[kbase + (size_t)key * D + e] : 0.f;
    v[e] = (key < Nk) ? V[kbase + (size_t)key * D + e] : 0.f;
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const int q_first = CAUSAL ? max(0, kt * kF32BT - off) : 0;
  for (int q = q_first; q < Nq; ++q) {
    __syncthreads();
    for (int e = threadIdx.x; e < D; e += kF32BT) {
      sq[e] = Q[qbase + (size_t)q * D + e];
      sdo[e] = dO[qbase + (size_t)q * D + e];
    }
    __syncthreads();
    const bool vis = key < Nk && (!CAUSAL || key <= q + off);
    if (!vis) continue;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      s = fmaf(sq[e], k[e], s);
      dp = fmaf(sdo[e], v[e], dp);
    }
    const float b = bias_h ? bias_h[(long long)q * bias.sq + key] : 0.f;
    const float p = expf(s * scale + b - L[(size_t)bh * Nq + q]);
    // Dropout (DROP): the kept probability times 1/keep feeds dV and the
    // masked, scaled dP feeds dS.
    const bool kept = !DROP || drop_byte(drop, bh, q, key) < drop.thresh;
    const float pd = kept ? (DROP ? p * drop.inv_keep : p) : 0.f;
    const float dpd = kept ? (DROP ? dp * drop.inv_keep : dp) : 0.f;
    const float ds =
        p * (dpd + LD[ld_index<DROP>(bh, q, (Nq + kLdRows - 1) / kLdRows) + ld_nd_off<DROP>()]);
#pragma unroll
    for (int e = 0; e < D; ++e) {
      dv[e] = fmaf(pd, sdo[e], dv[e]);
      dk[e] = fmaf(ds, sq[e], dk[e]);
    }
  }
  if (key < Nk) {
#pragma unroll
    for (int e = 0; e < D; ++e) {
      dK[kbase + (size_t)key * D + e] = dk[e] * scale;
      dV[kbase + (size_t)key * D + e] = dv[e];
    }
  }
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kF32BT) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ L, const float* __restrict__ dO, const float* __restrict__ LD,
    float* __restrict__ dQ, int Nq, int Nk, int nqt, float scale, int off, BiasDev bias,
    DropDev drop) {
  __shared__ float sk[D], sv[D];
  const int bh = blockIdx.x / nqt;
  const int qt = blockIdx.x - bh * nqt;
  const int q = qt * kF32BT + threadIdx.x;
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
  const float* brow = nullptr;  // this row's additive bias, if any
  if (bias.ptr && q < Nq) {
    const int b = bh / bias.H, h = bh - b * bias.H;
    brow = (const float*)bias.ptr + b * bias.sb + h * bias.sh + (long long)q * bias.sq;
  }
  float qv[D], dov[D], dq[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = (q < Nq) ? Q[qbase + (size_t)q * D + e] : 0.f;
    dov[e] = (q < Nq) ? dO[qbase + (size_t)q * D + e] : 0.f;
    dq[e] = 0.f;
  }
  const float lq = (q < Nq) ? L[(size_t)bh * Nq + q] : 0.f;
  const float ndq =  // -D
      (q < Nq) ? LD[ld_index<DROP>(bh, q, (Nq + kLdRows - 1) / kLdRows) + ld_nd_off<DROP>()] : 0.f;
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, qt * kF32BT + kF32BT + off);
  for (int key = 0; key < kend; ++key) {
    __syncthreads();
    for (int e = threadIdx.x; e < D; e += kF32BT) {
      sk[e] = K[kbase + (size_t)key * D + e];
      sv[e] = V[kbase + (size_t)key * D + e];
    }
    __syncthreads();
    const bool vis = q < Nq && (!CAUSAL || key <= q + off);
    if (!vis) continue;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      s = fmaf(qv[e], sk[e], s);
      dp = fmaf(dov[e], sv[e], dp);
    }
    const float p = expf(s * scale + (brow ? brow[key] : 0.f) - lq);
    const bool kept = !DROP || drop_byte(drop, bh, q, key) < drop.thresh;
    const float ds = p * ((kept ? (DROP ? dp * drop.inv_keep : dp) : 0.f) + ndq);
#pragma unroll
    for (int e = 0; e < D; ++e) dq[e] = fmaf(ds, sk[e], dq[e]);
  }
  if (q < Nq) {
#pragma unroll
    for (int e = 0; e < D; ++e) dQ[qbase + (size_t)q * D + e] = dq[e] * scale;
  }
}

template <int D, typename T>
hipError_t launch_pre(const BwdArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int nblk = (a.Nq + kLdRows - 1) / kLdRows;
  constexpr int RPB = 256 / (D / 8);
  const long nb = (long)BH * nblk * (kLdRows / RPB);  // workgroups (rows padded per head)
  if (nb == 0) return hipSuccess;
  // the layout of the (L2, -D) blocks follows the kernels that read them
  if (a.drop.on)
    hipLaunchKernelGGL((bwd_pre_kernel<D, T, true>), dim3((unsigned)nb), dim3(256), 0, s,
                       (const T*)a.O, (const T*)a.dO, a.L, a.LD, a.Nq, nblk);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<D, T, false>), dim3((unsigned)nb), dim3(256), 0, s,
                       (const T*)a.O, (const T*)a.dO, a.L, a.LD, a.Nq, nblk);
  return hipGetLastError();
}

}  // namespace

namespace {

DropDev drop_dev(const DropArgs& d) {
  return DropDev{d.seed_lo, d.seed_hi, d.offset, d.on ? d.thresh : 256u, d.on ? d.inv_keep : 1.f};
}

// Key blocks that go before the dQ workgroups in the fused launch: those whose
// chain of 32-row query blocks is longer than a dQ workgroup's key tiles, in
// units of a dK/dV query block.  A dK/dV wave spends 32 MFMAs (d = 128; 16 at
// d = 64) and 16 exponentials on a query block, a dQ wave 48 (24) and 32 on a
// 64-key tile: about 1.5x at d = 128, where the MFMAs dominate, and 1.07x at
// d = 64 (measured per step on one head).  Without a causal mask every key
// block is longer than every dQ workgroup.
int fused_split(const BwdArgs& a, int nkt, int nqt, int kv_bc) {
  if (!a.causal) return nkt;
  const int off = a.Nk - a.Nq;
  const double r = (a.d == 128) ? 1.5 : 1.07;
  auto tiles = [&](int t) {  // 64-key tiles of 128-row query tile t
    return (std::min(a.Nk, (t + 1) * kDqBR + off) + kDqBC - 1) / kDqBC;
  };
  const double dq_len = r * (tiles(0) + (nqt > 1 ? tiles(nqt - 1) : 0));
  const int nqb = (a.Nq + kKvBR - 1) / kKvBR;
  for (int kt = 0; kt < nkt; ++kt) {
    const int first = std::max(0, kt * kv_bc - off) / kKvBR;
    if (nqb - first < dq_len) return kt;
  }
  return nkt;
}

template <typename T, bool BIAS, bool DROP>
hipError_t launch_bwd_mfma(const BwdArgs& a, int stages, hipStream_t s) {
  const int BH = a.B * a.H;
  const float c = a.scale * kLog2e;
  const int off = a.Nk - a.Nq;
  const T* Q = (const T*)a.Q;
  const T* K = (const T*)a.K;
  const T* V = (const T*)a.V;
  const T* dO = (const T*)a.dO;
  const BiasDev bias = bias_dev(a.bias, a.B, a.H, a.scale);
  const DropDev drop = drop_dev(a.drop);
  if (stages & 1) {
    const hipError_t e = (a.d == 128) ? launch_pre<128, T>(a, s) : launch_pre<64, T>(a, s);
    if (e != hipSuccess) return e;
  }
  if (a.dS != nullptr) {
    // stored dS (set only with Nq, Nk > 0): dK/dV writes dS, dQ = scale *
    // dS K reads it (stage 4 needs stage 2 to have run on the same workspace)
    T* const dS = (T*)a.dS;
    if ((stages & 2) && a.Nk > 0 && a.Nq > 0) {
      constexpr int kKvBC = KvShape<BIAS>::kBC;
      const int nkt = (a.Nk + kKvBC - 1) / kKvBC;
      const int hpx = (BH % kNumXcd == 0) ? BH / kNumXcd : 0;
#define FA_DKDV_DS_LAUNCH(DD, CC)                                                              \
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, DD, CC, BIAS, DROP, true>), dim3(nkt * BH),           \
                     dim3(KvShape<BIAS>::kThreads), 0, s, Q, K, V, dO, a.LD, (T*)a.dK,        \
                     (T*)a.dV, a.Nq, a.Nk, nkt, BH, hpx, c, a.scale, off, bias, drop, dS)
      if (a.d == 128) {
        if (a.causal) FA_DKDV_DS_LAUNCH(128, true); else FA_DKDV_DS_LAUNCH(128, false);
      } else {
        if (a.causal) FA_DKDV_DS_LAUNCH(64, true); else FA_DKDV_DS_LAUNCH(64, false);
      }
#undef FA_DKDV_DS_LAUNCH
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if ((stages & 4) && a.Nq > 0) {
      const int nqt = (a.Nq + kDqBR - 1) / kDqBR;
      const int nblocks = (a.causal ? (nqt + 1) / 2 : nqt) * BH;
#define FA_DQ_DS_LAUNCH(DD, CC)                                                                \
  hipLaunchKernelGGL((bwd_dq_ds_kernel<T, DD, CC>), dim3(nblocks), dim3(kDqThreads), 0, s, K, \
                     (const T*)dS, (T*)a.dQ, a.Nq, a.Nk, nqt, a.scale, off, bias)
      if (a.d == 128) {
        if (a.causal) FA_DQ_DS_LAUNCH(128, true); else FA_DQ_DS_LAUNCH(128, false);
      } else {
        if (a.causal) FA_DQ_DS_LAUNCH(64, true); else FA_DQ_DS_LAUNCH(64, false);
      }
#undef FA_DQ_DS_LAUNCH
      return hipGetLastError();
    }
    return hipSuccess;
  }
  if constexpr (!BIAS) {
    if ((stages & 6) == 6 && a.Nk > 0 && a.Nq > 0) {
      constexpr int kKvBC = KvShape<false>::kBC;
      const int nkt = (a.Nk + kKvBC - 1) / kKvBC;
      const int nkv = nkt * BH;
      const int hpx = (BH % kNumXcd == 0) ? BH / kNumXcd : 0;
      const int nqt = (a.Nq + kDqBR - 1) / kDqBR;
      const int nq = (a.causal ? (nqt + 1) / 2 : nqt) * BH;
      const int nqpad = (nq + kNumXcd - 1) / kNumXcd * kNumXcd;
      const int n1 = fused_split(a, nkt, nqt, kKvBC) * BH / kNumXcd * kNumXcd;
#define FA_FUSED_LAUNCH(DD, CC)                                                                 \
  hipLaunchKernelGGL((bwd_fused_kernel<T, DD, CC, DROP>), dim3(nkv + nqpad), dim3(kDqThreads), 0,\
                     s, Q, K, V, dO, a.LD, (T*)a.dQ, (T*)a.dK, (T*)a.dV, a.Nq, a.Nk, nkt, BH,  \
                     hpx, n1, nqpad, nq, nqt, c, a.scale, off, bias, drop)
      if (a.d == 128) {
        if (a.causal) FA_FUSED_LAUNCH(128, true); else FA_FUSED_LAUNCH(128, false);
      } else {
        if (a.causal) FA_FUSED_LAUNCH(64, true); else FA_FUSED_LAUNCH(64, false);
      }
#undef FA_FUSED_LAUNCH
      return hipGetLastError();
    }
  }
  if ((stages & 2) && a.Nk > 0) {
    constexpr int kKvBC = KvShape<BIAS>::kBC;
    const int nkt = (a.Nk + kKvBC - 1) / kKvBC;
    const int nblocks = nkt * BH;
    const int hpx = (BH % kNumXcd == 0) ? BH / kNumXcd : 0;
#define FA_DKDV_LAUNCH(DD, CC)                                                                 \
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, DD, CC, BIAS, DROP, false>), dim3(nblocks),             \
                     dim3(KvShape<BIAS>::kThreads),                                             \
                     0, s, Q, K, V, dO, a.LD, (T*)a.dK, (T*)a.dV, a.Nq, a.Nk, nkt, BH, hpx, c,  \
                     a.scale, off, bias, drop, nullptr)
    if (a.d == 128) {
      if (a.causal) FA_DKDV_LAUNCH(128, true); else FA_DKDV_LAUNCH(128, false);
    } else {
      if (a.causal) FA_DKDV_LAUNCH(64, true); else FA_DKDV_LAUNCH(64, false);
    }
#undef FA_DKDV_LAUNCH
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & 4) && a.Nq > 0) {
    const int nqt = (a.Nq + kDqBR - 1) / kDqBR;
    const int nblocks = (a.causal ? (nqt + 1) / 2 : nqt) * BH;  // causal: query tile pairs
#define FA_DQ_LAUNCH(DD, CC)                                                                   \
  hipLaunchKernelGGL((bwd_dq_kernel<T, DD, CC, BIAS, DROP>), dim3(nblocks), dim3(kDqThreads), 0, \
                     s, Q, K, V, dO, a.LD, (T*)a.dQ, a.Nq, a.Nk, nqt, c, a.scale, off, bias, drop)
    if (a.d == 128) {
      if (a.causal) FA_DQ_LAUNCH(128, true); else FA_DQ_LAUNCH(128, false);
    } else {
      if (a.causal) FA_DQ_LAUNCH(64, true); else FA_DQ_LAUNCH(64, false);
    }
#undef FA_DQ_LAUNCH
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_bwd_typed(const BwdArgs& a, int stages, hipStream_t s) {
  if (a.drop.on)
    return a.bias.ptr ? launch_bwd_mfma<T, true, true>(a, stages, s)
                      : launch_bwd_mfma<T, false, true>(a, stages, s);
  return a.bias.ptr ? launch_bwd_mfma<T, true, false>(a, stages, s)
                    : launch_bwd_mfma<T, false, false>(a, stages, s);
}

}  // namespace

size_t bwd_ds_bytes(int BH, int Nq, int Nk) {
  return (size_t)BH * ((Nq + 31) / 32) * ds_chunks_per_row(Nk) * kDsChunk * 2;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int stages, hipStream_t s) {
  return launch_bwd_typed<bf16>(a, stages, s);
}
hipError_t launch_bwd_f16(const BwdArgs& a, int stages, hipStream_t s) {
  return launch_bwd_typed<f16>(a, stages, s);
}

hipError_t launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t s) {
  const int BH = a.B * a.H;
  if (stages & 1) {
    const hipError_t e = (a.d == 128) ? launch_pre<128, float>(a, s) : launch_pre<64, float>(a, s);
    if (e != hipSuccess) return e;
  }
  const int nkt = (a.Nk + kF32BT - 1) / kF32BT;
  const int nqt = (a.Nq + kF32BT - 1) / kF32BT;
  const int off = a.Nk - a.Nq;
  const float* Q = (const float*)a.Q;
  const float* K = (const float*)a.K;
  const float* V = (const float*)a.V;
  const float* dO = (const float*)a.dO;
  const BiasDev bias = bias_dev(a.bias, a.B, a.H, a.scale);
  const DropDev drop = drop_dev(a.drop);
  if ((stages & 2) && nkt > 0) {
#define FA_DKDV32_LAUNCH(DD, CC)                                                             \
  do {                                                                                       \
    if (a.drop.on)                                                                           \
      hipLaunchKernelGGL((bwd_dkdv_f32_kernel<DD, CC, true>), dim3(nkt * BH), dim3(kF32BT), 0, \
                         s, Q, K, V, a.L, dO, a.LD, (float*)a.dK, (float*)a.dV, a.Nq, a.Nk,  \
                         nkt, a.scale, off, bias, drop);                                     \
    else                                                                                     \
      hipLaunchKernelGGL((bwd_dkdv_f32_kernel<DD, CC, false>), dim3(nkt * BH), dim3(kF32BT),  \
                         0, s, Q, K, V, a.L, dO, a.LD, (float*)a.dK, (float*)a.dV, a.Nq,     \
                         a.Nk, nkt, a.scale, off, bias, drop);                               \
  } while (0)
    if (a.d == 128) {
      if (a.causal) FA_DKDV32_LAUNCH(128, true); else FA_DKDV32_LAUNCH(128, false);
    } else {
      if (a.causal) FA_DKDV32_LAUNCH(64, true); else FA_DKDV32_LAUNCH(64, false);
    }
#undef FA_DKDV32_LAUNCH
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & 4) && nqt > 0) {
#define FA_DQ32_LAUNCH(DD, CC)                                                               \
  do {                                                                                       \
    if (a.drop.on)                                                                           \
      hipLaunchKernelGGL((bwd_dq_f32_kernel<DD, CC, true>), dim3(nqt * BH), dim3(kF32BT), 0,  \
                         s, Q, K, V, a.L, dO, a.LD, (float*)a.dQ, a.Nq, a.Nk, nqt, a.scale,  \
                         off, bias, drop);                                                   \
    else                                                                                     \
      hipLaunchKernelGGL((bwd_dq_f32_kernel<DD, CC, false>), dim3(nqt * BH), dim3(kF32BT), 0, \
                         s, Q, K, V, a.L, dO, a.LD, (float*)a.dQ, a.Nq, a.Nk, nqt, a.scale,  \
                         off, bias, drop);                                                   \
  } while (0)
    if (a.d == 128) {
      if (a.causal) FA_DQ32_LAUNCH(128, true); else FA_DQ32_LAUNCH(128, false);
    } else {
      if (a.causal) FA_DQ32_LAUNCH(64, true); else FA_DQ32_LAUNCH(64, false);
    }
#undef FA_DQ32_LAUNCH
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace fa
