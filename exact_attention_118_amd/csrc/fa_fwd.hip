// Forward pass kernels: O = softmax(scale * Q K^T + mask) V, L = row logsumexp.
//
// Method: FlashAttention's tiled online softmax (the CSDN post "Flash Attention1",
// section "Flash Attention" and its 1 x N walk-through: a running row max and
// running row sum let each block of keys be folded into the output without
// ever storing the N x N score matrix), in the loop order of FlashAttention-2
// (the 51CTO FlashAttention V1/V2 notes, "Sequence Length 并行" and "Thread Block Level 并行": the Q tile is
// the outer, parallel dimension -- one workgroup per Q tile -- and K/V tiles
// are the inner loop; O stays on chip and is written once).  Normalisation by
// the row sum is deferred to the epilogue and only L is kept for the backward
// pass (the 51CTO FlashAttention V1/V2 notes, "FlashAttention V2 相比V1有哪些改进").  The exponent uses
// exp2 with scale*log2(e) folded on the host (the 51CTO FlashAttention V1/V2 notes, "指令级别的优化").
//
// gfx950 mapping (bf16 kernel):
//  * 256 threads = 4 waves; the workgroup owns BR = 128 query rows and each
//    wave owns 32 of them ("sliced-Q", the 51CTO FlashAttention V1/V2 notes "Warp Level 并行": all waves
//    read the same K/V tile, so no cross-wave reduction is needed).
//  * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16
//    MFMA: each lane then holds 16 scores of ONE query row (its lane % 32), so
//    row max / row sum are lane-local plus a single exchange with lane ^ 32.
//  * O^T = V^T P^T reuses the S^T accumulator registers directly as the
//    P operand (no LDS round trip); V^T is read from the row-major V tile with
//    the LDS transpose read ds_read_b64_tr_b16.
//  * K/V tiles of BC = 64 keys are staged in LDS; the next tile's global
//    loads are issued before the current tile's math (register prefetch).
//  * Causal: tiles beyond the diagonal are never loaded, the mask is applied
//    only on tiles that straddle it (the 51CTO FlashAttention V1/V2 notes, "FlashAttention V2 相比V1有哪些改进"),
//    and a wave whose rows see none of a tile skips its math.
//  * Grid: one workgroup per (Q tile, batch*head), remapped so each XCD gets a
//    contiguous range of Q tiles of the same heads (K/V stay in that XCD's L2;
//    the 51CTO FlashAttention V1/V2 notes, "Thread Block Level 并行", grid order with the Q tile fastest),
//    causal tiles longest first.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kFwdBR = 128;  // query rows per workgroup
constexpr int kFwdBC = 64;   // keys per K/V tile
constexpr int kFwdThreads = 256;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ L, int Nq, int Nk, int nqt, float c, int off) {
  constexpr int BR = kFwdBR, BC = kFwdBC;
  constexpr int KSTR = D + 8;    // LDS row pitch (elements) of the K tile
  constexpr int VSTR = D + 16;   // LDS row pitch (elements) of the V tile
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int NLD = BC * CPR / kFwdThreads;
  constexpr int NKK = D / 16;    // MFMA k-steps over the head dim
  constexpr int NNT = D / 32;    // 32-wide output tiles over the head dim
  static_assert(NLD * kFwdThreads == BC * CPR, "tile load must divide evenly");

  __shared__ __attribute__((aligned(16))) bf16 sK[BC * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 sV[BC * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqt;
  const int t = logical - bh * nqt;
  const int qt = CAUSAL ? (nqt - 1 - t) : t;
  const int q0 = qt * BR;
  const size_t qbase = (size_t)bh * Nq * D;
  const size_t kbase = (size_t)bh * Nk * D;

  // This lane's query row and its Q^T fragments (B operand of S^T = K Q^T).
  const int qrow = q0 + wave * 32 + l32;
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qf[kk] = (qrow < Nq) ? *(const bf16x8*)(Q + qbase + (size_t)qrow * D + kk * 16 + half * 8)
                         : zero_bf16x8();
  }

  // Keys this workgroup needs: all, or (causal) up to the last row's diagonal.
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, q0 + BR + off);
  const int ntiles = (kend + BC - 1) / BC;
  const int wrow_lo = q0 + wave * 32;  // smallest query row of this wave

  bf16x8 kreg[NLD], vreg[NLD];
  auto gload = [&](int tile) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + u * kFwdThreads;
      const int r = idx / CPR, ch = idx - r * CPR;
      const int key = tile * BC + r;
      if (key < Nk) {
        kreg[u] = *(const bf16x8*)(K + kbase + (size_t)key * D + ch * 8);
        vreg[u] = *(const bf16x8*)(V + kbase + (size_t)key * D + ch * 8);
      } else {
        kreg[u] = zero_bf16x8();
        vreg[u] = zero_bf16x8();
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + u * kFwdThreads;
      const int r = idx / CPR, ch = idx - r * CPR;
      *(bf16x8*)(sK + r * KSTR + ch * 8) = kreg[u];
      *(bf16x8*)(sV + r * VSTR + ch * 8) = vreg[u];
    }
  };

  float m_run = -INFINITY;  // running max of scores * c (log2 domain)
  float l_run = 0.f;        // running sum of this lane half's probabilities
  f32x16 oacc[NNT];
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) oacc[nt] = (f32x16){};

  gload(0);
  sstore();
  __syncthreads();

  // Per-lane constant parts of the LDS addresses.
  const int g = lane >> 4, s16 = lane & 15;
  // V^T operand via transpose read: this lane supplies row (s16/4) and
  // column ((g%2)*16 + (s16%4)*4) of a 4-row block; rows offset by half*4.
  const int vrow_lane = (g >> 1) * 4 + (s16 >> 2);
  const int vcol_lane = (g & 1) * 16 + (s16 & 3) * 4;

  for (int j = 0; j < ntiles; ++j) {
    if (j + 1 < ntiles) gload(j + 1);
    const int k0 = j * BC;
    const bool wave_idle = CAUSAL && (k0 > wrow_lo + 31 + off);
    if (!wave_idle) {
      // S^T tile pair: keys [k0, k0+64) x this wave's 32 rows.
      f32x16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        sacc[mt] = (f32x16){};
        const bf16* krow = sK + (mt * 32 + l32) * KSTR + half * 8;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const bf16x8 a = *(const bf16x8*)(krow + kk * 16);
          sacc[mt] = mfma32(a, qf[kk], sacc[mt]);
        }
      }
      const bool need_mask = (k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > wrow_lo + off));
      if (need_mask) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + mt * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            const bool vis = (key < Nk) && (!CAUSAL || key <= qrow + off);
            if (!vis) sacc[mt][i] = -INFINITY;
          }
      }
      // Online softmax (the CSDN post "Flash Attention1" walk-through; deferred normalisation).
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mt][i]);
      mx = fmaxf(mx, wave_shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * c);
      const float m_base = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_base);
      float rs = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(sacc[mt][i], c, -m_base));
          sacc[mt][i] = p;
          rs += p;
        }
      l_run = fmaf(l_run, alpha, rs);
      m_run = m_new;
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt) oacc[nt] *= alpha;

      // P^T fragments for the four 16-key chunks (B operand of O^T = V^T P^T).
      bf16x8 pf[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[kc][e] = (bf16)sacc[kc >> 1][(kc & 1) * 8 + e];

#pragma unroll
      for (int nt = 0; nt < NNT; ++nt) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16* vp = sV + (kc * 16 + vrow_lane) * VSTR + nt * 32 + vcol_lane;
          const bf16x4 lo = lds_read_tr(to_lds(vp));
          const bf16x4 hi = lds_read_tr(to_lds(vp + 8 * VSTR));
          oacc[nt] = mfma32(concat(lo, hi), pf[kc], oacc[nt]);
        }
      }
    }
    __syncthreads();
    if (j + 1 < ntiles) {
      sstore();
      __syncthreads();
    }
  }

  // Epilogue: O = O_acc / l, L = (m + log2 l) * ln 2.
  const float l_tot = l_run + wave_shfl_xor(l_run, 32);
  if (qrow < Nq) {
    const float inv = 1.f / l_tot;
    bf16* orow = O + qbase + (size_t)qrow * D;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[nt][gg * 4 + e] * inv);
        *(bf16x4*)(orow + nt * 32 + gg * 8 + half * 4) = v;
      }
    if (half == 0) L[(size_t)bh * Nq + qrow] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 forward: one thread per query row, K/V tiles of 16 keys in LDS, exact
// fp32 arithmetic with expf.  A correctness path for fp32 inputs.
constexpr int kF32Rows = 64;
constexpr int kF32Keys = 16;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32Rows) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ L, int Nq, int Nk, int nqt, float scale, int off) {
  __shared__ float sK[kF32Keys][D];
  __shared__ float sV[kF32Keys][D];
  const int bh = blockIdx.x / nqt;
  const int qt = blockIdx.x - bh * nqt;
  const int tid = threadIdx.x;
  const int row = qt * kF32Rows + tid;
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = (row < Nq) ? Q[qbase + (size_t)row * D + e] : 0.f;
    o[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, qt * kF32Rows + kF32Rows + off);
  for (int k0 = 0; k0 < kend; k0 += kF32Keys) {
    for (int idx = tid; idx < kF32Keys * D; idx += kF32Rows) {
      const int r = idx / D, e = idx - r * D;
      const int key = k0 + r;
      sK[r][e] = (key < Nk) ? K[kbase + (size_t)key * D + e] : 0.f;
      sV[r][e] = (key < Nk) ? V[kbase + (size_t)key * D + e] : 0.f;
    }
    __syncthreads();
    float s[kF32Keys];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kF32Keys; ++jj) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) acc = fmaf(q[e], sK[jj][e], acc);
      const int key = k0 + jj;
      const bool vis = key < Nk && (!CAUSAL || key <= row + off);
      s[jj] = vis ? acc * scale : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m_run - m_base);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= alpha;
#pragma unroll
    for (int jj = 0; jj < kF32Keys; ++jj) {
      const float p = expf(s[jj] - m_base);
      l_run += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = fmaf(p, sV[jj][e], o[e]);
    }
    m_run = m_new;
    __syncthreads();
  }
  if (row < Nq) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int e = 0; e < D; ++e) O[qbase + (size_t)row * D + e] = o[e] * inv;
    L[(size_t)bh * Nq + row] = m_run + logf(l_run);
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int nqt = (a.Nq + kFwdBR - 1) / kFwdBR;
  const int nblocks = nqt * BH;
  const float c = a.scale * kLog2e;
  const int off = a.Nk - a.Nq;
  const bf16* Q = (const bf16*)a.Q;
  const bf16* K = (const bf16*)a.K;
  const bf16* V = (const bf16*)a.V;
  bf16* O = (bf16*)a.O;
#define FA_FWD_LAUNCH(DD, CC)                                                                  \
  hipLaunchKernelGGL((fwd_bf16_kernel<DD, CC>), dim3(nblocks), dim3(kFwdThreads), 0, s, Q, K, V, \
                     O, a.L, a.Nq, a.Nk, nqt, c, off)
  if (a.d == 128) {
    if (a.causal) FA_FWD_LAUNCH(128, true); else FA_FWD_LAUNCH(128, false);
  } else {
    if (a.causal) FA_FWD_LAUNCH(64, true); else FA_FWD_LAUNCH(64, false);
  }
#undef FA_FWD_LAUNCH
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int nqt = (a.Nq + kF32Rows - 1) / kF32Rows;
  const int nblocks = nqt * BH;
  const int off = a.Nk - a.Nq;
  const float* Q = (const float*)a.Q;
  const float* K = (const float*)a.K;
  const float* V = (const float*)a.V;
  float* O = (float*)a.O;
#define FA_FWD32_LAUNCH(DD, CC)                                                               \
  hipLaunchKernelGGL((fwd_f32_kernel<DD, CC>), dim3(nblocks), dim3(kF32Rows), 0, s, Q, K, V, O, \
                     a.L, a.Nq, a.Nk, nqt, a.scale, off)
  if (a.d == 128) {
    if (a.causal) FA_FWD32_LAUNCH(128, true); else FA_FWD32_LAUNCH(128, false);
  } else {
    if (a.causal) FA_FWD32_LAUNCH(64, true); else FA_FWD32_LAUNCH(64, false);
  }
#undef FA_FWD32_LAUNCH
  return hipGetLastError();
}

}  // namespace fa
