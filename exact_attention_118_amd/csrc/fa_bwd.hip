// Backward pass kernels: dQ, dK, dV of f = sum(dO * O).
//
// Method: FlashAttention's backward pass recomputes the probabilities from
// Q, K and the forward logsumexp L instead of storing them (the Huawei Cloud post "FlashAttention", section 3
// "Recomputation"; the 51CTO FlashAttention V1/V2 notes: the backward pass needs only L, and takes the
// per-row auxiliary D, which the softmax Jacobian fixes as D = rowsum(dO * O)).
// Five GEMMs per (key block, query block) pair (the 51CTO FlashAttention V1/V2 notes, "FlashAttention V2
// 相比V1有哪些改进": fwd 2 GEMMs, bwd 5):
//     S = Q K^T            P  = exp(S * scale - L)
//     dP = dO V^T          dS = P * (dP - D)
//     dV += P^T dO         dK += scale * dS^T Q         dQ += scale * dS K
// The grid is parallel over key blocks (the 51CTO FlashAttention V1/V2 notes, "Thread
// Block Level 并行": the backward pass splits the key sequence across blocks); each workgroup keeps its dK and dV block on chip and
// loops over query blocks.  dQ receives contributions from every key block
// and is reduced with fp32 global atomic adds into a workspace accumulator
// (the 51CTO FlashAttention V1/V2 notes, "Sequence Parallel": bf16 atomics would be a performance disaster,
// so the accumulator is fp32 and is converted once at the end); consecutive
// workgroups start their query loop at different blocks so that their atomic
// adds target different rows at any moment (the 51CTO FlashAttention V1/V2 notes: place tiles whose
// atomics would collide in different waves).
//
// gfx950 mapping (bf16 kernel):
//  * 256 threads = 4 waves, BC = 128 keys per workgroup, 32 keys per wave:
//    dK and dV stay wave-private (the 51CTO FlashAttention V1/V2 notes, "Warp Level 并行", the partition in
//    which dV, dS and dK need no cross-warp sync and only dQ does).
//  * Accumulators are laid out with the key index along lanes (S = Q K^T with
//    the 32x32x16 bf16 MFMA), so P and dS feed dV^T = dO^T P and dK^T = Q^T dS
//    straight from registers; dO^T and Q^T come from the row-major LDS tiles
//    via the transpose read ds_read_b64_tr_b16.
//  * dS^T is written once to LDS; dQ = dS K is then split over the waves by
//    output tile, so the cross-wave reduction happens inside the MFMA k-loop
//    and each dQ element gets one atomic add per (query block, key block).
//  * Q, dO, L and D of the next query block are prefetched into registers
//    while the current block is processed.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBwdBC = 128;  // keys per workgroup
constexpr int kBwdBR = 64;   // query rows per inner iteration
constexpr int kBwdThreads = 256;

// D_i = sum_k dO_ik O_ik in fp32, and clear the fp32 dQ accumulator rows.
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O,
                                                      const T* __restrict__ dO,
                                                      float* __restrict__ Dvec,
                                                      float* __restrict__ dQacc, long rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t base = (size_t)row * D + part * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)O[base + e], (float)dO[base + e], acc);
    float4* z = (float4*)(dQacc + base);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int msk = TPR / 2; msk >= 1; msk >>= 1) acc += __shfl_xor(acc, msk, 64);
  if (row < rows && part == 0) Dvec[row] = acc;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ L, const bf16* __restrict__ dO, const float* __restrict__ Dvec,
    float* __restrict__ dQacc, bf16* __restrict__ dK, bf16* __restrict__ dV, int Nq, int Nk,
    int nkt, float c, float scale, int off) {
  constexpr int BC = kBwdBC, BR = kBwdBR;
  constexpr int TSTR = D + 16;    // LDS pitch of K, Q, dO tiles (elements)
  constexpr int SSTR = BR + 16;   // LDS pitch of the dS^T tile (elements)
  constexpr int CPR = D / 8;
  constexpr int NLQ = BR * CPR / kBwdThreads;  // 16-byte loads per thread per Q-block tensor
  constexpr int NKK = D / 16;
  constexpr int NNT = D / 32;
  constexpr int NQT_W = NNT / 2;  // dQ output tiles (over d) per wave
  static_assert(NLQ * kBwdThreads == BR * CPR, "tile load must divide evenly");

  __shared__ __attribute__((aligned(16))) bf16 sK[BC * TSTR];
  __shared__ __attribute__((aligned(16))) bf16 sQ[BR * TSTR];
  __shared__ __attribute__((aligned(16))) bf16 sdO[BR * TSTR];
  __shared__ __attribute__((aligned(16))) bf16 sdS[BC * SSTR];
  __shared__ __attribute__((aligned(16))) float sL2[BR];
  __shared__ __attribute__((aligned(16))) float sD[BR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, s16 = lane & 15;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nkt;
  const int kt = logical - bh * nkt;
  const int k0 = kt * BC;
  const int kw0 = k0 + wave * 32;  // this wave's first key
  const size_t qbase = (size_t)bh * Nq * D;
  const size_t kbase = (size_t)bh * Nk * D;
  const size_t lbase = (size_t)bh * Nq;

  // Stage the K block in LDS (for the dQ GEMM) and keep this wave's K and V
  // rows in registers (B operands of S = Q K^T and dP = dO V^T).
  for (int idx = tid; idx < BC * CPR; idx += kBwdThreads) {
    const int r = idx / CPR, ch = idx - r * CPR;
    const int key = k0 + r;
    *(bf16x8*)(sK + r * TSTR + ch * 8) =
        (key < Nk) ? *(const bf16x8*)(K + kbase + (size_t)key * D + ch * 8) : zero_bf16x8();
  }
  const int mykey = kw0 + l32;
  bf16x8 kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const size_t o = kbase + (size_t)mykey * D + kk * 16 + half * 8;
    kf[kk] = (mykey < Nk) ? *(const bf16x8*)(K + o) : zero_bf16x8();
    vf[kk] = (mykey < Nk) ? *(const bf16x8*)(V + o) : zero_bf16x8();
  }

  f32x16 dkacc[NNT], dvacc[NNT];
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) {
    dkacc[nt] = (f32x16){};
    dvacc[nt] = (f32x16){};
  }

  // Query blocks that can see any of this workgroup's keys.
  const int nqb = (Nq + BR - 1) / BR;
  const int qb_first = CAUSAL ? max(0, k0 - off) / BR : 0;
  const int nloop = nqb - qb_first;
  // Stagger the start so concurrent workgroups of one head add into different dQ rows.
  const int rot = CAUSAL ? 0 : (nloop > 0 ? kt % nloop : 0);

  bf16x8 qreg[NLQ], doreg[NLQ];
  float lreg = 0.f;
  auto gload = [&](int qb) {
    const int qi0 = qb * BR;
#pragma unroll
    for (int u = 0; u < NLQ; ++u) {
      const int idx = tid + u * kBwdThreads;
      const int r = idx / CPR, ch = idx - r * CPR;
      const int q = qi0 + r;
      if (q < Nq) {
        qreg[u] = *(const bf16x8*)(Q + qbase + (size_t)q * D + ch * 8);
        doreg[u] = *(const bf16x8*)(dO + qbase + (size_t)q * D + ch * 8);
      } else {
        qreg[u] = zero_bf16x8();
        doreg[u] = zero_bf16x8();
      }
    }
    if (tid < 2 * BR) {
      const int q = qi0 + (tid & (BR - 1));
      if (tid < BR) lreg = (q < Nq) ? L[lbase + q] * kLog2e : INFINITY;
      else lreg = (q < Nq) ? Dvec[lbase + q] : 0.f;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int u = 0; u < NLQ; ++u) {
      const int idx = tid + u * kBwdThreads;
      const int r = idx / CPR, ch = idx - r * CPR;
      *(bf16x8*)(sQ + r * TSTR + ch * 8) = qreg[u];
      *(bf16x8*)(sdO + r * TSTR + ch * 8) = doreg[u];
    }
    if (tid < BR) sL2[tid] = lreg;
    else if (tid < 2 * BR) sD[tid - BR] = lreg;
  };

  if (nloop > 0) {
    gload(qb_first + rot);
    sstore();
  }
  __syncthreads();

  // Lane-constant parts of the transpose-read addresses.
  const int tr_row = (g >> 1) * 4 + (s16 >> 2);     // row within a 16-row chunk (+8 for hi)
  const int tr_col = (g & 1) * 16 + (s16 & 3) * 4;  // column within a 32-wide tile
  // dQ tiles of this wave: query rows [mq*32, mq*32+32), d columns nt0*32 ...
  const int mq = wave & 1;
  const int nt0 = (wave >> 1) * NQT_W;

  for (int it = 0; it < nloop; ++it) {
    const int qb = qb_first + (it + rot) % nloop;
    const int qi0 = qb * BR;
    if (it + 1 < nloop) gload(qb_first + (it + 1 + rot) % nloop);

    const bool wave_idle = CAUSAL && (qi0 + BR - 1 + off < kw0);
    bf16x8 dsf[4];
    if (!wave_idle) {
      // S = Q K^T and dP = dO V^T for 64 query rows x this wave's 32 keys.
      f32x16 sacc[2], dpacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        sacc[mt] = (f32x16){};
        dpacc[mt] = (f32x16){};
        const bf16* qrow = sQ + (mt * 32 + l32) * TSTR + half * 8;
        const bf16* dorow = sdO + (mt * 32 + l32) * TSTR + half * 8;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          sacc[mt] = mfma32(*(const bf16x8*)(qrow + kk * 16), kf[kk], sacc[mt]);
          dpacc[mt] = mfma32(*(const bf16x8*)(dorow + kk * 16), vf[kk], dpacc[mt]);
        }
      }
      const bool need_mask = (qi0 + BR > Nq) || (k0 + BC > Nk) ||
                             (CAUSAL && (qi0 + off < kw0 + 31));
      // P = exp2(S*c - L*log2e), dS = P * (dP - D).
      bf16x8 pf[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int ql = mt * 32 + i4 * 8 + half * 4;
          const float4 l2 = *(const float4*)(sL2 + ql);
          const float4 dd = *(const float4*)(sD + ql);
          const float l2v[4] = {l2.x, l2.y, l2.z, l2.w};
          const float ddv[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i4 * 4 + e;
            float p = fast_exp2(fmaf(sacc[mt][i], c, -l2v[e]));
            if (need_mask) {
              const int q = qi0 + ql + e;
              const bool vis = (q < Nq) && (mykey < Nk) && (!CAUSAL || mykey <= q + off);
              if (!vis) p = 0.f;
            }
            const float ds = p * (dpacc[mt][i] - ddv[e]);
            const int kc = mt * 2 + (i4 >> 1);
            const int slot = (i4 & 1) * 4 + e;
            pf[kc][slot] = (bf16)p;
            dsf[kc][slot] = (bf16)ds;
          }
        }
      // dV^T += dO^T P and dK^T += Q^T dS (A operands by LDS transpose reads).
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const int off_lo = (kc * 16 + tr_row) * TSTR + nt * 32 + tr_col;
          const bf16x8 a_do = concat(lds_read_tr(to_lds(sdO + off_lo)),
                                     lds_read_tr(to_lds(sdO + off_lo + 8 * TSTR)));
          dvacc[nt] = mfma32(a_do, pf[kc], dvacc[nt]);
          const bf16x8 a_q = concat(lds_read_tr(to_lds(sQ + off_lo)),
                                    lds_read_tr(to_lds(sQ + off_lo + 8 * TSTR)));
          dkacc[nt] = mfma32(a_q, dsf[kc], dkacc[nt]);
        }
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) dsf[kc] = zero_bf16x8();
    }
    // dS^T -> LDS: row = key, 4 consecutive query columns per store.
    {
      bf16* srow = sdS + (wave * 32 + l32) * SSTR + half * 4;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = dsf[kc][hh * 4 + e];
          *(bf16x4*)(srow + kc * 16 + hh * 8) = v;
        }
    }
    __syncthreads();

    // dQ (unscaled) = dS K over the 128 keys of this workgroup, then atomics.
    {
      f32x16 qacc[NQT_W];
#pragma unroll
      for (int n = 0; n < NQT_W; ++n) qacc[n] = (f32x16){};
#pragma unroll
      for (int kc = 0; kc < BC / 16; ++kc) {
        const int srow_lo = kc * 16 + half * 8 + (s16 >> 2);
        const bf16* ap = sdS + srow_lo * SSTR + mq * 32 + (g & 1) * 16 + (s16 & 3) * 4;
        const bf16x8 a = concat(lds_read_tr(to_lds(ap)), lds_read_tr(to_lds(ap + 4 * SSTR)));
#pragma unroll
        for (int n = 0; n < NQT_W; ++n) {
          const bf16* bp = sK + srow_lo * TSTR + (nt0 + n) * 32 + (g & 1) * 16 + (s16 & 3) * 4;
          const bf16x8 b = concat(lds_read_tr(to_lds(bp)), lds_read_tr(to_lds(bp + 4 * TSTR)));
          qacc[n] = mfma32(a, b, qacc[n]);
        }
      }
#pragma unroll
      for (int n = 0; n < NQT_W; ++n) {
        const int dc = (nt0 + n) * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = qi0 + mq * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
          if (q < Nq)
            __hip_atomic_fetch_add(dQacc + (qbase + (size_t)q * D + dc), qacc[n][i],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();
    if (it + 1 < nloop) {
      sstore();
      __syncthreads();
    }
  }

  // Epilogue: dK = scale * dK_acc, dV = dV_acc; lane holds key kw0 + l32.
  if (mykey < Nk) {
    bf16* dkrow = dK + kbase + (size_t)mykey * D;
    bf16* dvrow = dV + kbase + (size_t)mykey * D;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        bf16x4 vk, vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vk[e] = (bf16)(dkacc[nt][gg * 4 + e] * scale);
          vv[e] = (bf16)(dvacc[nt][gg * 4 + e]);
        }
        *(bf16x4*)(dkrow + nt * 32 + gg * 8 + half * 4) = vk;
        *(bf16x4*)(dvrow + nt * 32 + gg * 8 + half * 4) = vv;
      }
  }
}

// dQ = dtype(scale * dQacc), 8 elements per thread.
template <typename T>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ dQacc,
                                                             T* __restrict__ dQ, float scale,
                                                             long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 a = ((const float4*)dQacc)[2 * i];
  const float4 b = ((const float4*)dQacc)[2 * i + 1];
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  if constexpr (sizeof(T) == 2) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)(v[e] * scale);
    ((bf16x8*)dQ)[i] = o;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) dQ[8 * i + e] = v[e] * scale;
  }
}

// ---------------------------------------------------------------------------
// fp32 backward (correctness path): one thread per key row for dK/dV, one
// thread per query row for dQ; plain fp32 FMAs and expf.
constexpr int kF32BT = 64;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32BT) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ L, const float* __restrict__ dO, const float* __restrict__ Dvec,
    float* __restrict__ dK, float* __restrict__ dV, int Nq, int Nk, int nkt, float scale,
    int off) {
  __shared__ float sq[D], sdo[D];
  const int bh = blockIdx.x / nkt;
  const int kt = blockIdx.x - bh * nkt;
  const int key = kt * kF32BT + threadIdx.x;
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
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
    const float p = expf(s * scale - L[(size_t)bh * Nq + q]);
    const float ds = p * (dp - Dvec[(size_t)bh * Nq + q]);
#pragma unroll
    for (int e = 0; e < D; ++e) {
      dv[e] = fmaf(p, sdo[e], dv[e]);
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32BT) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ L, const float* __restrict__ dO, const float* __restrict__ Dvec,
    float* __restrict__ dQ, int Nq, int Nk, int nqt, float scale, int off) {
  __shared__ float sk[D], sv[D];
  const int bh = blockIdx.x / nqt;
  const int qt = blockIdx.x - bh * nqt;
  const int q = qt * kF32BT + threadIdx.x;
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
  float qv[D], dov[D], dq[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = (q < Nq) ? Q[qbase + (size_t)q * D + e] : 0.f;
    dov[e] = (q < Nq) ? dO[qbase + (size_t)q * D + e] : 0.f;
    dq[e] = 0.f;
  }
  const float lq = (q < Nq) ? L[(size_t)bh * Nq + q] : 0.f;
  const float dq_aux = (q < Nq) ? Dvec[(size_t)bh * Nq + q] : 0.f;
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
    const float p = expf(s * scale - lq);
    const float ds = p * (dp - dq_aux);
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
  const long rows = (long)a.B * a.H * a.Nq;
  constexpr int RPB = 256 / (D / 8);
  const long nb = (rows + RPB - 1) / RPB;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_pre_kernel<D, T>), dim3((unsigned)nb), dim3(256), 0, s,
                     (const T*)a.O, (const T*)a.dO, a.Dvec, a.dQacc, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int stages, hipStream_t s) {
  const int BH = a.B * a.H;
  if (stages & 1) {
    const hipError_t e = (a.d == 128) ? launch_pre<128, bf16>(a, s) : launch_pre<64, bf16>(a, s);
    if (e != hipSuccess) return e;
  }
  if (stages & 2) {
    const int nkt = (a.Nk + kBwdBC - 1) / kBwdBC;
    const int nblocks = nkt * BH;
    const float c = a.scale * kLog2e;
    const int off = a.Nk - a.Nq;
#define FA_BWD_LAUNCH(DD, CC)                                                                   \
  hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<DD, CC>), dim3(nblocks), dim3(kBwdThreads), 0, s,     \
                     (const bf16*)a.Q, (const bf16*)a.K, (const bf16*)a.V, a.L,                  \
                     (const bf16*)a.dO, a.Dvec, a.dQacc, (bf16*)a.dK, (bf16*)a.dV, a.Nq, a.Nk,   \
                     nkt, c, a.scale, off)
    if (a.d == 128) {
      if (a.causal) FA_BWD_LAUNCH(128, true); else FA_BWD_LAUNCH(128, false);
    } else {
      if (a.causal) FA_BWD_LAUNCH(64, true); else FA_BWD_LAUNCH(64, false);
    }
#undef FA_BWD_LAUNCH
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & 4) {
    const long n8 = (long)BH * a.Nq * a.d / 8;
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dq_convert_kernel<bf16>), dim3((unsigned)((n8 + 255) / 256)),
                       dim3(256), 0, s, a.dQacc, (bf16*)a.dQ, a.scale, n8);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t s) {
  const int BH = a.B * a.H;
  if (stages & 1) {
    const hipError_t e = (a.d == 128) ? launch_pre<128, float>(a, s) : launch_pre<64, float>(a, s);
    if (e != hipSuccess) return e;
  }
  if (!(stages & 2)) return hipSuccess;  // the fp32 path writes dQ directly in its main stage
  const int nkt = (a.Nk + kF32BT - 1) / kF32BT;
  const int nqt = (a.Nq + kF32BT - 1) / kF32BT;
  const int off = a.Nk - a.Nq;
  const float* Q = (const float*)a.Q;
  const float* K = (const float*)a.K;
  const float* V = (const float*)a.V;
  const float* dO = (const float*)a.dO;
#define FA_BWD32_LAUNCH(DD, CC)                                                                  \
  do {                                                                                            \
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<DD, CC>), dim3(nkt * BH), dim3(kF32BT), 0, s, Q, K,   \
                       V, a.L, dO, a.Dvec, (float*)a.dK, (float*)a.dV, a.Nq, a.Nk, nkt, a.scale,  \
                       off);                                                                      \
    if (nqt > 0)                                                                                  \
      hipLaunchKernelGGL((bwd_dq_f32_kernel<DD, CC>), dim3(nqt * BH), dim3(kF32BT), 0, s, Q, K,   \
                         V, a.L, dO, a.Dvec, (float*)a.dQ, a.Nq, a.Nk, nqt, a.scale, off);        \
  } while (0)
  if (a.d == 128) {
    if (a.causal) FA_BWD32_LAUNCH(128, true); else FA_BWD32_LAUNCH(128, false);
  } else {
    if (a.causal) FA_BWD32_LAUNCH(64, true); else FA_BWD32_LAUNCH(64, false);
  }
#undef FA_BWD32_LAUNCH
  return hipGetLastError();
}

}  // namespace fa
