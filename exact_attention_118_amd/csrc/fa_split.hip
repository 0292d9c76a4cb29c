// Split-key forward for a single query row per head (decode shape), and the
// logsumexp-weighted combine of the per-split partial results.
//
// Method: with one query row, the query dimension offers no parallelism, so
// the keys are split across workgroups and a reduction rescales and sums the
// partial outputs (the 51CTO FlashAttention V1/V2 notes, "Sequence Length 并行": Flash-Decoding parallelises
// over the K/V sequence when the query length is 1; and the last paragraph of
// "Sequence Parallel": partial softmax results are combined by a reduction
// kernel that rescales them).  Each split runs the online softmax of the CSDN "Flash Attention1" post's
// walk-through over its keys and emits its normalised output O_s and
// logsumexp L_s; the combine forms L = log sum_s exp(L_s) and
// O = sum_s exp(L_s - L) O_s.
//
// This path moves K and V exactly once and does 4*d flops per key, so it is
// bound by HBM bandwidth; it uses plain vector loads and VALU dot products
// (MFMA would idle on a single query row).
//  * 256 threads = 4 waves; in a wave, D/8 lanes share one key row (16 bytes
//    each), so a wave covers 64/(D/8) keys per load pass and 8 passes per
//    iteration, all loads of an iteration in flight together.
//  * Each wave keeps its own running max / sum / output; the four waves are
//    merged through LDS at the end, so the key loop has no barriers.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kSplitThreads = 256;
constexpr int kSplitPasses = 8;

template <typename T, int D>
__global__ __launch_bounds__(kSplitThreads) void fwd_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    float* __restrict__ part_o, float* __restrict__ part_l, int Nk, int splits, int chunk,
    int BH, float c) {
  constexpr int TPR = D / 8;          // lanes per key row
  constexpr int KPP = 64 / TPR;       // keys per pass per wave
  constexpr int KPW = KPP * kSplitPasses;  // keys per iteration per wave
  __shared__ float sM[4], sL[4];
  __shared__ __attribute__((aligned(16))) float sO[4][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x / splits;
  const int sp = blockIdx.x - bh * splits;
  const int kb = sp * chunk;
  const int ke = min(Nk, kb + chunk);
  const int dpart = lane % TPR;   // this lane's 8 dims: [dpart*8, dpart*8+8)
  const int kgrp = lane / TPR;    // key within a pass
  const size_t kbase = (size_t)bh * Nk * D;

  float q[8];
  {
    const typename Vec<T>::x8 qv = *(const typename Vec<T>::x8*)(Q + (size_t)bh * D + dpart * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = (float)qv[e];
  }
  float m_run = -INFINITY, l_run = 0.f;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  for (int base = kb + wave * KPW; base < ke; base += 4 * KPW) {
    typename Vec<T>::x8 kv[kSplitPasses], vv[kSplitPasses];
#pragma unroll
    for (int p = 0; p < kSplitPasses; ++p) {
      const int key = base + p * KPP + kgrp;
      if (key < ke) {
        // Every K/V byte is read once: non-temporal loads stream it past the
        // caches (6.1 -> 6.9 TB/s on B16 H32 Nk16384 d128).
        kv[p] = __builtin_nontemporal_load(
            (const typename Vec<T>::x8*)(K + kbase + (size_t)key * D + dpart * 8));
        vv[p] = __builtin_nontemporal_load(
            (const typename Vec<T>::x8*)(V + kbase + (size_t)key * D + dpart * 8));
      } else {
        kv[p] = zero8<typename Vec<T>::x8>();
        vv[p] = zero8<typename Vec<T>::x8>();
      }
    }
    float s[kSplitPasses];
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < kSplitPasses; ++p) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(q[e], (float)kv[p][e], acc);
#pragma unroll
      for (int msk = TPR / 2; msk >= 1; msk >>= 1) acc += __shfl_xor(acc, msk, 64);
      const int key = base + p * KPP + kgrp;
      s[p] = (key < ke) ? acc : -INFINITY;
      mx = fmaxf(mx, s[p]);
    }
#pragma unroll
    for (int msk = TPR; msk < 64; msk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, msk, 64));
    const float m_new = fmaxf(m_run, mx * c);
    const float m_base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_base);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int p = 0; p < kSplitPasses; ++p) {
      const float pr = fast_exp2(fmaf(s[p], c, -m_base));
      l_run += pr;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(pr, (float)vv[p][e], o[e]);
    }
    m_run = m_new;
  }
  // Merge the key groups of the wave (lanes with equal dpart), then the waves.
#pragma unroll
  for (int msk = TPR; msk < 64; msk <<= 1) {
    l_run += __shfl_xor(l_run, msk, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], msk, 64);
  }
  if (lane < TPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sO[wave][dpart * 8 + e] = o[e];
    if (lane == 0) {
      sM[wave] = m_run;
      sL[wave] = l_run;
    }
  }
  __syncthreads();
  if (tid < D) {
    float M = fmaxf(fmaxf(sM[0], sM[1]), fmaxf(sM[2], sM[3]));
    const float Mb = (M == -INFINITY) ? 0.f : M;
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = fast_exp2(sM[w] - Mb);
      lsum = fmaf(sL[w], wt, lsum);
      acc = fmaf(sO[w][tid], wt, acc);
    }
    part_o[((size_t)sp * BH + bh) * D + tid] = acc / lsum;
    if (tid == 0) part_l[(size_t)sp * BH + bh] = (M + log2f(lsum)) * kLn2;
  }
}

// One workgroup of D threads per output row (rows = B*H*Nq, row-major like O):
// L = log sum_s exp(L_s), O = sum_s exp(L_s - L) O_s.  A split that saw no key
// of the row has L_s = -inf and weight 0; every row sees some key overall.
template <typename T, int D>
__global__ __launch_bounds__(D) void split_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_l,
                                                          T* __restrict__ O,
                                                          float* __restrict__ L, int splits,
                                                          int rows) {
  const int r = blockIdx.x, e = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_l[(size_t)s * rows + r]);
  float sum = 0.f;
  for (int s = 0; s < splits; ++s) sum += expf(part_l[(size_t)s * rows + r] - M);
  const float Lt = M + logf(sum);
  float acc = 0.f;
  for (int s = 0; s < splits; ++s)
    acc = fmaf(expf(part_l[(size_t)s * rows + r] - Lt), part_o[((size_t)s * rows + r) * D + e], acc);
  O[(size_t)r * D + e] = (T)acc;
  if (e == 0) L[r] = Lt;
}

template <typename T>
hipError_t launch_combine(const FwdArgs& a, int splits, int rows, const float* part_o,
                          const float* part_l, hipStream_t s) {
  if (a.d == 128) {
    hipLaunchKernelGGL((split_combine_kernel<T, 128>), dim3(rows), dim3(128), 0, s, part_o, part_l,
                       (T*)a.O, a.L, splits, rows);
  } else {
    hipLaunchKernelGGL((split_combine_kernel<T, 64>), dim3(rows), dim3(64), 0, s, part_o, part_l,
                       (T*)a.O, a.L, splits, rows);
  }
  return hipGetLastError();
}

}  // namespace

int split_chunk(int Nk, int splits) { return (Nk + splits - 1) / splits; }

namespace {

template <typename T>
hipError_t launch_split(const FwdArgs& a, int splits, float* part_o, float* part_l,
                        hipStream_t s) {
  const int BH = a.B * a.H;
  const int chunk = split_chunk(a.Nk, splits);
  const float c = a.scale * kLog2e;
  const unsigned nblocks = (unsigned)splits * (unsigned)BH;
  if (a.d == 128) {
    hipLaunchKernelGGL((fwd_split_kernel<T, 128>), dim3(nblocks), dim3(kSplitThreads), 0, s,
                       (const T*)a.Q, (const T*)a.K, (const T*)a.V, part_o, part_l, a.Nk, splits,
                       chunk, BH, c);
  } else {
    hipLaunchKernelGGL((fwd_split_kernel<T, 64>), dim3(nblocks), dim3(kSplitThreads), 0, s,
                       (const T*)a.Q, (const T*)a.K, (const T*)a.V, part_o, part_l, a.Nk, splits,
                       chunk, BH, c);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine<T>(a, splits, BH, part_o, part_l, s);
}

}  // namespace

hipError_t launch_fwd_split_bf16(const FwdArgs& a, int splits, float* part_o, float* part_l,
                                 hipStream_t s) {
  return launch_split<bf16>(a, splits, part_o, part_l, s);
}
hipError_t launch_fwd_split_f16(const FwdArgs& a, int splits, float* part_o, float* part_l,
                                hipStream_t s) {
  return launch_split<f16>(a, splits, part_o, part_l, s);
}

hipError_t launch_split_combine_bf16(const FwdArgs& a, int splits, const float* part_o,
                                     const float* part_l, hipStream_t s) {
  return launch_combine<bf16>(a, splits, a.B * a.H * a.Nq, part_o, part_l, s);
}
hipError_t launch_split_combine_f16(const FwdArgs& a, int splits, const float* part_o,
                                    const float* part_l, hipStream_t s) {
  return launch_combine<f16>(a, splits, a.B * a.H * a.Nq, part_o, part_l, s);
}

}  // namespace fa
