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
// gfx950 mapping (bf16 / fp16 kernel):
//  * 256 or 512 threads = 4 or 8 waves; the workgroup owns BR = 128 or 256
//    query rows and each wave owns 32 of them ("sliced-Q", the 51CTO
//    FlashAttention V1/V2 notes "Warp Level 并行": all waves read the same K/V
//    tile, so no cross-wave reduction is needed).
//  * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16/fp16
//    MFMA: each lane then holds 16 scores of ONE query row (its lane % 32), so
//    row max / row sum are lane-local plus a single exchange with lane ^ 32.
//  * O^T = V^T P^T reuses the S^T accumulator registers directly as the
//    P operand (no LDS round trip); V^T is read from the row-major V tile with
//    the LDS transpose read ds_read_b64_tr_b16.  The row sums of the rounded
//    P that normalise O come from one 16x16x32 MFMA per 16-key chunk, not
//    from vector instructions.
//  * K/V tiles of BC = 64 keys are staged in LDS, double-buffered and loaded
//    straight from HBM into LDS (global_load_lds_dwordx4) in an XOR-swizzled
//    layout that keeps both the row reads and the transpose reads free of
//    bank conflicts; the loads of tiles j+1/j+2 are spread over tile j's
//    MFMA steps, and tile j's exponentials over tile j+1's score MFMAs.
//  * Causal: tiles beyond the diagonal are never loaded and the mask is
//    applied only on tiles that straddle it (the 51CTO FlashAttention V1/V2
//    notes, "FlashAttention V2 相比V1有哪些改进").
//  * Grid: one workgroup per (Q tile, batch*head), remapped so each XCD gets a
//    contiguous range of Q tiles of the same heads (K/V stay in that XCD's L2;
//    the 51CTO FlashAttention V1/V2 notes, "Thread Block Level 并行", grid order with the Q tile fastest).
//    Causal: a workgroup takes Q tiles t and nqt-1-t in turn, so all carry
//    the same number of key tiles and no CU idles half-empty at the end.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

BiasDev bias_dev(const BiasArgs& b, int B, int H, float scale) {
  return make_bias_dev(b.ptr, b.sb, b.sh, b.sq, B, H, scale, b.tmap, b.tm_sb, b.tm_sh, b.nkt4);
}


// A workgroup of NW waves owns 32 * NW query rows: NW = 4 (128 rows, two
// workgroups per CU) or NW = 8 (256 rows, one per CU: each K/V tile staged
// in LDS then serves twice the rows, halving the L2 -> LDS traffic per MFMA).
constexpr int kFwdBC = 64;   // keys per K/V tile
constexpr int kFwdBR4 = 128;  // query rows of the 4-wave shape (bias tile-map granularity)
// The exponentials of the online softmax are taken against a reference that
// lags the row max (see the tile step): every probability stays at or below
// prob_limit<T>().  Floating point keeps its relative precision at any
// magnitude, so the limit only has to keep P, O and l finite: 2^40 for bf16
// (sums of 2^40-sized terms over any key count stay far below the fp32
// range), 2^15 for fp16, whose largest finite value is 65504.  The higher the
// limit, the more rarely the reference has to move.
template <typename T>
constexpr float prob_limit() {
  return std::is_same<T, f16>::value ? 32768.f : 1099511627776.f;
}

// Key splits (SPLIT): each workgroup takes one query tile and one chunk of
// `chunk` keys (a multiple of 2 * BC), and writes its normalised partial
// output and logsumexp in fp32 to part_o [splits, rows, D] and part_l
// [splits, rows] (rows = B*H*Nq) for the combine kernel (the 51CTO notes,
// "Sequence Length 并行" and the end of "Sequence Parallel": Flash-Decoding
// splits the keys when the query length gives too few workgroups).  A row
// that sees no key of its chunk writes 0 and -inf.
struct SplitDev {
  float* part_o;
  float* part_l;
  int splits, chunk, rows;
};

template <typename T, int D, bool CAUSAL, bool BIAS, bool DROP, bool SPLIT, int NW>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                T* __restrict__ O, float* __restrict__ L, int Nq, int Nk, int nqt, float c,
                int off, BiasDev bias, DropDev drop, SplitDev split) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int kFwdThreads = 64 * NW;
  constexpr int BR = 32 * NW, BC = kFwdBC;
  constexpr int NKK = D / 16;  // MFMA k-steps over the head dim
  constexpr int NNT = D / 32;  // 32-wide output tiles over the head dim
  constexpr int TILE = BC * D;  // elements per K or V tile
  constexpr float kProbLimit = prob_limit<T>();

  // K tiles j+1 (read) and j+2 (loading) at buffers 0/1, V tiles j (read) and
  // j+1 (loading) at buffers 2/3; all swizzled (see swz).  Tile j's buffers
  // are j & 1; the loop below is unrolled by two so that every LDS address
  // offset is a compile-time constant.
  // Bias staging (BIAS), after the tiles: a region of 32 rows x BC keys per
  // wave, rows of 8 chunks of 16 bytes, chunk c of row r at c ^ ((r / 2) % 8)
  // so that a read of one chunk per row takes the minimum two LDS passes.
  constexpr int BSTAGE = BIAS ? (kFwdThreads / 64) * 32 * BC : 0;
  __shared__ __attribute__((aligned(1024))) T smem[4 * TILE + BSTAGE];
  T* const sK0 = smem;
  T* const sV0 = smem + 2 * TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T* const sBw = smem + 4 * TILE + wave * 32 * BC;  // this wave's bias region (BIAS)
  const int half = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, s16 = lane & 15;

  // Grid: one workgroup per (query tile, batch*head); causal, one per pair of
  // query tiles (t, nqt-1-t) of a head, processed one after the other, so that
  // every workgroup has the same number of key tiles (a query tile's count
  // grows with its index).  Remapped so each XCD serves a contiguous range of
  // workgroups of the same heads (K/V stay in that XCD's L2; the 51CTO notes,
  // "Thread Block Level 并行", grid order with the query tile fastest).
  constexpr bool PAIRED = CAUSAL && !SPLIT;
  const int nwg = PAIRED ? (nqt + 1) / 2 : nqt;  // workgroups per head (and split)
  int logical = xcd_remap(blockIdx.x, gridDim.x);
  int sp = 0;  // key split (SPLIT)
  if constexpr (SPLIT) {
    sp = logical % split.splits;
    logical /= split.splits;
  }
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

  using KV = BufTile<D, BC, kFwdThreads>;
  const KV kv(wave, lane);
  static_assert(2 * KV::PER <= NKK, "tile loads fit the even score steps");
  // With key splits (a few query rows against many keys) each K/V tile is
  // read by one workgroup only: its loads are non-temporal (B4 H32 Nq16
  // Nk16384: 209 -> 178 us).  The tiled path re-reads every tile once per
  // query tile from the L2, where non-temporal loads cost 7%.
  constexpr int KV_AUX = SPLIT ? kLoadNonTemporal : 0;

  // The sums of the rounded probabilities that normalise O (see lq_run),
  // without dropout formed on the matrix cores: one 16x16x32 MFMA per
  // 16-key chunk of P, P as the B operand (lane l: row l % 32, one half of
  // the chunk's keys) and as the A operand ones in rows 0 and 8 of k-blocks
  // 0 and 2 and in rows 4 and 12 of k-blocks 1 and 3.  Element 0 of every
  // lane's result is then the chunk's sum for the lane's own row, both
  // halves included, in place of 16 v_dot2c per tile.  With a bias, whose
  // kernels are short of registers, the operand is made per tile instead of
  // being kept.
  auto make_asel = [](int ln) {
    const int m16 = ln & 15, kb = ln >> 4;
    const bool one = (m16 & 3) == 0 && ((m16 >> 2) & 1) == (kb & 1);
    T8 a;
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = one ? (T)1.f : (T)0.f;
    return a;
  };
  [[maybe_unused]] T8 asel_kept;
  if constexpr (!BIAS) asel_kept = make_asel(lane);

  // Byte offsets, within a tile, of this lane's LDS operand reads; the row
  // block and the buffer are added as instruction offsets.  S^T = K Q^T: the
  // A fragment of step st is K row (st&1)*32 + l32, 16-byte chunk
  // 2*(st>>1) + half.  O^T += V^T P^T: step st reads V^T for the 16 keys of
  // chunk st / NNT and head-dim tile st % NNT, two transpose reads
  // (hi = 0, 1) per fragment.
  unsigned ka[NKK], va[2 * NNT];
  {
    const SwzRow<D> krow(l32, half);
    const int tr_row = (g >> 1) * 4 + (s16 >> 2);     // row in a 16-row chunk
    const int tr_col = (g & 1) * 16 + (s16 & 3) * 4;  // column in a 32-wide tile
    const SwzTr<D> vtr(tr_row, tr_col);
#pragma unroll
    for (int i = 0; i < NKK; ++i) ka[i] = krow.off(0, 2 * i);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt) va[hi * NNT + nt] = vtr.off(0, hi, nt * 32);
  }
  auto kfrag = [&](int buf, int st) {
    return *at_byte<T8>(sK0 + buf * TILE, ka[st >> 1] + (st & 1) * 32 * 2 * D);
  };
  auto vfrag = [&](int buf, int st) {
    const unsigned rb = (st / NNT) * 16 * 2 * D;
    const T* base = sV0 + buf * TILE;
    return concat(lds_read_tr<T>(to_lds(at_byte<T>(base, va[st % NNT] + rb))),
                  lds_read_tr<T>(to_lds(at_byte<T>(base, va[NNT + st % NNT] + rb))));
  };
  // LDS fragments read ahead of their MFMAs (shallower with a bias, for registers)
  constexpr int KRING = BIAS ? 3 : 4, VRING = BIAS ? 2 : 3;

  for (int pass = 0; pass < (PAIRED ? 2 : 1); ++pass) {
    const int qt = !PAIRED ? t : (pass == 0 ? nqt - 1 - t : t);
    if (PAIRED && pass == 1 && t == nqt - 1 - t) break;  // odd count: the middle tile once
    if (pass == 1) __syncthreads();  // the first tile's last LDS reads precede the new loads
    const int q0 = qt * BR;

    // This lane's query row and its Q^T fragments (B operand of S^T = K Q^T).
    const int qrow = q0 + wave * 32 + l32;
    T8 qf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = (qrow < Nq) ? *(const T8*)(Q + qbase + (size_t)qrow * D + kk * 16 + half * 8)
                           : zero8<T8>();

    // Keys this workgroup needs: all, or (causal) up to the last row's diagonal.
    // With SPLIT, only the keys of chunk sp: tiles jbeg .. ntiles-1 (jbeg even,
    // so tile j still uses buffers j & 1).
    const int kbeg = SPLIT ? sp * split.chunk : 0;
    const int kend = min(CAUSAL ? min(Nk, q0 + BR + off) : Nk, SPLIT ? kbeg + split.chunk : Nk);
    int ntiles = (kend + BC - 1) / BC;
    int jbeg = kbeg / BC;
    // Bias tile map (BIAS): only the key tiles from the first to the last that
    // hold an entry above -inf for this query tile (jbeg stays even).
    if constexpr (BIAS) {
      static_assert(BR == kMapRows && BC == kMapKeys, "tile map granularity");
      if (bias.tmap) {
        const int b = bh / bias.H, h = bh - b * bias.H;
        int lo, hi;
        map_range(bias.tmap + b * bias.tm_sb + h * bias.tm_sh + (size_t)qt * bias.nkt4,
                  (Nk + BC - 1) / BC, lane, lo, hi);
        if (lo > hi) {
          ntiles = jbeg;
        } else {
          jbeg = max(jbeg, lo & ~1);
          ntiles = min(ntiles, hi + 1);
        }
      }
    }
    const int kfirst = jbeg * BC;
    const int wrow_lo = q0 + wave * 32;  // smallest query row of this wave

    float m_run = -INFINITY;  // reference of the exponentials (row max so far, log2 units)
    float l_run = 0.f;        // running sum of this lane half's probabilities (fp32, for L)
    // running sum of the same probabilities as rounded to T for P V: O is
    // normalised by it, so a dominant probability's rounding cancels between
    // numerator and denominator (fp32 l would leave up to 2^-9 of it in O)
    // (kept here with dropout, whose sums are taken before the mask; without
    // dropout element 0 of lacc holds it, from the matrix cores)
    [[maybe_unused]] float lq_run = 0.f;
    f32x4 lacc = (f32x4){};
    f32x16 oacc[NNT];
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) oacc[nt] = (f32x16){};

    // Keys past the end and, causal, keys after the row's diagonal get score
    // -inf.  Only tiles that cross the diagonal or the end need it; lane holds
    // row qrow, keys k0 + mt*32 + (i/4)*8 + half*4 + i%4.
    auto mask_tile = [&](f32x16 (&sc)[2], int k0) {
      if ((k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > wrow_lo + off))) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + mt * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            const bool vis = (key < Nk) && (!CAUSAL || key <= qrow + off);
            if (!vis) sc[mt][i] = -INFINITY;
          }
      }
    };
    // Scores of one K tile (2 x NKK MFMA steps) from LDS buffer buf.
    auto scores = [&](int buf, f32x16 (&sc)[2]) {
      T8 ring[KRING];
#pragma unroll
      for (int st = 0; st < KRING; ++st) ring[st] = kfrag(buf, st);
      sc[0] = (f32x16){};
      sc[1] = (f32x16){};
#pragma unroll
      for (int st = 0; st < 2 * NKK; ++st) {
        const T8 a = ring[st % KRING];
        if (st + KRING < 2 * NKK) ring[st % KRING] = kfrag(buf, st + KRING);
        sc[st & 1] = mfma32(a, qf[st >> 1], sc[st & 1]);
      }
    };
    // Bias of the score tile at key k0b: lane row qrow holds keys
    // k0b + mt*32 + g*8 + half*4 + 0..3 in elements i = g*4 .. g*4+3 of sc[mt];
    // rows past Nq read zeros, keys past Nk are masked afterwards.  Each wave
    // stages its 32 rows x BC keys in its own LDS region with four
    // direct-to-LDS loads of whole 128-byte rows (bias_issue), then reads its
    // lanes' pieces back (bias_fetch); no other wave touches the region.
    typedef typename Vec<T>::x4 BT4;
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
    auto bias_add = [&](f32x16 (&sc)[2], const BT4 (&bb)[8], int q0b) {
#pragma unroll
      for (int q = q0b; q < q0b + 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc[q >> 2][(q & 3) * 4 + e] = fmaf((float)bb[q][e], bias.inv_scale, sc[q >> 2][(q & 3) * 4 + e]);
    };
    auto row_max = [&](const f32x16 (&sc)[2]) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[mt][i]);
      return xor32_max(mx);
    };

    // Prologue: K tiles 0 and 1, V tile 0; scores, mask and row max of tile 0.
    kv.template tile<KV_AUX>(Kh, kfirst, Nk, sK0);
    kv.template tile<KV_AUX>(Kh, kfirst + BC, Nk, sK0 + TILE);
    kv.template tile<KV_AUX>(Vh, kfirst, Nk, sV0);
    vm_wait_all();
    __syncthreads();
    f32x16 sA[2], sB[2];
    if constexpr (BIAS) bias_issue(kfirst);
    scores(0, sA);
    if constexpr (BIAS) {
      BT4 bb[8];
      vm_wait_all();
      bias_fetch(bb, 0);
      bias_add(sA, bb, 0);
      bias_fetch(bb, 4);
      bias_add(sA, bb, 4);
    }
    mask_tile(sA, kfirst);
    m_run = row_max(sA) * c;  // the reference starts at tile 0's row max
    __syncthreads();  // every wave is done with K tile 0 before tile 2 replaces it

    // One key tile j (P = buffer parity j & 1, a constant at both inlined
    // call sites): scores of tile j are in scur, those of tile j+1 go to snext.
    auto tile_step = [&](const int P, int j, f32x16 (&scur)[2], f32x16 (&snext)[2])
                         __attribute__((always_inline)) {
      const int k0 = j * BC;
      // Online softmax (the CSDN post "Flash Attention1", 例子说明: running max
      // and running sum), normalised once in the epilogue.  The exponentials
      // are taken against a reference m_run, which only has to bound them:
      // the result is the same in exact arithmetic for any reference, since
      // O and l are both scaled by 2^-m_run.  So the reference is not moved
      // to each tile's row max.  Instead the row sums of the tile's
      // probabilities (two halves, each checked before its 16-bit values
      // enter P V) show whether any probability of the wave exceeds
      // kProbLimit; only then is the reference moved to the tile's row max,
      // what was accumulated rescaled, and that half recomputed.  A row that
      // has seen no finite score yet (m_run = -inf) always takes that path, so
      // that its first finite scores set the reference.
      float m_ref = (m_run == -INFINITY) ? 0.f : m_run;
      auto rebase = [&](float& part0, float& part1, float& partq) {
        const float m_new = fmaxf(m_run, row_max(scur) * c);
        const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
        l_run *= alpha;
        lq_run *= alpha;
        lacc *= alpha;
        part0 *= alpha;
        part1 *= alpha;
        partq *= alpha;
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) oacc[nt] *= alpha;
        m_run = m_new;
        m_ref = (m_run == -INFINITY) ? 0.f : m_run;
      };

      // The 32 probabilities of this lane's row in tile j, as 16 pairs (pair
      // pr: probabilities 2pr, 2pr+1 of chunk pr/4, converted together).  The
      // score block below is short of vector-ALU time and the P V block has
      // spare: with D = 128 the first kPairsA pairs go with the score MFMAs
      // and the rest with the first P V steps, which do not yet read them.
      constexpr int NPAIR = 16;
      constexpr int kPairsA = (D == 128) ? 8 : NPAIR;
      static_assert(NPAIR - kPairsA <= 2 * NNT, "late pairs fit before chunk 2 is read");
      T8 pf[4];
      // row sums of this lane's probabilities: rs[0..1] the early pairs,
      // rs[2..3] the late ones (two accumulators each)
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
      // with dropout, the same sums over the rounded probabilities: rq[0]
      // early, rq[1] late
      float rq[2] = {0.f, 0.f};
      // Dropout (DROP): the random bytes of this lane's scores of tile j,
      // keys k0 + mt*32 + ... in rb[mt], each made just before its pairs (the
      // second half after the score block when its pairs go with P V); the
      // row sums take the probabilities before dropout, P V after it (the
      // 1 / keep-probability factor is applied with 1 / l at the end).
      unsigned rb[2][4];
      if constexpr (DROP) {
        drop_bytes_rows(rb[0], drop, bh, qrow, k0 + half * 4, lane);
        if constexpr (kPairsA > 8) drop_bytes_rows(rb[1], drop, bh, qrow, k0 + 32 + half * 4, lane);
      }
      auto prob_pair = [&](int pr) {
        const int el = 2 * pr, kc = el >> 3, e = el & 7;
        const int mt = kc >> 1, i = (kc & 1) * 8 + e;
        const float p0 = fast_exp2(fmaf(scur[mt][i], c, -m_ref));
        const float p1 = fast_exp2(fmaf(scur[mt][i + 1], c, -m_ref));
        float& ra = rs[pr < kPairsA ? 0 : 2];
        float& rb_ = rs[pr < kPairsA ? 1 : 3];
        float& rq_ = rq[pr < kPairsA ? 0 : 1];
        // the first pair of each group starts its sums (0 + p = p exactly for
        // p >= 0), without an add into a zeroed register
        const bool first = (pr == 0 || pr == kPairsA);
        ra = first ? p0 : ra + p0;
        rb_ = first ? p1 : rb_ + p1;
        pf[kc][e] = (T)p0;
        pf[kc][e + 1] = (T)p1;
        if constexpr (DROP) rq_ = add_pair(pf[kc][e], pf[kc][e + 1], first ? 0.f : rq_);
        if constexpr (DROP) {
          if (!drop_keep(rb[mt][i >> 2], i & 3, drop.thresh)) pf[kc][e] = (T)0.f;
          if (!drop_keep(rb[mt][i >> 2], (i + 1) & 3, drop.thresh)) pf[kc][e + 1] = (T)0.f;
        }
        pin(pf[kc]);
        pin(ra);
        pin(rb_);
        if constexpr (DROP) pin(rq_);
      };

      // Scores of tile j+1 on the MFMA pipe, interleaved step by step with
      // exponentials of tile j on the vector ALU and with the direct-to-LDS
      // loads of K tile j+2 (over tile j's buffer, last read for tile j's
      // scores) and V tile j+1.  The last iterations also compute scores of a
      // stale buffer and load rows past the end (as zeros): that extra work
      // keeps this block free of branches, so the three kinds of work stay
      // interleaved.  With a bias, its values for tile j+1 are loaded first
      // and added once the scores are complete.
      if constexpr (BIAS) bias_issue(k0 + BC);
      {
        constexpr int SA = 2 * NKK;
        T8 ring[KRING];
#pragma unroll
        for (int st = 0; st < KRING; ++st) ring[st] = kfrag(1 - P, st);
        snext[0] = (f32x16){};
        snext[1] = (f32x16){};
#pragma unroll
        for (int st = 0; st < SA; ++st) {
          const T8 a = ring[st % KRING];
          if (st + KRING < SA) ring[st % KRING] = kfrag(1 - P, st + KRING);
          snext[st & 1] = mfma32(a, qf[st >> 1], snext[st & 1]);
          if ((st & 1) == 0) {
            const int di = st >> 1;
            if (di < KV::PER)
              kv.template part<KV_AUX>(Kh, k0 + 2 * BC, Nk, sK0 + P * TILE, di);
            else if (di < 2 * KV::PER)
              kv.template part<KV_AUX>(Vh, k0 + BC, Nk, sV0 + (1 - P) * TILE, di - KV::PER);
          }
#pragma unroll
          for (int pr = 0; pr < kPairsA; ++pr)
            if (pr * SA / kPairsA == st) prob_pair(pr);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // The early pairs, about to enter P V: redo them against the tile's row
      // max if some lane's sum of them exceeds the limit (nothing of tile j
      // has been accumulated yet).
      if (__builtin_amdgcn_ballot_w64(rs[0] + rs[1] > kProbLimit || m_run == -INFINITY) != 0) {
        rebase(rs[0], rs[1], rq[0]);
        rs[0] = rs[1] = 0.f;
        rq[0] = 0.f;
#pragma unroll
        for (int pr = 0; pr < kPairsA; ++pr) prob_pair(pr);
      }
      if constexpr (BIAS) {
        // the NKK tile loads of this block were issued after the bias loads
        // and complete in order: waiting for all but NKK waits for the bias
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NKK) : "memory");
        BT4 bnext[8];
        bias_fetch(bnext, 0);
        bias_add(snext, bnext, 0);
        __builtin_amdgcn_sched_barrier(0);  // half the bias registers live at a time
        bias_fetch(bnext, 4);
        bias_add(snext, bnext, 4);
      }
      mask_tile(snext, k0 + BC);
      if constexpr (DROP && kPairsA <= 8)
        drop_bytes_rows(rb[1], drop, bh, qrow, k0 + 32 + half * 4, lane);

      // O^T += V^T P^T for tile j (step st reads chunk st / NNT of P),
      // interleaved with the remaining probability pairs.
      {
        // While a wave is in this block its issue priority is raised, so that
        // the two waves of a SIMD tend to alternate: one issuing P V MFMAs,
        // the other the exponentials of its score block (about 2% faster
        // than equal priorities, measured on the long-sequence forward).
        __builtin_amdgcn_s_setprio(1);
        T8 asel;
        if constexpr (BIAS) {
          int ln = lane;
          pin(ln);  // made here, not kept across the tiles
          asel = make_asel(ln);
        } else {
          asel = asel_kept;
        }
        T8 ring[VRING];
#pragma unroll
        for (int st = 0; st < VRING; ++st) ring[st] = vfrag(P, st);
#pragma unroll
        for (int st = 0; st < 4 * NNT; ++st) {
          if (kPairsA < NPAIR && st == NPAIR - kPairsA) {
            // The late pairs are complete and their chunks not yet read: the
            // same check, now rescaling the early pairs' share of O and l.
            if (__builtin_amdgcn_ballot_w64(rs[2] + rs[3] > kProbLimit) != 0) {
              rebase(rs[0], rs[1], rq[0]);
              rs[2] = rs[3] = 0.f;
              rq[1] = 0.f;
#pragma unroll
              for (int pr = kPairsA; pr < NPAIR; ++pr) prob_pair(pr);
            }
          }
          const T8 a = ring[st % VRING];
          if (st + VRING < 4 * NNT) ring[st % VRING] = vfrag(P, st + VRING);
          oacc[st % NNT] = mfma32(a, pf[st / NNT], oacc[st % NNT]);
          if constexpr (!DROP) {
            if (st % NNT == 0) lacc = mfma16(asel, pf[st / NNT], lacc);
          }
          if (kPairsA + st < NPAIR) prob_pair(kPairsA + st);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
      if constexpr (DROP) lq_run += rq[0] + rq[1];
      vm_wait_all();  // this wave's part of tiles K j+2 and V j+1 has landed
      __syncthreads();
    };

    // Causal: tiles whose first key lies past the diagonal of this wave's
    // last row contribute nothing to its rows (with 256-row workgroups the
    // first waves reach them up to three tiles before the last ones).  The
    // wave runs the tile steps up to its last useful tile, then only takes
    // its part in the loads and barriers of the workgroup's remaining tiles.
    const int jact = (CAUSAL && !BIAS) ? min(ntiles, (wrow_lo + 31 + off) / BC + 1) : ntiles;
    for (int j = jbeg; j < jact; j += 2) {
      tile_step(0, j, sA, sB);
      if (j + 1 < jact) tile_step(1, j + 1, sB, sA);
    }
    for (int j = max(jact, jbeg); j < ntiles; ++j) {
      const int P = (j - jbeg) & 1;
#pragma unroll
      for (int di = 0; di < KV::PER; ++di) {
        kv.template part<KV_AUX>(Kh, (j + 2) * BC, Nk, sK0 + P * TILE, di);
        kv.template part<KV_AUX>(Vh, (j + 1) * BC, Nk, sV0 + (1 - P) * TILE, di);
      }
      vm_wait_all();
      __syncthreads();
    }

    // Epilogue: O = O_acc / lq (times 1 / keep-probability with dropout), lq
    // the sum of the rounded probabilities; L = (m + log2 l) * ln 2 with the
    // fp32 sum l.
    const float l_tot = xor32_sum(l_run);
    const float lq_tot = DROP ? xor32_sum(lq_run) : lacc[0];
    if constexpr (SPLIT) {
      if (qrow < Nq) {
        const size_t prow = (size_t)sp * split.rows + (size_t)bh * Nq + qrow;
        const bool any = l_tot > 0.f;  // some key of the chunk is visible to this row
        const float inv = any ? 1.f / lq_tot : 0.f;
        float* po = split.part_o + prow * D;
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = oacc[nt][gg * 4 + e] * inv;
            *(f32x4*)(po + nt * 32 + gg * 8 + half * 4) = v;
          }
        if (half == 0) split.part_l[prow] = any ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
      }
    } else if (qrow < Nq) {
      const float inv = (DROP ? drop.inv_keep : 1.f) / lq_tot;
      T* orow = O + qbase + (size_t)qrow * D;
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          T4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (T)(oacc[nt][gg * 4 + e] * inv);
          *(T4*)(orow + nt * 32 + gg * 8 + half * 4) = v;
        }
      if (half == 0) L[(size_t)bh * Nq + qrow] = (m_run + log2f(l_tot)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 forward: one thread per query row, K/V tiles of 16 keys in LDS, exact
// fp32 arithmetic with expf.  A correctness path for fp32 inputs.
constexpr int kF32Rows = 64;
constexpr int kF32Keys = 16;

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kF32Rows) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ L, int Nq, int Nk, int nqt, float scale, int off,
    BiasDev bias, DropDev drop) {
  __shared__ float sK[kF32Keys][D];
  __shared__ float sV[kF32Keys][D];
  const int bh = blockIdx.x / nqt;
  const int qt = blockIdx.x - bh * nqt;
  const int tid = threadIdx.x;
  const int row = qt * kF32Rows + tid;
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
  const float* brow = nullptr;  // this row's additive bias, if any
  if (bias.ptr && row < Nq) {
    const int b = bh / bias.H, h = bh - b * bias.H;
    brow = (const float*)bias.ptr + b * bias.sb + h * bias.sh + (long long)row * bias.sq;
  }
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
      s[jj] = vis ? acc * scale + (brow ? brow[key] : 0.f) : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m_run - m_base);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= alpha;
    // Dropout (DROP): one Philox call per 4 keys of this row; word row % 4
    // holds the row's 4 bytes.
    unsigned rbyte[kF32Keys / 4];
    if constexpr (DROP) {
#pragma unroll
      for (int kb = 0; kb < kF32Keys / 4; ++kb) {
        unsigned w[4] = {(unsigned)(k0 + 4 * kb) >> 2, (unsigned)row >> 2, (unsigned)bh,
                         drop.offset};
        philox4x32_10(w, drop.seed_lo, drop.seed_hi);
        const int r = row & 3;
        rbyte[kb] = r == 0 ? w[0] : r == 1 ? w[1] : r == 2 ? w[2] : w[3];
      }
    }
#pragma unroll
    for (int jj = 0; jj < kF32Keys; ++jj) {
      const float p = expf(s[jj] - m_base);
      l_run += p;
      const float pd = (DROP && !drop_keep(rbyte[jj >> 2], jj & 3, drop.thresh)) ? 0.f : p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = fmaf(pd, sV[jj][e], o[e]);
    }
    m_run = m_new;
    __syncthreads();
  }
  if (row < Nq) {
    const float inv = (DROP ? drop.inv_keep : 1.f) / l_run;
#pragma unroll
    for (int e = 0; e < D; ++e) O[qbase + (size_t)row * D + e] = o[e] * inv;
    L[(size_t)bh * Nq + row] = m_run + logf(l_run);
  }
}

}  // namespace

namespace {

DropDev drop_dev(const DropArgs& d) {
  return DropDev{d.seed_lo, d.seed_hi, d.offset, d.on ? d.thresh : 256u, d.on ? d.inv_keep : 1.f};
}

// Workgroup count of the tiled forward grid with NW-wave workgroups.
int fwd_blocks(const FwdArgs& a, int nw) {
  const int nqt = (a.Nq + 32 * nw - 1) / (32 * nw);
  // Causal: one workgroup per pair of query tiles (t, nqt-1-t).
  return (a.causal ? (nqt + 1) / 2 : nqt) * a.B * a.H;
}

template <typename T, bool BIAS, bool DROP, int NW>
hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t s) {
  const int nqt = (a.Nq + 32 * NW - 1) / (32 * NW);
  const int nblocks = fwd_blocks(a, NW);
  const float c = a.scale * kLog2e;
  const int off = a.Nk - a.Nq;
  const T* Q = (const T*)a.Q;
  const T* K = (const T*)a.K;
  const T* V = (const T*)a.V;
  T* O = (T*)a.O;
  const BiasDev bias = bias_dev(a.bias, a.B, a.H, a.scale);
  const DropDev drop = drop_dev(a.drop);
  const SplitDev nosplit{nullptr, nullptr, 1, 0, 0};
#define FA_FWD_LAUNCH(DD, CC)                                                                 \
  hipLaunchKernelGGL((fwd_kernel<T, DD, CC, BIAS, DROP, false, NW>), dim3(nblocks),           \
                     dim3(64 * NW), 0, s, Q, K, V, O, a.L, a.Nq, a.Nk, nqt, c, off, bias,     \
                     drop, nosplit)
  if (a.d == 128) {
    if (a.causal) FA_FWD_LAUNCH(128, true); else FA_FWD_LAUNCH(128, false);
  } else {
    if (a.causal) FA_FWD_LAUNCH(64, true); else FA_FWD_LAUNCH(64, false);
  }
#undef FA_FWD_LAUNCH
  return hipGetLastError();
}

// 8-wave workgroups when they still give every CU one (the bias path keeps
// 4 waves: its tile map and staging regions are laid out for 128-row tiles).
template <typename T, bool BIAS, bool DROP>
hipError_t launch_fwd_shape(const FwdArgs& a, hipStream_t s) {
  if constexpr (!BIAS) {
    if (fwd_blocks(a, 8) >= kNumCu) return launch_fwd_mfma<T, BIAS, DROP, 8>(a, s);
  }
  return launch_fwd_mfma<T, BIAS, DROP, 4>(a, s);
}

// Key splits for a few query rows: (query tile, key chunk, batch*head) per
// workgroup into the partial buffers; the caller runs the combine.
template <typename T>
hipError_t launch_fwd_rows_split(const FwdArgs& a, int splits, int chunk, float* part_o,
                                 float* part_l, hipStream_t s) {
  const int BH = a.B * a.H;
  const int nqt = (a.Nq + kFwdBR4 - 1) / kFwdBR4;
  const int nblocks = nqt * BH * splits;
  const float c = a.scale * kLog2e;
  const int off = a.Nk - a.Nq;
  const T* Q = (const T*)a.Q;
  const T* K = (const T*)a.K;
  const T* V = (const T*)a.V;
  const BiasDev nobias = bias_dev(BiasArgs{}, a.B, a.H, 1.f);
  const DropDev nodrop = drop_dev(DropArgs{});
  const SplitDev split{part_o, part_l, splits, chunk, BH * a.Nq};
#define FA_FWD_SPLIT_LAUNCH(DD, CC)                                                           \
  hipLaunchKernelGGL((fwd_kernel<T, DD, CC, false, false, true, 4>), dim3(nblocks),           \
                     dim3(256), 0, s, Q, K, V, (T*)a.O, a.L, a.Nq, a.Nk, nqt, c, off, \
                     nobias, nodrop, split)
  if (a.d == 128) {
    if (a.causal) FA_FWD_SPLIT_LAUNCH(128, true); else FA_FWD_SPLIT_LAUNCH(128, false);
  } else {
    if (a.causal) FA_FWD_SPLIT_LAUNCH(64, true); else FA_FWD_SPLIT_LAUNCH(64, false);
  }
#undef FA_FWD_SPLIT_LAUNCH
  return hipGetLastError();
}

template <typename T>
hipError_t launch_fwd_typed(const FwdArgs& a, hipStream_t s) {
  if (a.drop.on)
    return a.bias.ptr ? launch_fwd_shape<T, true, true>(a, s) : launch_fwd_shape<T, false, true>(a, s);
  return a.bias.ptr ? launch_fwd_shape<T, true, false>(a, s) : launch_fwd_shape<T, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) { return launch_fwd_typed<bf16>(a, s); }
hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t s) { return launch_fwd_typed<f16>(a, s); }

hipError_t launch_fwd_rows_split_bf16(const FwdArgs& a, int splits, int chunk, float* part_o,
                                      float* part_l, hipStream_t s) {
  return launch_fwd_rows_split<bf16>(a, splits, chunk, part_o, part_l, s);
}
hipError_t launch_fwd_rows_split_f16(const FwdArgs& a, int splits, int chunk, float* part_o,
                                     float* part_l, hipStream_t s) {
  return launch_fwd_rows_split<f16>(a, splits, chunk, part_o, part_l, s);
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
  const BiasDev bias = bias_dev(a.bias, a.B, a.H, a.scale);
  const DropDev drop = drop_dev(a.drop);
#define FA_FWD32_LAUNCH(DD, CC)                                                              \
  do {                                                                                       \
    if (a.drop.on)                                                                           \
      hipLaunchKernelGGL((fwd_f32_kernel<DD, CC, true>), dim3(nblocks), dim3(kF32Rows), 0, s, \
                         Q, K, V, O, a.L, a.Nq, a.Nk, nqt, a.scale, off, bias, drop);        \
    else                                                                                     \
      hipLaunchKernelGGL((fwd_f32_kernel<DD, CC, false>), dim3(nblocks), dim3(kF32Rows), 0,   \
                         s, Q, K, V, O, a.L, a.Nq, a.Nk, nqt, a.scale, off, bias, drop);     \
  } while (0)
  if (a.d == 128) {
    if (a.causal) FA_FWD32_LAUNCH(128, true); else FA_FWD32_LAUNCH(128, false);
  } else {
    if (a.causal) FA_FWD32_LAUNCH(64, true); else FA_FWD32_LAUNCH(64, false);
  }
#undef FA_FWD32_LAUNCH
  return hipGetLastError();
}

}  // namespace fa
