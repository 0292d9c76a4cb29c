/*
 * libfa -- fused scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * The operation (FlashAttention, as described on the pages this library is
 * built from):
 *
 *   S = scale * Q K^T  (+ causal mask),   P = softmax(S) row-wise,   O = P V
 *
 * the CSDN post "Flash Attention1" (section "Flash Attention": the three-line
 * formula and the blockwise running-max / running-sum softmax); the 51CTO FlashAttention V1/V2 notes
 * (FlashAttention V1 vs V2 notes, section "FlashAttention V2 相比V1有哪些改进":
 * the forward pass keeps only the row logsumexp L for the backward pass, and
 * causal masking skips the blocks above the diagonal).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are contiguous row-major [B, H, N, d] with d fastest.  Q, O, dO,
 *    dQ are [B, H, Nq, d]; K, V, dK, dV are [B, H, Nk, d].  L is [B, H, Nq]
 *    float32.  Element type of Q, K, V, O, dO, dQ, dK, dV is `dtype`.
 *  - Causal masking keeps key j for query row i iff j <= i + (Nk - Nq)
 *    (bottom-right alignment; the usual lower triangle when Nq == Nk).
 *  - L is the natural-log logsumexp of the scaled, masked score row.
 *  - All pointers are DEVICE pointers on the current HIP device, 16-byte
 *    aligned.  The caller owns every buffer; the library never allocates,
 *    frees or synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL
 *    means the default stream) and is asynchronous.
 *  - Arguments are checked before anything is enqueued; on any error status
 *    nothing is launched and no buffer is written.  FA_ERR_HIP reports a
 *    failed launch (hipGetLastError).  Faults inside a kernel surface at the
 *    caller's next synchronisation, as for any HIP kernel.
 *  - An empty problem (B*H*Nq == 0) returns FA_OK and launches nothing.
 *  - Supported: dtypes FA_BF16 and FA_FP16 with d in {64, 128} for every
 *    entry point (MFMA kernels, fp32 accumulation and statistics); dtype
 *    FA_FP32 with d in {64, 128} for fa_fwd (non-split) and fa_bwd.
 *  - Thread safety: the only global mutable state is fa_bwd_noalloc's scratch
 *    array; other concurrent calls on different streams with disjoint
 *    buffers are safe.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* negative size, Nk == 0 with Nq > 0, causal with Nq > Nk, size overflow */
  FA_ERR_UNSUPPORTED = 3, /* dtype / head dim / option combination not implemented */
  FA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than the query function returns */
  FA_ERR_HIP = 6          /* a kernel launch failed */
} fa_status;

typedef enum fa_dtype { FA_BF16 = 0, FA_FP32 = 1, FA_FP16 = 2 } fa_dtype;

/*
 * Forward pass: O = softmax(scale * Q K^T + mask) V and L = logsumexp of each
 * scaled, masked score row (the CSDN post "Flash Attention1", section "Flash Attention"; the 51CTO FlashAttention V1/V2 notes,
 * "FlashAttention V2 相比V1有哪些改进").
 *
 *  Q [B,H,Nq,d], K and V [B,H,Nk,d] (read); O [B,H,Nq,d] and L [B,H,Nq] fp32
 *  (written, every element).  scale is the score multiplier (usually
 *  1/sqrt(d)); it must be finite and > 0, else FA_ERR_UNSUPPORTED.
 *  causal != 0 applies the mask above.
 *
 *  num_splits chooses the key-split ("Flash-Decoding", the 51CTO FlashAttention
 *  V1/V2 notes, "Sequence Length 并行" and the last paragraph of "Sequence
 *  Parallel") path, available for Nq <= 128 with FA_BF16 or FA_FP16:
 *    0  = automatic: Nq == 1 always splits; 1 < Nq <= 128 splits when the
 *         query tiles alone give few workgroups and the keys are many;
 *         otherwise the tiled path,
 *    1  = tiled path for Nq > 1; for Nq == 1 the split path with one split,
 *    >1 = split path with at most that many key chunks (Nq <= 128, else
 *         FA_ERR_UNSUPPORTED; for Nq > 1 chunks are whole multiples of 128
 *         keys, so fewer may be used, and one chunk means the tiled path).
 *  fa_fwd_num_splits reports the count that will be used.  The split path
 *  needs a workspace of fa_fwd_workspace_size() bytes (fp32 partial outputs
 *  and logsumexps per split and query row); the tiled path needs none (pass
 *  NULL, 0).
 */
fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L,
                 int B, int H, int Nq, int Nk, int d, float scale, int causal,
                 fa_dtype dtype, int num_splits, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Backward pass: dQ, dK, dV of f = sum(dO * O) for the forward above,
 * recomputing P from Q, K and L instead of storing it (the Huawei Cloud post
 * "FlashAttention", section 3, Recomputation; the 51CTO FlashAttention V1/V2
 * notes, "FlashAttention V2相比V1有哪些改进": only L is kept for the backward
 * pass, which also takes the per-row auxiliary D = rowsum(dO * O)).
 *
 *  Q, K, V, O (from fa_fwd), L (from fa_fwd), dO: read.  dQ [B,H,Nq,d],
 *  dK, dV [B,H,Nk,d]: overwritten, every element (not accumulated into).
 *  workspace: fa_bwd_workspace_size() bytes of device memory, 16-byte
 *  aligned, written by the first stage: per head and block of 32 query rows
 *  64 fp32, the rows' L*log2(e) and -D, D = rowsum(dO * O) (rows past Nq
 *  zero), laid out for the kernels that read them (by row pair with dropout,
 *  as two runs of 32 without).  dK and dV are computed per key block by
 *  workgroups that recompute P and dP for their rows.  dQ comes one of two
 *  ways, with no atomic operations either way, so every output is
 *  deterministic:
 *   - stored dS (bf16 and fp16, d = 128, Nq and Nk >= 1024, at least 512
 *     128-key blocks over all heads, B*H*ceil(min(Nq, Nk)/128), or 1024 with
 *     a causal mask, a dS buffer of at most 8 GiB; with or without a bias;
 *     fa_bwd_stores_ds tells): the dK/dV workgroups also
 *     store dS, in a buffer after the per-row block (2 bytes per query-key
 *     pair, padded to 32 x 32 blocks and keys to 256:
 *     B*H*ceil(Nq/32)*ceil(Nk/256)*16 KiB), and a second launch forms
 *     dQ = scale * dS K from it: the five GEMMs per tile pair of the 51CTO
 *     notes ("FlashAttention V2相比V1有哪些改进");
 *   - otherwise, workgroups per query block recompute P and dP for their
 *     rows and accumulate dQ in registers, in one launch with the dK/dV
 *     workgroups (seven GEMMs; faster at d = 64 and on small grids, where
 *     the dQ workgroups run on CUs that the key blocks' chains leave idle).
 */
fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* L,
                 const void* dO, void* dQ, void* dK, void* dV,
                 int B, int H, int Nq, int Nk, int d, float scale, int causal,
                 fa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward pass in stages, for callers that schedule or time them
 * separately.  Same arguments as fa_bwd plus `stages`, a bit mask:
 *   FA_BWD_PREPROCESS (1): L*log2(e) and -D, D = rowsum(dO * O), into the workspace;
 *   FA_BWD_DKDV       (2): dK and dV written (reads the workspace);
 *   FA_BWD_DQ         (4): dQ written (reads the workspace).
 * fa_bwd(...) is fa_bwd_stages(..., FA_BWD_ALL).  Stages 2 and 4 need stage 1
 * to have run on the same workspace, and on the stored-dS path stage 4 reads
 * the dS that stage 2 stored there; a mask of 0 or above 7 returns
 * FA_ERR_UNSUPPORTED.  Stages 2 and 4 in one mask run as one launch (as two
 * with a bias or stored dS); the results are the same bit for bit either way.
 */
enum { FA_BWD_PREPROCESS = 1, FA_BWD_DKDV = 2, FA_BWD_DQ = 4, FA_BWD_ALL = 7 };
fa_status fa_bwd_stages(const void* Q, const void* K, const void* V, const void* O,
                        const float* L, const void* dO, void* dQ, void* dK, void* dV,
                        int B, int H, int Nq, int Nk, int d, float scale, int causal,
                        fa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream,
                        int stages);

/*
 * fa_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments and results as fa_bwd without the workspace.  The per-row
 * L*log2(e) and -D go to a scratch array inside the library instead, one per
 * GPU, of fa_bwd_noalloc_max_rows() rows (16 MiB; held until the process
 * ends).  B*H*ceil(Nq/32)*32 rows (each head's rows padded to a multiple of
 * 32) beyond that return FA_ERR_WORKSPACE before any launch.
 * The first call on a GPU looks up the array's address there; no call
 * allocates or frees memory.  Calls on one GPU share the array, so calls
 * that overlap on one GPU (different streams, or threads) race: serialise
 * them.  Every row the kernels read is written earlier in the same call.
 * dQ is always recomputed (no dS buffer): where fa_bwd takes the stored-dS
 * path, dQ may differ from its result in the last bits (dK and dV do not).
 */
fa_status fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                         const float* L, const void* dO, void* dQ, void* dK, void* dV,
                         int B, int H, int Nq, int Nk, int d, float scale, int causal,
                         fa_dtype dtype, void* stream);

/* Largest B*H*Nq that fa_bwd_noalloc accepts. */
size_t fa_bwd_noalloc_max_rows(void);

/*
 * Forward and backward passes with an additive bias -- the mask term of the
 * method's formula taken in general: O = softmax(scale * Q K^T + bias
 * (+ causal mask)) V (the CSDN post "Flash Attention1", section "Flash
 * Attention", the score line of the formula; the 51CTO FlashAttention V1/V2
 * notes name custom masks among the reasons to write one's own kernel).
 *
 *  bias: element type `dtype` (the same as Q); element (b, h, i, j) is
 *  bias[b*bias_sb + h*bias_sh + i*bias_sq + j].  bias_sb and bias_sh may be 0
 *  to broadcast over batches or heads.  A NULL bias is FA_ERR_NULL; bias_sb,
 *  bias_sh >= 0 and bias_sq >= Nk, else FA_ERR_SHAPE; bias_sb, bias_sh and
 *  bias_sq are multiples of 8 elements and the pointer is 16-byte aligned,
 *  else FA_ERR_ALIGN; (Nq - 1) * bias_sq + Nk <= 2^30, else FA_ERR_SHAPE.
 *  Only entries at rows < Nq and keys < Nk enter the result; the kernels may
 *  also read the rest of a 16-byte aligned block that holds such an entry.
 *  -inf entries remove keys; every score row must keep at least one finite
 *  entry, or that row of O is NaN.  The bias is a constant of the
 *  computation: fa_bwd_bias forms no gradient for it, and fa_bwd_bias must be
 *  given the bias that fa_fwd_bias used (it recomputes P with it).
 *  fa_fwd_bias always takes the tiled path and needs no workspace; the other
 *  arguments, rules and errors are those of fa_fwd and fa_bwd.
 */
fa_status fa_fwd_bias(const void* Q, const void* K, const void* V, const void* bias,
                      long long bias_sb, long long bias_sh, long long bias_sq, void* O, float* L,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal,
                      fa_dtype dtype, void* stream);

fa_status fa_bwd_bias(const void* Q, const void* K, const void* V, const void* bias,
                      long long bias_sb, long long bias_sh, long long bias_sq, const void* O,
                      const float* L, const void* dO, void* dQ, void* dK, void* dV, int B, int H,
                      int Nq, int Nk, int d, float scale, int causal, fa_dtype dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward and backward passes with an optional additive bias (as
 * fa_fwd_bias / fa_bwd_bias take it; bias == NULL: none) and optional
 * dropout on the normalised probabilities, O = (P * Z) V (the 51CTO
 * FlashAttention V1/V2 notes, section "FlashAttention V2 相比 V1 有哪些改进": the
 * V1 algorithm draws dropout on P inside its loop).
 *
 *  dropout_p: probability of dropping a score, 0 <= p < 1 (else
 *  FA_ERR_UNSUPPORTED).  The keep threshold is T = round((1 - p) * 256),
 *  rounded half to even in double precision from the float p; T = 0 is
 *  FA_ERR_UNSUPPORTED and T = 256 (p < 1/512) means no dropout.  A score is
 *  kept iff its random byte is below T, and Z = 256 / T where kept, 0 where
 *  dropped, so E[Z] = 1.  L stays the logsumexp of the scores before
 *  dropout.
 *  Random bytes: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
 *  Random Numbers: As Easy as 1, 2, 3", SC 2011) with key (seed mod 2^32,
 *  seed div 2^32) and counter (j div 4, i div 4, b*H + h, offset) for the
 *  score of query row i and key j of head (b, h); byte j mod 4 of output
 *  word i mod 4 is that score's byte.  A new offset (or seed) gives a new
 *  mask; fa_bwd_ex must be given the dropout_p, seed and offset (and bias)
 *  that fa_fwd_ex used, and regenerates the mask from them.
 *  bias_tile_map: NULL, or the map that fa_bias_tile_map wrote for this
 *  bias and these B, H, Nq, Nk (16-byte aligned; it needs a bias and a
 *  16-bit dtype, else FA_ERR_UNSUPPORTED), in device memory of
 *  bias_tile_map_bytes bytes: fewer than fa_bias_tile_map_size() for these
 *  bias strides and sizes is FA_ERR_WORKSPACE (0 with a NULL map).  The map's
 *  contents are trusted: a map built for another bias gives wrong results
 *  (never an access outside the map or the bias).  With it the kernels skip the
 *  tiles of all -inf entries at the ends of each query tile's key range and
 *  of each key block's query range; the results are the same as without it.
 *  Both always take the tiled path (no key splits; fa_fwd_ex needs no
 *  workspace); the other arguments, rules and errors are those of fa_fwd,
 *  fa_bwd and fa_fwd_bias.
 */
fa_status fa_fwd_ex(const void* Q, const void* K, const void* V, const void* bias,
                    long long bias_sb, long long bias_sh, long long bias_sq,
                    const unsigned char* bias_tile_map, size_t bias_tile_map_bytes,
                    float dropout_p, unsigned long long seed, unsigned int offset, void* O,
                    float* L, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                    fa_dtype dtype, void* stream);

fa_status fa_bwd_ex(const void* Q, const void* K, const void* V, const void* bias,
                    long long bias_sb, long long bias_sh, long long bias_sq,
                    const unsigned char* bias_tile_map, size_t bias_tile_map_bytes,
                    float dropout_p, unsigned long long seed, unsigned int offset,
                    const void* O, const float* L, const void* dO, void* dQ,
                    void* dK, void* dV, int B, int H, int Nq, int Nk, int d, float scale,
                    int causal, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Tile map of an additive bias, for skipping all-masked tiles: one byte per
 * tile of 128 query rows x 64 keys of each bias head, 1 iff the tile holds an
 * entry above -inf (NaN counts as present), else 0.  Layout [Bb][Hb][nqt][nkt4]
 * with Bb = (bias_sb ? B : 1), Hb = (bias_sh ? H : 1), nqt = ceil(Nq / 128),
 * nkt4 = ceil(Nk / 64) rounded up to a multiple of 4 (padding bytes 0).  A
 * block-sparse bias (a band, blocks along the diagonal, key padding) is the
 * intended use: the custom masks the 51CTO FlashAttention V1/V2 notes cite as
 * a reason for one's own kernel.  The kernel reads the bias once; compute the
 * map once per bias and pass it to every fa_fwd_ex / fa_bwd_ex call with it.
 * bias arguments as for fa_fwd_bias; bf16 or fp16 only (FA_ERR_UNSUPPORTED
 * otherwise); tile_map_bytes below fa_bias_tile_map_size: FA_ERR_WORKSPACE.
 */
size_t fa_bias_tile_map_size(long long bias_sb, long long bias_sh, int B, int H, int Nq, int Nk);

fa_status fa_bias_tile_map(const void* bias, long long bias_sb, long long bias_sh,
                           long long bias_sq, int B, int H, int Nq, int Nk, fa_dtype dtype,
                           unsigned char* tile_map, size_t tile_map_bytes, void* stream);

/* Workspace bytes fa_fwd needs for these arguments (0 when none). */
size_t fa_fwd_workspace_size(int B, int H, int Nq, int Nk, int d, fa_dtype dtype, int num_splits);

/* Workspace bytes fa_bwd, fa_bwd_stages, fa_bwd_bias and fa_bwd_ex need for
 * these arguments, causal or not: the per-row block, and the dS buffer where
 * the stored-dS path runs for a non-causal call (see fa_bwd; a causal call
 * with the same sizes uses it or needs less). */
size_t fa_bwd_workspace_size(int B, int H, int Nq, int Nk, int d, fa_dtype dtype);

/* 1 when fa_bwd (and fa_bwd_stages, fa_bwd_bias, fa_bwd_ex) with these
 * arguments stores dS and forms dQ from it, 0 when it recomputes dQ (and for
 * invalid arguments).  fa_bwd_noalloc always recomputes. */
int fa_bwd_stores_ds(int B, int H, int Nq, int Nk, int d, int causal, fa_dtype dtype);

/* Number of key splits fa_fwd uses for these arguments (1 on the tiled path). */
int fa_fwd_num_splits(int B, int H, int Nq, int Nk, int d, fa_dtype dtype, int num_splits);

/* Static, human-readable name of a status code. */
const char* fa_status_string(fa_status s);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
