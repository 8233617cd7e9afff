/*
 * fa_fwd.h: C ABI of the MI355X (gfx950) FlashAttention-2 forward library.
 *
 * The operation is exact scaled-dot-product attention, for every batch b, head
 * h and query position i (square: N queries attend over N keys):
 *
 *   out[b,h,i,:] = sum_{j in A(i)} softmax_j(scale * q_i . k_j) * v_j
 *   lse[b,h,i]   = ln sum_{j in A(i)} exp(scale * q_i . k_j)
 *
 * with A(i) = {0 .. N-1}, or {0 .. i} when causal (a token attends to itself and
 * to earlier tokens only).  This is the attention rule of "4 Triton and Custom
 * Kernels" (aisyseng.dev), section 4.7, equation 4.1, with an explicit scale;
 * the log-sum-exp side output is the one FlashAttention's forward pass stores
 * per query row ("FlashAttention and kernels", gtadkapally.com, section
 * "FlashAttention's forward pass", step 4): the natural log of the softmax
 * denominator of the scaled scores.  It is computed one key tile at a time with
 * the online-softmax recurrence (same page, "From a sum to an output row"),
 * so the N x N score matrix never reaches device memory.
 *
 * Plain C99; no HIP or torch types.  Link against libfa_fwd.so.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  Every argument check happens on the host before any HIP call,
 * so on an error nothing is launched and out/lse are untouched. */
enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,       /* a pointer argument is NULL                            */
  FA_ERR_SHAPE = 2,      /* B, H or N < 1, or the sizes overflow the index range  */
  FA_ERR_HEAD_DIM = 3,   /* d is not 32, 64, 128 or 256                           */
  FA_ERR_SCALE = 4,      /* scale is not finite and > 0                           */
  FA_ERR_ARG = 5,        /* causal not 0/1, unknown dtype, or a tile configuration
                            that is not compiled in                               */
  FA_ERR_ALIGN = 6,      /* q, k, v, out not 16-byte aligned, or lse not 4-byte   */
  FA_ERR_ALIAS = 7,      /* out or lse overlaps q, k, v or each other             */
  FA_ERR_NO_DEVICE = 8,  /* no current HIP device, or it is not gfx950            */
  FA_ERR_LAUNCH = 9,     /* the kernel launch was rejected by the HIP runtime     */
  FA_ERR_INTERNAL = 10,  /* anything else (no C++ exception crosses this ABI)     */
  FA_ERR_STRIDE = 11,    /* a stride is negative, misaligned, smaller than a row, or
                            puts a head beyond the 32-bit addressing of one head  */
  FA_ERR_WORKSPACE = 12, /* split-key workspace missing, misaligned or too small   */
  FA_ERR_SCRATCH = 13    /* fa_fwd_splitkv_noalloc: the partial results need more
                            than FA_SPLITKV_NOALLOC_MAX_BYTES                     */
};

/*
 * fa_fwd: enqueue the attention forward pass on `stream`.
 *
 *   q, k, v  device pointers, bfloat16 bit patterns, contiguous [B, H, N, d]:
 *            element (b, h, i, c) at index ((b*H + h)*N + i)*d + c.  Read only.
 *   out      device pointer, bfloat16, contiguous [B, H, N, d].  Written.
 *   lse      device pointer, float32, contiguous [B, H, N]: the natural-log
 *            log-sum-exp of each query row's scaled scores.  Written.
 *   B, H, N  batch, heads, sequence length (>= 1); B*H*N*d must stay below
 *            2^31 elements per tensor and (N + 256)*d below 2^30, so that one
 *            head's bytes stay within the 32-bit offsets of a buffer resource
 *            (else FA_ERR_SHAPE).
 *   d        head dimension: 32, 64, 128 or 256.
 *   scale    softmax scale applied to q.k (typically 1/sqrt(d)); finite, > 0
 *            (the running maximum is kept in scaled units, which needs scale > 0).
 *   causal   0: every key is visible; 1: key j is visible to query i iff j <= i.
 *   stream   a hipStream_t handle, or NULL for the null stream.
 *
 * Ownership: the caller allocates and owns every buffer, on the current HIP
 * device; the library allocates no device memory, keeps no pointer after the
 * call returns and holds no state beyond a per-device property cache.
 * Asynchrony: on FA_OK the kernel is queued and the call returns without
 * synchronising; results are valid once the stream has been synchronised, and
 * a device fault surfaces at that synchronisation.  Results are bit-identical
 * from run to run (no atomics, fixed reduction order).
 */
int fa_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
           int B, int H, int N, int d, float scale, int causal, void *stream);

/* Tile configuration of one compiled kernel variant:
 *   qb      32-query column blocks owned by each 64-lane wavefront (1 or 2);
 *   waves   wavefronts per workgroup;
 *   bk      keys per K/V tile staged through LDS;
 *   ksplit  0 or 1: each wavefront owns its queries (the workgroup owns
 *           waves*qb*32 of them); 4 (with qb 1, waves 4, bk 32): the four
 *           wavefronts share one block of 32 queries, wavefront w sweeps key
 *           tiles w, w+4, w+8, ..., and their partial softmax states are merged
 *           at the end of the workgroup (Flash-Decoding's split of the keys, "FlashAttention
 *           and kernels", "FlashAttention-2, -3, and what came after").  Values
 *           returned by the library set 1 for the former.
 * (Since version 600 the struct has four members; earlier versions had three.) */
typedef struct fa_tile_cfg {
  int qb;
  int waves;
  int bk;
  int ksplit;
} fa_tile_cfg;

/* fa_fwd with an explicit tile configuration (for measurements and sweeps).
 * Same arguments and contract as fa_fwd; returns FA_ERR_ARG if `cfg` is NULL or
 * names a variant that is not compiled in. */
int fa_fwd_cfg(const void *q, const void *k, const void *v, void *out, float *lse,
               int B, int H, int N, int d, float scale, int causal, void *stream,
               const fa_tile_cfg *cfg);

/*
 * General layouts and lengths: N_q query rows attend over N_k key rows, and
 * every tensor is addressed by element strides.  Same operation as fa_fwd with
 * A(i) = {0 .. N_k-1}, or, when causal, {j < N_k : j <= i}: the top-left
 * alignment of the causal mask, under which every query row sees at least key
 * 0 (the convention a non-square causal check uses in "How to profile and
 * optimise kernels", dev.to, Round 4, causal tile-skipping; N_QUERIES and
 * N_KEYS are separate lengths in "FlashAttention 2 from PyTorch to Triton").
 *
 *   q    16-bit elements of type `dtype`, element (b, h, i, c) at
 *        q[b*q_stride[0] + h*q_stride[1] + i*q_stride[2] + c],
 *        i < Nq;  k, v likewise with i < Nk;  out like q.  The head dimension is
 *        contiguous.  A [B, N, H, d] tensor has strides {N*H*d, d, H*d}.
 *   lse  fp32, element (b, h, i) at lse[b*lse_stride[0] + h*lse_stride[1] + i].
 *
 * Stride rules (else FA_ERR_STRIDE): every stride >= 0 and a multiple of 8
 * elements (16 bytes), every row stride >= d, and (N + 256) * row stride < 2^30
 * for each tensor's own N, so that one head stays within 32-bit byte offsets.
 * lse strides >= 0.  Pointers: q, k, v, out 16-byte aligned, lse 4-byte.
 * dtype: FA_DTYPE_BF16 (0, so a zero-initialised descriptor means bfloat16),
 * FA_DTYPE_F16 (IEEE binary16) or FA_DTYPE_F32 (IEEE binary32) for q, k, v and
 * out alike; scores, the softmax statistics and the accumulators are fp32 in
 * every case and lse is fp32.  fp16 inputs must be finite (|x| <= 65504).
 * FA_DTYPE_F32 runs on the fp32 matrix instruction (P stays fp32) for d = 64
 * or 128 (else FA_ERR_HEAD_DIM) and is not available to fa_fwd_splitkv
 * (FA_ERR_ARG).  Strides are in elements of the chosen type; the rules below
 * read "multiple of 16 bytes" for "multiple of 8 elements" and apply the 2^30
 * bound to bytes / 2.
 * Aliasing (FA_ERR_ALIAS) is judged on each tensor's whole byte extent: out
 * and lse must not overlap q, k, v or each other (inputs may overlap each
 * other, e.g. three views of one packed QKV tensor, or k, v with head stride
 * 0 shared by every query head); and out and lse must not overlap themselves
 * (with its dimensions ordered by stride, each stride at least the span of the
 * smaller ones, size-1 dimensions aside), so that no element is written twice.
 * Other arguments, ownership, asynchrony and determinism as for fa_fwd.
 */
typedef struct fa_fwd_desc {
  const void *q, *k, *v;
  void *out;
  float *lse;
  int B, H, Nq, Nk, d;
  long long q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  long long lse_stride[2];
  float scale;
  int causal;
  void *stream;
  int dtype;
} fa_fwd_desc;

/* Element types of fa_fwd_desc.dtype. */
enum fa_dtype { FA_DTYPE_BF16 = 0, FA_DTYPE_F16 = 1, FA_DTYPE_F32 = 2 };

int fa_fwd_ex(const fa_fwd_desc *desc);

/* fa_fwd_ex with an explicit tile configuration (FA_ERR_ARG if NULL or not compiled in). */
int fa_fwd_ex_cfg(const fa_fwd_desc *desc, const fa_tile_cfg *cfg);

/*
 * Split keys (Flash-Decoding): the same operation as fa_fwd_ex, computed by
 * splitting each head's keys into S contiguous ranges of whole 64-key tiles;
 * one pass produces every range's normalised partial output and log-sum-exp,
 * and a second kernel merges them per query row with the rule that combines
 * two partial (m, l, o) states ("FlashAttention and kernels", gtadkapally.com:
 * the online max/sum exercise with its merge of partial states, and the
 * Flash-Decoding paragraph of "FlashAttention-2, -3, and what came after").
 * It fills the GPU when B*H*ceil(Nq/256) is small (short prompts, decoding with
 * few query rows); results agree with fa_fwd_ex to rounding.
 *
 *   num_splits  requested S (1..1024), or 0 for fa_splitkv_default_splits; the
 *               number used is ceil(Nk / chunk) with chunk = ceil(Nk / S)
 *               rounded up to a multiple of 64 keys.
 *   workspace   caller-owned device memory, 256-byte aligned, at least
 *               fa_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits) bytes;
 *               scratch: its contents on entry are ignored and on return are
 *               unspecified.  It must not overlap any tensor (FA_ERR_ALIAS), and
 *               two calls in flight must not share it.
 * Errors: as fa_fwd_ex, plus FA_ERR_WORKSPACE, and FA_ERR_ARG for num_splits
 * outside 0..1024.  Two kernels are enqueued on desc->stream.
 */
int fa_fwd_splitkv(const fa_fwd_desc *desc, int num_splits, void *workspace, long long workspace_bytes);

/*
 * fa_fwd_splitkv without an allocation, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same operation, arguments (minus
 * the workspace), kernels and results as fa_fwd_splitkv; the partial results
 * go to a static device array inside the library instead, one per GPU, held
 * from the first call on that GPU until the process ends.  Up to
 * FA_SPLITKV_NOALLOC_MAX_BYTES of it is used: a call whose
 * fa_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits) exceeds that returns
 * FA_ERR_SCRATCH and launches nothing.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); the first call on a GPU
 * looks up the array's device address.  Every call on one GPU shares that
 * GPU's array: two calls that may run at the same time on one GPU (different
 * streams, or different host threads) race and give undefined results; calls
 * ordered on one stream do not.  Nothing in the array needs to start at zero
 * (every partial result the merge reads is written by the same call).
 */
#define FA_SPLITKV_NOALLOC_MAX_BYTES (32LL << 20)
int fa_fwd_splitkv_noalloc(const fa_fwd_desc *desc, int num_splits);

/* Workspace bytes for fa_fwd_splitkv (>= 0), or minus an error code. */
long long fa_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits);

/* The split count fa_fwd_splitkv uses for num_splits = 0 (>= 1), or minus an
 * error code.  The split path runs the key-split tile (one block of 32 queries,
 * four wavefronts splitting each split's keys again) when Nq <= 32 and d <= 128,
 * with about 256 workgroups and at least 512 keys per split; 128-query
 * workgroups when Nq <= 128 (d <= 128), else fa_fwd's tile, with about 512
 * workgroups and at least 256 keys per split. */
int fa_splitkv_default_splits(int B, int H, int Nq, int Nk, int d, int causal);

/* The configuration for (N, d, causal) on a grid that gives every compute unit
 * a workgroup; FA_OK or an error code.  (Host only; no device needed.) */
int fa_default_cfg(int N, int d, int causal, fa_tile_cfg *cfg);

/* The configuration fa_fwd and fa_fwd_ex pick for these sizes and element type
 * on the current device.  d = 256 and fp32 keep fa_default_cfg's 4-wavefront
 * tile.  At d = 32, 64 or 128 (bf16 or fp16), with w8 = B*H*ceil(Nq/256)
 * workgroups of (1, 8, 64) and w4 = B*H*ceil(Nq/128) of (1, 4, 64):
 * - non-causal: the key-split tile (1, 4, 32, ksplit 4) while 2*w4 <= CUs
 *   (d = 128: and 4*w4 <= CUs or Nq >= 1024); (1, 4, 64) while w4 <= CUs
 *   (d = 32: while w8 <= CUs); beyond, of
 *   (1, 8, 64), (1, 8, 32) and (1, 12, 64) (d = 64 only) and (1, 4, 64) the
 *   tile that leaves the busiest compute unit the least work: ceil(workgroups
 *   / CUs) * waves, weighed by the tile's measured speed (8 waves 1.000, 12
 *   waves 0.975, 4 waves 1.025 at d = 32, 1.030 at d = 64 and 1.050 at
 *   d = 128; (1, 8, 32), whose workgroups run two per CU, 0.970 when the grid
 *   has more workgroups than CUs, else 1.075); ties keep (1, 8, 64);
 * - causal: the key-split tile while w8 < CUs (d = 128: while w4 < CUs, or
 *   w4 = CUs with Nq >= 2048; d = 32: while w8 <= 1.5 CUs); beyond, the launch
 *   orders of (1, 8, 64) and (1, 4, 64) are replayed on the host (up to 16
 *   layers of CUs; past that both count as even) and their balance (mean over
 *   largest per-CU tile count) compared: (1, 8, 64) if its balance is above
 *   (1, 4, 64)'s; else (1, 4, 64) if the balance of (1, 8, 64) is below 0.97;
 *   else (both even) (1, 4, 64) from 4 layers of CUs on at d = 64, and at
 *   d = 32 for Nq <= 4096, and (1, 8, 64) otherwise.  The last few answers are
 *   remembered per host thread.
 * FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEAD_DIM, FA_ERR_ARG (causal, dtype)
 * or FA_ERR_NO_DEVICE. */
int fa_launch_cfg(int B, int H, int Nq, int d, int causal, int dtype, fa_tile_cfg *cfg);

/* Number of compiled variants, the i-th one (for d, causal given), and its
 * element type (an fa_dtype, or minus an error code).  fa_fwd and fa_fwd_cfg
 * use the bfloat16 variants; fa_fwd_ex and fa_fwd_ex_cfg pick by desc->dtype. */
int fa_num_variants(void);
int fa_variant(int i, int *d, int *causal, fa_tile_cfg *cfg);
int fa_variant_dtype(int i);

/* Static text for a status code. */
const char *fa_strerror(int status);

/* Library version, major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
