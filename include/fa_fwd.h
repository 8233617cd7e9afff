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
  FA_ERR_HEAD_DIM = 3,   /* d is not 64 or 128                                    */
  FA_ERR_SCALE = 4,      /* scale is not finite and > 0                           */
  FA_ERR_ARG = 5,        /* causal not 0/1, or an unknown tile configuration       */
  FA_ERR_ALIGN = 6,      /* q, k, v, out not 16-byte aligned, or lse not 4-byte   */
  FA_ERR_ALIAS = 7,      /* out or lse overlaps q, k, v or each other             */
  FA_ERR_NO_DEVICE = 8,  /* no current HIP device, or it is not gfx950            */
  FA_ERR_LAUNCH = 9,     /* the kernel launch was rejected by the HIP runtime     */
  FA_ERR_INTERNAL = 10   /* anything else (no C++ exception crosses this ABI)     */
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
 *            2^31 elements per tensor and N*d below 2^31.
 *   d        head dimension: 64 or 128.
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
 *   qb     32-query column blocks owned by each 64-lane wavefront (1 or 2);
 *   waves  wavefronts per workgroup (the workgroup owns waves*qb*32 queries);
 *   bk     keys per K/V tile staged through LDS. */
typedef struct fa_tile_cfg {
  int qb;
  int waves;
  int bk;
} fa_tile_cfg;

/* fa_fwd with an explicit tile configuration (for measurements and sweeps).
 * Same arguments and contract as fa_fwd; returns FA_ERR_ARG if `cfg` is NULL or
 * names a variant that is not compiled in. */
int fa_fwd_cfg(const void *q, const void *k, const void *v, void *out, float *lse,
               int B, int H, int N, int d, float scale, int causal, void *stream,
               const fa_tile_cfg *cfg);

/* The configuration fa_fwd picks for (N, d, causal); FA_OK or an error code. */
int fa_default_cfg(int N, int d, int causal, fa_tile_cfg *cfg);

/* Number of compiled variants, and the i-th one (for d, causal given). */
int fa_num_variants(void);
int fa_variant(int i, int *d, int *causal, fa_tile_cfg *cfg);

/* Static text for a status code. */
const char *fa_strerror(int status);

/* Library version, major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
