/*
 * fa_bwd.h: C ABI of the backward pass of the gfx950 FlashAttention-2 library
 * (same shared library and status codes as fa_fwd.h).
 *
 * Given the forward's inputs q, k, v, its output out and log-sum-exp lse, and
 * the gradient dout of a scalar loss with respect to out, computes the
 * gradients of that loss with respect to q, k and v for the attention of
 * fa_fwd (square heads, optional causal mask):
 *
 *   P  = exp(scale * q k^T - lse)           (row i over the keys A(i))
 *   dv = P^T dout,   dP = dout v^T,   D_i = sum_c dout[i,c] * out[i,c],
 *   dS = P o (dP - D),   dq = scale * dS k,   dk = scale * dS^T q.
 *
 * This is the chain rule through the softmax that FlashAttention's backward
 * applies, rebuilding P tile by tile from the saved per-row statistic instead
 * of storing the N x N matrix ("FlashAttention and kernels", gtadkapally.com,
 * section "The backward pass: recompute instead of remember"; D is the per-row
 * correction term of the softmax Jacobian).  No atomics are used; results are
 * deterministic.
 */
#ifndef FA_BWD_H
#define FA_BWD_H

#include "fa_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_bwd_workspace_bytes: bytes of device workspace fa_bwd needs for these
 * sizes (8 * B * H * N: D and lse * log2(e), fp32 per query row), or a negative
 * fa_status for invalid sizes.
 */
long long fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_bwd: enqueue the attention backward pass on `stream` (three kernels).
 *
 *   q, k, v     device pointers, bfloat16, contiguous [B, H, N, d] (as fa_fwd).
 *   out, lse    the forward's outputs for these q, k, v, scale and causal flag:
 *               bfloat16 [B, H, N, d] and float32 [B, H, N].  Read only.
 *   dout        device pointer, bfloat16 [B, H, N, d]: d loss / d out.  Read only.
 *   dq, dk, dv  device pointers, bfloat16 [B, H, N, d].  Written; every element.
 *   B, H, N, scale, causal   as for fa_fwd; d is 32, 64 or 128 (the backward
 *               holds a wavefront's dK and dV rows in registers, which d = 256
 *               would overflow; FA_ERR_HEAD_DIM).
 *   workspace   device memory of at least fa_bwd_workspace_bytes(B, H, N, d)
 *               bytes, 256-byte aligned, owned by the caller; its contents on
 *               entry are ignored and on return are unspecified.  Calls that
 *               share a workspace must be ordered (one stream).
 *   stream      hipStream_t as void* (NULL = default stream).
 *
 * Errors (checked on the host, in this order, before any launch; on an error
 * nothing is written): FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEAD_DIM,
 * FA_ERR_SCALE, FA_ERR_ARG (causal not 0/1), FA_ERR_ALIGN (tensors not 16-byte
 * aligned, lse not 4-byte), FA_ERR_WORKSPACE (too small or not 256-byte
 * aligned), FA_ERR_ALIAS (dq, dk, dv or the workspace overlap one another or
 * any input; the inputs may overlap each other), FA_ERR_NO_DEVICE,
 * FA_ERR_LAUNCH.  Asynchronous like fa_fwd.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* workspace,
           long long workspace_bytes, void* stream);

/*
 * General layouts, lengths and fp16: the operation of fa_bwd on tensors
 * addressed by element strides (the head dimension contiguous), in bfloat16 or
 * IEEE fp16, for N query rows over Nk key rows per head.  The formulas are
 * those of fa_bwd; the mask is fa_fwd_ex's: A(i) = all Nk keys, or when causal
 * {j < Nk : j <= i} (top-left alignment; with N < Nk the keys j >= N are seen by
 * no query and get dk = dv = 0).  out and lse must be fa_fwd_ex's outputs for
 * the same lengths, scale and mask.
 *
 *   q, out, dout         read only, i < N rows per head; element (b, h, i, c)
 *                        of q at
 *                        q[b*q_stride[0] + h*q_stride[1] + i*q_stride[2] + c],
 *                        and likewise for each tensor with its own strides.
 *                        A [B, N, H, d] tensor has strides {N*H*d, d, H*d}.
 *   k, v                 read only, Nk rows per head, addressed the same way.
 *   lse                  fp32, element (b, h, i) at
 *                        lse[b*lse_stride[0] + h*lse_stride[1] + i].  Read only.
 *   dq                   written, N rows per head; dk, dv written, Nk rows;
 *                        every element, with their own strides.
 *   Nk                   key rows per head; 0 means Nk = N (so a zero-
 *                        initialised descriptor keeps square heads).
 *   dtype                FA_DTYPE_BF16 (0) or FA_DTYPE_F16 for all nine 16-bit
 *                        tensors alike (else FA_ERR_ARG); products accumulate in
 *                        fp32 and P, dS enter the matrix instruction in dtype.
 *                        fp16 inputs must be finite.
 *   workspace            as for fa_bwd (fa_bwd_workspace_bytes(B, H, N, d)).
 * Stride rules (else FA_ERR_STRIDE): those of fa_fwd_desc for 16-bit
 * elements: every stride >= 0 and a multiple of 8 elements, every row stride
 * >= d, (rows + 256) * row stride < 2^30 with each tensor's own row count; lse
 * strides >= 0.  The workspace is sized by the query rows:
 * fa_bwd_workspace_bytes(B, H, N, d).
 * Errors, in this order: FA_ERR_NULL (desc or a pointer), FA_ERR_SHAPE (B, H,
 * N or Nk < 1, or B*H*max(N, Nk) >= 2^31), FA_ERR_HEAD_DIM, FA_ERR_STRIDE, FA_ERR_SCALE,
 * FA_ERR_ARG (causal, dtype), FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_ALIAS,
 * FA_ERR_NO_DEVICE, FA_ERR_LAUNCH.
 * Aliasing (FA_ERR_ALIAS): dq, dk, dv and the workspace must not overlap one
 * another or any input.  Two tensors overlap when their byte extents meet,
 * unless both are views with one row stride rs, batch strides that are
 * multiples of rs and all heads of a row within rs bytes, whose base addresses
 * modulo rs start intervals (of the row's span) that do not meet: then their
 * bytes are provably disjoint -- dq, dk, dv interleaved in one packed
 * [B, N, 3, H, d] buffer, for instance.  And dq, dk, dv must not overlap
 * themselves: with the dimensions ordered by stride, each stride at least the
 * span of the smaller ones (size-1 dimensions aside).  So a zero head stride,
 * e.g. for keys shared by several query heads, is refused for dk and dv: such
 * gradients must be summed, which the caller does over per-head buffers.  When every tensor is contiguous [B, H, N, d] (lse [B, H, N])
 * the call runs the same kernels as fa_bwd, with identical results for bf16.
 */
typedef struct fa_bwd_desc {
  const void *q, *k, *v, *out;
  const float *lse;
  const void *dout;
  void *dq, *dk, *dv;
  int B, H, N, d;
  long long q_stride[3], k_stride[3], v_stride[3], o_stride[3], do_stride[3];
  long long dq_stride[3], dk_stride[3], dv_stride[3];
  long long lse_stride[2];
  float scale;
  int causal;
  int dtype;
  void *workspace;
  long long workspace_bytes;
  void *stream;
  int Nk;
} fa_bwd_desc;

int fa_bwd_ex(const fa_bwd_desc *desc);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H */
