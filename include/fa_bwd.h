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
 *   B, H, N, d, scale, causal   as for fa_fwd.
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

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H */
