// FlashAttention-2 forward for fp32 inputs and outputs on gfx950: the same
// algorithm as fa_fwd_kernel (one workgroup per query tile, K/V tiles through a
// double-buffered LDS ring, online softmax with a lazy reference maximum,
// causal skipping), on the fp32 matrix instruction v_mfma_f32_32x32x2_f32.
//
// Operand mapping (32x32x2: a lane holds ONE element of each operand; lane half
// g = lane / 32 supplies k index g):
// * S^T = K Q^T: MFMA step (j, e) pairs head-dim columns 8j + e (half 0) and
//   8j + 4 + e (half 1).  A lane reads the four columns 8j + 4g .. 8j + 4g + 3 of
//   its key row with one ds_read_b128 and feeds them to four steps; Q sits in
//   VGPRs in the same order (D/2 floats per lane).  The K tile keeps the 16-byte
//   XOR swizzle of the 16-bit kernels (rows of 4D bytes), which keeps these
//   reads of 16 rows x one chunk on distinct banks.
// * O^T += V^T P^T: the S^T fragment gives lane half g the keys
//   8(r/4) + 4g + r%4 in register r, so step r pairs keys 8(r/4) + r%4 and
//   that + 4, and the B operand is the lane's own P register r.  The A operand
//   is V[key][c] for the lane's column c: one ds_read_b32 per step from an
//   unswizzled V tile (the two lane halves read two rows: at most a 2-way bank
//   conflict, and every address is a per-lane base plus an immediate).
// P is never rounded: the product runs at fp32 throughout.
#pragma once
#include "fa_fwd_kernel.hpp"

namespace fa {

template <int D, bool CAUSAL, int WAVES, int BK, bool STRIDED>
__global__ __launch_bounds__(WAVES * 64) void fa_fwd_f32_kernel(const Params pr) {
  static_assert(D == 64 || D == 128, "fp32 head dim");
  static_assert(BK == 32 || BK == 64, "key tile");
  constexpr int kRowBytes = D * 4;
  constexpr int kSw = 2 * D;                    // swz<kSw> / lds_offset<kSw> address rows of 4D bytes
  constexpr int kTileBytes = BK * kRowBytes;    // one K or V tile
  constexpr int kStageBytes = 2 * kTileBytes;   // K then V
  constexpr int kBlocks = kTileBytes / 1024;
  constexpr int kBlocksPerWave = (kBlocks + WAVES - 1) / WAVES;
  constexpr int kBQ = WAVES * 32;
  static_assert(kTileBytes % 1024 == 0 && 2 * kStageBytes <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char lds0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kStageBytes];

  const int BH = pr.BH, Nq = pr.Nq, Nk = pr.Nk, nqt = pr.nqt;
  const float qk_scale = pr.qk_scale;
  const int q_rs = STRIDED ? pr.q_rs : D, k_rs = STRIDED ? pr.k_rs : D;
  const int v_rs = STRIDED ? pr.v_rs : D, o_rs = STRIDED ? pr.o_rs : D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, lr = lane & 31;

  // ---- (head, query tile), as in fa_fwd_kernel --------------------------------
  const int total = (int)gridDim.x, i = (int)blockIdx.x;
  const bool xcd = (BH % 8) == 0;
  const int t = xcd ? (i & 7) * (total >> 3) + (i >> 3) : i;
  int bh, qt;
  if (CAUSAL) {
    if (xcd) {
      const int per = total >> 3, hpx = BH >> 3;
      const int chunk = t / per, j = t - chunk * per;
      bh = chunk * hpx + j % hpx;
      qt = nqt - 1 - j / hpx;
    } else {
      bh = t % BH;
      qt = nqt - 1 - t / BH;
    }
  } else {
    bh = t / nqt;
    qt = t - bh * nqt;
  }
  const int batch = bh / pr.H, hd = bh - batch * pr.H;
  const float* qp = reinterpret_cast<const float*>(pr.q);
  const float* kp = reinterpret_cast<const float*>(pr.k);
  const float* vp = reinterpret_cast<const float*>(pr.v);
  const long long q_off = STRIDED ? batch * pr.q_sb + hd * pr.q_sh : (long long)bh * Nq * D;
  const long long k_off = STRIDED ? batch * pr.k_sb + hd * pr.k_sh : (long long)bh * Nk * D;
  const long long v_off = STRIDED ? batch * pr.v_sb + hd * pr.v_sh : (long long)bh * Nk * D;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qp + q_off, (uint32_t)((Nq - 1) * q_rs + D) * 4);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp + k_off, (uint32_t)((Nk - 1) * k_rs + D) * 4);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp + v_off, (uint32_t)((Nk - 1) * v_rs + D) * 4);
  const int q0 = qt * kBQ;
  const int qw = q0 + wave * 32;
  const int query = qw + lr;

  // ---- Q row -> VGPRs: qreg[j] = columns 8j + 4g .. 8j + 4g + 3 ----------------
  f32x4 qreg[D / 8];
#pragma unroll
  for (int j = 0; j < D / 8; ++j) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(qrs, (query * q_rs + 8 * j + 4 * g) * 4, 0, 0);
    qreg[j] = __builtin_bit_cast(f32x4, x);
  }

  // ---- per-lane LDS offsets ------------------------------------------------------
  uint32_t dma_k[kBlocksPerWave], dma_v[kBlocksPerWave];
#pragma unroll
  for (int n = 0; n < kBlocksPerWave; ++n) {
    const int p = (wave + WAVES * n) * 64 + lane;
    const int row = p / (D / 4), pos = p % (D / 4);  // 16-byte chunk pos of row
    dma_k[n] = row * k_rs * 4 + ((pos ^ swz<kSw>(row)) << 4);
    dma_v[n] = row * v_rs * 4 + (pos << 4);
  }
  int koff[D / 8];  // K row lr, chunk 2j + g
#pragma unroll
  for (int j = 0; j < D / 8; ++j) koff[j] = lds_offset<kSw>(lr, 2 * j + g);
  const int vbase = 4 * g * kRowBytes + lr * 4;  // V row 4g, column lr

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -__builtin_inff(), l = 0.f;

  const int kend = CAUSAL ? min(q0 + kBQ, Nk) : Nk;
  const int ntiles = (kend + BK - 1) / BK;

  auto issue_tile = [&](int j, int stage) {
    const uint32_t gk = (uint32_t)(j * BK) * k_rs * 4, gv = (uint32_t)(j * BK) * v_rs * 4;
#pragma unroll
    for (int n = 0; n < kBlocksPerWave; ++n) {
      const int b = wave + WAVES * n;
      if (kBlocks % WAVES == 0 || b < kBlocks) {
        char* kdst = (stage ? lds1 : lds0) + b * 1024;
        dma16(krs, kdst, dma_k[n] + gk);
        dma16(vrs, kdst + kTileBytes, dma_v[n] + gv);
      }
    }
  };

  auto compute_tile = [&](const char* kst, int k0, bool masked) {
    const char* vst = kst + kTileBytes;
    // ---- S^T = K Q^T (lane = query, 16 keys per 32-key block) -------------------
    f32x16 s[BK / 32];
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int j = 0; j < D / 8; ++j) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(kst + kb * 32 * kRowBytes + koff[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qreg[j][e], s[kb], 0, 0, 0);
      }
    }
    // ---- mask, online softmax (lazy reference maximum) ----------------------------
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if ((CAUSAL && key > query) || key >= Nk) s[kb][r] = -__builtin_inff();
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = lane_swap_max(mx);
    const float mt = mx * qk_scale;
    const float m_new = (mt > m + kLazyMax) ? mt : m;
    const float m_sub = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_sub);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], qk_scale, -m_sub));
        s[kb][r] = e;
        rs += e;
      }
    l = fmaf(alpha, l, rs);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    // ---- O^T += V^T P^T -------------------------------------------------------------
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = kb * 32 + 8 * (r >> 2) + (r & 3);  // + 4g in vbase
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const float a = *reinterpret_cast<const float*>(vst + vbase + row * kRowBytes + db * 128);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][r], oacc[db], 0, 0, 0);
        }
      }
  };

  auto step = [&](int j, int stage) {
    if (j + 1 < ntiles) issue_tile(j + 1, stage ^ 1);
    const int k0 = j * BK;
    const bool skip = CAUSAL && (k0 > qw + 31);
    const bool masked = (CAUSAL && (k0 + BK - 1 > qw)) || (k0 + BK > Nk);
    if (!skip) compute_tile(stage ? lds1 : lds0, k0, masked);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
  };

  issue_tile(0, 0);  // ntiles >= 1: q0 < Nq and Nk >= 1
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(j, 0);
    step(j + 1, 1);
  }
  if (j < ntiles) step(j, 0);

  // ---- epilogue: O / l (fp32), LSE = (m + log2 l) ln 2 ------------------------------
  const float lt = lane_swap_sum(l);
  const float inv = 1.0f / lt;
  if (query < Nq) {
    const long long o_off = STRIDED ? batch * pr.o_sb + hd * pr.o_sh : (long long)bh * Nq * D;
    float* orow = reinterpret_cast<float*>(pr.out) + o_off + (long long)query * o_rs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x4 w = {oacc[db][4 * rr + 0] * inv, oacc[db][4 * rr + 1] * inv, oacc[db][4 * rr + 2] * inv,
                         oacc[db][4 * rr + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * rr + 4 * g) = w;
      }
    const long long l_off = STRIDED ? batch * pr.l_sb + hd * pr.l_sh : (long long)bh * Nq;
    if (g == 0) pr.lse[l_off + query] = (m + log2f(lt)) * kLn2;
  }
}

}  // namespace fa
