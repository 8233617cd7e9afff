// FlashAttention-2 forward for gfx950 (CDNA4), hand-written HIP.
//
// One workgroup owns a tile of BQ = WAVES*QB*32 query rows of one (batch, head);
// each 64-lane wavefront owns QB blocks of 32 whole query rows, so row
// statistics never cross wavefronts (the FA-2 split of queries, not keys, across
// the warps of a program: "FlashAttention and kernels", gtadkapally.com, section
// "FlashAttention-2, -3, and what came after").  The workgroup sweeps the keys
// in tiles of BK, staging K and V through a double-buffered LDS ring, and folds
// every tile into per-row running state with the online-softmax update (same
// page, "From a sum to an output row"; "4 Triton and Custom Kernels",
// section 4.8, the four-step update):
//
//   m_new = max(m, rowmax(S)),  alpha = exp(m - m_new),
//   l     = alpha*l + rowsum(exp(S - m_new)),  O = alpha*O + exp(S - m_new) V.
//
// Scores stay in registers; the N x N matrix never reaches HBM.
//
// Layout choices (gfx950 MFMA, v_mfma_f32_32x32x16_bf16):
// * S^T = K Q^T: the A operand is a K row segment (16 contiguous bytes of a key,
//   read from LDS), the B operand a Q row segment held in VGPRs for the whole
//   sweep.  The 32x32 fp32 result gives each lane ONE query (lane % 32) and 16
//   keys, so the row max and row sum are in-lane reductions plus one
//   v_permlane32_swap between the two lane halves.
// * O^T += V^T P^T: the probabilities of a lane's query, packed to bf16, are
//   already laid out as the B operand; V enters as the A operand from a V^T copy
//   in LDS (transposed while being staged), whose key order inside each 16-key
//   step matches the order in which the S^T accumulator holds the keys.  The
//   alpha rescale of O is a per-lane scalar multiply.
// * Scores are kept raw; the softmax scale and log2(e) are folded into one
//   multiply-add before v_exp_f32, which computes 2^x natively, and the running
//   maximum lives in log2 units of the scaled scores (the exp2 change of "How to
//   profile and optimise kernels", dev.to/lewis_won, Round 4, "exp2").
// * Causal: key tiles wholly before the workgroup's first query run unmasked;
//   tiles straddling the diagonal are masked per element; tiles after the
//   workgroup's last query are never visited; inside a straddling tile a
//   wavefront whose queries all precede the tile skips it (same article, Round
//   4, "Causal tile-skipping").  Longest query tiles are launched first.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

template <int D, int QB, int WAVES, int BK>
struct Tile {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kBQ = WAVES * QB * 32;
  static constexpr int kChunksPerRow = D / 8;            // 16-byte chunks per K/V row
  static constexpr int kKBytes = BK * D * 2;             // one K tile (bf16)
  static constexpr int kVBytes = BK * D * 2;             // one V^T tile (bf16)
  static constexpr int kStageBytes = kKBytes + kVBytes;
  static constexpr int kLdsBytes = 2 * kStageBytes;      // double-buffered ring
  static constexpr int kKChunks = BK * kChunksPerRow;    // 16-byte chunks per K tile
  static constexpr int kVUnits = (BK / 2) * kChunksPerRow;  // (key pair, 8 dims) units
  static constexpr int kKIters = (kKChunks + kThreads - 1) / kThreads;
  static constexpr int kVIters = (kVUnits + kThreads - 1) / kThreads;
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(BK % 32 == 0 && BK >= 64 && BK <= 128, "key tile");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one CU");
};

// K tile in LDS: row = key, 16-byte chunk c stored at chunk position c ^ (row & 7),
// so the 8 lanes of one ds_read_b128 phase (8 rows, one chunk) hit 8 distinct
// bank groups.
template <int D>
__device__ __forceinline__ int k_lds_offset(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ (row & 7)) << 4);
}

// V^T tile in LDS: row = head-dim index, BK keys per row in 8-byte chunks of 4
// keys; chunk c stored at position c ^ f(row) with f(row) = (row ^ (row >> 3)) & 15.
// Reads (16 rows, one chunk) and the transposing writes (rows 8 apart) are
// both spread across distinct banks by it.
template <int BK>
__device__ __forceinline__ int vt_lds_offset(int row, int key) {
  const int f = (row ^ (row >> 3)) & 15;
  return row * (BK * 2) + (((key >> 2) ^ f) << 3) + ((key & 3) << 1);
}

__device__ __forceinline__ float lane_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

template <int D, int QB, int WAVES, int BK>
struct Regs {
  using T = Tile<D, QB, WAVES, BK>;
  u32x4 k[T::kKIters];
  u32x4 va[T::kVIters];
  u32x4 vb[T::kVIters];
};

// Global -> registers for key tile starting at k0 (rows >= N are zero-filled).
template <int D, int QB, int WAVES, int BK>
__device__ __forceinline__ void load_tile(Regs<D, QB, WAVES, BK>& r, const uint16_t* __restrict__ kh,
                                          const uint16_t* __restrict__ vh, int k0, int N, int tid) {
  using T = Tile<D, QB, WAVES, BK>;
#pragma unroll
  for (int it = 0; it < T::kKIters; ++it) {
    const int u = tid + it * T::kThreads;
    const int row = u / T::kChunksPerRow, c = u % T::kChunksPerRow;
    const int key = k0 + row;
    u32x4 x = {0u, 0u, 0u, 0u};
    if ((T::kKChunks % T::kThreads == 0 || u < T::kKChunks) && key < N)
      x = *reinterpret_cast<const u32x4*>(kh + (size_t)key * D + c * 8);
    r.k[it] = x;
  }
#pragma unroll
  for (int it = 0; it < T::kVIters; ++it) {
    const int u = tid + it * T::kThreads;
    const int kp = u / T::kChunksPerRow, c = u % T::kChunksPerRow;
    const int key = k0 + 2 * kp;
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    const bool live = (T::kVUnits % T::kThreads == 0 || u < T::kVUnits);
    if (live && key < N) a = *reinterpret_cast<const u32x4*>(vh + (size_t)key * D + c * 8);
    if (live && key + 1 < N) b = *reinterpret_cast<const u32x4*>(vh + (size_t)(key + 1) * D + c * 8);
    r.va[it] = a;
    r.vb[it] = b;
  }
}

// Registers -> LDS stage: K as is (swizzled), V transposed into V^T.
template <int D, int QB, int WAVES, int BK>
__device__ __forceinline__ void store_tile(const Regs<D, QB, WAVES, BK>& r, char* stage, int tid) {
  using T = Tile<D, QB, WAVES, BK>;
#pragma unroll
  for (int it = 0; it < T::kKIters; ++it) {
    const int u = tid + it * T::kThreads;
    if (T::kKChunks % T::kThreads == 0 || u < T::kKChunks) {
      const int row = u / T::kChunksPerRow, c = u % T::kChunksPerRow;
      *reinterpret_cast<u32x4*>(stage + k_lds_offset<D>(row, c)) = r.k[it];
    }
  }
  char* vt = stage + T::kKBytes;
#pragma unroll
  for (int it = 0; it < T::kVIters; ++it) {
    const int u = tid + it * T::kThreads;
    if (T::kVUnits % T::kThreads == 0 || u < T::kVUnits) {
      const int kp = u / T::kChunksPerRow, c = u % T::kChunksPerRow;
      const int key = 2 * kp;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a = r.va[it][e >> 1], b = r.vb[it][e >> 1];
        const uint32_t w = (e & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
        *reinterpret_cast<uint32_t*>(vt + vt_lds_offset<BK>(c * 8 + e, key)) = w;
      }
    }
  }
}

template <int D, bool CAUSAL, int QB, int WAVES, int BK>
__global__ __launch_bounds__(WAVES * 64) void fa_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, float* __restrict__ lse, int BH, int N, int nqt, float qk_scale) {
  using T = Tile<D, QB, WAVES, BK>;
  __shared__ __attribute__((aligned(16))) char lds[T::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;   // lane half: selects k-slots 8g..8g+7 of an MFMA operand
  const int lr = lane & 31;  // this lane's query column inside a 32-query block

  // ---- which (head, query tile) this workgroup owns -------------------------
  // Workgroups are dispatched round-robin over the 8 XCDs; when the head count
  // allows, the ids are remapped so that each XCD works through a contiguous
  // set of heads (their K/V stay in that XCD's L2).  Causal tiles run longest
  // first, all heads' longest tiles before any shorter one.
  const int total = gridDim.x;
  const int i = blockIdx.x;
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

  const size_t head = (size_t)bh * N * D;
  const uint16_t* qh = q + head;
  const uint16_t* kh = k + head;
  const uint16_t* vh = v + head;
  const int q0 = qt * T::kBQ;
  const int qw = q0 + wave * (QB * 32);  // first query of this wavefront

  // ---- Q block -> VGPRs, as the B operand of S^T = K Q^T ---------------------
  bf16x8 qreg[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw + qb * 32 + lr;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < N) x = *reinterpret_cast<const u32x4*>(qh + (size_t)row * D + ks * 16 + g * 8);
      qreg[qb][ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[QB][D / 32];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -__builtin_inff();
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  }

  // Causal: keys at or after min(q0 + BQ, N) are invisible to the whole tile.
  const int kend = CAUSAL ? min(q0 + T::kBQ, N) : N;
  const int ntiles = (kend + BK - 1) / BK;

  Regs<D, QB, WAVES, BK> regs;
  load_tile<D, QB, WAVES, BK>(regs, kh, vh, 0, N, tid);
  store_tile<D, QB, WAVES, BK>(regs, lds, tid);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    char* stage = lds + (j & 1) * T::kStageBytes;
    const int k0 = j * BK;
    const bool more = j + 1 < ntiles;
    if (more) load_tile<D, QB, WAVES, BK>(regs, kh, vh, k0 + BK, N, tid);

    // Wave-uniform classification of this key tile for this wavefront.
    const bool skip = CAUSAL && (k0 > qw + QB * 32 - 1);
    const bool masked = (CAUSAL && (k0 + BK - 1 > qw)) || (k0 + BK > N);
    if (!skip) {
      // ---- S^T = K_j Q^T --------------------------------------------------
      f32x16 s[QB][BK / 32];
#pragma unroll
      for (int kb = 0; kb < BK / 32; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(stage + k_lds_offset<D>(kb * 32 + lr, 2 * ks + g));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][ks], s[qb][kb], 0, 0, 0);
        }
      }

      // ---- mask, online softmax, P -> bf16 ---------------------------------
      bf16x8 p[QB][BK / 16];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (masked) {
          const int query = qw + qb * 32 + lr;
#pragma unroll
          for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
              if ((CAUSAL && key > query) || key >= N) s[qb][kb][r] = -__builtin_inff();
            }
        }
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        mx = lane_swap_max(mx);
        const float m_new = fmaxf(m[qb], mx * qk_scale);
        // A row that has seen no visible key yet keeps m = -inf; subtract 0 then
        // so that exp2(-inf - (-inf)) never appears.
        const float m_sub = (m_new == -__builtin_inff()) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m[qb] - m_sub);
        m[qb] = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r], qk_scale, -m_sub));
            s[qb][kb][r] = e;
            rs += e;
          }
        l[qb] = fmaf(alpha, l[qb], rs);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[qb][db] *= alpha;
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(s[qb][kb][8 * h + 2 * e], s[qb][kb][8 * h + 2 * e + 1]);
            p[qb][2 * kb + h] = __builtin_bit_cast(bf16x8, w);
          }
      }

      // ---- O^T += V_j^T P^T ------------------------------------------------
      const char* vt = stage + T::kKBytes;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int row = db * 32 + lr;
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int key = kb * 32 + 16 * h + 4 * g;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vt + vt_lds_offset<BK>(row, key));
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vt + vt_lds_offset<BK>(row, key + 8));
            const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
            const bf16x8 a = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[qb][2 * kb + h], oacc[qb][db], 0, 0, 0);
          }
      }
    }

    if (more) store_tile<D, QB, WAVES, BK>(regs, lds + ((j + 1) & 1) * T::kStageBytes, tid);
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16, LSE = (m + log2 l) ln 2 ------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lane_swap_sum(l[qb]);
    const float inv = 1.0f / lt;
    const int query = qw + qb * 32 + lr;
    if (query < N) {
      uint16_t* orow = out + head + (size_t)query * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          u32x2 w;
          w[0] = pack_bf16x2(oacc[qb][db][4 * rr + 0] * inv, oacc[qb][db][4 * rr + 1] * inv);
          w[1] = pack_bf16x2(oacc[qb][db][4 * rr + 2] * inv, oacc[qb][db][4 * rr + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * rr + 4 * g) = w;
        }
      if (g == 0) lse[(size_t)bh * N + query] = (m[qb] + log2f(lt)) * kLn2;
    }
  }
}

}  // namespace fa
