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
// (here with a lazy m: it is raised only when rowmax(S) exceeds it by more than
// a fixed margin, which leaves O / l and m + log l unchanged and skips most
// rescales; see kLazyMax).
//
// Scores stay in registers; the N x N matrix never reaches HBM.
//
// gfx950 mapping (v_mfma_f32_32x32x16_bf16, or _f16 for fp16 inputs: the element
// type E only picks the MFMA and the packing; accumulators in VGPRs):
// * S^T = K Q^T: the A operand is a 16-byte K row segment read from LDS
//   (ds_read_b128), the B operand a Q row segment held in VGPRs for the whole
//   sweep.  The 32x32 fp32 result gives each lane ONE query (lane % 32) and 16
//   keys, so the row max and row sum are in-lane reductions plus one
//   v_permlane32_swap between the two lane halves.
// * O^T += V^T P^T: a lane's probabilities, packed to bf16, are already laid out
//   as the B operand.  V stays row-major in LDS and enters as the A operand
//   through ds_read_b64_tr_b16, which hands each lane one head-dim column of a
//   4-key x 16-column block; the key order inside each 16-key step matches the
//   order in which the S^T accumulator holds the keys.  The alpha rescale of O
//   is a per-lane scalar multiply, skipped when no lane's reference maximum
//   moved; the reference moves only when a tile's maximum passes it by more
//   than kLazyMax (a factor 2^8 in P), so after a row's first tiles it rarely
//   does.
// * K and V tiles go HBM -> LDS directly (buffer_load_dwordx4 ... lds), 16 bytes
//   per lane; rows past the last key fall outside the buffer's range and read
//   as zero.
//   LDS rows are XOR-swizzled at 16-byte granularity (the swizzle is applied to
//   the global address, since the direct loads fill LDS lane-linearly).
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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLazyMax = 8.0f;  // see the online-softmax update in fa_fwd_kernel
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
#ifndef FA_CAUSAL_GROUP
#define FA_CAUSAL_GROUP 2  // heads per causal launch-order group on one XCD
#endif

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b);
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b);

// Element types of Q, K, V and O (16 bits each; scores, statistics and
// accumulators are fp32 either way): the MFMA operand vector, the 32x32x16
// MFMA, and the round-to-nearest-even packing of two fp32 values.
struct Bf16 {
  typedef bf16x8 v8;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
};
struct F16 {
  typedef f16x8 v8;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16x2(a, b); }
};

template <int D, int QB, int WAVES, int BK>
struct Tile {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kBQ = WAVES * QB * 32;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = BK * kRowBytes;       // one K or V tile (bf16)
  static constexpr int kStageBytes = 2 * kTileBytes;      // K then V
  static constexpr int kLdsBytes = 2 * kStageBytes;       // double-buffered ring
  static constexpr int kBlocks = kTileBytes / 1024;       // 1 KB direct-load blocks per tile
  static constexpr int kBlocksPerWave = (kBlocks + WAVES - 1) / WAVES;
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head dim");
  static_assert(BK % 32 == 0 && BK >= 32 && BK <= 128, "key tile");
  static_assert(kTileBytes % 1024 == 0, "tile = whole 1 KB blocks");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one CU");
};

// Swizzle of the 16-byte chunks of LDS row `row` (K and V tiles alike):
// chunk c is stored at position c ^ swz(row).  The 64 banks span 256 bytes, so
// a chunk's bank group is (row * D / 8 + position) mod 16.  For 64-byte rows
// (d = 32: four rows per bank row) the position depends on row bits 2..3; for
// 128-byte rows (d = 64) on row bits 1..3 (bit-reversed); for 256- and 512-byte
// rows (d = 128, 256) on row bits 0..3 (2-bit fields swapped, low four position
// bits only).  Each keeps the K fragment reads (16 rows, one chunk) and the V
// transpose reads (4 rows, 4 chunks) on distinct bank groups.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 32) {
    return (row >> 2) & 3;
  } else if constexpr (D == 64) {
    const int m = (row >> 1) & 7;
    return ((m & 1) << 2) | (m & 2) | ((m >> 2) & 1);
  } else {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  }
}

template <int D>
__device__ __forceinline__ int lds_offset(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ swz<D>(row)) << 4);
}

// Maximum of two scores.  The operands are MFMA results or -inf, never NaN,
// so the IEEE maximum (no quieting of signalling NaNs needed, unlike fmaxf)
// gives the same value and lowers to v_maximum3_f32 chains.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float lane_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f32x2 f = {a, b};
  f16x2 h = __builtin_convertvector(f, f16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

// 16 bytes per lane, global -> LDS: lane l's bytes land at dst + 16*l (dst is
// wave-uniform).  Kept out of the kernel template: called directly from a
// template body, this builtin stops the host pass from emitting launch stubs.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, char* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, voffset, 0, 0, 0);
}

// Kernel arguments.  Tensors are addressed by element strides (batch, head,
// row); the head dimension is contiguous.  Row strides fit 32 bits and every
// head's Q, K, V extent fits the 32-bit byte range of a buffer resource (the
// host checks both).
struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh, l_sb, l_sh;
  int q_rs, k_rs, v_rs, o_rs;
  int H, BH, Nq, Nk, nqt;
  float qk_scale;
  // Split keys (SPLIT kernels only): workgroup split s covers keys
  // [s * chunk, min(Nk, (s + 1) * chunk)) and writes fp32 partial results
  // part_o [nsplit, BH, Nq, d] (normalised over its keys) and part_lse
  // [nsplit, BH, Nq] (natural log; -inf for a row that sees none of them).
  float* part_o;
  float* part_lse;
  int chunk, nsplit;
  // Causal launch order (not SPLIT): workgroups resident per CU at a time for
  // this kernel, and the device's CU count.
  int resident, cus;
};

// Causal launch order of fa_fwd_kernel: workgroup i of total = BH * nqt ->
// head bh and query tile qt.  Workgroups are dispatched round-robin over the 8
// XCDs; when the head count allows, ids are remapped so that each XCD works
// through a contiguous set of heads (their K/V stay in that XCD's L2).  Tiles
// run longest first within groups of FA_CAUSAL_GROUP heads of an XCD, one group
// after the other: a group's lengths n, n, n-1, n-1, ... and the next group's in
// the same order fill the compute units evenly (a unit freed by a tile of
// length i takes the next of length n + 1 - i), while only one group's K/V are
// live at the start of the group.  When res > 1 workgroups fit on a CU, the
// first res layers of cus workgroups start together and workgroups b and b + cus
// share a CU; every odd full layer then runs in reverse order, so a long tile
// shares its CU with a short one instead of one of the same length.  The host's
// tile rule replays this order to judge how evenly a launch loads the CUs.
__host__ __device__ __forceinline__ void causal_order(int i, int total, int BH, int nqt, int res, int cus, int& bh,
                                                      int& qt) {
  const bool xcd = (BH % 8) == 0;
  const int t = xcd ? (i & 7) * (total >> 3) + (i >> 3) : i;
  if (xcd) {
    const int per = total >> 3, hpx = BH >> 3;
    const int chunk = t / per;
    int j = t - chunk * per;
    const int cpx = cus >> 3;  // CUs per XCD
    if (res > 1 && cpx > 0 && (cus & 7) == 0) {
      const int l = j / cpx, p = j - l * cpx;
      if ((l & 1) && l < res && (l + 1) * cpx <= per) j = l * cpx + (cpx - 1 - p);
    }
    const int gs = (hpx % FA_CAUSAL_GROUP) == 0 ? FA_CAUSAL_GROUP : hpx;
    const int grp = j / (gs * nqt), r = j - grp * gs * nqt;
    bh = chunk * hpx + grp * gs + r % gs;
    qt = nqt - 1 - r / gs;
  } else {
    int u = t;
    if (res > 1 && cus > 0) {
      const int l = u / cus, p = u - l * cus;
      if ((l & 1) && l < res && (l + 1) * cus <= total) u = l * cus + (cus - 1 - p);
    }
    bh = u % BH;
    qt = nqt - 1 - u / BH;
  }
}

// STRIDED = false: every tensor is contiguous [B, H, N, d] (lse [B, H, Nq]) and
// the strides in `pr` are ignored; the addressing then needs fewer registers.
// SPLIT = true: one key split per workgroup, partial results to the workspace
// (the per-worker (m, l, o) states that Flash-Decoding merges afterwards:
// "FlashAttention and kernels", gtadkapally.com, section "FlashAttention-2, -3,
// and what came after").
template <int D, bool CAUSAL, int QB, int WAVES, int BK, bool STRIDED, bool SPLIT = false, typename E = Bf16>
__global__ __launch_bounds__(WAVES * 64) void fa_fwd_kernel(const Params pr) {
  using T = Tile<D, QB, WAVES, BK>;
  using v8 = typename E::v8;
  const int BH = pr.BH, Nq = pr.Nq, Nk = pr.Nk, nqt = pr.nqt;
  const float qk_scale = pr.qk_scale;
  const int q_rs = STRIDED ? pr.q_rs : D, k_rs = STRIDED ? pr.k_rs : D;
  const int v_rs = STRIDED ? pr.v_rs : D, o_rs = STRIDED ? pr.o_rs : D;
  // One array per ring stage: distinct objects let the compiler see that the
  // direct loads into one stage never alias the fragment reads of the other,
  // so it does not wait for the prefetch before reading the current tile.
  __shared__ __attribute__((aligned(1024))) char lds0[T::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[T::kStageBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;   // lane half: selects k-slots 8g..8g+7 of an MFMA operand
  const int lr = lane & 31;  // this lane's query column inside a 32-query block

  // ---- which (head, query tile) this workgroup owns -------------------------
  // Non-causal: ids remapped so that each XCD takes a contiguous set of heads
  // when the head count allows; causal: causal_order.
  const int split = SPLIT ? (int)(blockIdx.x % pr.nsplit) : 0;
  const int total = SPLIT ? (int)(gridDim.x / pr.nsplit) : (int)gridDim.x;
  const int i = SPLIT ? (int)(blockIdx.x / pr.nsplit) : (int)blockIdx.x;
  int bh, qt;
  if (CAUSAL) {
    causal_order(i, total, BH, nqt, SPLIT ? 1 : pr.resident, pr.cus, bh, qt);
  } else {
    const int t = (BH % 8) == 0 ? (i & 7) * (total >> 3) + (i >> 3) : i;
    bh = t / nqt;
    qt = t - bh * nqt;
  }

  // Per-head bases.  A buffer resource ends at the head's last row, so rows at
  // or past Nq (Nk) read as zero.
  const int batch = bh / pr.H, hd = bh - batch * pr.H;
  const long long q_off = STRIDED ? batch * pr.q_sb + hd * pr.q_sh : (long long)bh * Nq * D;
  const long long k_off = STRIDED ? batch * pr.k_sb + hd * pr.k_sh : (long long)bh * Nk * D;
  const long long v_off = STRIDED ? batch * pr.v_sb + hd * pr.v_sh : (long long)bh * Nk * D;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(pr.q + q_off, (uint32_t)((Nq - 1) * q_rs + D) * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(pr.k + k_off, (uint32_t)((Nk - 1) * k_rs + D) * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(pr.v + v_off, (uint32_t)((Nk - 1) * v_rs + D) * 2);
  const int q0 = qt * T::kBQ;
  const int qw = q0 + wave * (QB * 32);  // first query of this wavefront

  // ---- Q block -> VGPRs, as the B operand of S^T = K Q^T (rows >= Nq read 0) ----
  v8 qreg[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw + qb * 32 + lr;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(qrs, (row * q_rs + ks * 16 + g * 8) * 2, 0, 0);
      qreg[qb][ks] = __builtin_bit_cast(v8, x);
    }
  }

  // ---- per-lane LDS offsets (loop invariant) ---------------------------------
  // Direct loads: this wave fills 1 KB blocks b = wave + WAVES*n of each tile;
  // lane l lands at byte 1024*b + 16*l, i.e. at LDS (row, position) and must
  // fetch global chunk position ^ swz(row) of that row.
  uint32_t dma_k[T::kBlocksPerWave], dma_v[T::kBlocksPerWave];
#pragma unroll
  for (int n = 0; n < T::kBlocksPerWave; ++n) {
    const int p = (wave + WAVES * n) * 64 + lane;  // 16-byte slot in the tile
    const int row = p / (D / 8), pos = p % (D / 8);
    const uint32_t col = (pos ^ swz<D>(row)) << 4;
    dma_k[n] = row * k_rs * 2 + col;
    dma_v[n] = row * v_rs * 2 + col;
  }
  // K fragment reads: key row kb*32 + lr, chunk 2*ks + g.
  int koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = lds_offset<D>(lr, 2 * ks + g);
  // V transpose reads: in each 16-lane group (s = lane / 16), lane 4r + tt
  // supplies 4 elements of key row (kbase + r) starting at column 4*tt of the
  // group's 16 columns; the group's columns are db*32 + 16*(s & 1) + 0..15 and
  // kbase = kb*32 + 16*h + 4*g (+8 for the upper half of the 8 k-slots).
  int voff[D / 32][2];
  {
    const int s = lane >> 4, jj = lane & 15, r = jj >> 2, tt = jj & 3;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int key = 4 * g + r + 8 * hi;
        const int col = db * 32 + 16 * (s & 1) + 4 * tt;
        voff[db][hi] = lds_offset<D>(key, col >> 3) + ((col & 4) << 1);
      }
  }

  // m: the lazy reference maximum (log2 units of the scaled scores); thr =
  // m + kLazyMax, the score above which m moves.  m starts at the lowest
  // finite float instead of -inf, so exp2(s - m) and exp2(m_old - m_new) never
  // see inf - inf: a row that has not met a visible key yet keeps it (its P are
  // exp2(-inf) = 0), and the first finite score moves it with alpha = 0.
  f32x16 oacc[QB][D / 32];
  float m[QB], thr[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -__FLT_MAX__;
    thr[qb] = -__FLT_MAX__;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  }

  // This workgroup's keys: [kbeg, klim) (all of them unless split).  Causal
  // (top-left: key j is visible to query i iff j <= i): keys at or after
  // q0 + BQ are invisible to the whole tile.
  const int kbeg = SPLIT ? split * pr.chunk : 0;
  const int klim = SPLIT ? min(Nk, kbeg + pr.chunk) : Nk;
  const int kend = CAUSAL ? min(q0 + T::kBQ, klim) : klim;
  const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  auto issue_tile = [&](int j, int stage) {
    const uint32_t gk = (uint32_t)(kbeg + j * BK) * k_rs * 2, gv = (uint32_t)(kbeg + j * BK) * v_rs * 2;
#pragma unroll
    for (int n = 0; n < T::kBlocksPerWave; ++n) {
      const int b = wave + WAVES * n;
      if (T::kBlocks % WAVES == 0 || b < T::kBlocks) {
        char* kdst = (stage ? lds1 : lds0) + b * 1024;
        // The whole offset goes in the VGPR operand so the range check sees it.
        dma16(krs, kdst, dma_k[n] + gk);
        dma16(vrs, kdst + T::kTileBytes, dma_v[n] + gv);
      }
    }
  };

  auto compute_tile = [&](const char* kst, int k0, bool masked) {
    const char* vst = kst + T::kTileBytes;
    // ---- S^T = K_j Q^T ------------------------------------------------------
    f32x16 s[QB][BK / 32];
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb) {
      v8 a[D / 16];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        a[ks] = *reinterpret_cast<const v8*>(kst + kb * 32 * (D * 2) + koff[ks]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s[qb][kb] = E::mfma(a[0], qreg[qb][0], f32x16{});
#pragma unroll
        for (int ks = 1; ks < D / 16; ++ks) s[qb][kb] = E::mfma(a[ks], qreg[qb][ks], s[qb][kb]);
      }
    }
    // ---- V fragments (issued early; consumed after the softmax) --------------
    v8 va[D / 32][BK / 16];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int rowoff = kk * 16 * (D * 2);  // keys kk*16 .. (kb = kk/2, h = kk%2)
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vst + rowoff + voff[db][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vst + rowoff + voff[db][1]));
        const u32x4 w = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                         __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
        va[db][kk] = __builtin_bit_cast(v8, w);
      }
    // ---- mask, online softmax, P -> bf16, O^T += V_j^T P^T ----------------------
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // The lane's maximum is taken before the masked branch, in the block of
      // the S^T MFMAs, so the first key block's maximum overlaps the second
      // block's products; a masked tile (diagonal or ragged) takes it again.
      auto lane_max = [&]() {
        float x = vmax(s[qb][0][0], s[qb][0][1]);
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
          for (int r = (kb == 0 ? 2 : 0); r < 16; ++r) x = vmax(x, s[qb][kb][r]);
        return x;
      };
      float mx = lane_max();
      if (masked) {
        // Element r of key block kb holds key k0 + 4g + o(kb, r) with the
        // compile-time offset o = 32 kb + 8 (r / 4) + r % 4; it is masked when
        // o >= lim (past the query causally, or past the last key).
        const int base = k0 + 4 * g;
        const int lim = CAUSAL ? min(qw + qb * 32 + lr + 1, klim) - base : klim - base;
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s[qb][kb][r] = -__builtin_inff();
        mx = lane_max();
      }
      mx = lane_swap_max(mx);
      // Lazy reference maximum: m moves only when the tile's maximum exceeds it
      // by more than kLazyMax (log2 units); until then P may reach 2^kLazyMax,
      // far from fp32 / bf16 / fp16 overflow for P and O.  O / l and
      // LSE = m + log2 l hold for any reference m, so most tiles skip the
      // rescale of O and l, and alpha, altogether.
      const float mt = mx * qk_scale;
      const bool moves = mt > thr[qb];
      if (__builtin_amdgcn_ballot_w64(moves)) {
        const float m_new = moves ? mt : m[qb];
        const float alpha = __builtin_amdgcn_exp2f(m[qb] - m_new);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[qb][db] *= alpha;
        l[qb] *= alpha;
        m[qb] = m_new;
        thr[qb] = m_new + kLazyMax;
      }
      const float m_sub = m[qb];
      // P for 16 keys at a time (half of an S^T block: elements 8h .. 8h + 7),
      // packed to the B operand and multiplied at once: the O^T += V^T P^T
      // products of the first keys run while the later keys' P is computed.
      // Row-sum and accumulation orders are the plain ones (keys ascending).
      float rs = 0.f;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int kb = kk >> 1, h = kk & 1;
        float e8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e8[i] = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][8 * h + i], qk_scale, -m_sub));
          rs = (kk == 0 && i == 0) ? e8[i] : rs + e8[i];
        }
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = E::pack(e8[2 * e], e8[2 * e + 1]);
        const v8 pk = __builtin_bit_cast(v8, w);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[qb][db] = E::mfma(va[db][kk], pk, oacc[qb][db]);
      }
      l[qb] += rs;
    }
    // The row sums are first needed by the next tile; without a use here the
    // compiler sinks their adds past the barrier, where they issue back to back
    // with no MFMA in flight.  Used here, they interleave with the O^T MFMAs.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) asm volatile("" ::"v"(l[qb]));
  };

  auto step = [&](int j, int stage) {
    if (j + 1 < ntiles) issue_tile(j + 1, stage ^ 1);
    const int k0 = kbeg + j * BK;
    // Wave-uniform classification of this key tile for this wavefront.
    const bool skip = CAUSAL && (k0 > qw + QB * 32 - 1);
    const bool masked = (CAUSAL && (k0 + BK - 1 > qw)) || (k0 + BK > klim);
    if (!skip) compute_tile(stage ? lds1 : lds0, k0, masked);
    // This wave's direct loads into the other stage have landed; after the
    // barrier every wave's have, and every wave is done reading this stage.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
  };

  if (ntiles > 0) {  // uniform over the workgroup
    issue_tile(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(j, 0);
    step(j + 1, 1);
  }
  if (j < ntiles) step(j, 0);

  if constexpr (SPLIT) {
    // ---- epilogue of a key split: fp32 O / l and LSE, or 0 and -inf for a row
    // that saw none of this split's keys ------------------------------------------
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = lane_swap_sum(l[qb]);
      const bool none = !(lt > 0.f);
      const float inv = none ? 0.f : 1.0f / lt;
      const int query = qw + qb * 32 + lr;
      if (query < Nq) {
        const long long row = ((long long)split * BH + bh) * Nq + query;
        float* orow = pr.part_o + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            f32x4 w = {oacc[qb][db][4 * rr + 0] * inv, oacc[qb][db][4 * rr + 1] * inv,
                       oacc[qb][db][4 * rr + 2] * inv, oacc[qb][db][4 * rr + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * rr + 4 * g) = w;
          }
        if (g == 0) pr.part_lse[row] = none ? -__builtin_inff() : (m[qb] + log2f(lt)) * kLn2;
      }
    }
    return;
  }

  // ---- epilogue: O / l -> bf16, LSE = (m + log2 l) ln 2 ------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lane_swap_sum(l[qb]);
    const float inv = 1.0f / lt;
    const int query = qw + qb * 32 + lr;
    if (query < Nq) {
      const long long o_off = STRIDED ? batch * pr.o_sb + hd * pr.o_sh : (long long)bh * Nq * D;
      uint16_t* orow = pr.out + o_off + (long long)query * o_rs;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          u32x2 w;
          w[0] = E::pack(oacc[qb][db][4 * rr + 0] * inv, oacc[qb][db][4 * rr + 1] * inv);
          w[1] = E::pack(oacc[qb][db][4 * rr + 2] * inv, oacc[qb][db][4 * rr + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * rr + 4 * g) = w;
        }
      const long long l_off = STRIDED ? batch * pr.l_sb + hd * pr.l_sh : (long long)bh * Nq;
      if (g == 0) pr.lse[l_off + query] = (m[qb] + log2f(lt)) * kLn2;
    }
  }
}

// s_waitcnt vmcnt(N): at most N of this wavefront's vector memory loads
// outstanding (N < 64; the count's high bits sit at bits 14..15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Key split inside one workgroup, for grids too small to give every SIMD a
// wavefront of its own queries.  The workgroup's S wavefronts share ONE block of
// 32 query rows; wavefront w sweeps key tiles w, w + S, w + 2S, ... through a
// double-buffered LDS ring of its own, waiting only on its own direct loads (no
// workgroup barrier in the sweep), and keeps the usual running state (m, l, O)
// over its keys.  The S partial states of each row are then merged through LDS:
// with M = max_w m_w and a_w = 2^(m_w - M), O = sum_w a_w O_w / sum_w a_w l_w and
// LSE = (M + log2 sum_w a_w l_w) ln 2.  This is Flash-Decoding's split of the
// keys over parallel workers followed by the merge of their partial (m, l, o)
// states ("FlashAttention and kernels", gtadkapally.com, section
// "FlashAttention-2, -3, and what came after", the Flash-Decoding paragraph; the
// merge of two partial states is that page's online max/sum exercise), done
// inside one launch instead of two.
//
// SPLIT = true: one workgroup per (split of the keys, head, query block), as
// fa_fwd_kernel's SPLIT instantiation: keys [s * chunk, min(Nk, (s + 1) *
// chunk)), partial results O / l (fp32) and LSE (or 0 and -inf for a row that
// sees none of them) into the caller's workspace for fa_merge_kernel.
template <int D, bool CAUSAL, int S, int BK, bool STRIDED, typename E = Bf16, bool SPLIT = false>
__global__ __launch_bounds__(S * 64) void fa_fwd_wsplit_kernel(const Params pr) {
  constexpr int kTileBytes = BK * D * 2;
  constexpr int kBlocks = kTileBytes / 1024;
  constexpr int kStage = 2 * kTileBytes;  // K then V
  constexpr int KS = D / 16, DB = D / 32;
  static_assert(S * 32 * D * 4 <= S * kStage, "merge buffer fits the first ring stage");
  static_assert(kTileBytes % 1024 == 0 && BK % 32 == 0, "tile");
  using v8 = typename E::v8;
  const int Nq = pr.Nq, Nk = pr.Nk, BH = pr.BH;
  const float qk_scale = pr.qk_scale;
  const int q_rs = STRIDED ? pr.q_rs : D, k_rs = STRIDED ? pr.k_rs : D;
  const int v_rs = STRIDED ? pr.v_rs : D, o_rs = STRIDED ? pr.o_rs : D;
  __shared__ __attribute__((aligned(1024))) char lds0[S * kStage];
  __shared__ __attribute__((aligned(1024))) char lds1[S * kStage];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, lr = lane & 31;
  // Causal: the longest query blocks first, one per head and then the next, so
  // with B*H a multiple of 8 each head's blocks land on one XCD (workgroups are
  // dealt round-robin over the 8 XCDs).  Non-causal: head-major, with ids
  // remapped as in fa_fwd_kernel so that each XCD works through a contiguous
  // set of heads and one L2 fetches a head's K and V.
  const int nqt = pr.nqt;
  const int split = SPLIT ? (int)(blockIdx.x % pr.nsplit) : 0;
  const int bid = SPLIT ? (int)(blockIdx.x / pr.nsplit) : (int)blockIdx.x;
  int bh, qt;
  if (CAUSAL) {
    bh = bid % BH;
    qt = nqt - 1 - bid / BH;
  } else {
    const int total = SPLIT ? (int)(gridDim.x / pr.nsplit) : (int)gridDim.x;
    const int t = (BH % 8) == 0 ? (bid & 7) * (total >> 3) + (bid >> 3) : bid;
    bh = t / nqt;
    qt = t - bh * nqt;
  }
  const int batch = bh / pr.H, hd = bh - batch * pr.H;
  const long long q_off = STRIDED ? batch * pr.q_sb + hd * pr.q_sh : (long long)bh * Nq * D;
  const long long k_off = STRIDED ? batch * pr.k_sb + hd * pr.k_sh : (long long)bh * Nk * D;
  const long long v_off = STRIDED ? batch * pr.v_sb + hd * pr.v_sh : (long long)bh * Nk * D;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(pr.q + q_off, (uint32_t)((Nq - 1) * q_rs + D) * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(pr.k + k_off, (uint32_t)((Nk - 1) * k_rs + D) * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(pr.v + v_off, (uint32_t)((Nk - 1) * v_rs + D) * 2);
  const int q0 = qt * 32;

  v8 qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(qrs, ((q0 + lr) * q_rs + ks * 16 + g * 8) * 2, 0, 0);
    qreg[ks] = __builtin_bit_cast(v8, x);
  }
  uint32_t dma_k[kBlocks], dma_v[kBlocks];
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) {
    const int p = b * 64 + lane, row = p / (D / 8), pos = p % (D / 8);
    const uint32_t col = (pos ^ swz<D>(row)) << 4;
    dma_k[b] = row * k_rs * 2 + col;
    dma_v[b] = row * v_rs * 2 + col;
  }
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = lds_offset<D>(lr, 2 * ks + g);
  int voff[DB][2];
  {
    const int s = lane >> 4, jj = lane & 15, r = jj >> 2, tt = jj & 3;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int key = 4 * g + r + 8 * hi;
        const int col = db * 32 + 16 * (s & 1) + 4 * tt;
        voff[db][hi] = lds_offset<D>(key, col >> 3) + ((col & 4) << 1);
      }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m = -__FLT_MAX__, thr = -__FLT_MAX__, l = 0.f;

  // Keys [kbeg, kend) in tiles of BK (all of them unless split; causal
  // top-left: none at or after q0 + 32); this wavefront's are tiles wave,
  // wave + S, ...
  const int kbeg = SPLIT ? split * pr.chunk : 0;
  const int klim = SPLIT ? min(Nk, kbeg + pr.chunk) : Nk;
  const int kend = CAUSAL ? min(q0 + 32, klim) : klim;
  const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int nmine = ntiles > wave ? (ntiles - 1 - wave) / S + 1 : 0;
  char* const st0 = lds0 + wave * kStage;
  char* const st1 = lds1 + wave * kStage;

  auto issue = [&](int j, char* dst) {
    const uint32_t gk = (uint32_t)(kbeg + j * BK) * k_rs * 2, gv = (uint32_t)(kbeg + j * BK) * v_rs * 2;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      dma16(krs, dst + b * 1024, dma_k[b] + gk);
      dma16(vrs, dst + kTileBytes + b * 1024, dma_v[b] + gv);
    }
  };

  // One key tile: the same steps, layouts and lazy reference maximum as
  // fa_fwd_kernel's compute_tile, for this wavefront's 32 queries.
  auto compute_tile = [&](const char* kst, int k0, bool masked) {
    const char* vst = kst + kTileBytes;
    f32x16 s[BK / 32];
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb) {
      v8 a[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[ks] = *reinterpret_cast<const v8*>(kst + kb * 32 * (D * 2) + koff[ks]);
      s[kb] = E::mfma(a[0], qreg[0], f32x16{});
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) s[kb] = E::mfma(a[ks], qreg[ks], s[kb]);
    }
    v8 va[DB][BK / 16];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int rowoff = kk * 16 * (D * 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vst + rowoff + voff[db][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vst + rowoff + voff[db][1]));
        const u32x4 w = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                         __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
        va[db][kk] = __builtin_bit_cast(v8, w);
      }
    if (masked) {
      const int base = k0 + 4 * g;
      const int lim = CAUSAL ? min(q0 + lr + 1, klim) - base : klim - base;
#pragma unroll
      for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s[kb][r] = -__builtin_inff();
    }
    float mx = vmax(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 2 : 0); r < 16; ++r) mx = vmax(mx, s[kb][r]);
    mx = lane_swap_max(mx);
    const float mt = mx * qk_scale;
    const bool moves = mt > thr;
    if (__builtin_amdgcn_ballot_w64(moves)) {
      const float m_new = moves ? mt : m;
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      l *= alpha;
      m = m_new;
      thr = m_new + kLazyMax;
    }
    const float m_sub = m;
    float rs = 0.f;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int kb = kk >> 1, h = kk & 1;
      float e8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e8[i] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * h + i], qk_scale, -m_sub));
        rs = (kk == 0 && i == 0) ? e8[i] : rs + e8[i];
      }
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = E::pack(e8[2 * e], e8[2 * e + 1]);
      const v8 pk = __builtin_bit_cast(v8, w);
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = E::mfma(va[db][kk], pk, oacc[db]);
    }
    l += rs;
  };

  // Local tile i: the load of tile i + 1 into the other stage (read two steps
  // ago; those reads completed before their products), then tile i, then the
  // wait for this wavefront's loads.  Stages are fixed per parity, so the
  // compiler sees that the loads and the fragment reads touch distinct arrays.
  auto step = [&](int i, char* cur, char* nxt) {
    const int j = wave + i * S;
    if (i + 1 < nmine) issue(j + S, nxt);
    const int k0 = kbeg + j * BK;
    const bool masked = (CAUSAL && (k0 + BK - 1 > q0)) || (k0 + BK > klim);
    compute_tile(cur, k0, masked);
    wait_vmcnt<0>();
  };
  if (nmine > 0) {
    issue(wave, st0);
    wait_vmcnt<0>();
  }
  int i = 0;
  for (; i + 1 < nmine; i += 2) {
    step(i, st0, st1);
    step(i + 1, st1, st0);
  }
  if (i < nmine) step(i, st0, st1);

  // ---- merge the S partial states of each query row through LDS ----------------
  // Every wavefront reaches this barrier once, after its last loads landed; the
  // rings are then reused: O_w (fp32, 16-byte chunks swizzled by row) in the
  // first, m_w and l_w in the second.  An empty sweep leaves m_w = -FLT_MAX,
  // l_w = 0 and O_w = 0, whose weight is 0.
  __syncthreads();
  float* po = reinterpret_cast<float*>(lds0);  // [S][32][D]
  float* pm = reinterpret_cast<float*>(lds1);  // [S][32]
  float* pl = pm + S * 32;                     // [S][32]
  const float lt = lane_swap_sum(l);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const f32x4 w = {oacc[db][4 * rr], oacc[db][4 * rr + 1], oacc[db][4 * rr + 2], oacc[db][4 * rr + 3]};
      const int cw = db * 8 + 2 * rr + g;  // 16-byte chunk, swizzled by row against bank conflicts
      *reinterpret_cast<f32x4*>(po + (wave * 32 + lr) * D + ((cw ^ (lr & 7)) << 2)) = w;
    }
  if (g == 0) {
    pm[wave * 32 + lr] = m;
    pl[wave * 32 + lr] = lt;
  }
  __syncthreads();
  // Wavefront w finishes head-dim columns [w D/S, (w + 1) D/S) of the 32 rows.
  float M = -__FLT_MAX__;
#pragma unroll
  for (int p = 0; p < S; ++p) M = fmaxf(M, pm[p * 32 + lr]);
  float wt[S], L = 0.f;
#pragma unroll
  for (int p = 0; p < S; ++p) {
    wt[p] = __builtin_amdgcn_exp2f(pm[p * 32 + lr] - M);
    L += wt[p] * pl[p * 32 + lr];
  }
  const int query = q0 + lr;
  constexpr int CPL = D / S / 2;  // columns per lane
  static_assert(CPL % 4 == 0, "columns per lane");
  const int c0 = wave * (D / S) + g * CPL;
  auto column = [&](int c) {  // columns c0 + c .. c0 + c + 3 of this row, unnormalised
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < S; ++p)
      acc += wt[p] * *reinterpret_cast<const f32x4*>(po + (p * 32 + lr) * D + ((((c0 + c) >> 2) ^ (lr & 7)) << 2));
    return acc;
  };
  if constexpr (SPLIT) {
    // A row that sees none of this split's keys has L = 0: O = 0, LSE = -inf.
    const bool none = !(L > 0.f);
    const float inv = none ? 0.f : 1.0f / L;
    if (query < Nq) {
      const long long row = ((long long)split * BH + bh) * Nq + query;
      float* orow = pr.part_o + row * D;
#pragma unroll
      for (int c = 0; c < CPL; c += 4) *reinterpret_cast<f32x4*>(orow + c0 + c) = column(c) * inv;
      if (wave == 0 && g == 0) pr.part_lse[row] = none ? -__builtin_inff() : (M + log2f(L)) * kLn2;
    }
    return;
  }
  const float inv = 1.0f / L;
  if (query < Nq) {
    const long long o_off = STRIDED ? batch * pr.o_sb + hd * pr.o_sh : (long long)bh * Nq * D;
    uint16_t* orow = pr.out + o_off + (long long)query * o_rs;
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
      const f32x4 acc = column(c);
      u32x2 w;
      w[0] = E::pack(acc[0] * inv, acc[1] * inv);
      w[1] = E::pack(acc[2] * inv, acc[3] * inv);
      *reinterpret_cast<u32x2*>(orow + c0 + c) = w;
    }
    const long long l_off = STRIDED ? batch * pr.l_sb + hd * pr.l_sh : (long long)bh * Nq;
    if (wave == 0 && g == 0) pr.lse[l_off + query] = (M + log2f(L)) * kLn2;
  }
}

// Combine the key splits of every query row: with M = max_s LSE_s and
// w_s = exp(LSE_s - M), O = sum_s w_s O_s / sum_s w_s and LSE = M + ln sum_s w_s
// -- the merge rule of two partial (m, l, o) states ("FlashAttention and
// kernels", the online max/sum exercise that merges partial states, and the
// Flash-Decoding paragraph of "FlashAttention-2, -3, and what came after"),
// applied to states already divided by their own l.  One thread per four
// consecutive head-dim elements of one row; reads are coalesced along d.
template <int D, typename E = Bf16>
__global__ __launch_bounds__(256) void fa_merge_kernel(const Params pr, long long rows) {
  constexpr int kTPR = D / 4;  // threads per row
  const long long r = (long long)blockIdx.x * (256 / kTPR) + threadIdx.x / kTPR;
  const int c = (threadIdx.x % kTPR) * 4;
  if (r >= rows) return;
  const int bh = (int)(r / pr.Nq), query = (int)(r - (long long)bh * pr.Nq);
  const long long plane = (long long)pr.BH * pr.Nq;
  float mx = -__builtin_inff();
  for (int s = 0; s < pr.nsplit; ++s) mx = fmaxf(mx, pr.part_lse[s * plane + r]);
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < pr.nsplit; ++s) {
    const float ls = pr.part_lse[s * plane + r];
    if (ls == -__builtin_inff()) continue;
    const float w = expf(ls - mx);
    wsum += w;
    acc += w * *reinterpret_cast<const f32x4*>(pr.part_o + (s * plane + r) * D + c);
  }
  const float inv = 1.0f / wsum;
  const int batch = bh / pr.H, hd = bh - batch * pr.H;
  uint16_t* orow = pr.out + batch * pr.o_sb + hd * pr.o_sh + (long long)query * pr.o_rs;
  u32x2 w2;
  w2[0] = E::pack(acc[0] * inv, acc[1] * inv);
  w2[1] = E::pack(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(orow + c) = w2;
  if (c == 0) pr.lse[batch * pr.l_sb + hd * pr.l_sh + query] = mx + logf(wsum);
}

}  // namespace fa
