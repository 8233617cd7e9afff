// FlashAttention-2 backward for gfx950 (CDNA4), hand-written HIP.
//
// Gradients of the exact attention O = softmax(scale * Q K^T) V with respect to
// Q, K, V, given dO.  P is never stored: each kernel recomputes it tile by tile
// from the log-sum-exp the forward saved, and follows the chain rule through
// the softmax ("FlashAttention and kernels", gtadkapally.com, section "The
// backward pass: recompute instead of remember"):
//
//   P  = exp(scale * Q K^T - LSE),   dV = P^T dO,   dP = dO V^T,
//   D  = rowsum(dO o O),             dS = P o (dP - D),
//   dQ = scale * dS K,               dK = scale * dS^T Q.
//
// Three kernels, no atomics (every output element is written once, by one
// lane, so results are deterministic):
// * fa_bwd_pre_kernel: D per query row, and LSE * log2(e) for the exp2 form.
// * fa_bwd_dkdv_kernel: one workgroup per key tile (32 keys per wavefront, K and
//   V of those keys held in VGPRs); it sweeps the query tiles that see those keys,
//   staging Q, dO, LSE and D through a double-buffered LDS ring, and accumulates
//   dK^T and dV^T in registers.
// * fa_bwd_dq_kernel: one workgroup per query tile (32 queries per wavefront, Q
//   and dO in VGPRs); it sweeps the key tiles like the forward, with K and V in
//   LDS, and accumulates dQ^T.
// The split into a key-major and a query-major pass recomputes S and dP twice
// (7 matrix products instead of 5) in exchange for no atomic traffic on dQ.
//
// Inputs and gradients are bf16 or fp16 (template E), contiguous or strided.
// MFMA mapping (v_mfma_f32_32x32x16_{bf16,f16}; C lane l, register r holds row
// 8(r/4) + 4(l/32) + r%4, column l%32):
// * dK/dV pass: S = Q K^T and dP = dO V^T with Q (dO) rows read from LDS as the A
//   operand and K (V) rows in VGPRs as the B operand, so a lane owns ONE key and
//   16 queries; P and dS packed to 16 bits are then already the B operand of
//   dV^T += dO^T P and dK^T += Q^T dS, whose A operands are dO and Q read
//   transposed from LDS (ds_read_b64_tr_b16) in the order the C layout holds the
//   queries.  Each lane needs LSE and D of its 16 queries: four 16-byte LDS
//   reads each per 32 queries.
// * dQ pass: S^T = K Q^T and dP^T = V dO^T (lane = one query, as in the
//   forward), dS^T packed to 16 bits is the B operand of dQ^T += K^T dS^T, with K
//   read transposed from LDS.
// LDS tiles use the forward's XOR swizzle, which keeps both the row reads and
// the transposed reads free of bank conflicts.
#pragma once
#include "fa_fwd_kernel.hpp"

namespace fa {

constexpr float kLog2e = 1.44269504088896340736f;

// Kernel arguments of the backward: Nq query rows (q, out, dout, dq, lse) over
// Nk key rows (k, v, dk, dv) per head.  Tensors are addressed by element
// strides (batch, head, row) with a contiguous head dimension; the STRIDED =
// false kernels assume contiguous [B, H, rows, d] (lse [B, H, Nq]) and ignore
// them.  The workspace holds lse2 and dsum, contiguous [B*H, Nq] fp32 each.
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* lse2;  // LSE * log2(e)
  float* dsum;  // D = rowsum(dO o O)
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh, do_sb, do_sh;
  long long dq_sb, dq_sh, dk_sb, dk_sh, dv_sb, dv_sh, l_sb, l_sh;
  int q_rs, k_rs, v_rs, o_rs, do_rs, dq_rs, dk_rs, dv_rs;
  int H, BH, Nq, Nk, ntiles;
  int nqt;  // query tiles of 64 rows per head: ceil(Nq / 64)
  float qk_scale;  // scale * log2(e)
  float scale;
  // Causal launch order: workgroups of the launched kernel resident per CU at a
  // time, and the device's CU count (set per launch).
  int resident, cus;
};

// Element offset of head bh of a tensor: strided, or contiguous [B, H, rows, D].
template <bool STRIDED, int D>
__device__ __forceinline__ long long head_off(long long sb, long long sh, int bh, int H, int rows) {
  if constexpr (STRIDED) {
    const int b = bh / H;
    return b * sb + (bh - b * H) * sh;
  } else {
    return (long long)bh * rows * D;
  }
}

// Two packed 16-bit elements of type E, widened.
template <typename E>
struct Unpack2;
template <>
struct Unpack2<Bf16> {
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
};
template <>
struct Unpack2<F16> {
  static __device__ __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
  static __device__ __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }
};

// 4 bytes per lane, global -> LDS: lane l's word lands at dst + 4*l.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rsrc, char* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 4, voffset, 0, 0, 0);
}

// A operand of 32x32x16 read transposed out of a row-major (swizzled) LDS
// tile: rows (keys or queries) 16*step + {4g + 0..3, 8 + 4g + 0..3}, columns
// db*32 + lane%32 -- the order in which a C fragment holds its rows.
template <typename E>
__device__ __forceinline__ typename E::v8 read_tr(const char* base, int lo, int hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + lo));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + hi));
  const u32x4 w = {__builtin_bit_cast(u32x2, a)[0], __builtin_bit_cast(u32x2, a)[1], __builtin_bit_cast(u32x2, b)[0],
                   __builtin_bit_cast(u32x2, b)[1]};
  return __builtin_bit_cast(typename E::v8, w);
}

// Per-lane byte offsets of read_tr inside a tile: [db][0] for the low four
// rows, [db][1] for the high four.  In each 16-lane group (s = lane / 16), lane
// 4r + tt supplies 4 elements of row (4g + r, +8 for the high half) starting at
// column db*32 + 16*(s & 1) + 4*tt.
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int (&off)[D / 32][2]) {
  const int g = lane >> 5, s = lane >> 4, jj = lane & 15, r = jj >> 2, tt = jj & 3;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = 4 * g + r + 8 * hi;
      const int col = db * 32 + 16 * (s & 1) + 4 * tt;
      off[db][hi] = lds_offset<D>(row, col >> 3) + ((col & 4) << 1);
    }
}

// Direct loads of a tile in 1 KB blocks: block b covers rows kRows * b ..
// kRows * (b + 1) - 1 (kRows = 512 / D) and lane l fills row kRows * b + l /
// (D / 8), LDS position l % (D / 8), fetching the global chunk that the
// swizzle puts there.  The swizzle depends on row bits 0..3 only, so when
// kRows * WAVES is a multiple of 16 the blocks b = wave + WAVES * n of one
// wave share a per-lane byte offset; block n then adds rows kRows * b.
template <int D, int WAVES>
struct BlockDma {
  static constexpr int kRows = 512 / D;
  static_assert((kRows * WAVES) % 16 == 0, "one lane offset per wave needs the swizzle's 16-row period");
  // Per-lane part of the byte offset, for a tensor with row stride rs.
  static __device__ __forceinline__ uint32_t lane_off(int lane, int wave, int rs) {
    const int row_l = lane / (D / 8), pos = lane % (D / 8);
    return row_l * rs * 2 + ((pos ^ swz<D>(kRows * wave + row_l)) << 4);
  }
  // First row of block n of this wave.
  static __device__ __forceinline__ int row0(int wave, int n) { return kRows * (wave + WAVES * n); }
};

// A C fragment's 16 values as two 16-bit B operands (16 rows each): element e
// of operand h is register 8h + e.
template <typename E>
__device__ __forceinline__ void pack_b(const f32x16& x, typename E::v8 (&b)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = E::pack(x[8 * h + 2 * e], x[8 * h + 2 * e + 1]);
    b[h] = __builtin_bit_cast(typename E::v8, w);
  }
}

// Workgroup -> (head, tile).  Round-robin dispatch over the 8 XCDs is undone
// when the head count allows, so that each XCD works through a contiguous set
// of heads; `rank` 0 is the tile to run first (the caller maps it to its
// longest tile when causal).
__device__ __forceinline__ void tile_of(int i, int total, int BH, int ntiles, bool causal, int resident, int cus,
                                        int& bh, int& rank) {
  const bool xcd = (BH % 8) == 0;
  const int t = xcd ? (i & 7) * (total >> 3) + (i >> 3) : i;
  if (causal) {
    // With several workgroups resident per CU, the first `resident` layers of
    // `cus` workgroups start together and workgroups i and i + cus share a CU:
    // every odd full layer runs in reverse, pairing long tiles with short ones.
    if (xcd) {
      const int per = total >> 3, hpx = BH >> 3;
      const int chunk = t / per;
      int j = t - chunk * per;
      const int cpx = cus >> 3;
      if (resident > 1 && cpx > 0 && (cus & 7) == 0) {
        const int l = j / cpx, p = j - l * cpx;
        if ((l & 1) && l < resident && (l + 1) * cpx <= per) j = l * cpx + (cpx - 1 - p);
      }
      bh = chunk * hpx + j % hpx;
      rank = j / hpx;
    } else {
      int u = t;
      if (resident > 1 && cus > 0) {
        const int l = u / cus, p = u - l * cus;
        if ((l & 1) && l < resident && (l + 1) * cus <= total) u = l * cus + (cus - 1 - p);
      }
      bh = u % BH;
      rank = u / BH;
    }
  } else {
    bh = t / ntiles;
    rank = t - bh * ntiles;
  }
}

// ---- D = rowsum(dO o O) and LSE * log2(e), one row per D/8 lanes ------------
template <int D, typename E, bool STRIDED>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(const BwdParams pr) {
  constexpr int kLanes = D / 8;  // 16 bytes of a row per lane
  const long long rows = (long long)pr.BH * pr.Nq;
  const long long r = (long long)blockIdx.x * (256 / kLanes) + threadIdx.x / kLanes;
  const int c = (threadIdx.x % kLanes) * 8;
  float acc = 0.f;
  int bh = 0, i = 0;
  if (r < rows) {
    bh = (int)(r / pr.Nq);
    i = (int)(r - (long long)bh * pr.Nq);
    const int o_rs = STRIDED ? pr.o_rs : D, do_rs = STRIDED ? pr.do_rs : D;
    const uint16_t* orow = pr.out + head_off<STRIDED, D>(pr.o_sb, pr.o_sh, bh, pr.H, pr.Nq) + (long long)i * o_rs;
    const uint16_t* grow = pr.dout + head_off<STRIDED, D>(pr.do_sb, pr.do_sh, bh, pr.H, pr.Nq) + (long long)i * do_rs;
    const u32x4 o = *reinterpret_cast<const u32x4*>(orow + c);
    const u32x4 g = *reinterpret_cast<const u32x4*>(grow + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(Unpack2<E>::lo(o[e]), Unpack2<E>::lo(g[e]), acc);
      acc = fmaf(Unpack2<E>::hi(o[e]), Unpack2<E>::hi(g[e]), acc);
    }
  }
#pragma unroll
  for (int m = kLanes / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kLanes);
  if (r < rows && c == 0) {
    pr.dsum[r] = acc;
    const long long l_off = STRIDED ? (long long)(bh / pr.H) * pr.l_sb + (bh % pr.H) * pr.l_sh : (long long)bh * pr.Nq;
    pr.lse2[r] = pr.lse[l_off + i] * kLog2e;
  }
}

// ---- dK, dV: one workgroup per WAVES*32 keys ---------------------------------
// VLDS = false: each wavefront holds its 32 K and V rows in VGPRs.  VLDS = true
// (d = 128): V rows stay in LDS for the whole sweep and are read as the B
// operand of dP = dO V^T, which frees the 32 VGPRs that let two wavefronts share
// a SIMD.
template <int D, bool CAUSAL, int WAVES, bool VLDS, typename E = Bf16, bool STRIDED = false>
__global__ __launch_bounds__(WAVES * 64) void fa_bwd_dkdv_kernel(const BwdParams pr) {
  typedef typename E::v8 v8;
  constexpr int BQ = 64;                          // queries per staged tile
  constexpr int kBK = WAVES * 32;                 // keys per workgroup
  constexpr int kTileBytes = BQ * D * 2;          // one Q or dO tile
  constexpr int kBlocks = kTileBytes / 1024;      // 1 KB direct-load blocks per tile
  constexpr int kBlocksPerWave = (kBlocks + WAVES - 1) / WAVES;
  constexpr int kStageBytes = 2 * kTileBytes + 2 * BQ * 4;  // Q, dO, lse2, dsum
  constexpr int kVBytes = VLDS ? kBK * D * 2 : 1024;        // resident V rows
  static_assert(WAVES >= 2 && kBK % BQ == 0, "tile shape");
  static_assert(2 * kStageBytes + (VLDS ? kVBytes : 0) <= 160 * 1024, "LDS budget of one CU");
  __shared__ __attribute__((aligned(1024))) char lds0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char vlds[kVBytes];

  const int Nq = pr.Nq, Nk = pr.Nk;
  const float qk_scale = pr.qk_scale;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lr = lane & 31;

  int bh, kt;
  tile_of((int)blockIdx.x, (int)gridDim.x, pr.BH, pr.ntiles, CAUSAL, pr.resident, pr.cus, bh, kt);
  const int q_rs = STRIDED ? pr.q_rs : D, do_rs = STRIDED ? pr.do_rs : D;
  const int k_rs = STRIDED ? pr.k_rs : D, v_rs = STRIDED ? pr.v_rs : D;
  const __amdgpu_buffer_rsrc_t qrs =
      make_rsrc(pr.q + head_off<STRIDED, D>(pr.q_sb, pr.q_sh, bh, pr.H, Nq), (uint32_t)((Nq - 1) * q_rs + D) * 2);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(pr.dout + head_off<STRIDED, D>(pr.do_sb, pr.do_sh, bh, pr.H, Nq),
                                               (uint32_t)((Nq - 1) * do_rs + D) * 2);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(pr.lse2 + (long long)bh * Nq, (uint32_t)Nq * 4);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(pr.dsum + (long long)bh * Nq, (uint32_t)Nq * 4);
  const int k0 = kt * kBK;
  const int kw = k0 + wave * 32;  // first key of this wavefront
  // Causal (top-left: key j is seen by queries i >= j): queries before k0 see
  // none of these keys, and when k0 >= Nq no query does (then no tile is
  // staged and dK = dV = 0 are written).
  // (Non-causal, the count is pr.nqt; the strided kernel takes it from there,
  // where its registers allocate with a quarter of the spill of the computed
  // form, 52 against 208 bytes per lane at d = 128.)
  static_assert(BQ == 64, "pr.nqt counts 64-row query tiles");
  const int qbeg = CAUSAL ? k0 : 0;
  const int ntiles = (STRIDED && !CAUSAL) ? pr.nqt : (qbeg < Nq ? (Nq - qbeg + BQ - 1) / BQ : 0);

  using Dma = BlockDma<D, WAVES>;
  const uint32_t dma_q = Dma::lane_off(lane, wave, q_rs), dma_d = Dma::lane_off(lane, wave, do_rs);
  int roff[D / 16];  // row reads: row lr, chunk 2*ks + g
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) roff[ks] = lds_offset<D>(lr, 2 * ks + g);
  int toff[D / 32][2];
  tr_offsets<D>(lane, toff);

  // ---- this wavefront's K rows (and V rows, or the workgroup's V -> LDS) -------
  v8 kreg[D / 16], vreg[VLDS ? 1 : D / 16];
  {
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc(pr.k + head_off<STRIDED, D>(pr.k_sb, pr.k_sh, bh, pr.H, Nk), (uint32_t)((Nk - 1) * k_rs + D) * 2);
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(pr.v + head_off<STRIDED, D>(pr.v_sb, pr.v_sh, bh, pr.H, Nk), (uint32_t)((Nk - 1) * v_rs + D) * 2);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const uint32_t koff = ((kw + lr) * k_rs + ks * 16 + g * 8) * 2;
      kreg[ks] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(krs, koff, 0, 0));
      if constexpr (!VLDS) {
        const uint32_t voff = ((kw + lr) * v_rs + ks * 16 + g * 8) * 2;
        vreg[ks] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff, 0, 0));
      }
    }
    if constexpr (VLDS) {
      // kBK rows of V, swizzled like a tile; rows >= Nk read 0.  Waited for
      // with the first Q / dO tile (or below, when there is none).
      constexpr int kVBlocksPerWave = kVBytes / 1024 / WAVES;
      const uint32_t dma_v = Dma::lane_off(lane, wave, v_rs);
#pragma unroll
      for (int n = 0; n < kVBlocksPerWave; ++n)
        dma16(vrs, vlds + ((CAUSAL && STRIDED) ? (tid >> 6) + WAVES * n : wave + WAVES * n) * 1024,
              dma_v + (uint32_t)(k0 + Dma::row0(wave, n)) * v_rs * 2);
    }
  }
  const char* vrow = vlds + wave * 32 * (D * 2);  // this wavefront's V rows

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dk[db] = dv[db] = f32x16{};


  auto issue_tile = [&](int j, int stage) {
    const int qs = qbeg + j * BQ;
    char* st = stage ? lds1 : lds0;
    const uint32_t gq = (uint32_t)qs * q_rs * 2, gd = (uint32_t)qs * do_rs * 2;
#pragma unroll
    for (int n = 0; n < kBlocksPerWave; ++n) {
      const int b = wave + WAVES * n;
      if (kBlocks % WAVES == 0 || b < kBlocks) {
        const uint32_t r0 = (uint32_t)Dma::row0(wave, n);
        // Block b's LDS slot.  The causal strided kernel takes it from the
        // per-lane wave index: from the scalar one this compiler emits an
        // LDS-aperture check it cannot encode (instruction selection error).
        char* dst = st + ((CAUSAL && STRIDED) ? (tid >> 6) + WAVES * n : b) * 1024;
        dma16(qrs, dst, dma_q + r0 * q_rs * 2 + gq);
        dma16(drs, dst + kTileBytes, dma_d + r0 * do_rs * 2 + gd);
      }
    }
    if (wave == 0) dma4(lrs, st + 2 * kTileBytes, (uint32_t)(qs + lane) * 4);
    if (wave == 1) dma4(srs, st + 2 * kTileBytes + BQ * 4, (uint32_t)(qs + lane) * 4);
  };

  auto compute_tile = [&](const char* st, int qs) {
    const char* qst = st;
    const char* dst = st + kTileBytes;
    const float* lst = reinterpret_cast<const float*>(st + 2 * kTileBytes);
    const float* sst = lst + BQ;
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      const int qbase = qs + qb * 32;
      // Multiples of 32 both: either every query of the block precedes every
      // key of the wavefront, or the block is the diagonal one, or it follows.
      if (CAUSAL && qbase < kw) continue;
      const bool diag = CAUSAL && qbase == kw;
      // ---- S = Q K^T, dP = dO V^T (lane = key, 16 queries) ------------------
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const v8 a = *reinterpret_cast<const v8*>(qst + qb * 32 * (D * 2) + roff[ks]);
        s = E::mfma(a, kreg[ks], s);
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const v8 a = *reinterpret_cast<const v8*>(dst + qb * 32 * (D * 2) + roff[ks]);
        v8 b;
        if constexpr (VLDS)
          b = *reinterpret_cast<const v8*>(vrow + roff[ks]);
        else
          b = vreg[ks];
        dp = E::mfma(a, b, dp);
      }
      // ---- P and dS -----------------------------------------------------------
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 L = *reinterpret_cast<const f32x4*>(lst + qb * 32 + 8 * j + 4 * g);
        const f32x4 Dq = *reinterpret_cast<const f32x4*>(sst + qb * 32 + 8 * j + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * j + e;
          float p = __builtin_amdgcn_exp2f(fmaf(s[r], qk_scale, -L[e]));
          if (diag && (lr > 8 * j + 4 * g + e)) p = 0.f;  // key > query
          s[r] = p;
          dp[r] = p * (dp[r] - Dq[e]);
        }
      }
      v8 pb[2], db16[2];
      pack_b<E>(s, pb);
      pack_b<E>(dp, db16);
      // ---- dV^T += dO^T P, dK^T += Q^T dS --------------------------------------
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rowoff = (2 * qb + h) * 16 * (D * 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = E::mfma(read_tr<E>(dst + rowoff, toff[db][0], toff[db][1]), pb[h], dv[db]);
          dk[db] = E::mfma(read_tr<E>(qst + rowoff, toff[db][0], toff[db][1]), db16[h], dk[db]);
        }
      }
      // At 256 VGPRs (d = 128) two query blocks in flight do not fit: keep the
      // scheduler from overlapping them.
      if constexpr (VLDS) __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto step = [&](int j, int stage) {
    if (j + 1 < ntiles) issue_tile(j + 1, stage ^ 1);
    compute_tile(stage ? lds1 : lds0, qbeg + j * BQ);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads landed
    __syncthreads();                     // ... every wave's, and this stage is free
  };

  if (ntiles > 0) issue_tile(0, 0);  // uniform over the workgroup
  // The first tile (and V) landed for every wave; with no tile, the V load is
  // drained before the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(j, 0);
    step(j + 1, 1);
  }
  if (j < ntiles) step(j, 0);

  // ---- epilogue: dK = scale * (dK^T)^T, dV -> E --------------------------------
  // The lane index is read again (mbcnt) rather than kept from the prologue, so
  // that no per-lane value has to live across the query-tile loop.
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int g_e = lane_e >> 5;
  const int key = kw + (lane_e & 31);
  if (key < Nk) {
    const int dk_rs = STRIDED ? pr.dk_rs : D, dv_rs = STRIDED ? pr.dv_rs : D;
    uint16_t* krow = pr.dk + head_off<STRIDED, D>(pr.dk_sb, pr.dk_sh, bh, pr.H, Nk) + (long long)key * dk_rs;
    uint16_t* vout = pr.dv + head_off<STRIDED, D>(pr.dv_sb, pr.dv_sh, bh, pr.H, Nk) + (long long)key * dv_rs;
    const float sc = pr.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        u32x2 a, b;
        a[0] = E::pack(dk[db][4 * rr + 0] * sc, dk[db][4 * rr + 1] * sc);
        a[1] = E::pack(dk[db][4 * rr + 2] * sc, dk[db][4 * rr + 3] * sc);
        b[0] = E::pack(dv[db][4 * rr + 0], dv[db][4 * rr + 1]);
        b[1] = E::pack(dv[db][4 * rr + 2], dv[db][4 * rr + 3]);
        *reinterpret_cast<u32x2*>(krow + db * 32 + 8 * rr + 4 * g_e) = a;
        *reinterpret_cast<u32x2*>(vout + db * 32 + 8 * rr + 4 * g_e) = b;
      }
  }
}

// ---- dQ: one workgroup per WAVES*32 queries, key tiles of BK -----------------
// Up to d = 64 the registers fit four wavefronts per SIMD (four workgroups per
// CU): the non-causal kernel needs 134 VGPRs unconstrained and 124 when asked to.
template <int D, bool CAUSAL, int WAVES, int BK, typename E = Bf16, bool STRIDED = false>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 4 : 1)))
void fa_bwd_dq_kernel(const BwdParams pr) {
  typedef typename E::v8 v8;
  constexpr int kBQ = WAVES * 32;
  constexpr int kTileBytes = BK * D * 2;  // one K or V tile
  constexpr int kBlocks = kTileBytes / 1024;
  constexpr int kBlocksPerWave = (kBlocks + WAVES - 1) / WAVES;
  constexpr int kStageBytes = 2 * kTileBytes;  // K then V
  static_assert(BK % 32 == 0 && kTileBytes % 1024 == 0, "key tile");
  static_assert(2 * kStageBytes <= 160 * 1024, "LDS budget of one CU");
  __shared__ __attribute__((aligned(1024))) char lds0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kStageBytes];

  const int Nq = pr.Nq, Nk = pr.Nk, nqt = pr.ntiles;
  const float qk_scale = pr.qk_scale;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lr = lane & 31;

  int bh, rank;
  tile_of((int)blockIdx.x, (int)gridDim.x, pr.BH, nqt, CAUSAL, pr.resident, pr.cus, bh, rank);
  const int qt = CAUSAL ? nqt - 1 - rank : rank;  // causal: longest (last) query tile first
  const int q_rs = STRIDED ? pr.q_rs : D, do_rs = STRIDED ? pr.do_rs : D;
  const int k_rs = STRIDED ? pr.k_rs : D, v_rs = STRIDED ? pr.v_rs : D;
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(pr.k + head_off<STRIDED, D>(pr.k_sb, pr.k_sh, bh, pr.H, Nk), (uint32_t)((Nk - 1) * k_rs + D) * 2);
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(pr.v + head_off<STRIDED, D>(pr.v_sb, pr.v_sh, bh, pr.H, Nk), (uint32_t)((Nk - 1) * v_rs + D) * 2);
  const int q0 = qt * kBQ;
  const int qw = q0 + wave * 32;
  const int query = qw + lr;

  // ---- Q and dO rows -> VGPRs (B operands), LSE and D of this lane's query ----
  v8 qreg[D / 16], doreg[D / 16];
  {
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(pr.q + head_off<STRIDED, D>(pr.q_sb, pr.q_sh, bh, pr.H, Nq), (uint32_t)((Nq - 1) * q_rs + D) * 2);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(pr.dout + head_off<STRIDED, D>(pr.do_sb, pr.do_sh, bh, pr.H, Nq),
                                                 (uint32_t)((Nq - 1) * do_rs + D) * 2);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const uint32_t qoff = (query * q_rs + ks * 16 + g * 8) * 2;
      const uint32_t doff = (query * do_rs + ks * 16 + g * 8) * 2;
      qreg[ks] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff, 0, 0));
      doreg[ks] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(drs, doff, 0, 0));
    }
  }
  float l2 = 0.f, dd = 0.f;
  if (query < Nq) {
    l2 = pr.lse2[(long long)bh * Nq + query];
    dd = pr.dsum[(long long)bh * Nq + query];
  }

  using Dma = BlockDma<D, WAVES>;
  const uint32_t dma_k = Dma::lane_off(lane, wave, k_rs), dma_v = Dma::lane_off(lane, wave, v_rs);
  int roff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) roff[ks] = lds_offset<D>(lr, 2 * ks + g);
  int toff[D / 32][2];
  tr_offsets<D>(lane, toff);

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  const int kend = CAUSAL ? min(q0 + kBQ, Nk) : Nk;
  const int ntiles = (kend + BK - 1) / BK;

  auto issue_tile = [&](int j, int stage) {
    const uint32_t gk = (uint32_t)(j * BK) * k_rs * 2, gv = (uint32_t)(j * BK) * v_rs * 2;
    char* st = stage ? lds1 : lds0;
#pragma unroll
    for (int n = 0; n < kBlocksPerWave; ++n) {
      const int b = wave + WAVES * n;
      if (kBlocks % WAVES == 0 || b < kBlocks) {
        const uint32_t r0 = (uint32_t)Dma::row0(wave, n);
        char* dst = st + b * 1024;
        dma16(krs, dst, dma_k + r0 * k_rs * 2 + gk);
        dma16(vrs, dst + kTileBytes, dma_v + r0 * v_rs * 2 + gv);
      }
    }
  };

  auto compute_tile = [&](const char* kst, int k0, bool masked) {
    const char* vst = kst + kTileBytes;
    v8 dsb[BK / 16];
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb) {
      // ---- S^T = K Q^T, dP^T = V dO^T (lane = query, 16 keys) ------------------
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const v8 a = *reinterpret_cast<const v8*>(kst + kb * 32 * (D * 2) + roff[ks]);
        s = E::mfma(a, qreg[ks], s);
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const v8 a = *reinterpret_cast<const v8*>(vst + kb * 32 * (D * 2) + roff[ks]);
        dp = E::mfma(a, doreg[ks], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(s[r], qk_scale, -l2));
        if (masked) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if ((CAUSAL && key > query) || key >= Nk) p = 0.f;
        }
        dp[r] = p * (dp[r] - dd);
      }
      v8 b2[2];
      pack_b<E>(dp, b2);
      dsb[2 * kb] = b2[0];
      dsb[2 * kb + 1] = b2[1];
    }
    // ---- dQ^T += K^T dS^T ---------------------------------------------------------
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        dq[db] = E::mfma(read_tr<E>(kst + kk * 16 * (D * 2), toff[db][0], toff[db][1]), dsb[kk], dq[db]);
  };

  auto step = [&](int j, int stage) {
    if (j + 1 < ntiles) issue_tile(j + 1, stage ^ 1);
    const int k0 = j * BK;
    const bool skip = CAUSAL && (k0 > qw + 31);
    const bool masked = (CAUSAL && (k0 + BK - 1 > qw)) || (k0 + BK > Nk);
    if (!skip) compute_tile(stage ? lds1 : lds0, k0, masked);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };

  issue_tile(0, 0);  // ntiles >= 1: kend >= 1
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(j, 0);
    step(j + 1, 1);
  }
  if (j < ntiles) step(j, 0);

  if (query < Nq) {
    const int dq_rs = STRIDED ? pr.dq_rs : D;
    uint16_t* row = pr.dq + head_off<STRIDED, D>(pr.dq_sb, pr.dq_sh, bh, pr.H, Nq) + (long long)query * dq_rs;
    const float sc = pr.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        u32x2 w;
        w[0] = E::pack(dq[db][4 * rr + 0] * sc, dq[db][4 * rr + 1] * sc);
        w[1] = E::pack(dq[db][4 * rr + 2] * sc, dq[db][4 * rr + 3] * sc);
        *reinterpret_cast<u32x2*>(row + db * 32 + 8 * rr + 4 * g) = w;
      }
  }
}

}  // namespace fa
