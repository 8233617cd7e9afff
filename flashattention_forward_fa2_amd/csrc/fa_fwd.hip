// C ABI of the gfx950 FlashAttention-2 forward library: argument checks, the
// table of compiled tile variants, and the launch.  Declared in include/fa_fwd.h.
#include "fa_fwd.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "fa_fwd_f32_kernel.hpp"
#include "fa_fwd_kernel.hpp"

namespace {

constexpr int kVersion = 600;  // 0.6.0: fa_tile_cfg.ksplit

using Launcher = hipError_t (*)(const fa::Params&, int B, hipStream_t);

struct Variant {
  int d, causal, qb, waves, bk, dtype;
  Launcher launch;          // contiguous [B, H, N, d] tensors
  Launcher launch_strided;  // any strides
  Launcher launch_split;    // any strides, one key split per workgroup (p.nsplit splits)
  int ksplit;               // wavefronts splitting one query block's keys (0 or 1: none)
  int (*resident)();        // fa_fwd_kernel tiles: workgroups of the contiguous kernel per CU
};

// 0 and 1 both mean "each wavefront owns its own queries".
int ksplit_of(int k) { return k > 1 ? k : 1; }

int device_cus();

// Workgroups of this kernel resident on one CU at a time (from the occupancy
// calculator, once per instantiation; at least 1).
template <int D, bool CAUSAL, int QB, int WAVES, int BK, bool STRIDED, bool SPLIT, typename E>
int resident_per_cu() {
  static std::atomic<int> cached{0};
  int r = cached.load(std::memory_order_relaxed);
  if (r == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fa::fa_fwd_kernel<D, CAUSAL, QB, WAVES, BK, STRIDED, SPLIT, E>,
                                                     WAVES * 64, 0) != hipSuccess || n < 1)
      n = 1;
    cached.store(n, std::memory_order_relaxed);
    r = n;
  }
  return r;
}

template <int D, bool CAUSAL, int QB, int WAVES, int BK, bool STRIDED, bool SPLIT, typename E>
hipError_t launch_variant(const fa::Params& p, int B, hipStream_t stream) {
  using T = fa::Tile<D, QB, WAVES, BK>;
  fa::Params pr = p;
  pr.nqt = (p.Nq + T::kBQ - 1) / T::kBQ;
  pr.resident = 1;
  pr.cus = 0;
  if (CAUSAL && !SPLIT) {
    pr.resident = resident_per_cu<D, CAUSAL, QB, WAVES, BK, STRIDED, SPLIT, E>();
    pr.cus = device_cus();
  }
  const long long blocks = (long long)B * p.H * pr.nqt * (SPLIT ? p.nsplit : 1);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa::fa_fwd_kernel<D, CAUSAL, QB, WAVES, BK, STRIDED, SPLIT, E>), dim3((unsigned)blocks),
                     dim3(T::kThreads), 0, stream, pr);
  return hipGetLastError();
}

// Key split inside the workgroup: S wavefronts share each block of 32 queries
// (SPLIT: one workgroup per key split as well, p.nsplit of them).
template <int D, bool CAUSAL, int S, int BK, bool STRIDED, typename E, bool SPLIT = false>
hipError_t launch_wsplit(const fa::Params& p, int B, hipStream_t stream) {
  fa::Params pr = p;
  pr.nqt = (p.Nq + 31) / 32;
  const long long blocks = (long long)B * p.H * pr.nqt * (SPLIT ? p.nsplit : 1);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa::fa_fwd_wsplit_kernel<D, CAUSAL, S, BK, STRIDED, E, SPLIT>), dim3((unsigned)blocks),
                     dim3(S * 64), 0, stream, pr);
  return hipGetLastError();
}

template <int D, typename E>
hipError_t launch_merge(const fa::Params& p, hipStream_t stream) {
  const long long rows = (long long)p.BH * p.Nq;
  const long long blocks = (rows + (256 / (D / 4)) - 1) / (256 / (D / 4));
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa::fa_merge_kernel<D, E>), dim3((unsigned)blocks), dim3(256), 0, stream, p, rows);
  return hipGetLastError();
}

// fp32 inputs: 4 wavefronts of 32 queries, BK-key tiles (no split variant).
template <int D, bool CAUSAL, int WAVES, int BK, bool STRIDED>
hipError_t launch_f32(const fa::Params& p, int B, hipStream_t stream) {
  fa::Params pr = p;
  pr.nqt = (p.Nq + WAVES * 32 - 1) / (WAVES * 32);
  const long long blocks = (long long)B * p.H * pr.nqt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa::fa_fwd_f32_kernel<D, CAUSAL, WAVES, BK, STRIDED>), dim3((unsigned)blocks),
                     dim3(WAVES * 64), 0, stream, pr);
  return hipGetLastError();
}

hipError_t run_merge(const fa::Params& p, int d, int dtype, hipStream_t s) {
  if (dtype == FA_DTYPE_F16) {
    switch (d) {
      case 32: return launch_merge<32, fa::F16>(p, s);
      case 64: return launch_merge<64, fa::F16>(p, s);
      case 128: return launch_merge<128, fa::F16>(p, s);
      default: return launch_merge<256, fa::F16>(p, s);
    }
  }
  switch (d) {
    case 32: return launch_merge<32, fa::Bf16>(p, s);
    case 64: return launch_merge<64, fa::Bf16>(p, s);
    case 128: return launch_merge<128, fa::Bf16>(p, s);
    default: return launch_merge<256, fa::Bf16>(p, s);
  }
}

#define FA_VARIANT_T(D, C, QB, W, BK, T, DT)                                                          \
  {D, C, QB, W, BK, DT, &launch_variant<D, (C) != 0, QB, W, BK, false, false, T>,                     \
   &launch_variant<D, (C) != 0, QB, W, BK, true, false, T>, &launch_variant<D, (C) != 0, QB, W, BK, true, true, T>, \
   0, &resident_per_cu<D, (C) != 0, QB, W, BK, false, false, T>}
#define FA_VARIANT(D, C, QB, W, BK) FA_VARIANT_T(D, C, QB, W, BK, fa::Bf16, FA_DTYPE_BF16)
#define FA_VARIANT16(D, C, QB, W, BK) FA_VARIANT_T(D, C, QB, W, BK, fa::F16, FA_DTYPE_F16)
#define FA_VARIANT32(D, C, W, BK)                                                                        \
  {D, C, 1, W, BK, FA_DTYPE_F32, &launch_f32<D, (C) != 0, W, BK, false>, &launch_f32<D, (C) != 0, W, BK, true>, \
   nullptr}
// The key-split tile (1, 4, 32) with ksplit 4: four wavefronts per 32-query
// block, 32-key tiles in a ring per wavefront (32 KB of LDS at d = 32, 64 KB at
// d = 64, 128 KB at d = 128); also the split path's tile for short query ranges.
#define FA_VARIANT_KS(D, C, T, DT)                                                                     \
  {D, C, 1, 4, 32, DT, &launch_wsplit<D, (C) != 0, 4, 32, false, T>, &launch_wsplit<D, (C) != 0, 4, 32, true, T>, \
   &launch_wsplit<D, (C) != 0, 4, 32, true, T, true>, 4}
#define FA_VARIANTS_KS(D, C) FA_VARIANT_KS(D, C, fa::Bf16, FA_DTYPE_BF16), FA_VARIANT_KS(D, C, fa::F16, FA_DTYPE_F16)
#define FA_VARIANTS_DC(D, C) \
  FA_VARIANT(D, C, 1, 4, 64), FA_VARIANT(D, C, 2, 4, 64), FA_VARIANT(D, C, 1, 8, 64)
// Head dims 32 and 256 and the fp16 element type: the default tile and the
// 4-wave tile of the split path (d = 256: 32-key tiles, one configuration).
#define FA_VARIANTS_SMALL(MAC, D, C) MAC(D, C, 1, 8, 64), MAC(D, C, 1, 4, 64)

const Variant kVariants[] = {
    FA_VARIANTS_DC(64, 0), FA_VARIANTS_DC(64, 1), FA_VARIANTS_DC(128, 0), FA_VARIANTS_DC(128, 1),
    FA_VARIANTS_SMALL(FA_VARIANT, 32, 0), FA_VARIANTS_SMALL(FA_VARIANT, 32, 1),
    FA_VARIANT(256, 0, 1, 4, 32), FA_VARIANT(256, 1, 1, 4, 32),
    FA_VARIANTS_SMALL(FA_VARIANT16, 32, 0), FA_VARIANTS_SMALL(FA_VARIANT16, 32, 1),
    FA_VARIANTS_SMALL(FA_VARIANT16, 64, 0), FA_VARIANTS_SMALL(FA_VARIANT16, 64, 1),
    FA_VARIANTS_SMALL(FA_VARIANT16, 128, 0), FA_VARIANTS_SMALL(FA_VARIANT16, 128, 1),
    FA_VARIANT16(256, 0, 1, 4, 32), FA_VARIANT16(256, 1, 1, 4, 32),
    // 12 wavefronts (three per SIMD) at d = 64, non-causal: grids that 384-query
    // tiles spread more evenly over the compute units than 256-query tiles
    FA_VARIANT(64, 0, 1, 12, 64), FA_VARIANT16(64, 0, 1, 12, 64),
    // 32-key tiles at d = 64, non-causal: few enough registers for two 8-wavefront
    // workgroups (four wavefronts) per SIMD
    FA_VARIANT(64, 0, 1, 8, 32), FA_VARIANT16(64, 0, 1, 8, 32),
    // one wavefront of 32 queries: the split path's tile for decoding (Nq <= 32)
    FA_VARIANT(64, 0, 1, 1, 64), FA_VARIANT(64, 1, 1, 1, 64), FA_VARIANT(128, 0, 1, 1, 32),
    FA_VARIANT(128, 1, 1, 1, 32), FA_VARIANT16(64, 0, 1, 1, 64), FA_VARIANT16(64, 1, 1, 1, 64),
    FA_VARIANT16(128, 0, 1, 1, 32), FA_VARIANT16(128, 1, 1, 1, 32),
    FA_VARIANT32(64, 0, 4, 32), FA_VARIANT32(64, 1, 4, 32), FA_VARIANT32(128, 0, 4, 32),
    FA_VARIANT32(128, 1, 4, 32),
    FA_VARIANTS_KS(32, 0), FA_VARIANTS_KS(32, 1), FA_VARIANTS_KS(64, 0), FA_VARIANTS_KS(64, 1),
    FA_VARIANTS_KS(128, 0), FA_VARIANTS_KS(128, 1),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

const Variant* find_variant(int d, int causal, const fa_tile_cfg& c, int dtype = FA_DTYPE_BF16) {
  for (const Variant& v : kVariants)
    if (v.d == d && v.causal == causal && v.dtype == dtype && v.qb == c.qb && v.waves == c.waves && v.bk == c.bk &&
        ksplit_of(v.ksplit) == ksplit_of(c.ksplit))
      return &v;
  return nullptr;
}

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

// 8 wavefronts of 32 queries, 64-key tiles; d = 256 (512-byte rows, twice the
// registers per query) takes 4 wavefronts and 32-key tiles.
fa_tile_cfg default_cfg(int /*N*/, int d, int /*causal*/) {
  return d == 256 ? fa_tile_cfg{1, 4, 32} : fa_tile_cfg{1, 8, 64};
}

// The fp32 path's one configuration: 4 wavefronts, 32-key tiles.
fa_tile_cfg default_cfg_dt(int N, int d, int causal, int dtype) {
  return dtype == FA_DTYPE_F32 ? fa_tile_cfg{1, 4, 32} : default_cfg(N, d, causal);
}

int elem_bytes(int dtype) { return dtype == FA_DTYPE_F32 ? 4 : 2; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + bn && pb < pa + an;
}

// Host-only argument checks, in a fixed order; no HIP call is made here.
int validate(const void* q, const void* k, const void* v, const void* out, const float* lse, int B, int H,
             int N, int d, float scale, int causal) {
  if (!q || !k || !v || !out || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEAD_DIM;
  const long long elems = (long long)B * H * N * d;
  if ((long long)(N + 256) * d >= (1LL << 30) || elems >= (1LL << 31)) return FA_ERR_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  if (!al(q, 16) || !al(k, 16) || !al(v, 16) || !al(out, 16) || !al(lse, 4)) return FA_ERR_ALIGN;
  const size_t tbytes = (size_t)elems * 2, lbytes = (size_t)B * H * N * 4;
  for (const void* in : {q, k, v})
    if (overlaps(out, tbytes, in, tbytes) || overlaps(lse, lbytes, in, tbytes)) return FA_ERR_ALIAS;
  if (overlaps(out, tbytes, lse, lbytes)) return FA_ERR_ALIAS;
  return FA_OK;
}

// Per-device "is this a gfx950" and compute-unit count cache, filled once per
// device.
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];
int g_dev_cus[kMaxDevices];

// FA_OK with *cus = the current device's compute units, or FA_ERR_NO_DEVICE.
int check_device(int* cus = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_NO_DEVICE;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t p;
    g_dev_ok[dev] = hipGetDeviceProperties(&p, dev) == hipSuccess && std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[dev] = g_dev_ok[dev] ? p.multiProcessorCount : 0;
  });
  if (cus) *cus = g_dev_cus[dev];
  return g_dev_ok[dev] ? FA_OK : FA_ERR_NO_DEVICE;
}

// The current device's compute units (0 when unknown); check_device has run.
int device_cus() {
  int cus = 0;
  return check_device(&cus) == FA_OK ? cus : 0;
}

// How evenly a causal launch of fa_fwd_kernel with `rows`-query tiles loads the
// compute units: the launch order (causal_order) replayed on one XCD (on each
// when the heads do not split evenly over the 8 XCDs), the first `res` layers
// of its workgroups placed round-robin over the XCD's CUs as the order assumes
// and every later one on the CU with the least work so far; a workgroup's work
// is the number of 64-key tiles it visits.  Returns the mean over the largest
// per-CU work (1: even), the smallest over the XCDs.
double causal_balance(int BH, int Nq, int rows, int res, int cus) {
  const int nqt = (Nq + rows - 1) / rows;
  const long long total = (long long)BH * nqt;
  const int cpx = std::max(1, cus / 8);
  const int xcds = ((BH % 8) == 0 && (cus % 8) == 0) ? 1 : 8;  // one XCD stands for all when they match
  std::vector<double> work(cpx);
  double worst = 1.0;
  for (int x = 0; x < xcds; ++x) {
    std::fill(work.begin(), work.end(), 0.0);
    long long k = 0;
    for (long long i = x; i < total; i += 8, ++k) {
      int bh, qt;
      fa::causal_order((int)i, (int)total, BH, nqt, res, cus, bh, qt);
      const double w = (double)((std::min(qt * rows + rows, Nq) + 63) / 64);
      const long long c = k < (long long)cpx * res ? k % cpx : std::min_element(work.begin(), work.end()) - work.begin();
      work[c] += w;
    }
    double sum = 0.0, mx = 0.0;
    for (double v : work) sum += v, mx = std::max(mx, v);
    if (mx > 0.0) worst = std::min(worst, sum / cpx / mx);
  }
  return worst;
}

// The tile a launch uses when the caller names none: default_cfg_dt (one tile
// at d = 256 and for fp32), and at d = 32, 64 and 128 (bf16, fp16) a choice by
// grid size, from tile sweeps on MI355X.  With w8 = B*H*ceil(Nq/256) workgroups
// of the 8-wavefront tile (one per CU at a time) and w4 = B*H*ceil(Nq/128) of
// the 4-wavefront tile (1, 4, 64):
// * Non-causal: the key-split tile (1, 4, 32, ksplit 4: four wavefronts share
//   each block of 32 queries and split its keys) while 2*w4 <= CUs (d = 128: its
//   one workgroup per CU needs 4*w4 <= CUs, or rows of 1024 or more); (1, 4, 64)
//   while w4 <= CUs (d = 32: while w8 <= CUs, five 4-wavefront workgroups fit
//   a CU there); beyond, every query tile costs the same, so a launch lasts
//   about as long as the busiest CU, which runs ceil(workgroups / CUs) tiles of
//   `waves` wavefronts each: of the 8-, 12- (d = 64) and 4-wavefront tiles and
//   the 8-wavefront tile with 32-key tiles (d = 64; 108 registers, so two of its
//   workgroups share a CU) the one with the least such work, each weighed by its
//   measured speed (per mille of the 8-wavefront tile's time: 12 waves 975,
//   4 waves 1025 at d = 32, 1030 at d = 64 and 1050 at d = 128, 32-key tiles 970
//   when some CU gets two workgroups and 1075 when none does); ties keep the
//   8-wavefront tile.
// * Causal: work per query tile grows along the diagonal.  The key-split tile
//   while w8 < CUs (at d = 128 only while w4 < CUs, or w4 = CUs with Nq >= 2048:
//   its 128 KB of LDS leave one workgroup per CU, and four layers of short
//   rows cost more than they balance; at d = 32, with 32 KB, up to w8 <= 1.5
//   CUs).  Beyond, (1, 4, 64) where the 8-wavefront tile's launch order loads
//   the CUs unevenly (causal_balance < 0.97: one layer of tiles, or groups of
//   heads that do not pair long tiles with short ones), since its smaller tiles
//   and several workgroups per CU even that out -- unless its own order balances
//   worse; where both are even, (1, 8, 64), except from 4 layers on at d = 64
//   (three 4-wavefront workgroups per CU against one of 8 wavefronts) and at
//   d = 32 for rows up to 4096.
fa_tile_cfg launch_cfg(int B, int H, int Nq, int d, int causal, int dtype, int cus) {
  const fa_tile_cfg c = default_cfg_dt(Nq, d, causal, dtype);
  if (c.waves != 8 || cus <= 0) return c;
  const fa_tile_cfg ks{1, 4, 32, 4}, four{1, 4, 64};
  auto wgs = [&](const fa_tile_cfg& t) {
    return (long long)B * H * ((Nq + t.qb * t.waves * 32 - 1) / (t.qb * t.waves * 32));
  };
  const long long w8 = wgs(c), w4 = wgs(four);
  const bool has_ks = find_variant(d, causal, ks, dtype) != nullptr;
  const Variant* v4 = find_variant(d, causal, four, dtype);
  if (!causal) {
    if (2 * w4 <= cus && has_ks && (d != 128 || 4 * w4 <= cus || Nq >= 1024)) return ks;
    if ((w4 <= cus || (d == 32 && w8 <= cus)) && v4) return four;
    // Per mille of the 8-wavefront tile's time per workgroup; the 32-key tile
    // (d = 64) runs two workgroups per CU, faster once some CU gets two.
    struct Option { fa_tile_cfg t; long long permille, permille_alone; };
    const long long p4 = d == 32 ? 1025 : d == 64 ? 1030 : 1050;
    const Option opts[] = {{{1, 8, 64}, 1000, 1000}, {{1, 8, 32}, 970, 1075}, {{1, 12, 64}, 975, 975}, {{1, 4, 64}, p4, p4}};
    fa_tile_cfg best = c;
    long long best_cost = -1;
    for (const Option& o : opts) {
      if (!find_variant(d, causal, o.t, dtype)) continue;
      const long long n = wgs(o.t);
      const long long cost = (n + cus - 1) / cus * o.t.waves * (n > cus ? o.permille : o.permille_alone);
      if (best_cost < 0 || cost < best_cost) best_cost = cost, best = o.t;
    }
    return best;
  }
  if (!v4) return c;
  if (has_ks && (w8 < cus ? d <= 64 || w4 < cus || (w4 == cus && Nq >= 2048) : d == 32 && 2 * w8 <= 3LL * cus))
    return ks;
  // The balance replay costs a few microseconds; remember the last answers.
  struct Memo { long long bh; int nq, d, dtype, cus; fa_tile_cfg cfg; };
  thread_local Memo memo[8];
  thread_local int memo_next = 0;
  const long long BH = (long long)B * H;
  for (const Memo& m : memo)
    if (m.bh == BH && m.nq == Nq && m.d == d && m.dtype == dtype && m.cus == cus) return m.cfg;
  auto res = [](const Variant* v) { return v && v->resident ? v->resident() : 1; };
  // Past 16 layers both orders are taken as even (the replay would cost more).
  const bool replay = w8 <= 16LL * cus;
  const double b8 = w8 < cus ? 0.0 : replay ? causal_balance((int)BH, Nq, 256, res(find_variant(d, causal, c, dtype)), cus) : 1.0;
  const double b4 = replay ? causal_balance((int)BH, Nq, 128, res(v4), cus) : 1.0;
  fa_tile_cfg pick = four;
  if (b4 < b8) {
    pick = c;
  } else if (b8 >= 0.97) {
    // Both even: from four layers on the 4-wavefront tile's extra workgroup
    // per CU wins at d = 64 (three against two wavefronts per SIMD) and, for
    // rows up to 4096, at d = 32; otherwise the 8-wavefront tile.
    const bool long_grid = w8 >= 4LL * cus;
    pick = long_grid && (d == 64 || (d == 32 && Nq <= 4096)) ? four : c;
  }
  memo[memo_next] = Memo{BH, Nq, d, dtype, cus, pick};
  memo_next = (memo_next + 1) % 8;
  return pick;
}

// Byte extent of a strided [B, H, N, d] tensor: from its base to one past its
// last element.
long long extent_bytes(const long long st[3], int B, int H, int N, int d, int elem) {
  return ((long long)(B - 1) * st[0] + (long long)(H - 1) * st[1] + (long long)(N - 1) * st[2] + d) * elem;
}

// Strides in elements of `elem` bytes: >= 0, whole 16-byte units, rows at
// least d long, and (N + 256) rows within 2^31 bytes (one head's buffer range).
bool strides_ok(const long long st[3], int N, int d, int elem = 2) {
  const long long unit = 16 / elem;
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || st[i] % unit != 0 || st[i] > (1LL << 40)) return false;
  return st[2] >= d && (long long)(N + 256) * st[2] * elem < (1LL << 31);
}

// Every element of a strided [B, H, N, d] view has an address of its own: with
// the dimensions ordered by stride, each stride is at least the span of all the
// smaller ones (the contiguous head dimension spans d; size-1 dimensions impose
// nothing).  Sufficient, and what a written tensor needs so that no two lanes
// store to one element.
bool self_disjoint(const long long st[3], int B, int H, int N, int d) {
  long long dims[3][2] = {{st[0], B}, {st[1], H}, {st[2], N}};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (dims[j][0] < dims[i][0]) std::swap(dims[i], dims[j]);
  long long span = d;
  for (const auto& dm : dims) {
    if (dm[1] == 1) continue;
    if (dm[0] < span) return false;
    span += dm[0] * (dm[1] - 1);
  }
  return true;
}

// Host-only checks of a descriptor, in a fixed order; no HIP call is made here.
int validate_desc(const fa_fwd_desc& a) {
  if (!a.q || !a.k || !a.v || !a.out || !a.lse) return FA_ERR_NULL;
  if (a.B < 1 || a.H < 1 || a.Nq < 1 || a.Nk < 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(a.d)) return FA_ERR_HEAD_DIM;
  if (a.dtype == FA_DTYPE_F32 && a.d != 64 && a.d != 128) return FA_ERR_HEAD_DIM;
  if ((long long)a.B * a.H > 0x7fffffffLL) return FA_ERR_SHAPE;
  const int eb = elem_bytes(a.dtype);
  if (!strides_ok(a.q_stride, a.Nq, a.d, eb) || !strides_ok(a.k_stride, a.Nk, a.d, eb) ||
      !strides_ok(a.v_stride, a.Nk, a.d, eb) || !strides_ok(a.o_stride, a.Nq, a.d, eb))
    return FA_ERR_STRIDE;
  if (a.lse_stride[0] < 0 || a.lse_stride[1] < 0 || a.lse_stride[0] > (1LL << 40) || a.lse_stride[1] > (1LL << 40))
    return FA_ERR_STRIDE;
  if (!std::isfinite(a.scale) || !(a.scale > 0.f)) return FA_ERR_SCALE;
  if (a.causal != 0 && a.causal != 1) return FA_ERR_ARG;
  if (a.dtype != FA_DTYPE_BF16 && a.dtype != FA_DTYPE_F16 && a.dtype != FA_DTYPE_F32) return FA_ERR_ARG;
  auto al = [](const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; };
  if (!al(a.q, 16) || !al(a.k, 16) || !al(a.v, 16) || !al(a.out, 16) || !al(a.lse, 4)) return FA_ERR_ALIGN;
  const long long qb = extent_bytes(a.q_stride, a.B, a.H, a.Nq, a.d, eb);
  const long long kb = extent_bytes(a.k_stride, a.B, a.H, a.Nk, a.d, eb);
  const long long vb = extent_bytes(a.v_stride, a.B, a.H, a.Nk, a.d, eb);
  const long long ob = extent_bytes(a.o_stride, a.B, a.H, a.Nq, a.d, eb);
  const long long lst[3] = {a.lse_stride[0], a.lse_stride[1], 1};
  const long long lb = extent_bytes(lst, a.B, a.H, a.Nq, 1, 4);
  const std::pair<const void*, long long> ins[3] = {{a.q, qb}, {a.k, kb}, {a.v, vb}};
  for (const auto& in : ins)
    if (overlaps(a.out, (size_t)ob, in.first, (size_t)in.second) || overlaps(a.lse, (size_t)lb, in.first, (size_t)in.second))
      return FA_ERR_ALIAS;
  if (overlaps(a.out, (size_t)ob, a.lse, (size_t)lb)) return FA_ERR_ALIAS;
  const long long lst2[3] = {a.lse_stride[0], a.lse_stride[1], 1};
  if (!self_disjoint(a.o_stride, a.B, a.H, a.Nq, a.d) || !self_disjoint(lst2, a.B, a.H, a.Nq, 1)) return FA_ERR_ALIAS;
  return FA_OK;
}

// Kernel arguments of a (validated) descriptor.
fa::Params make_params(const fa_fwd_desc& a) {
  fa::Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.out = static_cast<uint16_t*>(a.out);
  p.lse = a.lse;
  p.q_sb = a.q_stride[0], p.q_sh = a.q_stride[1], p.q_rs = (int)a.q_stride[2];
  p.k_sb = a.k_stride[0], p.k_sh = a.k_stride[1], p.k_rs = (int)a.k_stride[2];
  p.v_sb = a.v_stride[0], p.v_sh = a.v_stride[1], p.v_rs = (int)a.v_stride[2];
  p.o_sb = a.o_stride[0], p.o_sh = a.o_stride[1], p.o_rs = (int)a.o_stride[2];
  p.l_sb = a.lse_stride[0], p.l_sh = a.lse_stride[1];
  p.H = a.H, p.BH = a.B * a.H, p.Nq = a.Nq, p.Nk = a.Nk;
  // Scores are kept raw; exp(scale*s - m) = 2^(s*scale*log2(e) - m') with m' in
  // log2 units, so the scale and log2(e) fold into one constant.
  p.qk_scale = (float)((double)a.scale * 1.4426950408889634);
  p.nsplit = 1;
  return p;
}

// cfg = nullptr: launch_cfg's choice for this device.
int run_desc(const fa_fwd_desc& a, const fa_tile_cfg* cfg) {
  const int st = validate_desc(a);
  if (st != FA_OK) return st;
  if (cfg && !find_variant(a.d, a.causal, *cfg, a.dtype)) return FA_ERR_ARG;
  int cus = 0;
  const int dst = check_device(&cus);
  if (dst != FA_OK) return dst;
  const Variant* var =
      find_variant(a.d, a.causal, cfg ? *cfg : launch_cfg(a.B, a.H, a.Nq, a.d, a.causal, a.dtype, cus), a.dtype);
  if (!var) return FA_ERR_INTERNAL;
  fa::Params p = make_params(a);
  auto contiguous = [&](const long long st[3], int n) {
    return st[0] == (long long)a.H * n * a.d && st[1] == (long long)n * a.d && st[2] == a.d;
  };
  const bool dense = contiguous(a.q_stride, a.Nq) && contiguous(a.k_stride, a.Nk) && contiguous(a.v_stride, a.Nk) &&
                     contiguous(a.o_stride, a.Nq) && a.lse_stride[0] == (long long)a.H * a.Nq &&
                     a.lse_stride[1] == a.Nq;
  const hipError_t e = (dense ? var->launch : var->launch_strided)(p, a.B, static_cast<hipStream_t>(a.stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// ---- key splits -------------------------------------------------------------------
// Keys per split: Nk / S rounded up to whole key tiles of 64.
constexpr int kSplitTile = 64;
int split_chunk(int Nk, int S) {
  const int c = (Nk + S - 1) / S;
  return (c + kSplitTile - 1) / kSplitTile * kSplitTile;
}
int split_count(int Nk, int S) {
  const int c = split_chunk(Nk, S);
  return (Nk + c - 1) / c;
}
long long split_workspace(int B, int H, int Nq, int d, int S_eff) {
  return (long long)S_eff * B * H * Nq * (d + 1) * 4;
}

// Tile configuration of the split path: short query ranges take smaller
// workgroups so fewer MFMA rows are padding -- the key-split tile when Nq <= 32
// (decoding: one block of 32 queries whose four wavefronts each stream their
// own key tiles, so four key streams per split are in flight), the 4-wave,
// 128-query tile when Nq <= 128 (d = 256 has the 4-wave tiles only).
fa_tile_cfg split_cfg(int Nq, int Nk, int d, int causal) {
  if (Nq <= 32 && d != 256) return fa_tile_cfg{1, 4, 32, 4};
  return Nq <= 128 && d != 256 ? fa_tile_cfg{1, 4, 64} : default_cfg(Nk, d, causal);
}

// (the same for both masks, so the workspace query needs no causal flag)
int default_splits(int B, int H, int Nq, int Nk, int d) {
  const fa_tile_cfg c = split_cfg(Nq, Nk, d, 0);
  const int rows = c.ksplit > 1 ? 32 : c.waves * c.qb * 32;  // query rows per workgroup
  const long long wgs = (long long)B * H * ((Nq + rows - 1) / rows);
  long long s;
  if (c.ksplit > 1) {
    // key-split tile: about 256 workgroups (one per CU at d = 128's 128 KB of
    // LDS), at least 512 keys per split (four 32-key tiles per wavefront)
    s = (256 + wgs - 1) / wgs;
    s = std::min<long long>(s, std::max(1, Nk / 512));
  } else {
    s = (512 + wgs - 1) / wgs;  // about 512 workgroups
    s = std::min<long long>(s, std::max(1, Nk / 256));  // at least 256 keys per split
  }
  return (int)std::max<long long>(1, std::min<long long>(s, 1024));
}

int run_splitkv(const fa_fwd_desc& a, int num_splits, void* ws, long long ws_bytes) {
  const int st = validate_desc(a);
  if (st != FA_OK) return st;
  if (a.dtype == FA_DTYPE_F32) return FA_ERR_ARG;  // no split instantiation of the fp32 kernel
  if (num_splits < 0 || num_splits > 1024) return FA_ERR_ARG;
  const int S = num_splits ? num_splits : default_splits(a.B, a.H, a.Nq, a.Nk, a.d);
  const int S_eff = split_count(a.Nk, S);
  const long long need = split_workspace(a.B, a.H, a.Nq, a.d, S_eff);
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) != 0 || ws_bytes < need) return FA_ERR_WORKSPACE;
  const std::pair<const void*, long long> others[5] = {
      {a.q, extent_bytes(a.q_stride, a.B, a.H, a.Nq, a.d, 2)},
      {a.k, extent_bytes(a.k_stride, a.B, a.H, a.Nk, a.d, 2)},
      {a.v, extent_bytes(a.v_stride, a.B, a.H, a.Nk, a.d, 2)},
      {a.out, extent_bytes(a.o_stride, a.B, a.H, a.Nq, a.d, 2)},
      {a.lse, 4 * ((long long)(a.B - 1) * a.lse_stride[0] + (long long)(a.H - 1) * a.lse_stride[1] + a.Nq)}};
  for (const auto& o : others)
    if (overlaps(ws, (size_t)need, o.first, (size_t)o.second)) return FA_ERR_ALIAS;
  const Variant* var = find_variant(a.d, a.causal, split_cfg(a.Nq, a.Nk, a.d, a.causal), a.dtype);
  if (!var) return FA_ERR_INTERNAL;
  const int dst = check_device();
  if (dst != FA_OK) return dst;
  fa::Params p = make_params(a);
  p.nsplit = S_eff;
  p.chunk = split_chunk(a.Nk, S);
  p.part_o = static_cast<float*>(ws);
  p.part_lse = p.part_o + (long long)S_eff * a.B * a.H * a.Nq * a.d;
  const hipStream_t stream = static_cast<hipStream_t>(a.stream);
  hipError_t e = var->launch_split(p, a.B, stream);
  if (e == hipSuccess) e = run_merge(p, a.d, a.dtype, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// ---- key splits without an allocation ---------------------------------------------
// The partial results of fa_fwd_splitkv_noalloc live in this file-scope device
// array instead of a caller's workspace: every GPU the library runs on holds
// one copy until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the device symbol); it
// uses the device address hipGetSymbolAddress returns, looked up once per
// device with that device current.
static __device__ __attribute__((aligned(256))) unsigned char scratch[FA_SPLITKV_NOALLOC_MAX_BYTES];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// FA_OK with *ptr = this device's copy of `scratch`, or an error code.
int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_NO_DEVICE;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_ptr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  if (!g_scratch_ptr[dev]) return FA_ERR_INTERNAL;
  *ptr = g_scratch_ptr[dev];
  return FA_OK;
}

int run_splitkv_noalloc(const fa_fwd_desc& a, int num_splits) {
  const int st = validate_desc(a);
  if (st != FA_OK) return st;
  if (a.dtype == FA_DTYPE_F32) return FA_ERR_ARG;
  if (num_splits < 0 || num_splits > 1024) return FA_ERR_ARG;
  const int S = num_splits ? num_splits : default_splits(a.B, a.H, a.Nq, a.Nk, a.d);
  if (split_workspace(a.B, a.H, a.Nq, a.d, split_count(a.Nk, S)) > FA_SPLITKV_NOALLOC_MAX_BYTES)
    return FA_ERR_SCRATCH;
  const int dst = check_device();
  if (dst != FA_OK) return dst;
  void* ws = nullptr;
  const int sst = scratch_address(&ws);
  if (sst != FA_OK) return sst;
  return run_splitkv(a, num_splits, ws, FA_SPLITKV_NOALLOC_MAX_BYTES);
}

// The square, contiguous call as a descriptor.
fa_fwd_desc square_desc(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N,
                        int d, float scale, int causal, void* stream) {
  fa_fwd_desc a{};
  a.q = q, a.k = k, a.v = v, a.out = out, a.lse = lse;
  a.B = B, a.H = H, a.Nq = N, a.Nk = N, a.d = d;
  const long long st[3] = {(long long)H * N * d, (long long)N * d, d};
  for (int i = 0; i < 3; ++i) a.q_stride[i] = a.k_stride[i] = a.v_stride[i] = a.o_stride[i] = st[i];
  a.lse_stride[0] = (long long)H * N, a.lse_stride[1] = N;
  a.scale = scale, a.causal = causal, a.stream = stream;
  return a;
}

int run(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N, int d,
        float scale, int causal, void* stream, const fa_tile_cfg* cfg) {
  const int st = validate(q, k, v, out, lse, B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  return run_desc(square_desc(q, k, v, out, lse, B, H, N, d, scale, causal, stream), cfg);
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N, int d,
           float scale, int causal, void* stream) {
  try {
    return run(q, k, v, out, lse, B, H, N, d, scale, causal, stream, nullptr);
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

int fa_fwd_cfg(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N, int d,
               float scale, int causal, void* stream, const fa_tile_cfg* cfg) {
  if (!cfg) return FA_ERR_ARG;
  try {
    return run(q, k, v, out, lse, B, H, N, d, scale, causal, stream, cfg);
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

int fa_fwd_ex(const fa_fwd_desc* desc) {
  if (!desc) return FA_ERR_NULL;
  try {
    return run_desc(*desc, nullptr);
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

int fa_fwd_ex_cfg(const fa_fwd_desc* desc, const fa_tile_cfg* cfg) {
  if (!desc) return FA_ERR_NULL;
  if (!cfg) return FA_ERR_ARG;
  try {
    return run_desc(*desc, cfg);
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

int fa_splitkv_default_splits(int B, int H, int Nq, int Nk, int d, int causal) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return -FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return -FA_ERR_HEAD_DIM;
  (void)causal;
  return default_splits(B, H, Nq, Nk, d);
}

long long fa_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return -FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return -FA_ERR_HEAD_DIM;
  if (num_splits < 0 || num_splits > 1024) return -FA_ERR_ARG;
  const int S = num_splits ? num_splits : default_splits(B, H, Nq, Nk, d);
  return split_workspace(B, H, Nq, d, split_count(Nk, S));
}

int fa_fwd_splitkv(const fa_fwd_desc* desc, int num_splits, void* workspace, long long workspace_bytes) {
  if (!desc) return FA_ERR_NULL;
  try {
    return run_splitkv(*desc, num_splits, workspace, workspace_bytes);
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

int fa_fwd_splitkv_noalloc(const fa_fwd_desc* desc, int num_splits) {
  if (!desc) return FA_ERR_NULL;
  try {
    return run_splitkv_noalloc(*desc, num_splits);
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

int fa_launch_cfg(int B, int H, int Nq, int d, int causal, int dtype, fa_tile_cfg* cfg) {
  if (!cfg) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d) || (dtype == FA_DTYPE_F32 && d != 64 && d != 128)) return FA_ERR_HEAD_DIM;
  if ((causal != 0 && causal != 1) || dtype < FA_DTYPE_BF16 || dtype > FA_DTYPE_F32) return FA_ERR_ARG;
  try {
    int cus = 0;
    const int st = check_device(&cus);
    if (st != FA_OK) return st;
    *cfg = launch_cfg(B, H, Nq, d, causal, dtype, cus);
    cfg->ksplit = ksplit_of(cfg->ksplit);
    return FA_OK;
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

int fa_default_cfg(int N, int d, int causal, fa_tile_cfg* cfg) {
  if (!cfg) return FA_ERR_NULL;
  if (N < 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEAD_DIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  *cfg = default_cfg(N, d, causal);
  cfg->ksplit = 1;
  return FA_OK;
}

int fa_num_variants(void) { return kNumVariants; }

int fa_variant(int i, int* d, int* causal, fa_tile_cfg* cfg) {
  if (i < 0 || i >= kNumVariants) return FA_ERR_ARG;
  if (!d || !causal || !cfg) return FA_ERR_NULL;
  *d = kVariants[i].d;
  *causal = kVariants[i].causal;
  *cfg = fa_tile_cfg{kVariants[i].qb, kVariants[i].waves, kVariants[i].bk, ksplit_of(kVariants[i].ksplit)};
  return FA_OK;
}

int fa_variant_dtype(int i) {
  if (i < 0 || i >= kNumVariants) return -FA_ERR_ARG;
  return kVariants[i].dtype;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer argument";
    case FA_ERR_SHAPE: return "B, H, N must be >= 1, tensors below 2^31 elements and (N + 256) * d below 2^30";
    case FA_ERR_HEAD_DIM: return "head dimension must be 32, 64, 128 or 256";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ARG: return "invalid argument (causal must be 0 or 1, dtype bf16, f16 or f32; tile configuration or path not compiled for it)";
    case FA_ERR_ALIGN: return "q, k, v, out must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ALIAS: return "out/lse overlap an input or each other";
    case FA_ERR_NO_DEVICE: return "no current HIP device, or it is not gfx950";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_INTERNAL: return "internal error";
    case FA_ERR_WORKSPACE: return "workspace missing, not 256-byte aligned or smaller than fa_splitkv_workspace_bytes";
    case FA_ERR_STRIDE: return "a stride is negative, not a multiple of 8 elements, shorter than a row, or too large";
    case FA_ERR_SCRATCH: return "the split-key partial results exceed the static scratch (FA_SPLITKV_NOALLOC_MAX_BYTES)";
    default: return "unknown status";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
