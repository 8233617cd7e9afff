// C ABI of the gfx950 FlashAttention-2 backward: argument checks and the three
// launches (D / LSE preprocessing, dK and dV, dQ), for bf16 or fp16 tensors,
// contiguous or strided.  Declared in include/fa_bwd.h.
#include "fa_bwd.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <utility>

#include "fa_bwd_kernel.hpp"

namespace {

// dK/dV workgroup: d = 64, 4 wavefronts with K and V in VGPRs (two workgroups
// per CU); d = 128, 8 wavefronts with V resident in LDS (one workgroup per CU,
// two wavefronts per SIMD either way).
#ifndef FA_DKDV_VLDS
#define FA_DKDV_VLDS 1
#endif
template <int D>
constexpr bool kDkdvVlds = D == 128 && FA_DKDV_VLDS;
template <int D>
constexpr int kDkdvWaves = kDkdvVlds<D> ? 8 : 4;
constexpr int kDqWaves = 4;    // 128 queries per dQ workgroup
// Key tile of the dQ sweep: 32 keys (at d = 128 this keeps the kernel within
// 256 registers, two wavefronts per SIMD; at d = 64, three).
template <int D>
constexpr int kDqBK = 32;

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + bn && pb < pa + an;
}

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

// Workgroups of `kernel` (launched with `threads` per workgroup) resident on one
// CU at a time, from the occupancy calculator, cached by the caller; at least 1.
template <typename K>
int occupancy(std::atomic<int>& cached, K kernel, int threads) {
  int r = cached.load(std::memory_order_relaxed);
  if (r == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) n = 1;
    cached.store(n, std::memory_order_relaxed);
    r = n;
  }
  return r;
}

int check_sizes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  const long long elems = (long long)B * H * N * d;
  if ((long long)(N + 256) * d >= (1LL << 30) || elems >= (1LL << 31)) return FA_ERR_SHAPE;
  return FA_OK;
}

long long workspace_bytes(int B, int H, int N) { return 8LL * B * H * N; }

// Byte extent of a strided [B, H, N, d] tensor of 2-byte elements (d = 1, elem
// = 4 for lse): from its base to one past its last element.
long long extent_bytes(const long long st[3], int B, int H, int N, int d, int elem) {
  return ((long long)(B - 1) * st[0] + (long long)(H - 1) * st[1] + (long long)(N - 1) * st[2] + d) * elem;
}

// Strides in 2-byte elements: >= 0, whole 16-byte units, rows at least d long,
// and (N + 256) rows within 2^31 bytes (one head's buffer range).
bool strides_ok(const long long st[3], int N, int d) {
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || st[i] % 8 != 0 || st[i] > (1LL << 40)) return false;
  return st[2] >= d && (long long)(N + 256) * st[2] * 2 < (1LL << 31);
}

// A tensor's bytes for the alias checks: the extent [base, base + extent) and,
// for a strided 16-bit view, its byte row stride rs and the bytes one row of all
// heads spans (row_span), with batch stride sb.  rs = 0: extent only.
struct Footprint {
  uintptr_t base;
  long long extent, sb, rs, row_span;
};

Footprint footprint(const void* p, const long long st[3], int B, int H, int N, int d) {
  return {reinterpret_cast<uintptr_t>(p), extent_bytes(st, B, H, N, d, 2), st[0] * 2, st[2] * 2,
          ((long long)(H - 1) * st[1] + d) * 2};
}

// False only when the two byte sets are provably disjoint: their extents do not
// meet, or both are views with one row stride rs, batch strides that are
// multiples of rs and all heads of a row within rs bytes, so that every byte of
// a view lies in the interval [base mod rs, base mod rs + row_span) modulo rs;
// disjoint intervals then mean disjoint views.  This admits dq, dk, dv written
// interleaved into one packed [B, N, 3, H, d] buffer.
bool may_overlap(const Footprint& a, const Footprint& b) {
  if (!overlaps(reinterpret_cast<const void*>(a.base), (size_t)a.extent, reinterpret_cast<const void*>(b.base),
                (size_t)b.extent))
    return false;
  const long long rs = a.rs;
  if (rs <= 0 || b.rs != rs || a.sb % rs != 0 || b.sb % rs != 0 || a.row_span > rs || b.row_span > rs) return true;
  const long long ra = (long long)(a.base % (uintptr_t)rs), rb = (long long)(b.base % (uintptr_t)rs);
  const long long ab = ((rb - ra) % rs + rs) % rs, ba = ((ra - rb) % rs + rs) % rs;
  return !(ab >= a.row_span && ba >= b.row_span);
}

// Every element of a strided [B, H, N, d] view has an address of its own: with
// the dimensions ordered by stride, each stride is at least the span of all the
// smaller ones (size-1 dimensions impose nothing).  Sufficient, and what a
// written gradient needs so that no two lanes store to one element.
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

bool contiguous(const long long st[3], int H, int N, int d) {
  return st[2] == d && st[1] == (long long)N * d && st[0] == (long long)H * N * d;
}

// Key rows per head of a descriptor (0 selects the square case).
int key_rows(const fa_bwd_desc& a) { return a.Nk == 0 ? a.N : a.Nk; }

// Host-only checks of a descriptor, in the documented order; no HIP call.
int validate(const fa_bwd_desc& a) {
  if (!a.q || !a.k || !a.v || !a.out || !a.lse || !a.dout || !a.dq || !a.dk || !a.dv || !a.workspace)
    return FA_ERR_NULL;
  const int Nk = key_rows(a);
  if (a.B < 1 || a.H < 1 || a.N < 1 || Nk < 1) return FA_ERR_SHAPE;
  if ((long long)a.B * a.H * std::max(a.N, Nk) >= (1LL << 31)) return FA_ERR_SHAPE;
  if (a.d != 32 && a.d != 64 && a.d != 128) return FA_ERR_HEAD_DIM;
  // q, out, dout, dq: N rows per head; k, v, dk, dv: Nk rows.
  const long long* tq[4] = {a.q_stride, a.o_stride, a.do_stride, a.dq_stride};
  const long long* tk[4] = {a.k_stride, a.v_stride, a.dk_stride, a.dv_stride};
  for (int i = 0; i < 4; ++i)
    if (!strides_ok(tq[i], a.N, a.d) || !strides_ok(tk[i], Nk, a.d)) return FA_ERR_STRIDE;
  for (int i = 0; i < 2; ++i)
    if (a.lse_stride[i] < 0 || a.lse_stride[i] > (1LL << 40)) return FA_ERR_STRIDE;
  if (!std::isfinite(a.scale) || !(a.scale > 0.f)) return FA_ERR_SCALE;
  if (a.causal != 0 && a.causal != 1) return FA_ERR_ARG;
  if (a.dtype != FA_DTYPE_BF16 && a.dtype != FA_DTYPE_F16) return FA_ERR_ARG;
  auto al = [](const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; };
  for (const void* t : {a.q, a.k, a.v, a.out, a.dout, (const void*)a.dq, (const void*)a.dk, (const void*)a.dv})
    if (!al(t, 16)) return FA_ERR_ALIGN;
  if (!al(a.lse, 4)) return FA_ERR_ALIGN;
  const long long need = workspace_bytes(a.B, a.H, a.N);
  if (!al(a.workspace, 256) || a.workspace_bytes < need) return FA_ERR_WORKSPACE;
  auto fq = [&](const void* p, const long long st[3]) { return footprint(p, st, a.B, a.H, a.N, a.d); };
  auto fk = [&](const void* p, const long long st[3]) { return footprint(p, st, a.B, a.H, Nk, a.d); };
  const long long lst[3] = {a.lse_stride[0], a.lse_stride[1], 1};
  const Footprint written[4] = {fq(a.dq, a.dq_stride), fk(a.dk, a.dk_stride), fk(a.dv, a.dv_stride),
                                {reinterpret_cast<uintptr_t>(a.workspace), need, 0, 0, 0}};
  const Footprint read[6] = {fq(a.q, a.q_stride),      fk(a.k, a.k_stride),      fk(a.v, a.v_stride),
                             fq(a.out, a.o_stride),    fq(a.dout, a.do_stride),
                             {reinterpret_cast<uintptr_t>(a.lse), extent_bytes(lst, a.B, a.H, a.N, 1, 4), 0, 0, 0}};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (may_overlap(written[i], written[j])) return FA_ERR_ALIAS;
    for (const auto& r : read)
      if (may_overlap(written[i], r)) return FA_ERR_ALIAS;
  }
  if (!self_disjoint(a.dq_stride, a.B, a.H, a.N, a.d) || !self_disjoint(a.dk_stride, a.B, a.H, Nk, a.d) ||
      !self_disjoint(a.dv_stride, a.B, a.H, Nk, a.d))
    return FA_ERR_ALIAS;
  return FA_OK;
}

template <int D, bool CAUSAL, typename E, bool STRIDED>
hipError_t launch(const fa::BwdParams& p0, hipStream_t stream) {
  fa::BwdParams p = p0;
  const long long rows = (long long)p.BH * p.Nq;
  constexpr int kRowsPerBlock = 256 / (D / 8);
  const long long pre_blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((fa::fa_bwd_pre_kernel<D, E, STRIDED>), dim3((unsigned)pre_blocks), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static std::atomic<int> dkdv_res{0}, dq_res{0};
  p.resident = 1;
  p.cus = 0;
  if (CAUSAL) {
    check_device(&p.cus);
    p.resident = occupancy(dkdv_res, fa::fa_bwd_dkdv_kernel<D, CAUSAL, kDkdvWaves<D>, kDkdvVlds<D>, E, STRIDED>,
                           kDkdvWaves<D> * 64);
  }
  constexpr int kBK = kDkdvWaves<D> * 32;
  p.ntiles = (p.Nk + kBK - 1) / kBK;  // key tiles
  hipLaunchKernelGGL((fa::fa_bwd_dkdv_kernel<D, CAUSAL, kDkdvWaves<D>, kDkdvVlds<D>, E, STRIDED>),
                     dim3((unsigned)(p.BH * p.ntiles)), dim3(kDkdvWaves<D> * 64), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (CAUSAL) p.resident = occupancy(dq_res, fa::fa_bwd_dq_kernel<D, CAUSAL, kDqWaves, kDqBK<D>, E, STRIDED>,
                                     kDqWaves * 64);
  constexpr int kBQ = kDqWaves * 32;
  p.ntiles = (p.Nq + kBQ - 1) / kBQ;  // query tiles
  hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<D, CAUSAL, kDqWaves, kDqBK<D>, E, STRIDED>),
                     dim3((unsigned)(p.BH * p.ntiles)), dim3(kDqWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dt(const fa::BwdParams& p, int dtype, bool strided, hipStream_t s) {
  if (dtype == FA_DTYPE_F16)
    return strided ? launch<D, CAUSAL, fa::F16, true>(p, s) : launch<D, CAUSAL, fa::F16, false>(p, s);
  return strided ? launch<D, CAUSAL, fa::Bf16, true>(p, s) : launch<D, CAUSAL, fa::Bf16, false>(p, s);
}

int run(const fa_bwd_desc& a) {
  const int st = validate(a);
  if (st != FA_OK) return st;
  const int dst = check_device();
  if (dst != FA_OK) return dst;
  fa::BwdParams p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.out = static_cast<const uint16_t*>(a.out);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.lse2 = static_cast<float*>(a.workspace);
  p.dsum = p.lse2 + (long long)a.B * a.H * a.N;
  p.q_sb = a.q_stride[0], p.q_sh = a.q_stride[1], p.q_rs = (int)a.q_stride[2];
  p.k_sb = a.k_stride[0], p.k_sh = a.k_stride[1], p.k_rs = (int)a.k_stride[2];
  p.v_sb = a.v_stride[0], p.v_sh = a.v_stride[1], p.v_rs = (int)a.v_stride[2];
  p.o_sb = a.o_stride[0], p.o_sh = a.o_stride[1], p.o_rs = (int)a.o_stride[2];
  p.do_sb = a.do_stride[0], p.do_sh = a.do_stride[1], p.do_rs = (int)a.do_stride[2];
  p.dq_sb = a.dq_stride[0], p.dq_sh = a.dq_stride[1], p.dq_rs = (int)a.dq_stride[2];
  p.dk_sb = a.dk_stride[0], p.dk_sh = a.dk_stride[1], p.dk_rs = (int)a.dk_stride[2];
  p.dv_sb = a.dv_stride[0], p.dv_sh = a.dv_stride[1], p.dv_rs = (int)a.dv_stride[2];
  p.l_sb = a.lse_stride[0], p.l_sh = a.lse_stride[1];
  p.H = a.H, p.BH = a.B * a.H, p.Nq = a.N, p.Nk = key_rows(a);
  p.nqt = (a.N + 63) / 64;
  p.qk_scale = (float)((double)a.scale * 1.4426950408889634);
  p.scale = a.scale;
  // Every tensor contiguous [B, H, N, d] (lse [B, H, N]): the kernels that
  // derive all addresses from (head, row).
  bool strided = a.lse_stride[1] != a.N || a.lse_stride[0] != (long long)a.H * a.N;
  for (const long long* t : {a.q_stride, a.o_stride, a.do_stride, a.dq_stride})
    strided = strided || !contiguous(t, a.H, a.N, a.d);
  for (const long long* t : {a.k_stride, a.v_stride, a.dk_stride, a.dv_stride})
    strided = strided || !contiguous(t, a.H, p.Nk, a.d);
  const hipStream_t s = static_cast<hipStream_t>(a.stream);
  hipError_t e;
  if (a.d == 32)
    e = a.causal ? launch_dt<32, true>(p, a.dtype, strided, s) : launch_dt<32, false>(p, a.dtype, strided, s);
  else if (a.d == 64)
    e = a.causal ? launch_dt<64, true>(p, a.dtype, strided, s) : launch_dt<64, false>(p, a.dtype, strided, s);
  else
    e = a.causal ? launch_dt<128, true>(p, a.dtype, strided, s) : launch_dt<128, false>(p, a.dtype, strided, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

void set_contiguous(long long st[3], int H, int N, int d) {
  st[0] = (long long)H * N * d, st[1] = (long long)N * d, st[2] = d;
}

}  // namespace

extern "C" {

long long fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  const int st = check_sizes(B, H, N, d);
  return st != FA_OK ? -st : workspace_bytes(B, H, N);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* workspace,
           long long ws_bytes, void* stream) {
  try {
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
    const int st = check_sizes(B, H, N, d);
    if (st != FA_OK) return st;
    fa_bwd_desc a{};
    a.q = q, a.k = k, a.v = v, a.out = out, a.lse = lse, a.dout = dout, a.dq = dq, a.dk = dk, a.dv = dv;
    a.B = B, a.H = H, a.N = N, a.d = d;
    for (long long* t : {a.q_stride, a.k_stride, a.v_stride, a.o_stride, a.do_stride, a.dq_stride, a.dk_stride,
                         a.dv_stride})
      set_contiguous(t, H, N, d);
    a.lse_stride[0] = (long long)H * N, a.lse_stride[1] = N;
    a.scale = scale, a.causal = causal, a.dtype = FA_DTYPE_BF16;
    a.workspace = workspace, a.workspace_bytes = ws_bytes, a.stream = stream;
    return run(a);
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

int fa_bwd_ex(const fa_bwd_desc* desc) {
  try {
    if (!desc) return FA_ERR_NULL;
    return run(*desc);
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

}  // extern "C"
