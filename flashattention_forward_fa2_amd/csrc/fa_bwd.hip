// C ABI of the gfx950 FlashAttention-2 backward: argument checks and the three
// launches (D / LSE preprocessing, dK and dV, dQ).  Declared in include/fa_bwd.h.
#include "fa_bwd.h"

#include <hip/hip_runtime.h>

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

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_NO_DEVICE;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t p;
    g_dev_ok[dev] = hipGetDeviceProperties(&p, dev) == hipSuccess && std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
  });
  return g_dev_ok[dev] ? FA_OK : FA_ERR_NO_DEVICE;
}

int check_sizes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  const long long elems = (long long)B * H * N * d;
  if ((long long)(N + 256) * d >= (1LL << 30) || elems >= (1LL << 31)) return FA_ERR_SHAPE;
  return FA_OK;
}

long long workspace_bytes(int B, int H, int N) { return 8LL * B * H * N; }

struct Args {
  const void *q, *k, *v, *out;
  const float* lse;
  const void* dout;
  void *dq, *dk, *dv;
  int B, H, N, d;
  float scale;
  int causal;
  void* ws;
  long long ws_bytes;
  void* stream;
};

// Host-only checks, in the documented order; no HIP call is made here.
int validate(const Args& a) {
  if (!a.q || !a.k || !a.v || !a.out || !a.lse || !a.dout || !a.dq || !a.dk || !a.dv || !a.ws) return FA_ERR_NULL;
  const int st = check_sizes(a.B, a.H, a.N, a.d);
  if (st != FA_OK) return st;
  if (!std::isfinite(a.scale) || !(a.scale > 0.f)) return FA_ERR_SCALE;
  if (a.causal != 0 && a.causal != 1) return FA_ERR_ARG;
  auto al = [](const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; };
  for (const void* t : {a.q, a.k, a.v, a.out, a.dout, (const void*)a.dq, (const void*)a.dk, (const void*)a.dv})
    if (!al(t, 16)) return FA_ERR_ALIGN;
  if (!al(a.lse, 4)) return FA_ERR_ALIGN;
  const long long need = workspace_bytes(a.B, a.H, a.N);
  if (!al(a.ws, 256) || a.ws_bytes < need) return FA_ERR_WORKSPACE;
  const size_t tb = (size_t)a.B * a.H * a.N * a.d * 2, lb = (size_t)a.B * a.H * a.N * 4;
  const std::pair<const void*, size_t> written[4] = {{a.dq, tb}, {a.dk, tb}, {a.dv, tb}, {a.ws, (size_t)need}};
  const std::pair<const void*, size_t> read[6] = {{a.q, tb}, {a.k, tb}, {a.v, tb}, {a.out, tb}, {a.dout, tb}, {a.lse, lb}};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(written[i].first, written[i].second, written[j].first, written[j].second)) return FA_ERR_ALIAS;
    for (const auto& r : read)
      if (overlaps(written[i].first, written[i].second, r.first, r.second)) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

template <int D, bool CAUSAL>
hipError_t launch(const fa::BwdParams& p0, hipStream_t stream) {
  fa::BwdParams p = p0;
  const long long rows = (long long)p.BH * p.N;
  constexpr int kRowsPerBlock = 256 / (D / 8);
  const long long pre_blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((fa::fa_bwd_pre_kernel<D>), dim3((unsigned)pre_blocks), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int kBK = kDkdvWaves<D> * 32;
  p.ntiles = (p.N + kBK - 1) / kBK;
  hipLaunchKernelGGL((fa::fa_bwd_dkdv_kernel<D, CAUSAL, kDkdvWaves<D>, kDkdvVlds<D>>),
                     dim3((unsigned)(p.BH * p.ntiles)), dim3(kDkdvWaves<D> * 64), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int kBQ = kDqWaves * 32;
  p.ntiles = (p.N + kBQ - 1) / kBQ;
  hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<D, CAUSAL, kDqWaves, kDqBK<D>>), dim3((unsigned)(p.BH * p.ntiles)),
                     dim3(kDqWaves * 64), 0, stream, p);
  return hipGetLastError();
}

int run(const Args& a) {
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
  p.lse2 = static_cast<float*>(a.ws);
  p.dsum = p.lse2 + (long long)a.B * a.H * a.N;
  p.BH = a.B * a.H, p.N = a.N;
  p.qk_scale = (float)((double)a.scale * 1.4426950408889634);
  p.scale = a.scale;
  const hipStream_t s = static_cast<hipStream_t>(a.stream);
  hipError_t e;
  if (a.d == 64)
    e = a.causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
  else
    e = a.causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
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
    const Args a{q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, workspace, ws_bytes, stream};
    return run(a);
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

}  // extern "C"
