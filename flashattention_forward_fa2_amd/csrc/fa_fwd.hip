// C ABI of the gfx950 FlashAttention-2 forward library: argument checks, the
// table of compiled tile variants, and the launch.  Declared in include/fa_fwd.h.
#include "fa_fwd.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "fa_fwd_kernel.hpp"

namespace {

constexpr int kVersion = 100;  // 0.1.0

using Launcher = hipError_t (*)(const void*, const void*, const void*, void*, float*, int BH, int N,
                                float qk_scale, hipStream_t);

struct Variant {
  int d, causal, qb, waves, bk;
  Launcher launch;
};

template <int D, bool CAUSAL, int QB, int WAVES, int BK>
hipError_t launch_variant(const void* q, const void* k, const void* v, void* out, float* lse, int BH,
                          int N, float qk_scale, hipStream_t stream) {
  using T = fa::Tile<D, QB, WAVES, BK>;
  const int nqt = (N + T::kBQ - 1) / T::kBQ;
  const long long blocks = (long long)BH * nqt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa::fa_fwd_kernel<D, CAUSAL, QB, WAVES, BK>), dim3((unsigned)blocks),
                     dim3(T::kThreads), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<uint16_t*>(out), lse, BH, N, nqt, qk_scale);
  return hipGetLastError();
}

#define FA_VARIANT(D, C, QB, W, BK) {D, C, QB, W, BK, &launch_variant<D, (C) != 0, QB, W, BK>}
#define FA_VARIANTS_DC(D, C) \
  FA_VARIANT(D, C, 1, 4, 64), FA_VARIANT(D, C, 2, 4, 64), FA_VARIANT(D, C, 1, 8, 64), FA_VARIANT(D, C, 2, 4, 128)

const Variant kVariants[] = {
    FA_VARIANTS_DC(64, 0), FA_VARIANTS_DC(64, 1), FA_VARIANTS_DC(128, 0), FA_VARIANTS_DC(128, 1),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

const Variant* find_variant(int d, int causal, const fa_tile_cfg& c) {
  for (const Variant& v : kVariants)
    if (v.d == d && v.causal == causal && v.qb == c.qb && v.waves == c.waves && v.bk == c.bk) return &v;
  return nullptr;
}

fa_tile_cfg default_cfg(int /*N*/, int /*d*/, int /*causal*/) { return fa_tile_cfg{1, 8, 64}; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + bn && pb < pa + an;
}

// Host-only argument checks, in a fixed order; no HIP call is made here.
int validate(const void* q, const void* k, const void* v, const void* out, const float* lse, int B, int H,
             int N, int d, float scale, int causal) {
  if (!q || !k || !v || !out || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  const long long elems = (long long)B * H * N * d;
  if ((long long)N * d >= (1LL << 31) || elems >= (1LL << 31)) return FA_ERR_SHAPE;
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

// Per-device "is this a gfx950" cache, filled once per device.
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

int run(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N, int d,
        float scale, int causal, void* stream, const fa_tile_cfg& cfg) {
  const int st = validate(q, k, v, out, lse, B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  const Variant* var = find_variant(d, causal, cfg);
  if (!var) return FA_ERR_ARG;
  const int dst = check_device();
  if (dst != FA_OK) return dst;
  // Scores are kept raw; exp(scale*s - m) = 2^(s*scale*log2(e) - m') with m' in
  // log2 units, so the scale and log2(e) fold into one constant.
  const float qk_scale = (float)((double)scale * 1.4426950408889634);
  const hipError_t e = var->launch(q, k, v, out, lse, B * H, N, qk_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N, int d,
           float scale, int causal, void* stream) {
  try {
    return run(q, k, v, out, lse, B, H, N, d, scale, causal, stream, default_cfg(N, d, causal));
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

int fa_fwd_cfg(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N, int d,
               float scale, int causal, void* stream, const fa_tile_cfg* cfg) {
  if (!cfg) return FA_ERR_ARG;
  try {
    return run(q, k, v, out, lse, B, H, N, d, scale, causal, stream, *cfg);
  } catch (...) {
    return FA_ERR_INTERNAL;
  }
}

int fa_default_cfg(int N, int d, int causal, fa_tile_cfg* cfg) {
  if (!cfg) return FA_ERR_NULL;
  if (N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  *cfg = default_cfg(N, d, causal);
  return FA_OK;
}

int fa_num_variants(void) { return kNumVariants; }

int fa_variant(int i, int* d, int* causal, fa_tile_cfg* cfg) {
  if (i < 0 || i >= kNumVariants) return FA_ERR_ARG;
  if (!d || !causal || !cfg) return FA_ERR_NULL;
  *d = kVariants[i].d;
  *causal = kVariants[i].causal;
  *cfg = fa_tile_cfg{kVariants[i].qb, kVariants[i].waves, kVariants[i].bk};
  return FA_OK;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer argument";
    case FA_ERR_SHAPE: return "B, H and N must be >= 1 and the tensors must have fewer than 2^31 elements";
    case FA_ERR_HEAD_DIM: return "head dimension must be 64 or 128";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ARG: return "invalid argument (causal must be 0 or 1; tile configuration not compiled in)";
    case FA_ERR_ALIGN: return "q, k, v, out must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ALIAS: return "out/lse overlap an input or each other";
    case FA_ERR_NO_DEVICE: return "no current HIP device, or it is not gfx950";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
