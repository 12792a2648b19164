// sdattn_api.hip -- the C ABI declared in include/sdattn.h: argument
// validation (host only, before any HIP call), device check, dispatch to
// the kernels (attention and GroupNorm), launch on the caller's stream.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "launch.hpp"
#include "sdattn.h"

namespace {

constexpr int kMaxDevices = 64;
#ifndef SDATTN_GN_TARGET_WGS
#define SDATTN_GN_TARGET_WGS 256  // one workgroup per MI355X CU
#endif
constexpr int64_t kGroupNormTargetWgs = SDATTN_GN_TARGET_WGS;

struct DeviceInfo {
  std::once_flag once;
  bool is_gfx950 = false;
};

DeviceInfo g_devices[kMaxDevices];

bool query_gfx950(int dev) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
  return strncmp(prop.gcnArchName, "gfx950", 6) == 0;
}

// Current device is a usable gfx950 (properties cached once per device).
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();  // do not leave the error for the caller's next call
    return SDATTN_ERR_DEVICE;
  }
  bool ok;
  if (dev < kMaxDevices) {
    DeviceInfo &di = g_devices[dev];
    std::call_once(di.once, [&] { di.is_gfx950 = query_gfx950(dev); });
    ok = di.is_gfx950;
  } else {
    ok = query_gfx950(dev);
  }
  return ok ? SDATTN_OK : SDATTN_ERR_DEVICE;
}

bool overlaps(const void *a, int64_t na, const void *b, int64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a);
  const uintptr_t pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

enum class Path { Auto, Short, Stream };

bool known_dtype(int dtype) {
  return dtype == SDATTN_DTYPE_F32 || dtype == SDATTN_DTYPE_BF16 ||
         dtype == SDATTN_DTYPE_BF16_F32OUT || dtype == SDATTN_DTYPE_F16 ||
         dtype == SDATTN_DTYPE_F16_F32OUT;
}

bool half_dtype(int dtype) {
  return dtype == SDATTN_DTYPE_F16 || dtype == SDATTN_DTYPE_F16_F32OUT;
}

bool f32_out(int dtype) {
  return dtype == SDATTN_DTYPE_F32 || dtype == SDATTN_DTYPE_BF16_F32OUT ||
         dtype == SDATTN_DTYPE_F16_F32OUT;
}

// Row strides of a call: 0 = contiguous [B, H, L, d]; otherwise token-major
// [B, L, ld] operands with head h in columns [h*d, h*d + d).
struct Strides {
  int ldq = 0, ldkv = 0, ldo = 0;
  bool token_major() const { return ldq != 0; }
};

sdattn::Layout layout_of(int H, int L, int d, int ld) {
  sdattn::Layout l;
  if (ld == 0) {
    l.sb = (long long)H * L * d;
    l.sh = L * d;
    l.sl = d;
  } else {
    l.sb = (long long)L * ld;
    l.sh = d;
    l.sl = ld;
  }
  return l;
}

// Elements from an operand's base to the end of its last element.
int64_t span_elems(int B, int H, int L, int d, int ld) {
  if (ld == 0) return (int64_t)B * H * L * d;
  return ((int64_t)B * L - 1) * ld + (int64_t)H * d;
}

int validate(const void *q, const void *k, const void *v, void *out, int B,
             int H, int Lq, int Lk, int d, float scale, int dtype, const Strides &st) {
  if (!known_dtype(dtype)) return SDATTN_ERR_INVALID_ARG;
  if (!q || !k || !v || !out) return SDATTN_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Lq < 1 || Lk < 1 || d < 1) return SDATTN_ERR_INVALID_ARG;
  if (!isfinite(scale)) return SDATTN_ERR_INVALID_ARG;
  if (st.token_major()) {
    // every row holds all heads; rows start 16-byte aligned
    const int64_t hd = (int64_t)H * d;
    for (int ld : {st.ldq, st.ldkv, st.ldo})
      if (ld < hd || ld % 8 != 0) return SDATTN_ERR_INVALID_ARG;
  }
  const int64_t nq = span_elems(B, H, Lq, d, st.ldq);
  const int64_t nk = span_elems(B, H, Lk, d, st.ldkv);
  const int64_t no = span_elems(B, H, Lq, d, st.ldo);
  if (nq > INT32_MAX || nk > INT32_MAX || no > INT32_MAX) return SDATTN_ERR_INVALID_ARG;
  // Kernels address a head's rows, and up to 64 rows past its end (read as
  // zero by the range check), with 32-bit byte offsets.
  const int64_t slq = st.ldq ? st.ldq : d, slk = st.ldkv ? st.ldkv : d;
  if ((Lq + 64) * slq > INT32_MAX || (Lk + 64) * slk > INT32_MAX) return SDATTN_ERR_INVALID_ARG;
  if (d % 8 != 0 || d > 256) return SDATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return SDATTN_ERR_MISALIGNED;
  const int64_t ein = (dtype == SDATTN_DTYPE_F32) ? 4 : 2;
  const int64_t eout = f32_out(dtype) ? 4 : 2;
  if (overlaps(out, no * eout, q, nq * ein) || overlaps(out, no * eout, k, nk * ein) ||
      overlaps(out, no * eout, v, nk * ein))
    return SDATTN_ERR_INVALID_ARG;
  return SDATTN_OK;
}

int run(const void *q, const void *k, const void *v, void *out, int B, int H,
        int Lq, int Lk, int d, float scale, int dtype, void *stream, Path path,
        const Strides &st = Strides()) {
  int rc = validate(q, k, v, out, B, H, Lq, Lk, d, scale, dtype, st);
  if (rc != SDATTN_OK) return rc;
  const int cap = sdattn::short_path_max_keys(d);
  if (path == Path::Short && Lk > cap) return SDATTN_ERR_UNSUPPORTED;
  rc = check_device();
  if (rc != SDATTN_OK) return rc;

  const sdattn::Layout lq = layout_of(H, Lq, d, st.ldq);
  const sdattn::Layout lk = layout_of(H, Lk, d, st.ldkv);
  const sdattn::Layout lo = layout_of(H, Lq, d, st.ldo);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (dtype == SDATTN_DTYPE_F32) {
    sdattn::F32Args a{};
    a.q = static_cast<const float *>(q);
    a.k = static_cast<const float *>(k);
    a.v = static_cast<const float *>(v);
    a.out = static_cast<float *>(out);
    a.H = H;
    a.lq = lq;
    a.lk = lk;
    a.lo = lo;
    a.Lq = Lq;
    a.Lk = Lk;
    a.d = d;
    a.scale = scale;
    err = sdattn::launch_f32(a, B * H, s);
  } else {
    sdattn::Args16 a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.out = out;
    a.H = H;
    a.lq = lq;
    a.lk = lk;
    a.lo = lo;
    a.Lq = Lq;
    a.Lk = Lk;
    a.d = d;
    a.c = fabsf(scale) * sdattn::kLog2e;
    a.qsign = (scale < 0.f) ? 0x80008000u : 0u;
    const bool short_path =
        (path == Path::Short) || (path == Path::Auto && Lk <= cap);
    err = sdattn::launch_16(a, B * H, short_path, f32_out(dtype), half_dtype(dtype), s);
  }
  return (err == hipSuccess) ? SDATTN_OK : SDATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int sdattn_fwd(const void *q, const void *k, const void *v, void *out, int B,
               int H, int Lq, int Lk, int d, float scale, int dtype,
               void *stream) {
  return run(q, k, v, out, B, H, Lq, Lk, d, scale, dtype, stream, Path::Auto);
}

int sdattn_cross_fwd(const void *q, const void *ctx_k, const void *ctx_v,
                     void *out, int B, int H, int Lq, int Lctx, int d,
                     float scale, int dtype, void *stream) {
  return run(q, ctx_k, ctx_v, out, B, H, Lq, Lctx, d, scale, dtype, stream,
             Path::Short);
}

int sdattn_stream_fwd(const void *q, const void *k, const void *v, void *out,
                      int B, int H, int Lq, int Lk, int d, float scale,
                      int dtype, void *stream) {
  return run(q, k, v, out, B, H, Lq, Lk, d, scale, dtype, stream, Path::Stream);
}

int sdattn_fwd_strided(const void *q, const void *k, const void *v, void *out, int B,
                       int H, int Lq, int Lk, int d, int ldq, int ldkv, int ldo,
                       float scale, int dtype, void *stream) {
  Strides st;
  st.ldq = ldq;
  st.ldkv = ldkv;
  st.ldo = ldo;
  if (ldq <= 0 || ldkv <= 0 || ldo <= 0) return SDATTN_ERR_INVALID_ARG;
  return run(q, k, v, out, B, H, Lq, Lk, d, scale, dtype, stream, Path::Auto, st);
}

int sdattn_group_norm(const void *x, const float *gamma, const float *beta, void *y,
                      int N, int C, int HW, int G, float eps, int silu, int dtype,
                      void *stream) {
  if (!known_dtype(dtype)) return SDATTN_ERR_INVALID_ARG;
  if (!x || !gamma || !beta || !y) return SDATTN_ERR_INVALID_ARG;
  if (N < 1 || C < 1 || HW < 1 || G < 1 || C % G != 0) return SDATTN_ERR_INVALID_ARG;
  if (!isfinite(eps) || eps < 0.f || (silu != 0 && silu != 1)) return SDATTN_ERR_INVALID_ARG;
  const int64_t n = (int64_t)N * C * HW;
  if (n > INT32_MAX || (int64_t)N * G > INT32_MAX) return SDATTN_ERR_INVALID_ARG;
  if (HW % 8 != 0 || C / G > sdattn::group_norm_max_channels_per_group())
    return SDATTN_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y) || (reinterpret_cast<uintptr_t>(gamma) & 3u) ||
      (reinterpret_cast<uintptr_t>(beta) & 3u))
    return SDATTN_ERR_MISALIGNED;
  const int64_t ein = (dtype == SDATTN_DTYPE_F32) ? 4 : 2;
  const int64_t eout = f32_out(dtype) ? 4 : 2;
  // In place (y == x) is allowed when input and output elements have the
  // same size: every element is read before the workgroup writes it.
  const bool in_place = (x == y) && ein == eout;
  if (!in_place && overlaps(y, n * eout, x, n * ein)) return SDATTN_ERR_INVALID_ARG;
  if (overlaps(y, n * eout, gamma, (int64_t)C * 4) || overlaps(y, n * eout, beta, (int64_t)C * 4))
    return SDATTN_ERR_INVALID_ARG;
  int rc = check_device();
  if (rc != SDATTN_OK) return rc;
  sdattn::GnArgs a{};
  a.x = x;
  a.gamma = gamma;
  a.beta = beta;
  a.y = y;
  a.N = N;
  a.C = C;
  a.S = HW;
  a.G = G;
  a.eps = eps;
  a.silu = silu;
  // Out of place with fewer groups than CUs: spread each group over up to 8
  // workgroups (in place keeps one workgroup per group).
  a.split = 1;
  if (!in_place && (int64_t)N * G < kGroupNormTargetWgs)
    a.split = (int)std::min<int64_t>(8, kGroupNormTargetWgs / ((int64_t)N * G));
  const int elem = (dtype == SDATTN_DTYPE_F32) ? 0 : half_dtype(dtype) ? 2 : 1;
  const hipError_t err = sdattn::launch_group_norm(a, elem, f32_out(dtype),
                                                   static_cast<hipStream_t>(stream));
  return (err == hipSuccess) ? SDATTN_OK : SDATTN_ERR_LAUNCH;
}

int sdattn_cross_max_ctx(int d, int dtype) {
  if (!known_dtype(dtype)) return 0;
  if (d < 8 || d > 256 || d % 8 != 0) return 0;
  return sdattn::short_path_max_keys(d);
}

const char *sdattn_strerror(int status) {
  switch (status) {
    case SDATTN_OK: return "success";
    case SDATTN_ERR_INVALID_ARG: return "invalid argument";
    case SDATTN_ERR_UNSUPPORTED: return "unsupported head dimension or context length";
    case SDATTN_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case SDATTN_ERR_DEVICE: return "no gfx950 HIP device is current";
    case SDATTN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown sdattn status";
  }
}

int sdattn_version(void) { return 10300; }

}  // extern "C"
