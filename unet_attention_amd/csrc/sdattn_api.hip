// sdattn_api.hip -- the C ABI declared in include/sdattn.h: argument
// validation (host only, before any HIP call), device check, dispatch to
// the kernels, launch on the caller's stream.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "launch.hpp"
#include "sdattn.h"

namespace {

constexpr int kMaxDevices = 64;

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

int validate(const void *q, const void *k, const void *v, void *out, int B,
             int H, int Lq, int Lk, int d, float scale, int dtype) {
  if (!known_dtype(dtype)) return SDATTN_ERR_INVALID_ARG;
  if (!q || !k || !v || !out) return SDATTN_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Lq < 1 || Lk < 1 || d < 1) return SDATTN_ERR_INVALID_ARG;
  if (!isfinite(scale)) return SDATTN_ERR_INVALID_ARG;
  const int64_t nq = (int64_t)B * H * Lq * d, nk = (int64_t)B * H * Lk * d;
  if (nq > INT32_MAX || nk > INT32_MAX) return SDATTN_ERR_INVALID_ARG;
  if (d % 8 != 0 || d > 256) return SDATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return SDATTN_ERR_MISALIGNED;
  const int64_t ein = (dtype == SDATTN_DTYPE_F32) ? 4 : 2;
  const int64_t eout = f32_out(dtype) ? 4 : 2;
  const int64_t nout = nq * eout;
  if (overlaps(out, nout, q, nq * ein) || overlaps(out, nout, k, nk * ein) ||
      overlaps(out, nout, v, nk * ein))
    return SDATTN_ERR_INVALID_ARG;
  return SDATTN_OK;
}

int run(const void *q, const void *k, const void *v, void *out, int B, int H,
        int Lq, int Lk, int d, float scale, int dtype, void *stream, Path path) {
  int rc = validate(q, k, v, out, B, H, Lq, Lk, d, scale, dtype);
  if (rc != SDATTN_OK) return rc;
  const int cap = sdattn::short_path_max_keys(d);
  if (path == Path::Short && Lk > cap) return SDATTN_ERR_UNSUPPORTED;
  rc = check_device();
  if (rc != SDATTN_OK) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (dtype == SDATTN_DTYPE_F32) {
    sdattn::F32Args a{};
    a.q = static_cast<const float *>(q);
    a.k = static_cast<const float *>(k);
    a.v = static_cast<const float *>(v);
    a.out = static_cast<float *>(out);
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

int sdattn_version(void) { return 10100; }

}  // extern "C"
