// abi_sanitize.cpp -- the host side of libsdattn (sdattn_api.hip: argument
// validation, device check, dispatch, layouts, status mapping) run on the
// CPU under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Test infrastructure, built by tests/test_sanitize.py: sdattn_api.hip is
// compiled host-only and linked with this file, which stands in for the
// three HIP runtime calls the layer makes (a fake device whose architecture
// the test chooses) and for the kernel launchers (stubs that record their
// arguments and return a chosen status).  No GPU, no HIP runtime library.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "launch.hpp"
#include "sdattn.h"

// ---------------------------------------------------------------------------
// fake runtime

static int g_have_device = 1;
static const char *g_arch = "gfx950:sramecc+:xnack-";
static int g_props_calls = 0;
static int g_last_error_calls = 0;

extern "C" hipError_t hipGetDevice(int *dev) {
  if (!g_have_device) return hipErrorNoDevice;
  *dev = 0;
  return hipSuccess;
}

extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_t *prop, int dev) {
  (void)dev;
  ++g_props_calls;
  memset(prop, 0, sizeof(*prop));
  strncpy(prop->gcnArchName, g_arch, sizeof(prop->gcnArchName) - 1);
  return hipSuccess;
}

extern "C" hipError_t hipGetLastError(void) {
  ++g_last_error_calls;
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// stub launchers

struct Launch {
  char kind;  // 'a' attention 16-bit, 'f' fp32, 'g' group norm
  sdattn::Args16 a16;
  sdattn::F32Args af;
  sdattn::GnArgs gn;
  int BH;
  bool short_path, out_f32, half;
  int elem;
};
static std::vector<Launch> g_launches;
static hipError_t g_launch_status = hipSuccess;

namespace sdattn {
int short_path_max_keys(int) { return 128; }
int group_norm_max_channels_per_group() { return 8192; }
hipError_t launch_16(const Args16 &a, int BH, bool short_path, bool out_f32, bool half,
                     hipStream_t) {
  Launch l{};
  l.kind = 'a';
  l.a16 = a;
  l.BH = BH;
  l.short_path = short_path;
  l.out_f32 = out_f32;
  l.half = half;
  g_launches.push_back(l);
  return g_launch_status;
}
hipError_t launch_f32(const F32Args &a, int BH, hipStream_t) {
  Launch l{};
  l.kind = 'f';
  l.af = a;
  l.BH = BH;
  g_launches.push_back(l);
  return g_launch_status;
}
hipError_t launch_group_norm(const GnArgs &a, int elem, bool out_f32, hipStream_t) {
  Launch l{};
  l.kind = 'g';
  l.gn = a;
  l.elem = elem;
  l.out_f32 = out_f32;
  g_launches.push_back(l);
  return g_launch_status;
}
}  // namespace sdattn

// ---------------------------------------------------------------------------

static int failures = 0;
#define CHECK(c)                                                             \
  do {                                                                       \
    if (!(c)) {                                                              \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

// Host buffers stand in for device pointers: the layer never dereferences
// them, it only checks alignment and overlap.
alignas(16) static uint8_t g_mem[1 << 22];

int main() {
  uint8_t *q = g_mem, *k = g_mem + (1 << 20), *v = g_mem + (2 << 20), *o = g_mem + (3 << 20);
  const float sc = 0.125f;

  // -- valid calls and their dispatch
  CHECK(sdattn_fwd(q, k, v, o, 2, 3, 100, 77, 40, sc, SDATTN_DTYPE_BF16, nullptr) == SDATTN_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].kind == 'a' && g_launches[0].short_path);
  CHECK(g_launches[0].BH == 6 && !g_launches[0].out_f32 && !g_launches[0].half);
  {
    const sdattn::Args16 &a = g_launches[0].a16;
    CHECK(a.Lq == 100 && a.Lk == 77 && a.d == 40 && a.H == 3);
    CHECK(a.lq.sb == 3LL * 100 * 40 && a.lq.sh == 100 * 40 && a.lq.sl == 40);
    CHECK(a.lk.sb == 3LL * 77 * 40 && a.lk.sh == 77 * 40 && a.lk.sl == 40);
    CHECK(fabsf(a.c - sc * 1.4426950408889634f) <= 1e-7f && a.qsign == 0u);
  }
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 64, 129, 64, -sc, SDATTN_DTYPE_BF16_F32OUT, nullptr) ==
        SDATTN_OK);
  CHECK(!g_launches.back().short_path && g_launches.back().out_f32);
  CHECK(g_launches.back().a16.qsign == 0x80008000u && g_launches.back().a16.c > 0.f);
  CHECK(sdattn_stream_fwd(q, k, v, o, 1, 1, 64, 10, 64, sc, SDATTN_DTYPE_F16, nullptr) ==
        SDATTN_OK);
  CHECK(!g_launches.back().short_path && g_launches.back().half);
  CHECK(sdattn_cross_fwd(q, k, v, o, 1, 2, 64, 128, 80, sc, SDATTN_DTYPE_F16_F32OUT, nullptr) ==
        SDATTN_OK);
  CHECK(g_launches.back().short_path && g_launches.back().half && g_launches.back().out_f32);
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 64, 77, 40, sc, SDATTN_DTYPE_F32, nullptr) == SDATTN_OK);
  CHECK(g_launches.back().kind == 'f' && g_launches.back().af.scale == sc);
  // token-major: [B, L, ld] with head h in columns [h*d, h*d + d)
  CHECK(sdattn_fwd_strided(q, k, v, o, 2, 4, 50, 60, 64, 3 * 256, 3 * 256, 256, sc,
                           SDATTN_DTYPE_BF16, nullptr) == SDATTN_OK);
  {
    const sdattn::Args16 &a = g_launches.back().a16;
    CHECK(a.lq.sb == 50LL * 768 && a.lq.sh == 64 && a.lq.sl == 768);
    CHECK(a.lk.sb == 60LL * 768 && a.lk.sh == 64 && a.lk.sl == 768);
    CHECK(a.lo.sb == 50LL * 256 && a.lo.sh == 64 && a.lo.sl == 256);
  }
  const size_t nvalid = g_launches.size();

  // -- launch status: the launcher's own status, and nothing else
  g_last_error_calls = 0;
  g_launch_status = hipErrorLaunchFailure;
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 64, 64, 64, sc, SDATTN_DTYPE_BF16, nullptr) ==
        SDATTN_ERR_LAUNCH);
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 64, 64, 64, sc, SDATTN_DTYPE_F32, nullptr) ==
        SDATTN_ERR_LAUNCH);
  CHECK(sdattn_group_norm(q, (const float *)k, (const float *)v, o, 1, 32, 64, 8, 1e-5f, 1,
                          SDATTN_DTYPE_BF16, nullptr) == SDATTN_ERR_LAUNCH);
  g_launch_status = hipSuccess;
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 64, 64, 64, sc, SDATTN_DTYPE_BF16, nullptr) == SDATTN_OK);
  CHECK(g_last_error_calls == 0);  // an earlier error on the thread is neither read nor cleared

  // -- invalid arguments: rejected before any launch
  const size_t before = g_launches.size();
  CHECK(sdattn_fwd(nullptr, k, v, o, 1, 1, 8, 8, 8, sc, 1, nullptr) == SDATTN_ERR_INVALID_ARG);
  CHECK(sdattn_fwd(q, k, v, nullptr, 1, 1, 8, 8, 8, sc, 1, nullptr) == SDATTN_ERR_INVALID_ARG);
  CHECK(sdattn_fwd(q, k, v, o, 0, 1, 8, 8, 8, sc, 1, nullptr) == SDATTN_ERR_INVALID_ARG);
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 8, 0, 8, sc, 1, nullptr) == SDATTN_ERR_INVALID_ARG);
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 8, 8, 8, sc, 7, nullptr) == SDATTN_ERR_INVALID_ARG);
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 8, 8, 8, NAN, 1, nullptr) == SDATTN_ERR_INVALID_ARG);
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 8, 8, 8, INFINITY, 1, nullptr) == SDATTN_ERR_INVALID_ARG);
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 8, 8, 12, sc, 1, nullptr) == SDATTN_ERR_UNSUPPORTED);
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 8, 8, 264, sc, 1, nullptr) == SDATTN_ERR_UNSUPPORTED);
  CHECK(sdattn_fwd(q + 2, k, v, o, 1, 1, 8, 8, 8, sc, 1, nullptr) == SDATTN_ERR_MISALIGNED);
  CHECK(sdattn_fwd(q, k, v, o + 8, 1, 1, 8, 8, 8, sc, 1, nullptr) == SDATTN_ERR_MISALIGNED);
  // out overlapping q, k or v
  CHECK(sdattn_fwd(q, k, v, q + 16, 1, 1, 8, 8, 8, sc, 1, nullptr) == SDATTN_ERR_INVALID_ARG);
  CHECK(sdattn_fwd(q, k, v, v, 1, 1, 8, 8, 8, sc, 1, nullptr) == SDATTN_ERR_INVALID_ARG);
  // more than 2^31 - 1 elements in one operand
  CHECK(sdattn_fwd(q, k, v, o, 65536, 8, 4096, 8, 8, sc, 1, nullptr) == SDATTN_ERR_INVALID_ARG);
  // cross entry above its context cap
  CHECK(sdattn_cross_fwd(q, k, v, o, 1, 1, 8, 129, 8, sc, 1, nullptr) ==
        SDATTN_ERR_UNSUPPORTED);
  // token-major strides
  CHECK(sdattn_fwd_strided(q, k, v, o, 1, 2, 8, 8, 8, 8, 16, 16, sc, 1, nullptr) ==
        SDATTN_ERR_INVALID_ARG);  // ld < H*d
  CHECK(sdattn_fwd_strided(q, k, v, o, 1, 2, 8, 8, 8, 20, 20, 20, sc, 1, nullptr) ==
        SDATTN_ERR_INVALID_ARG);  // ld % 8
  CHECK(sdattn_fwd_strided(q, k, v, o, 1, 2, 8, 8, 8, 0, 16, 16, sc, 1, nullptr) ==
        SDATTN_ERR_INVALID_ARG);
  // group norm
  const float *gam = (const float *)k, *bet = (const float *)v;
  CHECK(sdattn_group_norm(q, gam, bet, o, 1, 30, 64, 8, 1e-5f, 0, 1, nullptr) ==
        SDATTN_ERR_INVALID_ARG);  // C % G
  CHECK(sdattn_group_norm(q, gam, bet, o, 1, 32, 64, 8, -1.f, 0, 1, nullptr) ==
        SDATTN_ERR_INVALID_ARG);
  CHECK(sdattn_group_norm(q, gam, bet, o, 1, 32, 64, 8, 1e-5f, 2, 1, nullptr) ==
        SDATTN_ERR_INVALID_ARG);
  CHECK(sdattn_group_norm(q, gam, bet, o, 1, 32, 60, 8, 1e-5f, 0, 1, nullptr) ==
        SDATTN_ERR_UNSUPPORTED);  // HW % 8
  CHECK(sdattn_group_norm(q, gam, bet, q + 64, 1, 32, 64, 8, 1e-5f, 0, 1, nullptr) ==
        SDATTN_ERR_INVALID_ARG);  // partial overlap
  CHECK(sdattn_group_norm(q, gam, bet, q, 1, 32, 64, 8, 1e-5f, 0, SDATTN_DTYPE_BF16_F32OUT,
                          nullptr) == SDATTN_ERR_INVALID_ARG);  // in place, sizes differ
  CHECK(g_launches.size() == before);

  // group norm: in place allowed; few groups out of place -> split form
  CHECK(sdattn_group_norm(q, gam, bet, q, 2, 64, 64, 32, 1e-5f, 1, 1, nullptr) == SDATTN_OK);
  CHECK(g_launches.back().kind == 'g' && g_launches.back().gn.split == 1);
  CHECK(sdattn_group_norm(q, gam, bet, o, 2, 64, 64, 32, 1e-5f, 1, 1, nullptr) == SDATTN_OK);
  CHECK(g_launches.back().gn.split == 4 && g_launches.back().elem == 1);

  // -- device check: cached once per device; another arch or no device fails
  CHECK(g_props_calls == 1);
  (void)nvalid;
  g_have_device = 0;
  CHECK(sdattn_fwd(q, k, v, o, 1, 1, 8, 8, 8, sc, 1, nullptr) == SDATTN_ERR_DEVICE);
  g_have_device = 1;

  // -- strings and constants
  for (int s = 0; s <= 6; ++s) CHECK(sdattn_strerror(s) != nullptr && sdattn_strerror(s)[0]);
  CHECK(sdattn_strerror(-1) != nullptr);
  CHECK(sdattn_cross_max_ctx(40, 1) == 128 && sdattn_cross_max_ctx(12, 1) == 0);
  CHECK(sdattn_cross_max_ctx(40, 9) == 0 && sdattn_cross_max_ctx(264, 1) == 0);
  CHECK(sdattn_version() > 0);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("host ABI sanitizer run: all checks passed\n");
  return 0;
}
