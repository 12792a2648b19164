// peak.hip -- attainable-peak microbenchmarks for gfx950 (MI355X), used by
// the benchmark to put each attention kernel's rate beside what the same
// chip reaches on the plain operation:
//
// * peak_mfma: back-to-back independent v_mfma_f32_32x32x16_bf16 on four
//   accumulators per wave, optionally with n_exp independent v_exp_f32 and
//   n_fma independent v_fma_f32 per matrix instruction -- the attainable
//   dense bf16 rate, and how much transcendental / FMA vector work the SIMD
//   issues under the matrix core (the softmax's share of the attention);
// * peak_copy: a 16-byte-per-lane device copy (the attainable HBM rate for
//   a transfer of a given size);
// * peak_lds: 16-byte LDS reads from every lane (LDS read bandwidth).
//
// Not part of libsdattn: a separate library with its own small C ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename A>
hipError_t launch1(void (*k)(A), dim3 g, dim3 b, size_t lds, hipStream_t s, A arg) {
  void *args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void *>(k), g, b, args, lds, s);
}

struct MfmaArgs {
  float *sink;
  int iters;
  float seed;
};

template <int NE, int NF>
__global__ __launch_bounds__(256) void k_mfma(MfmaArgs a) {
  const int lane = threadIdx.x & 63;
  bf16x8 x, y;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = (__bf16)(a.seed * (float)(lane + i));
    y[i] = (__bf16)(a.seed * (float)(lane - i));
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  float e[NE > 0 ? NE : 1], f[NF > 0 ? NF : 1];
#pragma unroll
  for (int k = 0; k < NE; ++k) e[k] = a.seed * (float)(lane + k) - 4.0f;
#pragma unroll
  for (int k = 0; k < NF; ++k) f[k] = a.seed * (float)(lane - k);
  for (int it = 0; it < a.iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc[j], 0, 0, 0);
      // exp2 of a value kept in [-4, 0): bounded, independent chains
#pragma unroll
      for (int k = 0; k < NE; ++k) e[k] = __builtin_amdgcn_exp2f(e[k]) - 4.0f;
#pragma unroll
      for (int k = 0; k < NF; ++k) f[k] = __builtin_fmaf(f[k], 0.999f, 0.001f);
    }
    // issue order: each matrix instruction followed by its share of the
    // vector work (an exp and an add per chain, an FMA per chain)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (2 * NE + NF > 0) __builtin_amdgcn_sched_group_barrier(0x002, 2 * NE + NF, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
#pragma unroll
  for (int k = 0; k < NE; ++k) s += e[k];
#pragma unroll
  for (int k = 0; k < NF; ++k) s += f[k];
  a.sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

struct CopyArgs {
  const u32x4 *src;
  u32x4 *dst;
  long long n;  // 16-byte chunks
};

// Each thread moves four 16-byte chunks per round (four loads in flight
// before the stores), chunks strided by the grid so every instruction is a
// contiguous 1 KB per wave.
__global__ __launch_bounds__(256) void k_copy(CopyArgs a) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < a.n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = a.src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) a.dst[i + u * stride] = v[u];
  }
  for (; i < a.n; i += stride) a.dst[i] = a.src[i];
}

struct LdsArgs {
  float *sink;
  int iters;
};

__global__ __launch_bounds__(256) void k_lds(LdsArgs a) {
  __shared__ u32x4 buf[4096];  // 64 KB
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int it = 0; it < a.iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= buf[(w * 1024 + j * 64 + lane + it) & 4095];
  }
  a.sink[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// One wave: the lane layouts the attention kernels rely on, written out for
// a test to compare with their documented form.
//  out[0 .. 1023]: v_mfma_f32_32x32x16_bf16 with A[r][k] = (k == r % 16) and
//    B[k][c] = k, the operands placed as documented (lane l supplies row /
//    column l % 32 and k = 8 (l / 32) .. +7): accumulator register i of lane
//    l, written at 16 l + i, must read (8 (i / 4) + 4 (l / 32) + i % 4) % 16;
//  out[1024 .. 2047]: the same with A[r][k] = (k == 0) and B[k][c] = c % 32:
//    register i of lane l must read l % 32;
//  out[2048 .. 2303]: ds_read_b64_tr_b16 from an LDS table holding value x
//    at halfword x, each lane addressing halfword 4 l: the four halfwords
//    lane l receives, at 4 l + j;
//  out[2304 .. 2431]: v_permlane32_swap with both operands 100 + l (the
//    form the kernels use): both results of each lane.
__global__ __launch_bounds__(64) void k_probe(int *out) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  __shared__ __attribute__((aligned(16))) uint16_t tab[512];
  const int l = threadIdx.x;
  for (int i = l; i < 512; i += 64) tab[i] = (uint16_t)i;
  __syncthreads();
  const int r = l % 32, kb = 8 * (l / 32);
  bf16x8 a1, b1, a2, b2;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = kb + j;
    a1[j] = (__bf16)(k == r % 16 ? 1.0f : 0.0f);
    b1[j] = (__bf16)(float)k;
    a2[j] = (__bf16)(k == 0 ? 1.0f : 0.0f);
    b2[j] = (__bf16)(float)(l % 32);
  }
  const f32x16 d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, f32x16{}, 0, 0, 0);
  const f32x16 d2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b2, f32x16{}, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    out[16 * l + i] = (int)d1[i];
    out[1024 + 16 * l + i] = (int)d2[i];
  }
  const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tab + 4 * l));
#pragma unroll
  for (int j = 0; j < 4; ++j) out[2048 + 4 * l + j] = (int)(uint16_t)t[j];
  const auto sw = __builtin_amdgcn_permlane32_swap((uint32_t)(100 + l), (uint32_t)(100 + l), false,
                                                   false);
  out[2304 + 2 * l] = (int)sw[0];
  out[2304 + 2 * l + 1] = (int)sw[1];
}

}  // namespace

extern "C" {

// Writes the 2432 ints described at k_probe to out (device memory).
int peak_probe_layouts(int *out, void *stream) {
  return (int)launch1(&k_probe, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out);
}


// n_exp in {0, 2, 4, 8}, n_fma in {0, 4, 8}; sink holds nwg * 256 floats.
int peak_mfma(int nwg, int iters, int n_exp, int n_fma, float *sink, void *stream) {
  MfmaArgs a{sink, iters, 1e-3f};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g(nwg), b(256);
#define PEAK_CASE(E, F) \
  if (n_exp == E && n_fma == F) return (int)launch1(&k_mfma<E, F>, g, b, 0, s, a);
  PEAK_CASE(0, 0) PEAK_CASE(2, 0) PEAK_CASE(4, 0) PEAK_CASE(8, 0)
  PEAK_CASE(0, 4) PEAK_CASE(0, 8) PEAK_CASE(4, 4) PEAK_CASE(2, 4)
#undef PEAK_CASE
  return (int)hipErrorInvalidValue;
}

// Copies bytes (a multiple of 16) from src to dst with nwg workgroups.
int peak_copy(const void *src, void *dst, long long bytes, int nwg, void *stream) {
  if (bytes % 16) return (int)hipErrorInvalidValue;
  CopyArgs a{static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), bytes / 16};
  return (int)launch1(&k_copy, dim3(nwg), dim3(256), 0, static_cast<hipStream_t>(stream), a);
}

// Each of nwg workgroups (4 waves) reads iters * 8 * 16 bytes per lane from LDS.
int peak_lds(int nwg, int iters, float *sink, void *stream) {
  LdsArgs a{sink, iters};
  return (int)launch1(&k_lds, dim3(nwg), dim3(256), 0, static_cast<hipStream_t>(stream), a);
}

}  // extern "C"
