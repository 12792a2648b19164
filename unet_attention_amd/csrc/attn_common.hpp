// attn_common.hpp -- device-side types and helpers shared by the bf16 and
// fp32 attention kernels of libsdattn (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kQW = 32;             // query rows owned by one wave (bf16 kernels)
constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescaling: the running maximum m (log2 domain) is only raised when a
// tile's maximum exceeds it by more than this many binary orders, so the
// unnormalised weights stay <= 2^kRescaleSlack.  The result is unchanged in
// exact arithmetic because l and O always share the same stale m.
constexpr float kRescaleSlack = 8.0f;

// Placement of one [B, H, L, d] operand: element (b, h, i, c) lives at
// b*sb + h*sh + i*sl + c elements from the base pointer.  Contiguous
// [B, H, L, d]: sb = H*L*d, sh = L*d, sl = d.  Token-major [B, L, ld] with
// head h in columns [h*d, h*d + d): sb = L*ld, sh = d, sl = ld.
struct Layout {
  long long sb;
  int sh, sl;
  __host__ __device__ size_t head(int bh, int H) const {
    const int b = bh / H;
    return (size_t)b * (size_t)sb + (size_t)(bh - b * H) * (size_t)sh;
  }
};

// Bytes from a head's first element to the end of its last row: rows at or
// past L start beyond this, so range-checked loads read them as zero.
__device__ __forceinline__ uint32_t head_span_bytes(int L, int sl, int d, int esz) {
  return (uint32_t)((L - 1) * sl + d) * (uint32_t)esz;
}

// Arguments common to the 16-bit (bf16 or fp16) kernels; q/k/v hold 16-bit
// element bit patterns, v is placed like k.
struct Args16 {
  const uint16_t *q;
  const uint16_t *k;
  const uint16_t *v;
  void *out;
  int H;
  Layout lq, lk, lo;
  int Lq, Lk, d;
  int qblocks;     // workgroups per (b, h)
  int nwg;         // total workgroups
  float c;         // |scale| * log2(e): scores enter exp2 as s * c
  uint32_t qsign;  // 0x80008000 flips Q's sign bits when scale < 0
};

struct F32Args {
  const float *q;
  const float *k;
  const float *v;
  float *out;
  int H;
  Layout lq, lk, lo;
  int Lq, Lk, d;
  int qblocks;
  float scale;
};

// GroupNorm (+ SiLU): x, y are [N, C, S] contiguous (S = H*W), G groups of
// C/G consecutive channels, per-channel fp32 gamma and beta.
struct GnArgs {
  const void *x;
  const float *gamma;
  const float *beta;
  void *y;
  int N, C, S, G;
  float eps;
  int silu;
  int split;  // workgroups per group (1: the group's own workgroup only)
};

// The dispatcher hands workgroup i to XCD (i mod 8).  Renumber so that the
// workgroups resident on one XCD get consecutive logical ids, i.e. the
// query blocks of one (b, h) share that XCD's L2 copy of its K and V.
// A bijection on [0, n) for every n.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = i & 7, k = i >> 3;
  return (x < rem) ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).
// Lane l supplies row (l % 32) of A / column (l % 32) of B with eight
// consecutive k values; the accumulator gives lane l column (l % 32) and
// rows 8*(i/4) + 4*(l/32) + (i%4) for register i.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The 16-bit element type of the matrix-core kernels: bf16 (H = false) or
// fp16 (H = true).  Operands travel as bit patterns in bf16x8 containers;
// only the matrix instruction, the packing of fp32 results and the constant
// one differ.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <bool H>
__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (H)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool H>
constexpr uint16_t one16() { return H ? 0x3C00 : 0x3F80; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) {
  return __builtin_bit_cast(bf16x8, x);
}

__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void st16(void *p, u32x4 x) {
  *reinterpret_cast<u32x4 *>(p) = x;
}

// Half-wave exchanges through v_permlane32_swap (a VALU op, no LDS trip).
// With both operands holding x, the swap leaves {x_lo, x_lo} in the first
// result and {x_hi, x_hi} in the second, lane by lane.
__device__ __forceinline__ void halves(float x, float &lo_bcast, float &hi_bcast) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  lo_bcast = __uint_as_float(r[0]);
  hi_bcast = __uint_as_float(r[1]);
}

// max over lanes l and l ^ 32.
__device__ __forceinline__ float max_halves(float x) {
  float a, b;
  halves(x, a, b);
  return fmaxf(a, b);
}

// sum over lanes l and l ^ 32.
__device__ __forceinline__ float sum_halves(float x) {
  float a, b;
  halves(x, a, b);
  return a + b;
}

// Every lane gets the value of lane (l % 32).
__device__ __forceinline__ float from_low_half(float x) {
  float a, b;
  halves(x, a, b);
  return a;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// bf16 bits of two floats packed low/high, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Same in the element type H (fp16: v_cvt_pk_f16_f32, round to nearest even).
template <bool H>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (H) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 p = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, p);
  } else {
    return pack_bf16x2(lo, hi);
  }
}

}  // namespace sdattn
