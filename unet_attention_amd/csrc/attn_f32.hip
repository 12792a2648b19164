// attn_f32.hip -- fp32 attention kernel (fp32 in, fp32 arithmetic, fp32 out).
//
// Same method as the bf16 kernels (page "Diffusion inference engine from
// scratch: Rust + wgpu", section 3.2: scores computed tile by tile with a
// running maximum and running sum, never stored), on the vector ALUs:
// one wave per 16 query rows; each lane scores one key of a 64-key tile
// against all 16 rows, wave reductions give each row's tile maximum and
// sum, the weights go through LDS and each lane accumulates O for its own
// head-dim columns.  This path exists for fp32 accuracy (~1e-6), not speed.
#include "attn_common.hpp"
#include "launch.hpp"

namespace sdattn {

namespace {

constexpr int kQB = 16;  // query rows per workgroup

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <int DU>  // ceil(d / 64): output columns per lane
__global__ __launch_bounds__(kWave) void attn_f32_kernel(F32Args a) {
  __shared__ __attribute__((aligned(16))) float qs[kQB * 256];
  __shared__ float ps[kQB * kWave];
  const int lane = threadIdx.x;
  const int bh = blockIdx.x / a.qblocks;
  const int q0 = (blockIdx.x - bh * a.qblocks) * kQB;
  const int d = a.d, Lq = a.Lq, Lk = a.Lk;
  const int slq = a.lq.sl, slk = a.lk.sl, slo = a.lo.sl;
  const float *qg = a.q + a.lq.head(bh, a.H);
  const float *kg = a.k + a.lk.head(bh, a.H);
  const float *vg = a.v + a.lk.head(bh, a.H);

  for (int idx = lane; idx < kQB * d; idx += kWave) {
    const int r = idx / d, cc = idx - r * d;
    qs[idx] = (q0 + r < Lq) ? qg[(size_t)(q0 + r) * slq + cc] : 0.f;
  }
  __syncthreads();

  float m[kQB], l[kQB], o[kQB][DU];
#pragma unroll
  for (int r = 0; r < kQB; ++r) {
    m[r] = -__builtin_inff();
    l[r] = 0.f;
#pragma unroll
    for (int u = 0; u < DU; ++u) o[r][u] = 0.f;
  }

  for (int j0 = 0; j0 < Lk; j0 += kWave) {
    const int j = j0 + lane;
    const bool valid = j < Lk;
    float s[kQB];
#pragma unroll
    for (int r = 0; r < kQB; ++r) s[r] = 0.f;
    const float *kr = kg + (size_t)(valid ? j : 0) * slk;
    for (int cc = 0; cc < d; cc += 4) {
      f32x4 kv = {0.f, 0.f, 0.f, 0.f};
      if (valid) kv = *reinterpret_cast<const f32x4 *>(kr + cc);
#pragma unroll
      for (int r = 0; r < kQB; ++r) {
        const f32x4 qv = *reinterpret_cast<const f32x4 *>(qs + r * d + cc);
        s[r] = __builtin_fmaf(qv[0], kv[0], s[r]);
        s[r] = __builtin_fmaf(qv[1], kv[1], s[r]);
        s[r] = __builtin_fmaf(qv[2], kv[2], s[r]);
        s[r] = __builtin_fmaf(qv[3], kv[3], s[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kQB; ++r) {
      const float t = valid ? s[r] * a.scale : -__builtin_inff();
      const float mn = fmaxf(m[r], wave_max(t));
      const float alpha = expf(m[r] - mn);
      const float p = valid ? expf(t - mn) : 0.f;
      l[r] = l[r] * alpha + wave_sum(p);
#pragma unroll
      for (int u = 0; u < DU; ++u) o[r][u] *= alpha;
      m[r] = mn;
      ps[r * kWave + lane] = p;
    }
    __syncthreads();
    const int nj = min(kWave, Lk - j0);
    for (int jj = 0; jj < nj; ++jj) {
      const float *vr = vg + (size_t)(j0 + jj) * slk;
      float vv[DU];
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        const int col = lane + kWave * u;
        vv[u] = (col < d) ? vr[col] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < kQB; ++r) {
        const float pr = ps[r * kWave + jj];
#pragma unroll
        for (int u = 0; u < DU; ++u) o[r][u] = __builtin_fmaf(pr, vv[u], o[r][u]);
      }
    }
    __syncthreads();
  }

  float *og = a.out + a.lo.head(bh, a.H);
#pragma unroll
  for (int r = 0; r < kQB; ++r) {
    if (q0 + r >= Lq) continue;
    const float inv = 1.0f / l[r];
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int col = lane + kWave * u;
      if (col < d) og[(size_t)(q0 + r) * slo + col] = o[r][u] * inv;
    }
  }
}

}  // namespace

hipError_t launch_f32(const F32Args &base, int BH, hipStream_t stream) {
  F32Args a = base;
  a.qblocks = (a.Lq + kQB - 1) / kQB;
  const dim3 grid(BH * a.qblocks), block(kWave);
  switch ((a.d + kWave - 1) / kWave) {
    case 1: return launch_kernel(&attn_f32_kernel<1>, grid, block, 0, stream, a);
    case 2: return launch_kernel(&attn_f32_kernel<2>, grid, block, 0, stream, a);
    case 3: return launch_kernel(&attn_f32_kernel<3>, grid, block, 0, stream, a);
    case 4: return launch_kernel(&attn_f32_kernel<4>, grid, block, 0, stream, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdattn
