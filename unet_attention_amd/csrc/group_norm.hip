// group_norm.hip -- GroupNorm, optionally fused with the SiLU that follows
// it, for gfx950 (MI355X).
//
// Method: the page "Diffusion inference engine from scratch: Rust + wgpu",
// section 3.1, normalises each group of consecutive channels with its mean
// and variance and 1/sqrt(var + eps) (it reduces partial sums through
// workgroup memory), and its model-level fusion list pairs GroupNorm with
// SiLU in one kernel.  The design here is CDNA4's own:
//
// * one workgroup (8 waves) per (sample, group); the group is contiguous in
//   [N, C, H*W] memory and is read with 16-byte loads;
// * groups of up to kMaxResident elements are read from HBM once into
//   registers (fp32), so the mean and the centred variance are exact
//   two-pass reductions on chip (wave shuffles, then one LDS exchange) and
//   the output is written once: the minimum traffic, one read and one write;
// * larger groups stream twice: moments for the statistics, then the
//   normalising pass.  Each thread sums its values shifted by its own first
//   value (so its sums cancel by at most a factor n + 1 for its n values),
//   and the per-thread (count, mean, M2) are merged pairwise with Chan's
//   update, which stays exact-in-form however far apart the partial means
//   are;
// * out of place, when there are fewer groups than CUs, several workgroups
//   share a group: each forms the group's statistics (from L2 after the
//   first read) and normalises its own slice;
// * per channel y = (x - mu) * (rstd * gamma) + beta, then SiLU
//   y / (1 + e^-y) when requested.
#include "attn_common.hpp"
#include "launch.hpp"

namespace sdattn {

namespace {

constexpr int kGnThreads = 512;                      // 8 waves
constexpr int kGnWaves = kGnThreads / kWave;
constexpr int kMaxChunksPerThread = 16;               // 8 elements per chunk
// Chunks of its own slice a split-form workgroup keeps in registers per
// thread (a larger slice is read again for the normalisation).
constexpr int kSliceChunks = 10;
constexpr int kMaxResident = kGnThreads * kMaxChunksPerThread * 8;  // 65536
constexpr int kMaxGroupChannels = 8192;  // gamma + beta of a group in <= 64 KB of LDS

// Element codes: 0 fp32, 1 bf16, 2 fp16.
template <int ET>
__device__ __forceinline__ void load8(const void *base, size_t e, float (&v)[8]) {
  if constexpr (ET == 0) {
    const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + e);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (ET == 1) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      } else {
        // Scalar halves: the two-lane vector form of this conversion was
        // miscompiled here (one half-pair replicated into all four).
        const uint32_t wi = w[i];
        v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wi & 0xffffu));
        v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wi >> 16));
      }
    }
  }
}

template <int ET, bool OUT_F32>
__device__ __forceinline__ void store8(void *base, size_t e, const float (&v)[8]) {
  if constexpr (OUT_F32 || ET == 0) {
    f32x4 *p = reinterpret_cast<f32x4 *>(static_cast<float *>(base) + e);
    p[0] = f32x4{v[0], v[1], v[2], v[3]};
    p[1] = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    constexpr bool H = (ET == 2);
    *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(base) + e) =
        u32x4{pack2<H>(v[0], v[1]), pack2<H>(v[2], v[3]), pack2<H>(v[4], v[5]),
              pack2<H>(v[6], v[7])};
  }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Sum over the workgroup; every thread gets the total.  red holds
// kGnWaves floats; the leading barrier keeps an earlier use of red safe.
__device__ __forceinline__ float block_sum(float x, float *red) {
  x = wave_sum(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = x;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kGnWaves; ++w) t += red[w];
  return t;
}

// Count, mean and sum of squared deviations of a set of values.
struct Moments {
  float n, mean, m2;
};

// Moments of the union of two disjoint sets (Chan, Golub and LeVeque's
// pairwise update).  Either set may be empty.
__device__ __forceinline__ Moments merge_moments(Moments a, Moments b) {
  const float n = a.n + b.n;
  if (n == 0.f) return a;
  const float dl = b.mean - a.mean;
  const float fb = b.n / n;
  return Moments{n, __builtin_fmaf(dl, fb, a.mean), a.m2 + b.m2 + dl * dl * a.n * fb};
}

// A thread's moments from its n values' sums about the shift x0:
// s1 = sum(x - x0), s2 = sum((x - x0)^2).
__device__ __forceinline__ Moments moments_from_shifted(float n, float x0, float s1, float s2) {
  if (n == 0.f) return Moments{0.f, 0.f, 0.f};
  const float d1 = s1 / n;
  return Moments{n, x0 + d1, fmaxf(s2 - s1 * d1, 0.f)};
}

// Moments of the whole workgroup's values, identical in every thread:
// pairwise merges across the wave, then the waves' results in wave order.
// red holds 3 * kGnWaves floats; the leading barrier keeps an earlier use
// of red safe.
__device__ __forceinline__ Moments block_moments(Moments m, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const Moments o{__shfl_xor(m.n, off), __shfl_xor(m.mean, off), __shfl_xor(m.m2, off)};
    m = merge_moments(m, o);
  }
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    const int w = threadIdx.x / kWave;
    red[3 * w] = m.n;
    red[3 * w + 1] = m.mean;
    red[3 * w + 2] = m.m2;
  }
  __syncthreads();
  Moments t{red[0], red[1], red[2]};
#pragma unroll
  for (int w = 1; w < kGnWaves; ++w) t = merge_moments(t, Moments{red[3 * w], red[3 * w + 1], red[3 * w + 2]});
  return t;
}

// y * sigmoid(y); the hardware reciprocal (1 ulp) in place of an IEEE
// division.  e^-y overflowing to +inf gives y * 0, the correct limit.
__device__ __forceinline__ float silu(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
}

// The group's gamma and beta slices (cpg values each) go to LDS once, at
// the start, while the activations are in flight; a per-chunk global read
// of them would put one memory latency per chunk on the critical path.
// gb holds gamma in [0, cpg) and beta in [cpg, 2*cpg); the reductions'
// barriers order these writes before any read.
__device__ __forceinline__ void stage_affine(const GnArgs &a, int c0, int cpg, float *gb) {
  for (int i = threadIdx.x; i < cpg; i += kGnThreads) {
    gb[i] = a.gamma[c0 + i];
    gb[cpg + i] = a.beta[c0 + i];
  }
}

// y = (x - mu) * a + beta with a = rstd * gamma, for the 8 values of one
// chunk (all in group-local channel cc).  Subtracting mu first keeps x near
// mu exact even when a is large (a near-constant group, var << eps); folding
// mu into the shift would cancel catastrophically there.
template <int ET, bool OUT_F32, bool SILU>
__device__ __forceinline__ void normalise_store(const GnArgs &a, size_t e, const float *gb,
                                                int cpg, int cc, float mu, float rstd,
                                                float (&v)[8]) {
  const float sc = rstd * gb[cc];
  const float sh = gb[cpg + cc];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = __builtin_fmaf(v[i] - mu, sc, sh);
    v[i] = SILU ? silu(y) : y;
  }
  store8<ET, OUT_F32>(a.y, e, v);
}

// Chunks of [ja, nch) this thread visits (ja + tid, ja + tid + kGnThreads, ...).
__device__ __forceinline__ int own_chunks(int ja, int nch) {
  const int first = ja + (int)threadIdx.x;
  return first < nch ? (nch - first + kGnThreads - 1) / kGnThreads : 0;
}

// The first value of chunk j (the first chunk this thread sums), the shift
// of its sums: being one of the thread's own values, it lies within the
// thread's spread.  0 for a thread with no chunk (j >= nch).
template <int ET>
__device__ __forceinline__ float thread_shift(const void *x, size_t base, int j, int nch) {
  if (j >= nch) return 0.f;
  float v[8];
  load8<ET>(x, base + (size_t)j * 8, v);
  return v[0];
}

// Shifted sums s1 += x - x0, s2 += (x - x0)^2 over this thread's chunks
// ja + tid, ja + tid + kGnThreads, ... of [ja, nch), U chunk loads in flight
// at a time (a chunk past the range adds x0, i.e. nothing).
template <int ET, int U>
__device__ __forceinline__ void shifted_sums(const void *x, size_t base, int ja, int nch,
                                             float x0, float &s1, float &s2) {
  for (int j0 = ja + (int)threadIdx.x; j0 < nch; j0 += U * kGnThreads) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * kGnThreads;
      if (j < nch) {
        load8<ET>(x, base + (size_t)j * 8, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[u][i] = x0;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = v[u][i] - x0;
        s1 += t;
        s2 = __builtin_fmaf(t, t, s2);
      }
  }
}

// Normalise chunks [j0, j1) of a group, U chunk loads in flight at a time.
template <int ET, bool OUT_F32, bool SILU, int U>
__device__ __forceinline__ void normalise_range(const GnArgs &a, size_t base, int j0, int j1,
                                                const float *gb, int cpg, float mu,
                                                float rstd) {
  const int cpc = a.S / 8;  // chunks per channel
  for (int jb = j0 + (int)threadIdx.x; jb < j1; jb += U * kGnThreads) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * kGnThreads;
      if (j < j1) load8<ET>(a.x, base + (size_t)j * 8, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * kGnThreads;
      if (j < j1)
        normalise_store<ET, OUT_F32, SILU>(a, base + (size_t)j * 8, gb, cpg, j / cpc,
                                           mu, rstd, v[u]);
    }
  }
}

// Register-resident path: KPT chunks of 8 elements per thread.
template <int ET, bool OUT_F32, bool SILU, int KPT>
__global__ __launch_bounds__(kGnThreads) void group_norm_resident(GnArgs a) {
  __shared__ float red[kGnWaves];
  extern __shared__ float gb[];
  const int ng = blockIdx.x;
  const int n = ng / a.G, g = ng - n * a.G;
  const int cpg = a.C / a.G;
  const size_t base = ((size_t)n * a.C + (size_t)g * cpg) * a.S;
  const int nch = cpg * a.S / 8;  // chunks in the group
  const int tid = threadIdx.x;

  float v[KPT][8];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int j = tid + k * kGnThreads;
    if (j < nch) {
      load8<ET>(a.x, base + (size_t)j * 8, v[k]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[k][i] = 0.f;
    }
  }
  stage_affine(a, g * cpg, cpg, gb);
#pragma unroll
  for (int k = 0; k < KPT; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[k][i];
  const float inv_m = 1.0f / (float)(nch * 8);
  const float mu = block_sum(s, red) * inv_m;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    if (tid + k * kGnThreads < nch) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = v[k][i] - mu;
        q = __builtin_fmaf(t, t, q);
      }
    }
  }
  const float var = block_sum(q, red) * inv_m;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  const int cpc = a.S / 8;  // chunks per channel
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int j = tid + k * kGnThreads;
    if (j < nch)
      normalise_store<ET, OUT_F32, SILU>(a, base + (size_t)j * 8, gb, cpg, j / cpc, mu, rstd,
                                         v[k]);
  }
}

// Streaming path for groups larger than kMaxResident: statistics from sums
// shifted by the group's first element, then a second pass that normalises.
template <int ET, bool OUT_F32, bool SILU>
__global__ __launch_bounds__(kGnThreads) void group_norm_stream(GnArgs a) {
  __shared__ float red[3 * kGnWaves];
  extern __shared__ float gb[];
  const int ng = blockIdx.x;
  const int n = ng / a.G, g = ng - n * a.G;
  const int cpg = a.C / a.G;
  const size_t base = ((size_t)n * a.C + (size_t)g * cpg) * a.S;
  const int nch = cpg * a.S / 8;
  const int tid = threadIdx.x;

  stage_affine(a, g * cpg, cpg, gb);
  // this thread's chunks are tid, tid + kGnThreads, ...; its shift is the
  // first value of its first chunk
  const float x0 = thread_shift<ET>(a.x, base, tid, nch);
  float s1 = 0.f, s2 = 0.f;
  shifted_sums<ET, 8>(a.x, base, 0, nch, x0, s1, s2);
  const Moments mo = block_moments(
      moments_from_shifted(8.0f * (float)own_chunks(0, nch), x0, s1, s2), red);
  const float mu = mo.mean;
  const float rstd = 1.0f / sqrtf(mo.m2 / mo.n + a.eps);
  // In place, each chunk is read and then written by the same thread after
  // every read of the statistics pass (the block sums are barriers).
  normalise_range<ET, OUT_F32, SILU, 4>(a, base, 0, nch, gb, cpg, mu, rstd);
}

// Split form (out of place only): K = a.split workgroups per group, placed on
// one XCD.  Each computes the whole group's statistics itself (shifted sums;
// after the first workgroup's misses the group comes from L2) and normalises
// only its 1/K slice, so the per-element work of a group spreads over K CUs
// with no workspace and no inter-workgroup wait.  Not used in place: a
// slice's writes would race with the other workgroups' statistics reads.
template <int ET, bool OUT_F32, bool SILU>
__global__ __launch_bounds__(kGnThreads) void group_norm_split(GnArgs a) {
  __shared__ float red[3 * kGnWaves];
  extern __shared__ float gb[];
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int K = a.split;
  const int ng = wg / K, k = wg - ng * K;
  const int n = ng / a.G, g = ng - n * a.G;
  const int cpg = a.C / a.G;
  const size_t base = ((size_t)n * a.C + (size_t)g * cpg) * a.S;
  const int nch = cpg * a.S / 8;
  const int tid = threadIdx.x;

  stage_affine(a, g * cpg, cpg, gb);
  const int j0 = (int)((long long)k * nch / K), j1 = (int)((long long)(k + 1) * nch / K);
  if (j1 - j0 <= kSliceChunks * kGnThreads) {
    // this thread sums its slice chunks, then its chunks of [0, j0) and of
    // [j1, nch); its shift is the first of these
    const int jf = (j0 + tid < j1) ? j0 + tid : (tid < j0) ? tid : j1 + tid;
    const float x0 = thread_shift<ET>(a.x, base, jf, nch);
    const float nt =
        8.0f * (float)(own_chunks(j0, j1) + own_chunks(0, j0) + own_chunks(j1, nch));
    // This workgroup's slice stays in registers from the statistics pass to
    // the normalisation (read once; its loads overlap the rest of the group).
    const int cpc = a.S / 8;
    float own[kSliceChunks][8];
#pragma unroll
    for (int u = 0; u < kSliceChunks; ++u) {
      const int j = j0 + tid + u * kGnThreads;
      if (j < j1) load8<ET>(a.x, base + (size_t)j * 8, own[u]);
    }
    float s1 = 0.f, s2 = 0.f;
    shifted_sums<ET, 8>(a.x, base, 0, j0, x0, s1, s2);
    shifted_sums<ET, 8>(a.x, base, j1, nch, x0, s1, s2);
#pragma unroll
    for (int u = 0; u < kSliceChunks; ++u) {
      if (j0 + tid + u * kGnThreads < j1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float t = own[u][i] - x0;
          s1 += t;
          s2 = __builtin_fmaf(t, t, s2);
        }
      }
    }
    const Moments mo = block_moments(moments_from_shifted(nt, x0, s1, s2), red);
    const float mu = mo.mean;
    const float rstd = 1.0f / sqrtf(mo.m2 / mo.n + a.eps);
#pragma unroll
    for (int u = 0; u < kSliceChunks; ++u) {
      const int j = j0 + tid + u * kGnThreads;
      if (j < j1)
        normalise_store<ET, OUT_F32, SILU>(a, base + (size_t)j * 8, gb, cpg, j / cpc, mu, rstd,
                                           own[u]);
    }
    return;
  }
  const float x0 = thread_shift<ET>(a.x, base, tid, nch);
  float s1 = 0.f, s2 = 0.f;
  shifted_sums<ET, 8>(a.x, base, 0, nch, x0, s1, s2);
  const Moments mo =
      block_moments(moments_from_shifted(8.0f * (float)own_chunks(0, nch), x0, s1, s2), red);
  const float mu = mo.mean;
  const float rstd = 1.0f / sqrtf(mo.m2 / mo.n + a.eps);
  normalise_range<ET, OUT_F32, SILU, 4>(a, base, j0, j1, gb, cpg, mu, rstd);
}

template <int ET, bool OUT_F32, bool SILU>
hipError_t launch_gn_et(const GnArgs &a, hipStream_t stream) {
  const int nch = a.C / a.G * a.S / 8;
  const dim3 grid(a.N * a.G), block(kGnThreads);
  const size_t lds = 2 * sizeof(float) * (a.C / a.G);  // the group's gamma and beta
  if (a.split > 1)
    return launch_kernel(&group_norm_split<ET, OUT_F32, SILU>, dim3(a.N * a.G * a.split), block,
                         lds, stream, a);
  const int kpt = (nch + kGnThreads - 1) / kGnThreads;
  if (kpt <= 2)
    return launch_kernel(&group_norm_resident<ET, OUT_F32, SILU, 2>, grid, block, lds, stream, a);
  if (kpt <= 4)
    return launch_kernel(&group_norm_resident<ET, OUT_F32, SILU, 4>, grid, block, lds, stream, a);
  if (kpt <= 8)
    return launch_kernel(&group_norm_resident<ET, OUT_F32, SILU, 8>, grid, block, lds, stream, a);
  if (kpt <= kMaxChunksPerThread)
    return launch_kernel(&group_norm_resident<ET, OUT_F32, SILU, kMaxChunksPerThread>, grid,
                         block, lds, stream, a);
  return launch_kernel(&group_norm_stream<ET, OUT_F32, SILU>, grid, block, lds, stream, a);
}

template <int ET, bool OUT_F32>
hipError_t launch_gn_out(const GnArgs &a, hipStream_t stream) {
  return a.silu ? launch_gn_et<ET, OUT_F32, true>(a, stream)
                : launch_gn_et<ET, OUT_F32, false>(a, stream);
}

}  // namespace

int group_norm_max_resident() { return kMaxResident; }

int group_norm_max_channels_per_group() { return kMaxGroupChannels; }

hipError_t launch_group_norm(const GnArgs &a, int elem, bool out_f32, hipStream_t stream) {
  switch (elem) {
    case 0: return launch_gn_out<0, true>(a, stream);
    case 1: return out_f32 ? launch_gn_out<1, true>(a, stream) : launch_gn_out<1, false>(a, stream);
    case 2: return out_f32 ? launch_gn_out<2, true>(a, stream) : launch_gn_out<2, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdattn
