// attn_bf16.hip -- bf16 fused attention kernels for gfx950 (MI355X).
//
// Method: the page "Diffusion inference engine from scratch: Rust + wgpu",
// section 3.2, computes cross-attention block by block with a running row
// maximum and running sum so the Q.K^T score matrix never reaches memory.
// Its WGSL tiles (64 x 64 x 32, 16 x 16 threads, fp32 scores in workgroup
// memory) target Vulkan/Metal-class GPUs; the design here is CDNA4's own:
//
// * one wave owns 32 query rows; both products run on the 32x32x16 bf16
//   matrix cores with fp32 accumulation;
// * scores are produced transposed, S^T = K Q^T, so lane l holds the scores
//   of query (l % 32) against 16 keys of each 32-key sub-tile: the row
//   maximum and row sum are in-lane plus one exchange between half-waves;
// * the S^T accumulator registers, rounded to bf16, are exactly the B
//   operand of O^T += V^T P^T, so the weights never leave registers; V is
//   stored transposed in LDS with its keys in the matching order;
// * the running maximum lives in the log2 domain (exp2 with scale*log2(e)
//   folded into one FMA) and is raised lazily, only when a tile's maximum
//   exceeds it by kRescaleSlack binary orders;
// * when the head dim is padded (d = 40 -> 64, 80 -> 96 columns of V^T), a
//   row of ones in the padding makes the matrix core produce the row sum l
//   for free;
// * streaming kernel: K and V^T tiles of 64 keys double-buffered in LDS,
//   prefetched into registers one tile ahead, one barrier per tile;
//   short-key kernel (text contexts, Lk <= 128): all keys loaded to LDS
//   once, single-pass softmax with no rescaling.
#include "attn_common.hpp"
#include "launch.hpp"

namespace sdattn {

namespace {

constexpr int kBN = 64;        // keys per streamed tile
constexpr int kShortMax = 128;  // keys held by the short-key kernel
constexpr uint16_t kBf16One = 0x3F80;

template <int DK>
struct Shape {
  static constexpr int DV = (DK + 31) / 32 * 32;   // O^T rows (32-row tiles)
  static constexpr bool kOnes = (DV > DK);         // padding holds a ones row
  static constexpr int DK8 = DK / 8;               // 16-byte chunks per row
  static constexpr int KST = DK + 8;               // K row stride in LDS
};

// Q fragments: B operand of S^T = K Q^T.  Lane l holds query q0 + l%32 and
// columns dk*16 + 8*(l/32) .. +7; rows past Lq and columns past d are zero.
template <int DK>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[DK / 16],
                                       const uint16_t *qg, int q0, int Lq,
                                       int d, uint32_t qsign, int lane) {
  const int qi = q0 + (lane & 31);
  const int cb = 8 * (lane >> 5);
#pragma unroll
  for (int dk = 0; dk < DK / 16; ++dk) {
    const int c0 = dk * 16 + cb;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < Lq && c0 < d) x = ld16(qg + (size_t)qi * d + c0);
    x ^= qsign;
    qf[dk] = as_bf16x8(x);
  }
}

// Transpose four key rows x eight columns (bf16) into eight columns x four
// keys and store them as 8-byte runs of V^T.  Within each 16-key chunk the
// keys are stored in the order in which one half-wave consumes them as an
// MFMA operand: slot 8*hh + 4*a + r holds key 8*a + 4*hh + r.
__device__ __forceinline__ void store_vt_unit(uint16_t *vt, int vst, int row0,
                                              int g, const u32x4 (&rows)[4]) {
  const int kc = g >> 2, gg = g & 3;
  const int slot = kc * 16 + 8 * (gg & 1) + 4 * (gg >> 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int w = i >> 1;
    uint32_t lo, hi;
    if (i & 1) {
      lo = (rows[0][w] >> 16) | (rows[1][w] & 0xFFFF0000u);
      hi = (rows[2][w] >> 16) | (rows[3][w] & 0xFFFF0000u);
    } else {
      lo = (rows[0][w] & 0xFFFFu) | (rows[1][w] << 16);
      hi = (rows[2][w] & 0xFFFFu) | (rows[3][w] << 16);
    }
    u32x2 pr = {lo, hi};
    *reinterpret_cast<u32x2 *>(vt + (row0 + i) * vst + slot) = pr;
  }
}

// Rows [d, DV) of V^T never change: zeros, plus a row of ones at d when the
// row sum is taken from the matrix core.
template <int DK>
__device__ __forceinline__ void init_vt_const(uint16_t *vt, int vst, int keys,
                                              int d, int tid, int nthreads) {
  using S = Shape<DK>;
  const int per_row = keys / 8;
  const int n = (S::DV - d) * per_row;
  for (int idx = tid; idx < n; idx += nthreads) {
    const int r = d + idx / per_row, c8 = idx % per_row;
    const uint32_t w = (S::kOnes && r == d) ? (uint32_t(kBf16One) * 0x10001u) : 0u;
    u32x4 x = {w, w, w, w};
    st16(vt + r * vst + c8 * 8, x);
  }
}

// K pad columns [d, DK) are zero in every row.
template <int DK>
__device__ __forceinline__ void init_k_pad(uint16_t *ks, int rows, int d,
                                           int tid, int nthreads) {
  using S = Shape<DK>;
  const int d8 = d >> 3, padc = S::DK8 - d8;
  const int n = rows * padc;
  for (int idx = tid; idx < n; idx += nthreads) {
    const int r = idx / padc, c = d8 + idx % padc;
    st16(ks + r * S::KST + c * 8, u32x4{0u, 0u, 0u, 0u});
  }
}

// One 32-key sub-tile of S^T for this wave: sum over head-dim chunks.
template <int DK>
__device__ __forceinline__ f32x16 scores_subtile(const uint16_t *ks, int row0,
                                                 const bf16x8 (&qf)[DK / 16],
                                                 int lane) {
  using S = Shape<DK>;
  f32x16 acc = {};
  const uint16_t *kp = ks + (row0 + (lane & 31)) * S::KST + 8 * (lane >> 5);
#pragma unroll
  for (int dk = 0; dk < DK / 16; ++dk)
    acc = mfma32x32x16(as_bf16x8(ld16(kp + dk * 16)), qf[dk], acc);
  return acc;
}

// O^T += V^T P^T over one 16-key chunk (keys kc*16 .. +15 of the LDS tile).
template <int DK>
__device__ __forceinline__ void pv_chunk(f32x16 (&o)[Shape<DK>::DV / 32],
                                         const uint16_t *vt, int vst, int kc,
                                         bf16x8 p, int lane) {
  using S = Shape<DK>;
  const uint16_t *vp = vt + (lane & 31) * vst + kc * 16 + 8 * (lane >> 5);
#pragma unroll
  for (int mt = 0; mt < S::DV / 32; ++mt)
    o[mt] = mfma32x32x16(as_bf16x8(ld16(vp + mt * 32 * vst)), p, o[mt]);
}

// Key index (relative to the sub-tile) of accumulator register i in this lane.
__device__ __forceinline__ int acc_key(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// Epilogue: divide by the row sum and store this wave's 32 rows.
template <int DK, bool OUT_F32>
__device__ __forceinline__ void store_out(const f32x16 (&o)[Shape<DK>::DV / 32],
                                          float lsum, void *outp, size_t obase,
                                          int q0, int Lq, int d, int lane) {
  using S = Shape<DK>;
  float l;
  if constexpr (S::kOnes) {
    // Row d of O^T holds sum_j p_j; it sits in the first half-wave.
    float lv = 0.f;
#pragma unroll
    for (int mt = 0; mt < S::DV / 32; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        if (mt * 32 + 8 * g4 == d) lv = o[mt][4 * g4];
    l = __shfl(lv, lane & 31);
  } else {
    l = lsum + swap_halves(lsum);
  }
  const float inv = 1.0f / l;
  const int qi = q0 + (lane & 31);
  if (qi >= Lq) return;
  const int hb = 4 * (lane >> 5);
#pragma unroll
  for (int mt = 0; mt < S::DV / 32; ++mt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c0 = mt * 32 + 8 * g4 + hb;
      if (c0 < d) {
        const float x0 = o[mt][4 * g4 + 0] * inv, x1 = o[mt][4 * g4 + 1] * inv;
        const float x2 = o[mt][4 * g4 + 2] * inv, x3 = o[mt][4 * g4 + 3] * inv;
        const size_t off = obase + (size_t)qi * d + c0;
        if constexpr (OUT_F32) {
          f32x4 x = {x0, x1, x2, x3};
          *reinterpret_cast<f32x4 *>(static_cast<float *>(outp) + off) = x;
        } else {
          u32x2 x = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
          *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(outp) + off) = x;
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Streaming kernel: any Lk >= 1.

template <int DK, int NW, bool OUT_F32>
__global__ __launch_bounds__(NW * kWave) void attn_stream_bf16(Bf16Args a) {
  using S = Shape<DK>;
  constexpr int NT = NW * kWave;
  constexpr int VST = kBN + 8;
  constexpr int KCH = (kBN * S::DK8 + NT - 1) / NT;
  constexpr int VU = (kBN / 4) * S::DK8;
  constexpr int VCH = (VU + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * S::KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][S::DV * VST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wg = xcd_remap(blockIdx.x, a.nwg);
  const int bh = wg / a.qblocks;
  const int q0 = (wg - bh * a.qblocks) * (NW * kQW) + wave * kQW;
  const int d = a.d, d8 = d >> 3, Lk = a.Lk, Lq = a.Lq;
  const uint16_t *kg = a.k + (size_t)bh * Lk * d;
  const uint16_t *vg = a.v + (size_t)bh * Lk * d;
  const float c = a.c;

  bf16x8 qf[DK / 16];
  load_q<DK>(qf, a.q + (size_t)bh * Lq * d, q0, Lq, d, a.qsign, lane);

  init_k_pad<DK>(&Ks[0][0], 2 * kBN, d, tid, NT);
  init_vt_const<DK>(&Vt[0][0], VST, kBN, d, tid, NT);
  init_vt_const<DK>(&Vt[1][0], VST, kBN, d, tid, NT);

  u32x4 kreg[KCH];
  u32x4 vreg[VCH][4];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int t = 0; t < KCH; ++t) {
      const int idx = tid + t * NT;
      const int row = idx / S::DK8, ch = idx % S::DK8, j = j0 + row;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (idx < kBN * S::DK8 && ch < d8 && j < Lk) x = ld16(kg + (size_t)j * d + ch * 8);
      kreg[t] = x;
    }
#pragma unroll
    for (int t = 0; t < VCH; ++t) {
      const int u = tid + t * NT;
      const int g = u % (kBN / 4), ch = u / (kBN / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * g + r;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (u < VU && ch < d8 && j < Lk) x = ld16(vg + (size_t)j * d + ch * 8);
        vreg[t][r] = x;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int t = 0; t < KCH; ++t) {
      const int idx = tid + t * NT;
      const int row = idx / S::DK8, ch = idx % S::DK8;
      if (idx < kBN * S::DK8 && ch < d8) st16(&Ks[buf][row * S::KST + ch * 8], kreg[t]);
    }
#pragma unroll
    for (int t = 0; t < VCH; ++t) {
      const int u = tid + t * NT;
      const int g = u % (kBN / 4), ch = u / (kBN / 4);
      if (u < VU && ch < d8) store_vt_unit(&Vt[buf][0], VST, ch * 8, g, vreg[t]);
    }
  };

  f32x16 o[S::DV / 32];
#pragma unroll
  for (int mt = 0; mt < S::DV / 32; ++mt) o[mt] = f32x16{};
  float m_run = -__builtin_inff();  // running max, log2 domain
  float lsum = 0.f;                 // partial row sum (when not from MFMA)

  const int ntiles = (Lk + kBN - 1) / kBN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1, j0 = t * kBN;
    const bool tail = (j0 + kBN > Lk);
    if (t + 1 < ntiles) load_tile(j0 + kBN);

    f32x16 s[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) s[nt] = scores_subtile<DK>(&Ks[buf][0], nt * 32, qf, lane);
    if (tail) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (j0 + nt * 32 + acc_key(i, lane) >= Lk) s[nt][i] = -__builtin_inff();
    }
    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
    mx = fmaxf(mx, swap_halves(mx));
    const float mt_new = mx * c;
    if (__any(mt_new > m_run + kRescaleSlack)) {
      const float mn = fmaxf(m_run, mt_new);
      const float alpha = fast_exp2(m_run - mn);
#pragma unroll
      for (int mt = 0; mt < S::DV / 32; ++mt) o[mt] *= alpha;
      lsum *= alpha;
      m_run = mn;
    }
    const float nm = -m_run;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * kk + j;
          float x = fast_exp2(__builtin_fmaf(s[nt][i], c, nm));
          if (tail && j0 + nt * 32 + acc_key(i, lane) >= Lk) x = 0.f;
          p[j] = x;
          if constexpr (!S::kOnes) lsum += x;
        }
        u32x4 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                    pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        pv_chunk<DK>(o, &Vt[buf][0], VST, nt * 2 + kk, as_bf16x8(pk), lane);
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  store_out<DK, OUT_F32>(o, lsum, a.out, (size_t)bh * Lq * d, q0, Lq, d, lane);
}

// ---------------------------------------------------------------------------
// Short-key kernel: Lk <= kShortMax, every key resident in LDS.

template <int DK, int NW, int QPW, bool OUT_F32>
__global__ __launch_bounds__(NW * kWave) void attn_short_bf16(Bf16Args a) {
  using S = Shape<DK>;
  constexpr int NT = NW * kWave;
  constexpr int NKT = kShortMax / 32;
  constexpr int VST = kShortMax + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kShortMax * S::KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[S::DV * VST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wg = xcd_remap(blockIdx.x, a.nwg);
  const int bh = wg / a.qblocks;
  const int qbase = (wg - bh * a.qblocks) * (NW * kQW * QPW);
  const int d = a.d, d8 = d >> 3, Lk = a.Lk, Lq = a.Lq;
  const uint16_t *qg = a.q + (size_t)bh * Lq * d;
  const uint16_t *kg = a.k + (size_t)bh * Lk * d;
  const uint16_t *vg = a.v + (size_t)bh * Lk * d;
  const float c = a.c;
  const int nkt = (Lk + 31) >> 5;
  const int keys = nkt * 32;

  // Issue the first query tile's loads before staging K and V.
  bf16x8 qf[DK / 16];
  load_q<DK>(qf, qg, qbase + wave * kQW, Lq, d, a.qsign, lane);

  init_k_pad<DK>(Ks, keys, d, tid, NT);
  init_vt_const<DK>(Vt, VST, keys, d, tid, NT);
  for (int idx = tid; idx < keys * S::DK8; idx += NT) {
    const int row = idx / S::DK8, ch = idx % S::DK8;
    if (ch < d8) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < Lk) x = ld16(kg + (size_t)row * d + ch * 8);
      st16(&Ks[row * S::KST + ch * 8], x);
    }
  }
  const int ngroups = keys / 4;
  for (int u = tid; u < ngroups * d8; u += NT) {
    const int g = u % ngroups, ch = u / ngroups;
    u32x4 rows[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * g + r;
      rows[r] = (j < Lk) ? ld16(vg + (size_t)j * d + ch * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    store_vt_unit(Vt, VST, ch * 8, g, rows);
  }
  __syncthreads();

  for (int t = 0; t < QPW; ++t) {
    const int q0 = qbase + (t * NW + wave) * kQW;
    bf16x8 qn[DK / 16];
    if (t + 1 < QPW) load_q<DK>(qn, qg, q0 + NW * kQW, Lq, d, a.qsign, lane);

    f32x16 s[NKT];
    float mx = -__builtin_inff();
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      if (nt < nkt) {
        s[nt] = scores_subtile<DK>(Ks, nt * 32, qf, lane);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (nt * 32 + acc_key(i, lane) >= Lk) s[nt][i] = -__builtin_inff();
          mx = fmaxf(mx, s[nt][i]);
        }
      }
    }
    mx = fmaxf(mx, swap_halves(mx));
    const float nm = -(mx * c);

    f32x16 o[S::DV / 32];
#pragma unroll
    for (int mt = 0; mt < S::DV / 32; ++mt) o[mt] = f32x16{};
    float lsum = 0.f;
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      if (nt < nkt) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 8 * kk + j;
            float x = fast_exp2(__builtin_fmaf(s[nt][i], c, nm));
            if (nt * 32 + acc_key(i, lane) >= Lk) x = 0.f;
            p[j] = x;
            if constexpr (!S::kOnes) lsum += x;
          }
          u32x4 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                      pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
          pv_chunk<DK>(o, Vt, VST, nt * 2 + kk, as_bf16x8(pk), lane);
        }
      }
    }
    store_out<DK, OUT_F32>(o, lsum, a.out, (size_t)bh * Lq * d, q0, Lq, d, lane);
    if (t + 1 < QPW) {
#pragma unroll
      for (int dk = 0; dk < DK / 16; ++dk) qf[dk] = qn[dk];
    }
  }
}

constexpr int kStreamWaves = 4;
constexpr int kShortWaves = 4;
constexpr int kShortTiles = 2;   // query tiles per wave in the short kernel

template <int DK>
hipError_t launch_dk(const Bf16Args &base, int BH, bool short_path, bool out_f32,
                     hipStream_t stream) {
  Bf16Args a = base;
  if (short_path) {
    const int per_wg = kShortWaves * kQW * kShortTiles;
    a.qblocks = (a.Lq + per_wg - 1) / per_wg;
    a.nwg = BH * a.qblocks;
    if (out_f32)
      hipLaunchKernelGGL((attn_short_bf16<DK, kShortWaves, kShortTiles, true>),
                         dim3(a.nwg), dim3(kShortWaves * kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_short_bf16<DK, kShortWaves, kShortTiles, false>),
                         dim3(a.nwg), dim3(kShortWaves * kWave), 0, stream, a);
  } else {
    const int per_wg = kStreamWaves * kQW;
    a.qblocks = (a.Lq + per_wg - 1) / per_wg;
    a.nwg = BH * a.qblocks;
    if (out_f32)
      hipLaunchKernelGGL((attn_stream_bf16<DK, kStreamWaves, true>),
                         dim3(a.nwg), dim3(kStreamWaves * kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_stream_bf16<DK, kStreamWaves, false>),
                         dim3(a.nwg), dim3(kStreamWaves * kWave), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

int short_path_max_keys() { return kShortMax; }

hipError_t launch_bf16(const Bf16Args &a, int BH, bool short_path, bool out_f32,
                       hipStream_t stream) {
  const int dk = (a.d + 15) / 16 * 16;
  switch (dk) {
    case 16: return launch_dk<16>(a, BH, short_path, out_f32, stream);
    case 32: return launch_dk<32>(a, BH, short_path, out_f32, stream);
    case 48: return launch_dk<48>(a, BH, short_path, out_f32, stream);
    case 64: return launch_dk<64>(a, BH, short_path, out_f32, stream);
    case 80: return launch_dk<80>(a, BH, short_path, out_f32, stream);
    case 96: return launch_dk<96>(a, BH, short_path, out_f32, stream);
    case 112: return launch_dk<112>(a, BH, short_path, out_f32, stream);
    case 128: return launch_dk<128>(a, BH, short_path, out_f32, stream);
    case 144: return launch_dk<144>(a, BH, short_path, out_f32, stream);
    case 160: return launch_dk<160>(a, BH, short_path, out_f32, stream);
    case 176: return launch_dk<176>(a, BH, short_path, out_f32, stream);
    case 192: return launch_dk<192>(a, BH, short_path, out_f32, stream);
    case 208: return launch_dk<208>(a, BH, short_path, out_f32, stream);
    case 224: return launch_dk<224>(a, BH, short_path, out_f32, stream);
    case 240: return launch_dk<240>(a, BH, short_path, out_f32, stream);
    case 256: return launch_dk<256>(a, BH, short_path, out_f32, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdattn
