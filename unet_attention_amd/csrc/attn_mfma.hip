// attn_mfma.hip -- 16-bit (bf16 / fp16) fused attention kernels for gfx950
// (MI355X).
//
// Method: the page "Diffusion inference engine from scratch: Rust + wgpu",
// section 3.2, computes cross-attention block by block with a running row
// maximum and running sum so the Q.K^T score matrix never reaches memory.
// Its WGSL tiles (64 x 64 x 32, 16 x 16 threads, fp32 scores in workgroup
// memory) target Vulkan/Metal-class GPUs; the design here is CDNA4's own.
//
// Common to every kernel:
// * one wave owns 32 query rows; both products run on the 32x32x16
//   matrix cores (bf16 or fp16 operands, fp32 accumulation), in VGPR form;
// * scores are produced transposed, S^T = K Q^T, so lane l holds the scores
//   of query (l % 32) against 16 keys of each 32-key sub-tile: row
//   reductions are in-lane plus one v_permlane32_swap between half-waves;
// * the S^T accumulator registers, rounded to 16 bits, are exactly the B
//   operand of O^T += V^T P^T, so the weights never leave registers;
// * exp2 with scale*log2(e) folded into one FMA; when the head dim is padded
//   (d = 40 -> 64, 80 -> 96 rows of V^T) a row of ones in the padding makes
//   the matrix core produce the row sum l;
// * Q, K and V are read through range-checked buffer descriptors: rows past
//   the end read as zero;
// * workgroup ids are renumbered so the query blocks of one head share an
//   XCD (and its L2 copy of that head's K and V).
//
// The kernels:
// * attn_stream_fix (self-attention, head dims <= 64): eight waves, 64-key
//   K and V tiles moved by buffer->LDS transfers into six LDS buffers each
//   (iteration j owns the transfers of K tile j+5 and V tile j+3); each
//   iteration computes the scores of tile t+1, the weights of tile t and
//   P.V of tile t-1 in one straight block against a fixed per-row reference
//   (the first processed tile's maximum; exact fallback on overflow); the
//   steady-state loop runs one barrier per pair of iterations; odd query
//   blocks walk the key tiles backwards;
// * attn_stream_rescale (head dims > 64): lazily rescaled running maximum,
//   three LDS buffers, and on small grids a two- or four-way split of every
//   key tile between waves that share a query block, merged through LDS;
// * attn_short (contexts of up to 128 keys, the text encoder's 77): all keys
//   resident in LDS, single-pass softmax (the maximum over every key is
//   known before any exponential), output written through LDS.
#include <type_traits>

#include "attn_common.hpp"
#include "launch.hpp"

namespace sdattn {

namespace {

// Keys held by the short-key kernel.  A 256-key instantiation (scores of all
// keys in registers beside O) measured slower than the streaming kernels
// beyond 128 keys for every head dim, so longer contexts stream.
template <int DK>
constexpr int short_cap() { return 128; }
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 raw buffer, range checked

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)bytes, kRsrcWord3);
}

// 16-byte load; a chunk at or past the buffer's size reads as zero.
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int DK>
struct Shape {
  static constexpr int DV = (DK + 31) / 32 * 32;   // O^T rows (32-row tiles)
  static constexpr bool kOnes = (DV > DK);         // padding holds a ones row
  static constexpr int DK8 = DK / 8;               // 16-byte chunks per row
  static constexpr int KST = DK + 8;               // K row stride in LDS
  static constexpr int MT = DV / 32;               // O^T accumulator tiles
};

// Two waves per SIMD keep the whole working set in <= 256 VGPRs (VGPR-form
// MFMA); the widest head dims need more registers and run one wave per SIMD.
// (The second __launch_bounds__ argument is this minimum waves per SIMD.)
template <int DK>
constexpr int waves_per_simd() { return DK <= 112 ? 2 : 1; }


// Q fragments: B operand of S^T = K Q^T.  Lane l holds query q0 + l%32 and
// columns dk*16 + 8*(l/32) .. +7; rows past Lq and columns past d are zero.
template <int DK>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[DK / 16], rsrc_t qr, int q0,
                                       int d, int sl, uint32_t qsign, int lane) {
  const int qi = q0 + (lane & 31);
  const int cb = 8 * (lane >> 5);
#pragma unroll
  for (int dk = 0; dk < DK / 16; ++dk) {
    const int c0 = dk * 16 + cb;
    u32x4 x = bload16(qr, (uint32_t)(qi * sl + c0) * 2u);
    if (c0 >= d) x = u32x4{0u, 0u, 0u, 0u};
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
    // v_perm_b32 byte selectors: {low halves of a, b} or {high halves}.
    const int w = i >> 1;
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
    u32x2 pr = {__builtin_amdgcn_perm(rows[1][w], rows[0][w], sel),
                __builtin_amdgcn_perm(rows[3][w], rows[2][w], sel)};
    *reinterpret_cast<u32x2 *>(vt + (row0 + i) * vst + slot) = pr;
  }
}

// Rows [d, DV) of V^T never change: zeros, plus a row of ones at d when the
// row sum is taken from the matrix core.  KEYS slots per row are written.
template <int DK, int KEYS, bool H = false>
__device__ __forceinline__ void init_vt_const(uint16_t *vt, int vst, int d, int tid,
                                              int nthreads) {
  using S = Shape<DK>;
  constexpr int per_row = KEYS / 8;
  const int n = (S::DV - d) * per_row;
  for (int idx = tid; idx < n; idx += nthreads) {
    const int r = d + idx / per_row, c8 = idx % per_row;
    const uint32_t w = (S::kOnes && r == d) ? (uint32_t(one16<H>()) * 0x10001u) : 0u;
    st16(vt + r * vst + c8 * 8, u32x4{w, w, w, w});
  }
}

// K pad columns [d, DK) are zero in every row.  d is a multiple of 8 and DK
// the next multiple of 16, so there is at most one 16-byte pad chunk.
template <int DK, int ROWS>
__device__ __forceinline__ void init_k_pad(uint16_t *ks, int d, int tid, int nthreads) {
  using S = Shape<DK>;
  if ((d >> 3) == S::DK8) return;
  for (int r = tid; r < ROWS; r += nthreads)
    st16(ks + r * S::KST + (S::DK8 - 1) * 8, u32x4{0u, 0u, 0u, 0u});
}

// One 32-key sub-tile of S^T for this wave: sum over head-dim chunks.
template <int DK, bool H = false>
__device__ __forceinline__ f32x16 scores_subtile(const uint16_t *kp,
                                                 const bf16x8 (&qf)[DK / 16]) {
  f32x16 acc = {};
#pragma unroll
  for (int dk = 0; dk < DK / 16; ++dk)
    acc = mma<H>(as_bf16x8(ld16(kp + dk * 16)), qf[dk], acc);
  return acc;
}

// O^T += V^T P^T over one 16-key chunk; vp points at this lane's row/slot.
template <int DK, bool H = false>
__device__ __forceinline__ void pv_chunk(f32x16 (&o)[Shape<DK>::MT],
                                         const uint16_t *vp, int vst, bf16x8 p) {
#pragma unroll
  for (int mt = 0; mt < Shape<DK>::MT; ++mt)
    o[mt] = mma<H>(as_bf16x8(ld16(vp + mt * 32 * vst)), p, o[mt]);
}

// Key index (relative to the sub-tile) of accumulator register i in this lane.
__device__ __forceinline__ int acc_key(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// Sequential chain: compiles to v_max3_f32, two new values per instruction.
__device__ __forceinline__ float max16(const f32x16 &s, float m) {
#pragma unroll
  for (int i = 0; i < 16; i += 2) m = fmaxf(fmaxf(m, s[i]), s[i + 1]);
  return m;
}

// Epilogue: divide by the row sum l and store this wave's 32 rows.
template <int DK, bool OUT_F32, bool H = false>
__device__ __forceinline__ void store_out_l(const f32x16 (&o)[Shape<DK>::MT], float l,
                                            void *outp, size_t obase, int q0, int Lq,
                                            int d, int sl, int lane) {
  using S = Shape<DK>;
  const float inv = 1.0f / l;
  const int qi = q0 + (lane & 31);
  if (qi >= Lq) return;
  const int hb = 4 * (lane >> 5);
#pragma unroll
  for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c0 = mt * 32 + 8 * g4 + hb;
      if (c0 < d) {
        const float x0 = o[mt][4 * g4 + 0] * inv, x1 = o[mt][4 * g4 + 1] * inv;
        const float x2 = o[mt][4 * g4 + 2] * inv, x3 = o[mt][4 * g4 + 3] * inv;
        const size_t off = obase + (size_t)qi * sl + c0;
        if constexpr (OUT_F32) {
          f32x4 x = {x0, x1, x2, x3};
          *reinterpret_cast<f32x4 *>(static_cast<float *>(outp) + off) = x;
        } else {
          u32x2 x = {pack2<H>(x0, x1), pack2<H>(x2, x3)};
          *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(outp) + off) = x;
        }
      }
    }
}

// Same, with l taken from the ones row of O^T (padded head dims) or from the
// per-lane partial sums lsum.
template <int DK, bool OUT_F32, bool H = false>
__device__ __forceinline__ void store_out(const f32x16 (&o)[Shape<DK>::MT],
                                          float lsum, void *outp, size_t obase,
                                          int q0, int Lq, int d, int sl, int lane) {
  using S = Shape<DK>;
  float l;
  if constexpr (S::kOnes) {
    // Row d of O^T holds sum_j p_j; it sits in the first half-wave.
    float lv = 0.f;
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        if (mt * 32 + 8 * g4 == d) lv = o[mt][4 * g4];
    l = from_low_half(lv);
  } else {
    l = sum_halves(lsum);
  }
  store_out_l<DK, OUT_F32, H>(o, l, outp, obase, q0, Lq, d, sl, lane);
}

// ---------------------------------------------------------------------------
// Streaming kernels: K and V tiles go from HBM straight into LDS with
// buffer->LDS transfers, so no registers, LDS writes or vector instructions
// are spent on staging, and several LDS buffers (three in the rescaling
// kernel, six in the fixed-reference one) let the transfers of later tiles
// overlap the computation of the current one.
//
// K keeps its row-major [key][DK+8] layout (the MFMA A operand of S^T is a
// plain 16-byte LDS read).  V is also kept row-major, [key][VSTR], and the A
// operand of O^T += V^T P^T is assembled by two transposing LDS reads
// (ds_read_b64_tr_b16): within each 16-lane group, output lane i, element j
// is element (i % 4) of the 8 bytes addressed by source lane 4*j + i/4.  With
// source lane 4*j + q of group g pointing at V[key0 + 4*(g/2) + j][16*(g%2) +
// 4*q], lane l receives row (l % 32) of V^T for keys key0 + 4*(l/32) + 0..3,
// and the second read (8 rows further) keys key0 + 8 + 4*(l/32) + 0..3:
// exactly the key order of the S^T accumulator registers.  Columns [d, DV)
// of every V row are constants written once (a column of ones at d when the
// row sum comes from the matrix core, zeros otherwise); the transfers skip
// them.

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 16-byte buffer -> LDS transfer issued from inline assembly.  Lane i
// writes lds + 16*i bytes (lds: byte address in LDS, wave-uniform); source
// offsets at or past the buffer size write zeros.  The compiler does not see
// the LDS write, so it adds no wait of its own before later LDS reads (it
// cannot tell that they touch other buffers, and would otherwise wait for
// every transfer in flight): the caller orders the transfer with an explicit
// vmcnt wait and barrier before the data is read, and issues it only into a
// buffer that every wave has finished reading.  No register receives data.
// M0 is declared clobbered; nothing the compiler generates for these kernels
// keeps a value in M0 (no compiler-issued LDS transfers, GWS or indexed
// register moves), so the clobber warning does not apply.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_raw(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  // One wait state between the scalar write of M0 and its read by the
  // transfer (a GFX9-family hazard).
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "m0");
}
#pragma clang diagnostic pop

// Raw buffer descriptor words (gfx9 layout: base, stride 0, size in bytes,
// range-checked raw access).
__device__ __forceinline__ u32x4 rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, bytes, kRsrcWord3};
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(lds_void *)const_cast<void *>(p);
}


__device__ __forceinline__ s16x4 ld_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<uint16_t *>(p));
}

// Wait until at most N of this wave's buffer loads are in flight and all of
// its LDS operations are done, then synchronise the workgroup.  (A plain
// __syncthreads would wait for every load, including the prefetch of the
// tile after next.)
template <int N>
__device__ __forceinline__ void vmcnt_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Same with a run-time count n in [0, MAXN] (wave-uniform).
template <int MAXN>
__device__ __forceinline__ void vmcnt_barrier_rt(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) {
      vmcnt_barrier<MAXN>();
      return;
    }
    vmcnt_barrier_rt<MAXN - 1>(n);
  } else {
    vmcnt_barrier<0>();
  }
}

// V row stride of the DMA kernel: an odd multiple of 64 bytes, so the four
// key rows one transposing read touches fall on distinct LDS banks.
template <int DK>
constexpr int dma_vstr() {
  return ((Shape<DK>::DV * 2) % 128 == 0) ? Shape<DK>::DV + 32 : Shape<DK>::DV;
}
// 64-key tiles when three K and three V buffers fit in the CU's 160 KB.
template <int DK>
constexpr int dma_bn() {
  return 3 * 64 * (Shape<DK>::KST + dma_vstr<DK>()) * 2 <= 160 * 1024 ? 64 : 32;
}

// 128-key tiles (for the four-way key split) when three K and three V
// buffers of that size fit in the CU's 160 KB.
template <int DK>
constexpr bool dma_fits_128() {
  return 3 * 128 * (Shape<DK>::KST + dma_vstr<DK>()) * 2 <= 160 * 1024;
}

template <int DK, int NW, int BN_ = dma_bn<DK>()>
struct DmaPlan {
  using S = Shape<DK>;
  static constexpr int BN = BN_;
  static constexpr int NSUB = BN / 32;
  static constexpr int NB = 3;                      // LDS buffers per operand
  static constexpr int KCR = S::KST / 8;            // 16-byte chunks per K row
  static constexpr int VSTR = dma_vstr<DK>();
  static constexpr int VCR = VSTR / 8;
  static constexpr int KBUF = BN * S::KST;          // elements per K buffer
  static constexpr int VBUF = BN * VSTR;            // elements per V buffer
  static constexpr int KI = (BN * KCR + 63) / 64;   // transfers (64 lanes) per K tile
  static constexpr int VI = (BN * VCR + 63) / 64;   // ... per V tile
  static constexpr int NI = KI + VI;
  static constexpr int NIW = (NI + NW - 1) / NW;    // per wave, upper bound
};

// KS = 2 (4) splits every 64-key (128-key) tile between KS waves that own
// the same 32 query rows, each taking one 32-key sub-tile: a workgroup then
// covers NW/KS query blocks, so small problems launch KS times as many
// waves.  Each wave keeps its own running maximum, row sum and O over its
// keys; the partial results are merged through LDS at the end
// (O = sum_w a_w O_w, l = sum_w a_w l_w, a_w = 2^(m_w - max_w m_w)).
template <int DK, int NW, bool OUT_F32, bool H, int KS = 1>
__global__ __launch_bounds__(NW * kWave, (waves_per_simd<DK>()))
void attn_stream_rescale(Args16 a) {
  using S = Shape<DK>;
  using P = DmaPlan<DK, NW, (KS == 4 ? 128 : dma_bn<DK>())>;
  constexpr int BN = P::BN, NSUB = P::NSUB;
  static_assert(KS == 1 || (KS == NSUB && NW % KS == 0), "one 32-key sub-tile per wave and tile");
  // merge area of the split form: per wave pair, O^T (MT x 16 floats per
  // lane), then m and l (one float per lane each)
  constexpr int kMergeFloats = S::MT * 16 * 64 + 2 * 64;
  static_assert(KS == 1 || (NW / KS) * (KS - 1) * kMergeFloats * 4 <=
                               P::NB * (P::KBUF + P::VBUF) * 2,
                "merge area fits in the tile buffers");
  __shared__ __attribute__((aligned(16))) uint16_t smem[P::NB * (P::KBUF + P::VBUF)];
  uint16_t *const Ks = smem;
  uint16_t *const Vs = smem + P::NB * P::KBUF;

  // The wave index is uniform: keep it (and everything derived from it, such
  // as the LDS destinations of the transfers) in scalar registers.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = xcd_remap(blockIdx.x, a.nwg);
  const int bh = wg / a.qblocks;
  const int qw = wave / KS;         // query block of this wave within the workgroup
  const int kh = wave - qw * KS;    // its sub-tile of every key tile (split form)
  const int q0 = (wg - bh * a.qblocks) * (NW / KS * kQW) + qw * kQW;
  const int d = a.d, d8 = d >> 3, Lk = a.Lk, Lq = a.Lq;
  const float c = a.c;
  const int slq = a.lq.sl, slk = a.lk.sl;
  const uint32_t kvbytes = head_span_bytes(Lk, slk, d, 2);
  const rsrc_t qr = make_rsrc(a.q + a.lq.head(bh, a.H), head_span_bytes(Lq, slq, d, 2));
  const u32x4 kw = rsrc_words(a.k + a.lk.head(bh, a.H), kvbytes);
  const u32x4 vw = rsrc_words(a.v + a.lk.head(bh, a.H), kvbytes);
  const int ntiles = (Lk + BN - 1) / BN;
  const bool ragged = (Lk % BN) != 0;

  // This wave's share of each tile's transfers: instruction i = wave + NW*r
  // covers 64 consecutive 16-byte chunks of the K (i < KI) or V buffer.
  uint32_t goff[P::NIW];  // source byte offset within a tile
  int loff[P::NIW];       // destination element offset within a buffer
  bool isk[P::NIW], act[P::NIW];
#pragma unroll
  for (int r = 0; r < P::NIW; ++r) {
    const int i = wave + NW * r;
    isk[r] = i < P::KI;
    const int blk = isk[r] ? i : i - P::KI;
    const int cpos = blk * 64 + lane;
    const int cr = isk[r] ? P::KCR : P::VCR;
    const int row = cpos / cr, col = cpos - row * cr;
    act[r] = (i < P::NI) && row < BN && col < d8;
    goff[r] = (uint32_t)(row * slk + col * 8) * 2u;
    loff[r] = blk * 512;
  }
  // Transfers this wave really issues per tile (one with no active lane is
  // branched over and does not count towards vmcnt).
  int my_count = 0;
#pragma unroll
  for (int r = 0; r < P::NIW; ++r)
    if (wave + NW * r < P::NI && __any(act[r])) ++my_count;
  auto issue = [&](int tt, int b) {
    const uint32_t toff = (uint32_t)(tt * BN * slk) * 2u;
#pragma unroll
    for (int r = 0; r < P::NIW; ++r) {
      if (wave + NW * r < P::NI) {
        if (isk[r]) {
          if (act[r]) dma16_raw(kw, toff + goff[r], lds_addr(Ks + b * P::KBUF + loff[r]));
        } else {
          if (act[r]) dma16_raw(vw, toff + goff[r], lds_addr(Vs + b * P::VBUF + loff[r]));
        }
      }
    }
  };

  bf16x8 qf[DK / 16];
  load_q<DK>(qf, qr, q0, d, slq, a.qsign, lane);
  issue(0, 0);
  if (ntiles > 1) issue(1, 1);

  // Constant columns, never touched by the transfers: K columns [d, DK) and
  // V columns [d, DV) (ones at d for the matrix-core row sum).
  if (d8 < S::DK8) {
    for (int r = tid; r < P::NB * BN; r += NW * kWave)
      st16(Ks + r * S::KST + d8 * 8, u32x4{0u, 0u, 0u, 0u});
  }
  for (int idx = tid; idx < P::NB * BN * (S::DV / 8); idx += NW * kWave) {
    const int r = idx / (S::DV / 8), c8 = idx - r * (S::DV / 8);
    if (c8 >= d8) {
      const uint32_t w0 = (S::kOnes && c8 == d8) ? uint32_t(one16<H>()) : 0u;
      st16(Vs + r * P::VSTR + c8 * 8, u32x4{w0, 0u, 0u, 0u});
    }
  }

  // Per-lane LDS read bases: K rows (l % 32); V rows for the transposing reads.
  const int koff = (lane & 31) * S::KST + 8 * (lane >> 5);
  const int g = lane >> 4, pl = lane & 15;
  const int voff = (4 * (g >> 1) + (pl >> 2)) * P::VSTR + 16 * (g & 1) + 4 * (pl & 3);

  f32x16 o[S::MT];
#pragma unroll
  for (int mt = 0; mt < S::MT; ++mt) o[mt] = f32x16{};
  float m_run = -__builtin_inff();
  float lsum = 0.f;

  // O^T += V^T P^T for one 16-key chunk, V^T assembled by transposing reads.
  auto pv = [&](const uint16_t *vb, int kc, bf16x8 pk) {
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt) {
      const uint16_t *vp = vb + voff + kc * 16 * P::VSTR + mt * 32;
      const s16x4 lo = ld_tr16(vp), hi = ld_tr16(vp + 8 * P::VSTR);
      const bf16x8 av =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[mt] = mma<H>(av, pk, o[mt]);
    }
  };

  // Softmax update for one 32-key sub-tile (scores s, first key key0), then
  // its two P.V chunks from V buffer vb.
  auto sub = [&](auto mask_c, f32x16 &s, int key0, const uint16_t *vb, int kc0) {
    constexpr bool MASK = decltype(mask_c)::value;
    if constexpr (MASK) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + acc_key(i, lane) >= Lk) s[i] = -__builtin_inff();
    }
    float mx = max16(s, -__builtin_inff());
    mx = max_halves(mx);
    const float mt_new = mx * c;
    if (__any(mt_new > m_run + kRescaleSlack)) {
      const float mn = fmaxf(m_run, mt_new);
      const float alpha = fast_exp2(m_run - mn);
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) o[mt] *= alpha;
      lsum *= alpha;
      m_run = mn;
    }
    const float nm = -m_run;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * kk + j;
        float x = fast_exp2(__builtin_fmaf(s[i], c, nm));
        if constexpr (MASK) {
          if (key0 + acc_key(i, lane) >= Lk) x = 0.f;
        }
        p[j] = x;
        if constexpr (!S::kOnes) lsum += x;
      }
      const u32x4 pk = {pack2<H>(p[0], p[1]), pack2<H>(p[2], p[3]),
                        pack2<H>(p[4], p[5]), pack2<H>(p[6], p[7])};
      pv(vb, kc0 + kk, as_bf16x8(pk));
    }
  };

  using Full = std::integral_constant<bool, false>;
  using Ragged = std::integral_constant<bool, true>;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;

  // Tile t, held in LDS buffer B (= t % 3, a compile-time constant): start
  // the transfer of tile t+2 into buffer (B+2) % 3, compute tile t, then wait
  // until tile t+1 has landed everywhere (tile t+2 may stay in flight).
  auto step = [&](auto b_c, auto mask_c, int t) {
    constexpr int B = decltype(b_c)::value;
    if (t + 2 < ntiles) issue(t + 2, (B + 2) % 3);
    const uint16_t *kb = Ks + B * P::KBUF + koff;
    const uint16_t *vb = Vs + B * P::VBUF;
    if constexpr (KS > 1) {
      f32x16 s0 = scores_subtile<DK, H>(kb + 32 * kh * S::KST, qf);
      sub(mask_c, s0, t * BN + 32 * kh, vb, 2 * kh);
    } else {
      f32x16 s0 = scores_subtile<DK, H>(kb, qf), s1;
      if constexpr (NSUB == 2) s1 = scores_subtile<DK, H>(kb + 32 * S::KST, qf);
      sub(mask_c, s0, t * BN, vb, 0);
      if constexpr (NSUB == 2) sub(mask_c, s1, t * BN + 32, vb, 2);
    }
    if (t + 1 < ntiles) vmcnt_barrier_rt<P::NIW>(t + 2 < ntiles ? my_count : 0);
  };

  // Tile 0 (and the constants) must have landed before anyone reads them;
  // tile 1's transfers may still be in flight.
  vmcnt_barrier_rt<P::NIW>(ntiles > 1 ? my_count : 0);

  const int nfull = ragged ? ntiles - 1 : ntiles;
  int t = 0;
  for (; t + 3 <= nfull; t += 3) {
    step(B0{}, Full{}, t);
    step(B1{}, Full{}, t + 1);
    step(B2{}, Full{}, t + 2);
  }
  if (t < nfull) {
    step(B0{}, Full{}, t);
    if (t + 1 < nfull) {
      step(B1{}, Full{}, t + 1);
      if (ragged) step(B2{}, Ragged{}, t + 2);
    } else if (ragged) {
      step(B1{}, Ragged{}, t + 1);
    }
  } else if (ragged) {
    step(B0{}, Ragged{}, t);
  }

  if constexpr (KS > 1) {
    // Every wave is done with the tile buffers (no transfer is in flight
    // after the last tile); they now hold the other waves' partial results,
    // KS-1 slots per query block.
    float *const mg = reinterpret_cast<float *>(smem) + qw * (KS - 1) * kMergeFloats;
    const float lw = S::kOnes ? 0.f : sum_halves(lsum);
    __syncthreads();
    if (kh > 0) {
      float *const slot = mg + (kh - 1) * kMergeFloats;
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) slot[(mt * 16 + i) * 64 + lane] = o[mt][i];
      slot[S::MT * 16 * 64 + lane] = m_run;
      slot[S::MT * 16 * 64 + 64 + lane] = lw;
    }
    __syncthreads();
    if (kh == 0) {
      // key 0 is in this wave's part, so m_run is finite; another part may
      // have seen no key (m = -inf, O = 0, l = 0): its factor is then 0
      float mx = m_run;
#pragma unroll
      for (int w = 1; w < KS; ++w) mx = fmaxf(mx, mg[(w - 1) * kMergeFloats + S::MT * 16 * 64 + lane]);
      const float a0 = fast_exp2(m_run - mx);
      float l = a0 * lw;
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) o[mt] *= a0;
#pragma unroll
      for (int w = 1; w < KS; ++w) {
        const float *slot = mg + (w - 1) * kMergeFloats;
        const float aw = fast_exp2(slot[S::MT * 16 * 64 + lane] - mx);
#pragma unroll
        for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[mt][i] += aw * slot[(mt * 16 + i) * 64 + lane];
        l += aw * slot[S::MT * 16 * 64 + 64 + lane];
      }
      if constexpr (S::kOnes) {
        store_out<DK, OUT_F32, H>(o, 0.f, a.out, a.lo.head(bh, a.H), q0, Lq, d, a.lo.sl, lane);
      } else {
        store_out_l<DK, OUT_F32, H>(o, l, a.out, a.lo.head(bh, a.H), q0, Lq, d, a.lo.sl, lane);
      }
    }
  } else {
    store_out<DK, OUT_F32, H>(o, lsum, a.out, a.lo.head(bh, a.H), q0, Lq, d, a.lo.sl, lane);
  }
}

// ---------------------------------------------------------------------------
// Streaming kernel, fixed-reference form.
//
// Subtracting the row maximum before exponentiating only keeps the weights
// inside fp32's range: any common reference gives the same normalised result
// in exact arithmetic, and the weights are rounded to bf16, whose exponent
// range is fp32's.  This kernel takes the maximum of the first key tile as
// the reference of the whole row and never rescales, so the loop keeps no
// running maximum, no per-tile reduction and no data-dependent branch: each
// iteration is one straight block in which the softmax of tile t (vector
// ALUs) is interleaved with the scores of tile t+1 and P.V of tile t-1
// (matrix cores).  Keys far below the reference underflow to zero, which is
// exact to fp32 precision because the key that set the reference has weight
// 1.  A key more than ~128 binary orders above it overflows; O or l then ends
// non-finite, and the wave recomputes its rows with the exact lazily
// rescaled recurrence, reading K and V straight from memory.
//
// fp16 weights have only 16 binary orders of headroom, so in fp16 (H) the
// kernel also takes each tile's row maximum and, when it exceeds the
// reference by more than kRescaleSlack, moves the reference up and rescales
// O: a lazy rescale at tile granularity, inside the same pipeline.

// Exact recurrence for this wave's 32 query rows (32-key sub-tiles, K and V
// read with buffer loads, no LDS).  Returns the row sum l; O^T in o.
template <int DK, bool H = false>
__device__ __forceinline__ float rows_exact(f32x16 (&o)[Shape<DK>::MT],
                                            const bf16x8 (&qf)[DK / 16], rsrc_t kr,
                                            rsrc_t vr, int Lk, int d, int sl, float c,
                                            int lane) {
  using S = Shape<DK>;
#pragma unroll
  for (int mt = 0; mt < S::MT; ++mt) o[mt] = f32x16{};
  float m_run = -__builtin_inff(), lsum = 0.f;
  const int h = lane >> 5, r32 = lane & 31;
  for (int key0 = 0; key0 < Lk; key0 += 32) {
    f32x16 sv = {};
#pragma unroll
    for (int dk = 0; dk < DK / 16; ++dk) {
      const int c0 = dk * 16 + 8 * h;
      u32x4 x = bload16(kr, (uint32_t)((key0 + r32) * sl + c0) * 2u);
      if (c0 >= d) x = u32x4{0u, 0u, 0u, 0u};
      sv = mma<H>(as_bf16x8(x), qf[dk], sv);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (key0 + acc_key(i, lane) >= Lk) sv[i] = -__builtin_inff();
    float mx = max16(sv, -__builtin_inff());
    mx = max_halves(mx) * c;  // finite: key0 < Lk is a valid key
    if (mx > m_run) {
      const float alpha = fast_exp2(m_run - mx);
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) o[mt] *= alpha;
      lsum *= alpha;
      m_run = mx;
    }
    u32x4 pk[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float p8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * kk + j;
        float x = fast_exp2(__builtin_fmaf(sv[i], c, -m_run));
        if (key0 + acc_key(i, lane) >= Lk) x = 0.f;
        lsum += x;
        p8[j] = x;
      }
      pk[kk] = u32x4{pack2<H>(p8[0], p8[1]), pack2<H>(p8[2], p8[3]),
                     pack2<H>(p8[4], p8[5]), pack2<H>(p8[6], p8[7])};
    }
    // V^T operand: lane l supplies column 32*mt + l%32 of V at the keys its
    // weight slots hold (slot j of half h: key 16*kk + 8*(j/4) + 4*h + j%4).
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) {
        const int col = 32 * mt + r32;
        uint32_t w[4];
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
          uint32_t e[2];
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const int j = 2 * j2 + e2;
            const int key = key0 + 16 * kk + 8 * (j >> 2) + 4 * h + (j & 3);
            e[e2] = col < d ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                  vr, (uint32_t)(key * sl + col) * 2u, 0, 0)
                            : 0u;
          }
          w[j2] = e[0] | (e[1] << 16);
        }
        o[mt] = mma<H>(as_bf16x8(u32x4{w[0], w[1], w[2], w[3]}),
                             as_bf16x8(pk[kk]), o[mt]);
      }
  }
  return sum_halves(lsum);
}

// LDS buffers per operand in the fixed-reference kernel: iteration j owns
// the transfers of K tile j+NB-1 and V tile j+NB-3; the steady-state loop
// runs one barrier per pair of iterations, which needs NB >= 4 (6: the
// transfers of a pair have a pair's time in flight before they are needed).
#ifndef SDATTN_FIX_BUFFERS
#define SDATTN_FIX_BUFFERS 6
#endif
constexpr int kFixBuffers = SDATTN_FIX_BUFFERS;
template <int V>
using IntC = std::integral_constant<int, V>;

// LDS layout of the fixed-reference kernel for head dim D (a multiple of 8,
// DK = D rounded up to 16): rows as short as the operands allow, so that
// few transfer lanes carry padding.
//  * K rows are D elements when D/8 is odd (an odd number of 16-byte chunks
//    puts the 16-byte reads of consecutive rows on distinct banks), else
//    D + 8.  With D < DK the reads of columns [D, DK) see the first columns
//    of the next row, which meet the zero columns of Q; each buffer ends in
//    a zero chunk for its last row.
//  * V rows hold D data columns plus, when DV > DK, the chunk with the
//    ones column.  Transposing reads of columns past that feed rows of O^T
//    at or beyond D, which are never stored; a row length that is a
//    multiple of 128 bytes (which would put the four key rows of one read on
//    the same banks) gets 64 bytes more.
template <int DK, int D, int NW>
struct FixPlan {
  using S = Shape<DK>;
  static_assert(D % 8 == 0 && D <= DK && D + 16 > DK, "D rounds up to DK");
  static constexpr int BN = 64;
  static constexpr int KST = ((D / 8) & 1) ? D : D + 8;
  static constexpr int KPAD = KST < DK ? 8 : 0;
  static constexpr int VNEED = D + (S::kOnes ? 8 : 0);
  static constexpr int VSTR = (VNEED * 2) % 128 == 0 ? VNEED + 32 : VNEED;
  static constexpr int VTAIL = S::DV > VSTR ? S::DV - VSTR : 0;
  static constexpr int KCR = KST / 8, VCR = VSTR / 8;
  static constexpr int KBUF = BN * KST + KPAD;  // elements per K buffer
  static constexpr int VBUF = BN * VSTR;        // elements per V buffer
  static constexpr int KI = (BN * KCR + 63) / 64;
  static constexpr int VI = (BN * VCR + 63) / 64;
  static constexpr int NI = KI + VI;
  static constexpr int NIW = (NI + NW - 1) / NW;
  // K rows without padding (KST == D) fill whole 64-lane transfers: every
  // lane of every K transfer is active.
  static constexpr bool KFULL = KST == D && (BN * KCR) % 64 == 0;
  static_assert((KBUF * 2) % 16 == 0 && (VBUF * 2) % 16 == 0, "16-byte aligned buffers");
};

template <int DK, int D, int NW, bool OUT_F32, bool H = false>
__global__ __launch_bounds__(NW * kWave, 2)
void attn_stream_fix(Args16 a) {
  using S = Shape<DK>;
  using P = FixPlan<DK, D, NW>;
  constexpr int BN = P::BN;
  constexpr int NB = kFixBuffers;  // LDS buffers per operand
  static_assert(NB == 6, "the steady-state loop folds six buffer phases");
  __shared__ __attribute__((aligned(16))) uint16_t
      smem[NB * (P::KBUF + P::VBUF) + (P::VTAIL + 7) / 8 * 8];
  uint16_t *const Ks = smem;
  uint16_t *const Vs = smem + NB * P::KBUF;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = xcd_remap(blockIdx.x, a.nwg);
  const int bh = wg / a.qblocks;
  const int q0 = (wg - bh * a.qblocks) * (NW * kQW) + wave * kQW;
  const int d = D, Lk = a.Lk, Lq = a.Lq;
  const float c = a.c;
  const int slq = a.lq.sl, slk = a.lk.sl;
  const uint16_t *const kbase = a.k + a.lk.head(bh, a.H);
  const uint16_t *const vbase = a.v + a.lk.head(bh, a.H);
  const uint32_t kvbytes = head_span_bytes(Lk, slk, d, 2);
  const rsrc_t qr = make_rsrc(a.q + a.lq.head(bh, a.H), head_span_bytes(Lq, slq, d, 2));
  const rsrc_t kr = make_rsrc(kbase, kvbytes);
  const rsrc_t vr = make_rsrc(vbase, kvbytes);
  const u32x4 kw = rsrc_words(kbase, kvbytes), vw = rsrc_words(vbase, kvbytes);
  const int n = (Lk + BN - 1) / BN;
  const bool ragged = (Lk % BN) != 0;
  // Odd query blocks walk the key tiles from the last one down.  When a
  // head has more query blocks than one round of its XCD's CUs takes (the
  // 128x128 latent: 64 blocks, 32 CUs), the next round then starts on the
  // tiles the previous one read last, still in L2, instead of re-reading
  // from HBM the ones it read first (evicted: a head's K and V outgrow the
  // 4 MB L2).  Any tile order gives the same result.  key_tile(j): the key
  // tile processed j-th; the ragged tile is processed first or last.
  const bool rev = ((wg - bh * a.qblocks) & 1) != 0;
  auto key_tile = [&](int j) { return rev ? n - 1 - j : j; };
  const bool ragged_first = ragged && rev && n > 1, ragged_last = ragged && !rev;

  // Transfers: instruction i = wave + NW*r covers 64 consecutive 16-byte
  // chunks of a K (i < KI) or V buffer.  K tile u goes to K buffer u % NB and
  // V tile u to V buffer u % NB; iteration j owns K tile j+NB-1 and V tile
  // j+NB-3 (the prologue plays iterations 1-NB .. -1).  Iteration t reads K
  // tile t+1 and V tile t-1; both are owned by iteration t+2-NB.
  uint32_t goff[P::NIW];
  uint32_t loff[P::NIW];  // byte offset within a buffer
  bool isk[P::NIW], act[P::NIW];
#pragma unroll
  for (int r = 0; r < P::NIW; ++r) {
    const int i = wave + NW * r;
    isk[r] = i < P::KI;
    const int blk = isk[r] ? i : i - P::KI;
    const int cpos = blk * 64 + lane;
    const int cr = isk[r] ? P::KCR : P::VCR;
    const int row = cpos / cr, col = cpos - row * cr;
    act[r] = (i < P::NI) && row < BN && col < D / 8;
    goff[r] = (uint32_t)(row * slk + col * 8) * 2u;
    loff[r] = (uint32_t)blk * 1024u;
  }
  // Transfers this wave issues per K tile and per V tile (an instruction
  // with no active lane is branched over and does not count in vmcnt).
  int kc = 0, vc = 0;
#pragma unroll
  for (int r = 0; r < P::NIW; ++r)
    if (wave + NW * r < P::NI && __any(act[r])) {
      if (isk[r]) ++kc; else ++vc;
    }
  // Which of its NIW slots this wave issues as a K or a V transfer, and each
  // slot's LDS byte offset within a buffer: wave-uniform values, taken into
  // scalar registers once so the issue code below is scalar arithmetic and
  // scalar branches (with per-lane conditions the compiler kept them as
  // lane masks and rebuilt each branch condition through vector
  // instructions, ~165 cycles per tile).
  int kon[P::NIW], von[P::NIW];
  uint32_t lofs[P::NIW];
#pragma unroll
  for (int r = 0; r < P::NIW; ++r) {
    const bool on = wave + NW * r < P::NI;
    kon[r] = __builtin_amdgcn_readfirstlane((on && isk[r]) ? 1 : 0);
    von[r] = __builtin_amdgcn_readfirstlane((on && !isk[r]) ? 1 : 0);
    lofs[r] = __builtin_amdgcn_readfirstlane(loff[r]);
  }
  const uint32_t ks_lds = lds_addr(Ks), vs_lds = lds_addr(Vs);
  auto issue_k = [&](int tt, int b) {
    const uint32_t toff = (uint32_t)(key_tile(tt) * BN * slk) * 2u;
    const uint32_t dst = ks_lds + (uint32_t)(b * P::KBUF) * 2u;
#pragma unroll
    for (int r = 0; r < P::NIW; ++r)
      if (kon[r]) {
        // readfirstlane: a no-op on a value already in a scalar register,
        // and a guarantee where the compiler would leave it in a vector one
        const uint32_t l = __builtin_amdgcn_readfirstlane(dst + lofs[r]);
        if constexpr (P::KFULL) dma16_raw(kw, toff + goff[r], l);
        else if (act[r]) dma16_raw(kw, toff + goff[r], l);
      }
  };
  auto issue_v = [&](int tt, int b) {
    const uint32_t toff = (uint32_t)(key_tile(tt) * BN * slk) * 2u;
    const uint32_t dst = vs_lds + (uint32_t)(b * P::VBUF) * 2u;
#pragma unroll
    for (int r = 0; r < P::NIW; ++r)
      if (von[r]) {
        const uint32_t l = __builtin_amdgcn_readfirstlane(dst + lofs[r]);
        if (act[r]) dma16_raw(vw, toff + goff[r], l);
      }
  };

  // Transfers this wave issues for iteration j (prologue included), and
  // iteration j's transfers themselves (the buffer of K tile j+NB-1 held K
  // tile j-1, read in iteration j-2; that of V tile j+NB-3 held V tile j-3,
  // read in iteration j-2).
  auto issued = [&](int j) {
    const int uk = j + NB - 1, uv = j + NB - 3;
    return (uk >= 0 && uk < n ? kc : 0) + (uv >= 0 && uv < n ? vc : 0);
  };
  auto issue_iter = [&](int j) {
    const int uk = j + NB - 1, uv = j + NB - 3;
    if (uk >= 0 && uk < n) issue_k(uk, uk % NB);
    if (uv >= 0 && uv < n) issue_v(uv, uv % NB);
  };

  bf16x8 qf[DK / 16];
  load_q<DK>(qf, qr, q0, d, slq, a.qsign, lane);
#pragma unroll
  for (int j = 1 - NB; j < 0; ++j) issue_iter(j);

  // Constants the transfers never write: the zero chunk after each K buffer
  // and the V chunk at column D (a one at D, zeros after it).
  if constexpr (P::KPAD > 0) {
    if (tid < NB) st16(Ks + tid * P::KBUF + BN * P::KST, u32x4{0u, 0u, 0u, 0u});
  }
  if constexpr (S::kOnes) {
    for (int r = tid; r < NB * BN; r += NW * kWave)
      st16(Vs + r * P::VSTR + D, u32x4{uint32_t(one16<H>()), 0u, 0u, 0u});
  }

  const int koff = (lane & 31) * P::KST + 8 * (lane >> 5);
  const int g = lane >> 4, pl = lane & 15;
  const int voff = (4 * (g >> 1) + (pl >> 2)) * P::VSTR + 16 * (g & 1) + 4 * (pl & 3);

  f32x16 o[S::MT];
#pragma unroll
  for (int mt = 0; mt < S::MT; ++mt) o[mt] = f32x16{};
  // Row sums for head dims whose V^T has no padding row to hold ones: an
  // all-ones A operand makes every row of this accumulator sum the bf16
  // weights exactly as P.V uses them.
  f32x16 lacc = {};
  const uint32_t one2 = uint32_t(one16<H>()) * 0x10001u;
  const bf16x8 ones8 = as_bf16x8(u32x4{one2, one2, one2, one2});

  auto scores = [&](int b, f32x16 &s0, f32x16 &s1) {
    const uint16_t *kb = Ks + b * P::KBUF + koff;
    s0 = scores_subtile<DK, H>(kb, qf);
    s1 = scores_subtile<DK, H>(kb + 32 * P::KST, qf);
  };
  auto pv = [&](int b, const u32x4 (&pk)[4]) {
    const uint16_t *vb = Vs + b * P::VBUF + voff;
#pragma unroll
    for (int kc4 = 0; kc4 < 4; ++kc4)
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) {
        const uint16_t *vp = vb + kc4 * 16 * P::VSTR + mt * 32;
        const s16x4 lo = ld_tr16(vp), hi = ld_tr16(vp + 8 * P::VSTR);
        const bf16x8 av =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[mt] = mma<H>(av, as_bf16x8(pk[kc4]), o[mt]);
        if constexpr (!S::kOnes)
          if (mt == 0) lacc = mma<H>(ones8, as_bf16x8(pk[kc4]), lacc);
      }
  };

  // Tile 0's K has landed (everything the prologue issued after it may be
  // in flight): scores and the reference of every row.
  {
    int after = issued(1 - NB) - kc;
#pragma unroll
    for (int j = 2 - NB; j < 0; ++j) after += issued(j);
    vmcnt_barrier_rt<NB * P::NIW>(after);
  }
  f32x16 sA0, sA1, sB0, sB1;
  scores(0, sA0, sA1);
  float nm;
  {
    f32x16 m0 = sA0, m1 = sA1;
    if ((n == 1 && ragged) || ragged_first) {
      const int key0 = key_tile(0) * BN;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (key0 + acc_key(i, lane) >= Lk) m0[i] = -__builtin_inff();
        if (key0 + 32 + acc_key(i, lane) >= Lk) m1[i] = -__builtin_inff();
      }
    }
    nm = -(max_halves(max16(m1, max16(m0, -__builtin_inff()))) * c);
  }

  // Weights of one tile relative to the fixed reference.
  auto weights = [&](auto mask_c, int key0, const f32x16 &s0, const f32x16 &s1, float nmt,
                     u32x4 (&pk)[4]) {
    constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float p8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * kk + j;
          float x = fast_exp2(__builtin_fmaf(u == 0 ? s0[i] : s1[i], c, nmt));
          if constexpr (MASK) {
            if (key0 + 32 * u + acc_key(i, lane) >= Lk) x = 0.f;
          }
          p8[j] = x;
        }
        pk[2 * u + kk] = u32x4{pack2<H>(p8[0], p8[1]), pack2<H>(p8[2], p8[3]),
                               pack2<H>(p8[4], p8[5]), pack2<H>(p8[6], p8[7])};
      }
  };

  // Iteration t: wait for K tile t+1 and V tile t-1 (owned by iteration
  // t+2-NB; later ones may stay in flight), then -- one block of
  // independent work -- scores of tile t+1 (into nx), weights of tile t
  // (from cu, into pout) and P.V of tile t-1 (weights pin), then issue
  // iteration t's transfers (into buffers every wave finished reading before
  // the last barrier).  Alternate register roles between consecutive
  // iterations avoid copies.
  // Steady state: one barrier per pair (t, t+1), t odd.  It waits for the
  // tiles of both blocks (owned by iterations up to t+3-NB; the transfers of
  // the previous pair may stay in flight: later_ss); the pair's second block
  // runs straight on, and both iterations issue their transfers after their
  // blocks (their buffers are read by neither block, NB >= 4).  Half the
  // barriers of one per iteration (measured: waits and transfer issue took
  // ~28 % of an iteration's cycles on the 64x64-latent workload).
  const int later_ss = __builtin_amdgcn_readfirstlane((NB - 4) * (kc + vc));
  // PH_c: -1 for the general iteration; else the steady-state form with
  // t % NB == PH (buffer numbers fold to constants; odd PH: first of a
  // pair, even PH: second) and every transfer issued (the wait count is
  // later_ss): far fewer scalar instructions per iteration.
  auto body = [&](auto pv_c, auto next_c, auto mask_c, auto ph_c, int t, const f32x16 &cu0,
                  const f32x16 &cu1, f32x16 &nx0, f32x16 &nx1, const u32x4 (&pin)[4],
                  u32x4 (&pout)[4]) {
    constexpr bool HAS_PV = decltype(pv_c)::value;
    constexpr bool HAS_NEXT = decltype(next_c)::value;
    constexpr int PH = decltype(ph_c)::value;
    int b1, b2;  // K buffer read by the scores, V buffer read by P.V
    if constexpr (PH >= 0) {
      if constexpr (PH % 2 == 1) vmcnt_barrier_rt<(NB - 4) * P::NIW>(later_ss);
      b1 = (PH + 1) % NB;
      b2 = (PH + NB - 1) % NB;
    } else {
      int later = 0;
#pragma unroll
      for (int j = t + 3 - NB; j < t; ++j) later += issued(j);
      vmcnt_barrier_rt<(NB - 3) * P::NIW>(later);
      const int b = t % NB;
      b1 = b == NB - 1 ? 0 : b + 1;
      b2 = b == 0 ? NB - 1 : b - 1;
    }
    // fp16 weights must stay below fp16's largest value: when a row's tile
    // maximum rises more than kRescaleSlack above the reference, the
    // reference moves up.  The tile maximum is computed beside the weights
    // (nothing waits for it) and checked after the block: in the rare case
    // the check fires, O -- which now holds tiles up to t-1 against the old
    // reference -- is scaled and tile t's weights are taken again against
    // the new one.  (Checking before the weights put the maximum, a
    // wave-wide vote and a branch ahead of the exponentials, and the
    // scheduler then ran all vector work of the block before all of its
    // matrix-core work.)
    float tmax = 0.f;
    if constexpr (H) {
      f32x16 m0 = cu0, m1 = cu1;
      if constexpr (decltype(mask_c)::value) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (key_tile(t) * BN + acc_key(i, lane) >= Lk) m0[i] = -__builtin_inff();
          if (key_tile(t) * BN + 32 + acc_key(i, lane) >= Lk) m1[i] = -__builtin_inff();
        }
      }
      tmax = max_halves(max16(m1, max16(m0, -__builtin_inff()))) * c;
    }
    // The softmax depends on nothing produced in this iteration; an opaque
    // copy of the reference keeps the compiler from hoisting it above the
    // barrier, so it stays in the block it is meant to overlap.
    float nmt = nm;
    asm volatile("" : "+v"(nmt));
    // The scheduler's built-in strategy 0 spreads the LDS reads among the
    // MFMAs of this block (measured 1-3 % faster than its default order).
    __builtin_amdgcn_iglp_opt(0);
    if constexpr (HAS_NEXT) scores(b1, nx0, nx1);
    weights(mask_c, key_tile(t) * BN, cu0, cu1, nmt, pout);
    if constexpr (HAS_PV) pv(b2, pin);
    if constexpr (H) {
      if (__any(tmax + nm > kRescaleSlack)) {
        // A real branch (if-converted it would run every tile); the opaque
        // use of the first weights keeps the compiler from sinking their
        // computation out of the block into the path that does not
        // recompute them.
        asm volatile("" ::"v"(pout[0]), "v"(pout[1]), "v"(pout[2]), "v"(pout[3]));
        const float mref = fmaxf(-nm, tmax);
        const float alpha = fast_exp2(-nm - mref);
        nm = -mref;
#pragma unroll
        for (int mt = 0; mt < S::MT; ++mt) o[mt] *= alpha;
        if constexpr (!S::kOnes) lacc *= alpha;
        weights(mask_c, key_tile(t) * BN, cu0, cu1, nm, pout);
      }
    }
    // The weights are consumed only in the next iteration.  This opaque use
    // keeps the compiler from sinking their computation below the next
    // barrier: it did so in every other iteration, leaving one block with
    // matrix-core work only and the next with two tiles' vector work.
    asm volatile("" : "+v"(pout[0]), "+v"(pout[1]), "+v"(pout[2]), "+v"(pout[3]));
    // Iteration t's transfers go out after its block: right after a barrier
    // every wave would issue at the same moment, with the matrix cores idle.
    if constexpr (PH >= 0) {
      issue_k(t + NB - 1, (PH + NB - 1) % NB);
      issue_v(t + NB - 3, (PH + NB - 3) % NB);
    } else {
      issue_iter(t);
    }
  };
  using F = std::integral_constant<bool, false>;
  using T = std::integral_constant<bool, true>;
  using G = std::integral_constant<int, -1>;

  u32x4 pA[4], pB[4];
  // Last iteration (no next tile) and the P.V of the last tile.
  auto finish = [&](int t, const f32x16 &cu0, const f32x16 &cu1, const u32x4 (&pin)[4],
                    u32x4 (&pout)[4]) {
    if (ragged_last) body(T{}, F{}, T{}, G{}, t, cu0, cu1, sA0, sA1, pin, pout);
    else body(T{}, F{}, F{}, G{}, t, cu0, cu1, sA0, sA1, pin, pout);
    vmcnt_barrier<0>();
    pv(t % NB, pout);
  };

  if (n == 1) {
    if (ragged) body(F{}, F{}, T{}, G{}, 0, sA0, sA1, sB0, sB1, pB, pA);
    else body(F{}, F{}, F{}, G{}, 0, sA0, sA1, sB0, sB1, pB, pA);
    vmcnt_barrier<0>();
    pv(0, pA);
  } else {
    if (ragged_first) body(F{}, T{}, T{}, G{}, 0, sA0, sA1, sB0, sB1, pB, pA);
    else body(F{}, T{}, F{}, G{}, 0, sA0, sA1, sB0, sB1, pB, pA);
    int t = 1;
    {
      // Steady state: six iterations (three pairs) run both register roles
      // through all six buffer phases (t = 1 mod 6 on entry).
      for (; t + 5 + NB < n; t += 6) {
        body(T{}, T{}, F{}, IntC<1>{}, t, sB0, sB1, sA0, sA1, pA, pB);
        body(T{}, T{}, F{}, IntC<2>{}, t + 1, sA0, sA1, sB0, sB1, pB, pA);
        body(T{}, T{}, F{}, IntC<3>{}, t + 2, sB0, sB1, sA0, sA1, pA, pB);
        body(T{}, T{}, F{}, IntC<4>{}, t + 3, sA0, sA1, sB0, sB1, pB, pA);
        body(T{}, T{}, F{}, IntC<5>{}, t + 4, sB0, sB1, sA0, sA1, pA, pB);
        body(T{}, T{}, F{}, IntC<0>{}, t + 5, sA0, sA1, sB0, sB1, pB, pA);
      }
    }
    for (; t + 2 < n; t += 2) {
      body(T{}, T{}, F{}, G{}, t, sB0, sB1, sA0, sA1, pA, pB);
      body(T{}, T{}, F{}, G{}, t + 1, sA0, sA1, sB0, sB1, pB, pA);
    }
    if (t + 1 < n) {
      body(T{}, T{}, F{}, G{}, t, sB0, sB1, sA0, sA1, pA, pB);
      finish(t + 1, sA0, sA1, pB, pA);
    } else {
      finish(t, sB0, sB1, pA, pB);
    }
  }

  float l;
  if constexpr (S::kOnes) {
    float lv = 0.f;
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        if (mt * 32 + 8 * g4 == d) lv = o[mt][4 * g4];
    l = from_low_half(lv);
  } else {
    l = lacc[0];
  }
  // Rows of O^T at or past D are never stored (some hold sums over padding
  // or neighbouring LDS rows): only rows < D and l decide the fallback.
  bool ok = __builtin_isfinite(l);
  const int hb = 4 * (lane >> 5);
#pragma unroll
  for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (mt * 32 + 8 * (i >> 2) + hb + (i & 3) < D) ok = ok && __builtin_isfinite(o[mt][i]);
  if (__any(!ok)) l = rows_exact<DK, H>(o, qf, kr, vr, Lk, d, slk, c, lane);

  store_out_l<DK, OUT_F32, H>(o, l, a.out, a.lo.head(bh, a.H), q0, Lq, d, a.lo.sl, lane);
}

// ---------------------------------------------------------------------------
// Short-key kernel: Lk <= KMAX (128 or 256), every key resident in LDS.

// Epilogue through LDS: the wave writes its normalised 32 x d tile into a
// private LDS region laid out exactly like the rows in HBM, then stores it
// with 16-byte contiguous chunks (whole cache lines per instruction).
template <int DK, bool OUT_F32, bool H = false>
__device__ __forceinline__ void store_out_staged(const f32x16 (&o)[Shape<DK>::MT],
                                                 float lsum, void *outp, size_t obase,
                                                 int q0, int Lq, int d, int sl, int lane,
                                                 uint8_t *stage) {
  using S = Shape<DK>;
  constexpr int ELT = OUT_F32 ? 4 : 2;
  float l;
  if constexpr (S::kOnes) {
    float lv = 0.f;
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        if (mt * 32 + 8 * g4 == d) lv = o[mt][4 * g4];
    l = from_low_half(lv);
  } else {
    l = sum_halves(lsum);
  }
  const float inv = 1.0f / l;
  const int r = lane & 31, hb = 4 * (lane >> 5);
#pragma unroll
  for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c0 = mt * 32 + 8 * g4 + hb;
      if (c0 < d) {
        const float x0 = o[mt][4 * g4 + 0] * inv, x1 = o[mt][4 * g4 + 1] * inv;
        const float x2 = o[mt][4 * g4 + 2] * inv, x3 = o[mt][4 * g4 + 3] * inv;
        uint8_t *dst = stage + (r * d + c0) * ELT;
        if constexpr (OUT_F32) {
          *reinterpret_cast<f32x4 *>(dst) = f32x4{x0, x1, x2, x3};
        } else {
          *reinterpret_cast<u32x2 *>(dst) = u32x2{pack2<H>(x0, x1), pack2<H>(x2, x3)};
        }
      }
    }
  // LDS operations of one wave complete in order, so the reads below see the
  // writes above.
  const int rows = min(kQW, Lq - q0);
  if (rows <= 0) return;
  const int cpr = d * ELT / 16;  // 16-byte chunks per row (d % 8 == 0)
  const int nchunks = rows * cpr;
  uint8_t *gdst = static_cast<uint8_t *>(outp) + (obase + (size_t)q0 * sl) * ELT;
  for (int ch = lane; ch < nchunks; ch += kWave) {
    const int r = ch / cpr, cc = ch - r * cpr;
    *reinterpret_cast<u32x4 *>(gdst + ((size_t)r * sl * ELT + cc * 16)) =
        *reinterpret_cast<const u32x4 *>(stage + ch * 16);
  }
}

template <int DK, int NW, int QPW, int KMAX, bool OUT_F32, bool H>
__global__ __launch_bounds__(NW * kWave, (waves_per_simd<DK>()))
void attn_short(Args16 a) {
  using S = Shape<DK>;
  constexpr int NT = NW * kWave;
  constexpr int NKT = KMAX / 32;
  constexpr int VST = KMAX + 8;
  constexpr int KCH = (KMAX * S::DK8 + NT - 1) / NT;        // K chunks / thread
  constexpr int VCH = ((KMAX / 4) * S::DK8 + NT - 1) / NT;  // V units / thread
  constexpr int STAGE = kQW * DK * (OUT_F32 ? 4 : 2);            // bytes per wave
  // Output staging only where K, V^T and the staging area fit in the LDS
  // share of one workgroup (half of the CU's for up to four waves: two
  // workgroups per CU; all of it for eight); otherwise rows are stored
  // directly.
  constexpr int KV_BYTES = (KMAX * S::KST + S::DV * VST) * 2;
  constexpr bool kStaged = KV_BYTES + NW * STAGE <= (NW >= 8 ? 160 : 80) * 1024;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KMAX * S::KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[S::DV * VST];
  __shared__ __attribute__((aligned(16))) uint8_t Ost[kStaged ? NW * STAGE : 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wg = xcd_remap(blockIdx.x, a.nwg);
  const int bh = wg / a.qblocks;
  const int qbase = (wg - bh * a.qblocks) * (NW * kQW * QPW);
  const int d = a.d, d8 = d >> 3, Lk = a.Lk, Lq = a.Lq;
  const float c = a.c;
  const int slq = a.lq.sl, slk = a.lk.sl;
  const uint32_t kvbytes = head_span_bytes(Lk, slk, d, 2);
  const rsrc_t qr = make_rsrc(a.q + a.lq.head(bh, a.H), head_span_bytes(Lq, slq, d, 2));
  const rsrc_t kr = make_rsrc(a.k + a.lk.head(bh, a.H), kvbytes);
  const rsrc_t vr = make_rsrc(a.v + a.lk.head(bh, a.H), kvbytes);
  const int nkt = (Lk + 31) >> 5;
  const int keys = nkt * 32;
  const int ngroups = keys / 4;

  // Issue every HBM load first (this wave's first Q tile, all of K, all of
  // V), so their latencies overlap; only then write LDS.
  bf16x8 qf[DK / 16];
  load_q<DK>(qf, qr, qbase + wave * kQW, d, slq, a.qsign, lane);
  u32x4 kreg[KCH];
  u32x4 vreg[VCH][4];
#pragma unroll
  for (int t = 0; t < KCH; ++t) {
    const int idx = tid + t * NT;
    const int row = idx / S::DK8, ch = idx - row * S::DK8;
    if (row < keys && ch < d8) kreg[t] = bload16(kr, (uint32_t)(row * slk + ch * 8) * 2u);
  }
#pragma unroll
  for (int t = 0; t < VCH; ++t) {
    const int u = tid + t * NT;
    const int g = u % (KMAX / 4), ch = u / (KMAX / 4);
    if (g < ngroups && ch < d8) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[t][r] = bload16(vr, (uint32_t)((4 * g + r) * slk + ch * 8) * 2u);
    }
  }

  init_k_pad<DK, KMAX>(Ks, d, tid, NT);
  init_vt_const<DK, KMAX, H>(Vt, VST, d, tid, NT);
#pragma unroll
  for (int t = 0; t < KCH; ++t) {
    const int idx = tid + t * NT;
    const int row = idx / S::DK8, ch = idx - row * S::DK8;
    if (row < keys && ch < d8) st16(&Ks[row * S::KST + ch * 8], kreg[t]);
  }
#pragma unroll
  for (int t = 0; t < VCH; ++t) {
    const int u = tid + t * NT;
    const int g = u % (KMAX / 4), ch = u / (KMAX / 4);
    if (g < ngroups && ch < d8) store_vt_unit(Vt, VST, ch * 8, g, vreg[t]);
  }
  __syncthreads();

  const int koff = (lane & 31) * S::KST + 8 * (lane >> 5);
  const int voff = (lane & 31) * VST + 8 * (lane >> 5);
  uint8_t *stage = Ost + (kStaged ? wave * STAGE : 0);

  for (int t = 0; t < QPW; ++t) {
    const int q0 = qbase + (t * NW + wave) * kQW;
    bf16x8 qn[DK / 16];
    if (t + 1 < QPW) load_q<DK>(qn, qr, q0 + NW * kQW, d, slq, a.qsign, lane);

    f32x16 s[NKT];
    float mx = -__builtin_inff();
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      if (nt < nkt) {
        s[nt] = scores_subtile<DK, H>(Ks + koff + nt * 32 * S::KST, qf);
        if (nt == nkt - 1) {
          // A real (uniform) branch: if-converted, the masking would run on
          // every sub-tile.
          asm volatile("");
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (nt * 32 + acc_key(i, lane) >= Lk) s[nt][i] = -__builtin_inff();
        }
        mx = max16(s[nt], mx);
      }
    }
    mx = max_halves(mx);
    const float nm = -(mx * c);

    f32x16 o[S::MT];
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt) o[mt] = f32x16{};
    float lsum = 0.f;
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      if (nt < nkt) {
        const bool last = (nt == nkt - 1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk == 1 && nt * 32 + 16 >= Lk) break;  // chunk entirely past Lk
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) p[j] = fast_exp2(__builtin_fmaf(s[nt][8 * kk + j], c, nm));
          if (last) {
            // masked scores are -inf, so these weights are already 0 unless
            // the scale is 0 (-inf * 0); zero them explicitly
            asm volatile("");
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (nt * 32 + acc_key(8 * kk + j, lane) >= Lk) p[j] = 0.f;
          }
          if constexpr (!S::kOnes) {
#pragma unroll
            for (int j = 0; j < 8; ++j) lsum += p[j];
          }
          const u32x4 pk = {pack2<H>(p[0], p[1]), pack2<H>(p[2], p[3]),
                            pack2<H>(p[4], p[5]), pack2<H>(p[6], p[7])};
          pv_chunk<DK, H>(o, Vt + voff + (nt * 2 + kk) * 16, VST, as_bf16x8(pk));
        }
      }
    }
    if constexpr (kStaged)
      store_out_staged<DK, OUT_F32, H>(o, lsum, a.out, a.lo.head(bh, a.H), q0, Lq, d, a.lo.sl, lane,
                                    stage);
    else
      store_out<DK, OUT_F32, H>(o, lsum, a.out, a.lo.head(bh, a.H), q0, Lq, d, a.lo.sl, lane);
    if (t + 1 < QPW) {
#pragma unroll
      for (int dk = 0; dk < DK / 16; ++dk) qf[dk] = qn[dk];
    }
  }
}

// Launch shapes (build-time knobs for tuning; the defaults are the tuned ones).
#ifndef SDATTN_STREAM_WAVES
#define SDATTN_STREAM_WAVES 4
#endif
#ifndef SDATTN_SHORT_WAVES
#define SDATTN_SHORT_WAVES 4
#endif
#ifndef SDATTN_SHORT_TILES
#define SDATTN_SHORT_TILES 1
#endif
#ifndef SDATTN_STREAM_FIX_MAX_DK
#define SDATTN_STREAM_FIX_MAX_DK 64
#endif
#ifndef SDATTN_STREAM_FIX_WAVES
#define SDATTN_STREAM_FIX_WAVES 8
#endif
constexpr int kStreamFixMaxDk = SDATTN_STREAM_FIX_MAX_DK;  // widest DK of the fixed-reference kernel
constexpr int kStreamFixWaves = SDATTN_STREAM_FIX_WAVES;
constexpr int kStreamWaves = SDATTN_STREAM_WAVES;          // rescaling streaming kernel
// Below this many workgroups of the plain form, the rescaling kernel splits
// each key tile between two waves (the chip has 256 compute units).
#ifndef SDATTN_SPLIT_BELOW
#define SDATTN_SPLIT_BELOW 256
#endif
constexpr int kSplitBelow = SDATTN_SPLIT_BELOW;
// Below this many workgroups of the two-way split, four waves share each
// query block (head dims whose 128-key tiles fit three times in LDS).
#ifndef SDATTN_SPLIT4_BELOW
#define SDATTN_SPLIT4_BELOW 512
#endif
constexpr int kSplit4Below = SDATTN_SPLIT4_BELOW;
constexpr int kShortWaves = SDATTN_SHORT_WAVES;
constexpr int kShortTiles = SDATTN_SHORT_TILES;   // query tiles per wave (short kernel)
// Below this many four-wave workgroups the short kernel runs two-wave ones.
#ifndef SDATTN_SHORT_NARROW_BELOW
#define SDATTN_SHORT_NARROW_BELOW 64
#endif
constexpr int kShortNarrowBelow = SDATTN_SHORT_NARROW_BELOW;
// From this many four-wave workgroups on (two waves per SIMD on every CU and
// more), the short kernel runs eight-wave ones: each workgroup stages the
// head's keys and values once for twice the query rows, halving the
// redundant K/V reads from L2.
#ifndef SDATTN_SHORT_WIDE_FROM
#define SDATTN_SHORT_WIDE_FROM 512
#endif
constexpr int kShortWideFrom = SDATTN_SHORT_WIDE_FROM;

template <int DK, bool H>
hipError_t launch_short(Args16 a, int BH, bool out_f32, hipStream_t stream) {
  constexpr int NW = kShortWaves, QPW = kShortTiles, KMAX = short_cap<DK>();
  const int per_wg = NW * kQW * QPW;
  a.qblocks = (a.Lq + per_wg - 1) / per_wg;
  a.nwg = BH * a.qblocks;
  if constexpr (NW == 4 && QPW == 1 && waves_per_simd<DK>() == 2) {
    if (a.nwg >= kShortWideFrom) {
      constexpr int NW8 = 8;
      a.qblocks = (a.Lq + NW8 * kQW - 1) / (NW8 * kQW);
      a.nwg = BH * a.qblocks;
      const dim3 grid(a.nwg), block(NW8 * kWave);
      return out_f32
                 ? launch_kernel(&attn_short<DK, NW8, 1, KMAX, true, H>, grid, block, 0, stream, a)
                 : launch_kernel(&attn_short<DK, NW8, 1, KMAX, false, H>, grid, block, 0, stream, a);
    }
  }
  if constexpr (NW == 4 && QPW == 1) {
    if (a.nwg < kShortNarrowBelow) {
      // few workgroups (the 16x16 level): two-wave workgroups spread the
      // same waves over twice as many CUs
      constexpr int NW2 = 2;
      a.qblocks = (a.Lq + NW2 * kQW - 1) / (NW2 * kQW);
      a.nwg = BH * a.qblocks;
      const dim3 grid(a.nwg), block(NW2 * kWave);
      return out_f32
                 ? launch_kernel(&attn_short<DK, NW2, 1, KMAX, true, H>, grid, block, 0, stream, a)
                 : launch_kernel(&attn_short<DK, NW2, 1, KMAX, false, H>, grid, block, 0, stream, a);
    }
  }
  const dim3 grid(a.nwg), block(NW * kWave);
  return out_f32 ? launch_kernel(&attn_short<DK, NW, QPW, KMAX, true, H>, grid, block, 0, stream, a)
                 : launch_kernel(&attn_short<DK, NW, QPW, KMAX, false, H>, grid, block, 0, stream, a);
}

template <int DK, bool H>
hipError_t launch_rescale(Args16 a, int BH, bool out_f32, hipStream_t stream) {
  constexpr int NW = kStreamWaves;
  a.qblocks = (a.Lq + NW * kQW - 1) / (NW * kQW);
  a.nwg = BH * a.qblocks;
  const dim3 block(NW * kWave);
  if constexpr (DmaPlan<DK, NW>::NSUB == 2) {
    if (a.nwg < kSplitBelow) {
      // few workgroups for the chip: two waves share each query block, or
      // four (one per SIMD, on 128-key tiles) when that still leaves fewer
      // than two waves per SIMD on the chip
      const int nwg2 = BH * ((a.Lq + NW / 2 * kQW - 1) / (NW / 2 * kQW));
      if constexpr (dma_fits_128<DK>()) {
        if (nwg2 < kSplit4Below) {
          // eight-wave workgroups (two query blocks x four key parts): the
          // 128-key tiles leave room for one workgroup per CU
          constexpr int NW8 = 8;
          a.qblocks = (a.Lq + NW8 / 4 * kQW - 1) / (NW8 / 4 * kQW);
          a.nwg = BH * a.qblocks;
          const dim3 grid(a.nwg), block8(NW8 * kWave);
          return out_f32
                     ? launch_kernel(&attn_stream_rescale<DK, NW8, true, H, 4>, grid, block8, 0, stream, a)
                     : launch_kernel(&attn_stream_rescale<DK, NW8, false, H, 4>, grid, block8, 0, stream, a);
        }
      }
      a.qblocks = (a.Lq + NW / 2 * kQW - 1) / (NW / 2 * kQW);
      a.nwg = nwg2;
      const dim3 grid(a.nwg);
      return out_f32
                 ? launch_kernel(&attn_stream_rescale<DK, NW, true, H, 2>, grid, block, 0, stream, a)
                 : launch_kernel(&attn_stream_rescale<DK, NW, false, H, 2>, grid, block, 0, stream, a);
    }
  }
  const dim3 grid(a.nwg);
  return out_f32 ? launch_kernel(&attn_stream_rescale<DK, NW, true, H>, grid, block, 0, stream, a)
                 : launch_kernel(&attn_stream_rescale<DK, NW, false, H>, grid, block, 0, stream, a);
}

template <int DK, bool H>
hipError_t launch_fix(Args16 a, int BH, bool out_f32, hipStream_t stream) {
  constexpr int NW = kStreamFixWaves;
  a.qblocks = (a.Lq + NW * kQW - 1) / (NW * kQW);
  a.nwg = BH * a.qblocks;
  const dim3 grid(a.nwg), block(NW * kWave);
  // d is DK or DK - 8 (d % 8 == 0); each has its own LDS layout.
  if (a.d == DK)
    return out_f32 ? launch_kernel(&attn_stream_fix<DK, DK, NW, true, H>, grid, block, 0, stream, a)
                   : launch_kernel(&attn_stream_fix<DK, DK, NW, false, H>, grid, block, 0, stream, a);
  return out_f32
             ? launch_kernel(&attn_stream_fix<DK, DK - 8, NW, true, H>, grid, block, 0, stream, a)
             : launch_kernel(&attn_stream_fix<DK, DK - 8, NW, false, H>, grid, block, 0, stream, a);
}

// Short-key kernel up to the key cap, else the fixed-reference kernel up to
// DK 64 and the rescaling kernel above.  In fp16 the fixed-reference kernel
// moves its reference up whenever a tile would push weights past 2^8 (fp16's
// range ends at 65504); bf16 weights share fp32's exponent range and never
// need that.
template <int DK>
hipError_t launch_dk(const Args16 &a, int BH, bool short_path, bool out_f32, bool half,
                     hipStream_t stream) {
  if (short_path)
    return half ? launch_short<DK, true>(a, BH, out_f32, stream)
                : launch_short<DK, false>(a, BH, out_f32, stream);
  if constexpr (DK <= kStreamFixMaxDk)
    return half ? launch_fix<DK, true>(a, BH, out_f32, stream)
                : launch_fix<DK, false>(a, BH, out_f32, stream);
  else
    return half ? launch_rescale<DK, true>(a, BH, out_f32, stream)
                : launch_rescale<DK, false>(a, BH, out_f32, stream);
}

}  // namespace

// Entry for one head-dim class (DK = head dim rounded up to 16).
template <int DK>
hipError_t launch_16_dk(const Args16 &a, int BH, bool short_path, bool out_f32, bool half,
                        hipStream_t stream) {
  return launch_dk<DK>(a, BH, short_path, out_f32, half, stream);
}

// The build compiles this file once per head-dim class (-DSDATTN_DK=16 ...
// 256, in parallel) and once with -DSDATTN_DK=0 for the dispatcher below;
// compiled without SDATTN_DK it holds everything.
#define SDATTN_FOR_EACH_DK(X) \
  X(16) X(32) X(48) X(64) X(80) X(96) X(112) X(128) X(144) X(160) X(176) X(192) X(208) \
  X(224) X(240) X(256)
#define SDATTN_INST(DK)                                                                  \
  template hipError_t launch_16_dk<DK>(const Args16 &, int, bool, bool, bool, hipStream_t);
#define SDATTN_EXTERN(DK)                                                                \
  extern template hipError_t launch_16_dk<DK>(const Args16 &, int, bool, bool, bool,    \
                                              hipStream_t);
#if defined(SDATTN_DK)
#if SDATTN_DK > 0
SDATTN_INST(SDATTN_DK)
#else
SDATTN_FOR_EACH_DK(SDATTN_EXTERN)
#endif
#else
SDATTN_FOR_EACH_DK(SDATTN_INST)
#endif

#if !defined(SDATTN_DK) || SDATTN_DK == 0
int short_path_max_keys(int d) {
  (void)d;
  return short_cap<16>();
}

hipError_t launch_16(const Args16 &a, int BH, bool short_path, bool out_f32, bool half,
                     hipStream_t stream) {
  const int dk = (a.d + 15) / 16 * 16;
  switch (dk) {
#define SDATTN_CASE(DK) \
  case DK: return launch_16_dk<DK>(a, BH, short_path, out_f32, half, stream);
    SDATTN_FOR_EACH_DK(SDATTN_CASE)
#undef SDATTN_CASE
    default: return hipErrorInvalidValue;
  }
}
#endif

}  // namespace sdattn
