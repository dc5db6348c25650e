// fa_kernel.h - gfx950 (CDNA4) exact-attention forward kernel.
//
// Method (the FlashAttention forward pass; pages: "FlashAttention 4: Snellere,
// Geheugenefficiente Aandacht voor LLM's" and "[RFC] FA4 - head_dim=256 & head_dim=512"):
//   one workgroup keeps a tile of queries resident and streams the K/V tiles of its head
//   through LDS; scores never leave the chip; a running row maximum and running row sums
//   carry the softmax across tiles ("Waarom aandachtkernels ..." section), and the output
//   accumulator is rescaled only when the row maximum has grown by more than a threshold
//   ("Slimmere Online Softmax-herwaardering" section).
//
// CDNA4 mapping (our own design, not the pages' Blackwell pipeline):
//   * a wave owns 32 query rows; a workgroup of NW waves owns BR = 32*NW rows;
//   * both products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation, in
//     transposed form:  S^T = K * Q^T  and  O^T += V^T * P^T.  In the MFMA C layout each
//     lane then holds ONE query row (column = lane % 32) and 16 keys (or 16 head-dim
//     values), so row max / row sums are lane-local, the rescale factor is a per-lane
//     scalar, and P^T feeds the second MFMA's B operand straight from registers;
//   * V^T is read with ds_read_b64_tr_b16 (LDS transpose read), so V stays in its natural
//     [key][d] layout in LDS;
//   * K/V tiles are double-buffered in LDS with an XOR swizzle of 16-byte chunks; the next
//     tile's global loads are issued before the current tile's math;
//   * softmax in base 2: p = exp2(s*c - m), c = scale*log2(e), on v_exp_f32;
//   * lazy rescale: the running max m (log2 units) is raised only when some row of the
//     wave sees a tile max above m + TAU; until then p <= 2^TAU;
//   * two row sums: lO = sum of the rounded P actually fed to the MFMA (normalises O, so the
//     rounding of P cancels in O = (P_b V) / sum P_b) and lL = fp32 sum of p (feeds the LSE).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Lazy-rescale threshold in log2 units: p = exp2(s*c - m) stays <= 2^TAU between rescales.
constexpr float TAU = 8.0f;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct Bf16 {
  using x8 = bf16x8;
  using x2 = bf16x2;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ x2 cvt2(float a, float b) {
    x2 r = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32, round to nearest even
    return r;
  }
  static __device__ __forceinline__ float dot2(x2 a, x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
  static __device__ __forceinline__ x2 ones() {
    x2 r = {(__bf16)1.0f, (__bf16)1.0f};
    return r;
  }
};

struct F16 {
  using x8 = f16x8;
  using x2 = f16x2;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ x2 cvt2(float a, float b) {
    x2 r = {(_Float16)a, (_Float16)b};
    return r;
  }
  static __device__ __forceinline__ float dot2(x2 a, x2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
  }
  static __device__ __forceinline__ x2 ones() {
    x2 r = {(_Float16)1.0f, (_Float16)1.0f};
    return r;
  }
};

struct FwdParams {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint8_t* o;
  float* lse;
  int B, Nq, Nk, Hq, Hkv;
  int group;      // Hq / Hkv
  int nqt;        // query tiles per (b, h)
  float c;        // scale * log2(e)
};

template <bool V> struct BoolC { static constexpr bool value = V; };

// XOR swizzle of the 16-byte chunk index inside an LDS row: 16 consecutive rows map one
// logical chunk to 16 different physical chunks (GEMM1 reads), and the 4-row groups read
// by ds_read_b64_tr_b16 land in 4 different chunk pairs.
__device__ __forceinline__ int swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }

// Block id -> (b*Hq + h, query tile). Workgroups are dispatched round-robin over the 8
// XCDs (bid % 8); when B*Hq is a multiple of 8, each XCD gets a contiguous set of heads so
// that workgroups sharing K/V run on the same XCD and share its L2. Causal work is ordered
// longest-first (highest query tile first) inside each XCD's share.
template <bool CAUSAL>
__device__ __forceinline__ void decode_block(int bid, const FwdParams& p, int& bh, int& qt) {
  const int BH = p.B * p.Hq;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3, hpx = BH >> 3;
    if (CAUSAL) {
      qt = p.nqt - 1 - slot / hpx;
      bh = xcd * hpx + slot % hpx;
    } else {
      bh = xcd * hpx + slot / p.nqt;
      qt = slot % p.nqt;
    }
  } else {
    if (CAUSAL) {
      qt = p.nqt - 1 - bid / BH;
      bh = bid % BH;
    } else {
      bh = bid / p.nqt;
      qt = bid % p.nqt;
    }
  }
}

template <int D, int NW, int BC, bool CAUSAL, class T>
__global__ void __launch_bounds__(NW * 64)
fwd_kernel(FwdParams p) {
  using x8 = typename T::x8;
  using x2 = typename T::x2;
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int KS1 = D / 16;       // GEMM1 k-steps (over head dim)
  constexpr int MT1 = BC / 32;      // score tiles (32 keys each) per K/V tile
  constexpr int MT2 = D / 32;       // output tiles (32 head-dim rows each)
  constexpr int KS2 = BC / 16;      // GEMM2 k-steps (over keys)
  constexpr int ROWB = D * 2;       // bytes per K/V row in LDS
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int TILEB = BC * ROWB;  // bytes per K or V tile
  constexpr int LOADS = BC * CPR / NT;
  static_assert((BC * CPR) % NT == 0, "tile chunks must divide over the workgroup");
  static_assert(BC % 32 == 0 && D % 32 == 0 && CPR >= 16, "tile shape");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // [2 buffers][K, V][TILEB]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int bh, qt;
  decode_block<CAUSAL>(blockIdx.x, p, bh, qt);
  const int b = bh / p.Hq;
  const int hq = bh - b * p.Hq;
  const int kvh = hq / p.group;
  const int Nq = p.Nq, Nk = p.Nk;

  const int q_wg0 = qt * BR;
  const int qw0 = q_wg0 + wave * 32;
  const int q_lane = qw0 + l32;
  const int q_ld = q_lane < Nq ? q_lane : Nq - 1;

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(Nq, q_wg0 + BR));
  const int ntiles = (kend + BC - 1) / BC;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query q_ld, dims 16t + 8hh .. +7
  x8 qf[KS1];
  {
    const uint8_t* qp = p.q + (((size_t)b * Nq + q_ld) * p.Hq + hq) * (size_t)(D * 2);
#pragma unroll
    for (int t = 0; t < KS1; ++t) {
      u32x4 raw = *(const u32x4*)(qp + (16 * t + 8 * hh) * 2);
      qf[t] = __builtin_bit_cast(x8, raw);
    }
  }

  f32x16 acc[MT2];
#pragma unroll
  for (int i = 0; i < MT2; ++i) acc[i] = f32x16{};
  float m_run = -__builtin_inff();
  float lL = 0.f, lO = 0.f;
  const float c = p.c;

  // ---- K/V staging: global -> registers -> LDS (swizzled)
  const size_t kv_row = (size_t)p.Hkv * D * 2;  // bytes between consecutive tokens
  const uint8_t* kbase = p.k + ((size_t)b * Nk * p.Hkv + kvh) * (size_t)(D * 2);
  const uint8_t* vbase = p.v + ((size_t)b * Nk * p.Hkv + kvh) * (size_t)(D * 2);
  u32x4 stK[LOADS], stV[LOADS];

  auto gload = [&](int tile) {
    const int k0 = tile * BC;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int pidx = tid + n * NT;
      const int row = pidx / CPR, ch = pidx % CPR;
      int key = k0 + row;
      key = key < Nk ? key : Nk - 1;
      const size_t off = (size_t)key * kv_row + ch * 16;
      stK[n] = *(const u32x4*)(kbase + off);
      stV[n] = *(const u32x4*)(vbase + off);
    }
  };
  auto swrite = [&](int buf) {
    uint8_t* kb = smem + buf * 2 * TILEB;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int pidx = tid + n * NT;
      const int row = pidx / CPR, ch = pidx % CPR;
      const int pos = row * ROWB + ((ch ^ swz(row)) << 4);
      *(u32x4*)(kb + pos) = stK[n];
      *(u32x4*)(kb + TILEB + pos) = stV[n];
    }
  };

  gload(0);
  swrite(0);
  __syncthreads();

  const x2 one2 = T::ones();

  // One K/V tile of work for this wave. SPLIT_P (used on the wave's first tile): P is fed to
  // the second product as hi + lo, two rounded parts whose sum carries ~16 significant bits,
  // so rows that have seen only a few keys are not limited by the 8-bit rounding of P.
  auto tile_step = [&](const int j, auto split_tag) {
    constexpr bool SPLIT_P = decltype(split_tag)::value;
    const int buf = j & 1;
    const int k0 = j * BC;
    const uint8_t* kl = smem + buf * 2 * TILEB;
    const uint8_t* vl = kl + TILEB;
    // ---- GEMM1: S^T[key][q] = sum_d K[key][d] Q[q][d]
    f32x16 s[MT1];
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt) {
      s[mt] = f32x16{};
      const int row = mt * 32 + l32;
      const uint8_t* rp = kl + row * ROWB;
      const int sw = swz(row);
#pragma unroll
      for (int t = 0; t < KS1; ++t) {
        const int ch = (2 * t + hh) ^ sw;
        u32x4 raw = *(const u32x4*)(rp + (ch << 4));
        s[mt] = T::mfma(__builtin_bit_cast(x8, raw), qf[t], s[mt]);
      }
    }
    // ---- mask: causal (key > query) and tail (key >= Nk); lane's query is q_lane,
    //      register r of score tile mt holds key k0 + 32mt + 8(r/4) + 4hh + r%4
    const bool need_mask = (k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > qw0));
    if (need_mask) {
#pragma unroll
      for (int mt = 0; mt < MT1; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool masked = (key >= Nk) || (CAUSAL && key > q_lane);
          if (masked) s[mt][r] = -__builtin_inff();
        }
    }
    // ---- row max (lane-local over its keys, then across the two lane halves)
    float mx = s[0][0];
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[mt][r]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const float mtile = mx * c;  // c >= 0, so max(s)*c == max(s*c)
    // ---- lazy rescale, decided per wave
    const bool grow = mtile > m_run + TAU;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = __builtin_fmaxf(m_run, mtile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);  // 0 on the first tile
#pragma unroll
      for (int i = 0; i < MT2; ++i) acc[i] *= alpha;
      lL *= alpha;
      lO *= alpha;
      m_run = mnew;
    }
    // ---- p = exp2(s*c - m); P rounded to the MFMA element type; two row sums
    const float negm = -m_run;
    x8 pf[KS2];
    x8 pl[SPLIT_P ? KS2 : 1];
    float sumL = 0.f, sumO = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][r], c, negm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][r + 1], c, negm));
        sumL += p0 + p1;
        const x2 pb = T::cvt2(p0, p1);
        sumO = T::dot2(pb, one2, sumO);
        const int u = mt * 2 + (r >> 3);
        pf[u][(r & 7)] = pb[0];
        pf[u][(r & 7) + 1] = pb[1];
        if constexpr (SPLIT_P) {
          const x2 lo = T::cvt2(p0 - (float)pb[0], p1 - (float)pb[1]);
          sumO = T::dot2(lo, one2, sumO);
          pl[u][(r & 7)] = lo[0];
          pl[u][(r & 7) + 1] = lo[1];
        }
      }
    lL += sumL;
    lO += sumO;
    // ---- GEMM2: O^T[d][q] += sum_key V^T[d][key] P^T[key][q]
    // k-step u covers keys 16u + {4hh + 0..3, 8 + 4hh + 0..3} (the order P^T holds them).
    // ds_read_b64_tr_b16: lane i of a 16-lane group reads row key0 + i/4, dims
    // d0 + 4(i%4) .. +3; lane c of the group receives V[key0 + 0..3][d0 + c].
    const int grp = lane >> 4, gi = lane & 15;
    const int rsub = gi >> 2;                          // row inside the 4-row block
    const int dsub = 2 * (grp & 1) + ((gi & 3) >> 1);  // 16-byte chunk inside 32 dims
    const int half8 = (gi & 1) * 8;                    // byte offset inside the chunk
#pragma unroll
    for (int md = 0; md < MT2; ++md)
#pragma unroll
      for (int u = 0; u < KS2; ++u) {
        s16x4 lo4, hi4;
        {
          const int row = 16 * u + 4 * (grp >> 1) + rsub;
          const int ch = (4 * md + dsub) ^ swz(row);
          lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + row * ROWB + (ch << 4) + half8));
        }
        {
          const int row = 16 * u + 8 + 4 * (grp >> 1) + rsub;
          const int ch = (4 * md + dsub) ^ swz(row);
          hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + row * ROWB + (ch << 4) + half8));
        }
        u32x4 raw;
        raw[0] = __builtin_bit_cast(u32x2, lo4)[0];
        raw[1] = __builtin_bit_cast(u32x2, lo4)[1];
        raw[2] = __builtin_bit_cast(u32x2, hi4)[0];
        raw[3] = __builtin_bit_cast(u32x2, hi4)[1];
        const x8 vfrag = __builtin_bit_cast(x8, raw);
        acc[md] = T::mfma(vfrag, pf[u], acc[md]);
        if constexpr (SPLIT_P) acc[md] = T::mfma(vfrag, pl[u], acc[md]);
      }
  };

  // tile 0 (never skipped: key 0 is visible to every query)
  if (ntiles > 1) gload(1);
  tile_step(0, BoolC<true>{});
  if (ntiles > 1) swrite(1);
  __syncthreads();
  for (int j = 1; j < ntiles; ++j) {
    if (j + 1 < ntiles) gload(j + 1);
    const bool skip = CAUSAL && (j * BC > qw0 + 31);  // every key after every query of this wave
    if (!skip) tile_step(j, BoolC<false>{});
    if (j + 1 < ntiles) swrite((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: combine the two lane halves' sums, normalise, store O and LSE
  lL += __shfl_xor(lL, 32);
  lO += __shfl_xor(lO, 32);
  if (q_lane < Nq) {
    const float inv = 1.0f / lO;
    uint8_t* op = p.o + (((size_t)b * Nq + q_lane) * p.Hq + hq) * (size_t)(D * 2);
#pragma unroll
    for (int md = 0; md < MT2; ++md)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const x2 a = T::cvt2(acc[md][4 * i + 0] * inv, acc[md][4 * i + 1] * inv);
        const x2 bb = T::cvt2(acc[md][4 * i + 2] * inv, acc[md][4 * i + 3] * inv);
        u32x2 w;
        w[0] = __builtin_bit_cast(unsigned, a);
        w[1] = __builtin_bit_cast(unsigned, bb);
        const int d = 32 * md + 8 * i + 4 * hh;
        *(u32x2*)(op + d * 2) = w;
      }
    if (hh == 0)
      p.lse[((size_t)b * p.Hq + hq) * Nq + q_lane] = (m_run + __builtin_amdgcn_logf(lL)) * LN2;
  }
}

}  // namespace fa
