// fa_bwd_kernel.h - gfx950 backward pass of exact attention (gradients of sum(O * dO)).
//
// The backward pass sits next to the forward on the pages ("[RFC] FA4 - head_dim=256 &
// head_dim=512", Phase 1 "Backward kernel" and the backward rows of "Performance
// Snapshot"). With S = scale*Q K^T, P = softmax(S) = exp(S - LSE) (the forward's LSE):
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),  D_i = sum_d dO_id O_id,
//     dQ = scale * dS K,   dK = scale * dS^T Q.
// Two kernels, neither needs atomics:
//   * dq kernel (query-major, the forward's structure): a wave owns 32 queries and keeps Q
//     and dO in registers; K and V tiles stream through LDS. It computes D for its rows
//     (and stores D for the second kernel), then per key tile
//         S^T = K Q^T,  dP^T = V dO^T  (A operand = K / V rows),
//         P^T = exp2(c S^T - LSE log2 e),  dS^T = P^T (dP^T - D)  (lane-local per query),
//         dQ^T += K^T dS^T  (K^T read with ds_read_b64_tr_b16, dS^T straight from registers);
//   * dkdv kernel (key-major): a wave owns 32 keys and keeps K and V in registers; Q, dO,
//     LSE and D tiles stream through LDS. Per query tile
//         S = Q K^T,  dP = dO V^T  (C layout: a lane owns one key, 16 query rows),
//         P = exp2(c S - LSE log2 e),  dS = P (dP - D)  (LSE, D per row from LDS),
//         dV^T += dO^T P,  dK^T += Q^T dS  (dO^T, Q^T via ds_read_b64_tr_b16);
//     for grouped-query heads the query heads of the group are visited in turn.
// P and dS enter the MFMAs rounded to the input element type (bf16/fp16); everything else is
// fp32. This is a plain, unscheduled implementation: each tile is loaded into LDS (double
// buffered, buffer loads straight to LDS), computed, and the workgroup synchronises.
#pragma once

#include "fa_kernel.h"

namespace fa {

struct BwdParams {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* o;
  const float* lse;
  const uint8_t* dout;
  uint8_t* dq;
  uint8_t* dk;
  uint8_t* dv;
  float* dsum;  // D = rowsum(dO * O), [B, Hq, Nq], written by the dq kernel
  int B, Nq, Nk, Hq, Hkv;
  int group;
  int ntile;    // work tiles per (b, head) of the kernel (query tiles or key tiles)
  float c;      // scale * log2(e), of either sign (P = exp2(c s - LSE log2(e)) needs no
                // running maximum; masked entries are set to 0 after the exp); log2(e) when
                // zero_scores is set
  float scale;  // the signed scale (dQ = scale dS K, dK = scale dS^T Q)
  int zero_scores;  // scale is zero (or below the normal range): every score is exactly 0
  unsigned order_mul, order_add;  // grid order (testing hook), as in FwdParams
};

template <int D>
struct BwdCfg {
  static constexpr int NW = 4;         // waves per workgroup, 32 rows each
  static constexpr int WPE = D == 128 ? 2 : 1;  // waves per SIMD the registers are sized for
  static constexpr int BT = 32;        // rows per streamed tile
  static constexpr int ROW = D * 2 + 16;  // padded LDS row pitch (bytes)
  static constexpr int TB = BT * ROW;     // bytes per streamed tile
};

// A transposed MFMA operand (8 values of one column over 16 rows) from an LDS tile with row
// pitch `row`: two ds_read_b64_tr_b16, rows 0..7 and 8..15 below `p`.
template <class X8>
__device__ __forceinline__ X8 bwd_tr_frag(const uint8_t* p, int row) {
  const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * row));
  u32x4 raw;
  raw[0] = __builtin_bit_cast(u32x2, lo4)[0];
  raw[1] = __builtin_bit_cast(u32x2, lo4)[1];
  raw[2] = __builtin_bit_cast(u32x2, hi4)[0];
  raw[3] = __builtin_bit_cast(u32x2, hi4)[1];
  return __builtin_bit_cast(X8, raw);
}

// LDS fragment reads are issued this many steps ahead of their MFMAs, in a fixed order
// (sched_barrier between steps): PF1 for the score products, PF2 for the transposed ones.
// 0: the compiler's order (the hd128 dk/dv kernel has no registers to spare for fragments
// read ahead: they spill).
constexpr int BWD_DQ_PF1 = 2, BWD_DQ_PF2 = 2;
template <int D> constexpr int bwd_kv_pf1() { return D == 128 ? 0 : 2; }
template <int D> constexpr int bwd_kv_pf2() { return D == 128 ? 0 : 2; }

// Load one BT-row tile of a [.., tokens, heads, D] tensor straight into LDS (padded rows).
// `base` points at (b, token 0, head); rows past `valid_rows` load zeros.
template <int D, int NW, bool SCALAR_DESC>
__device__ __forceinline__ void bwd_load_rows(const uint8_t* base, uint32_t row_bytes, int row0,
                                              int valid_rows, uint8_t* ldst, int wave, int lane) {
  using C = BwdCfg<D>;
  constexpr int SL = C::ROW / 16, CPR = D / 8;
  constexpr int NI = (C::BT * SL + 63) / 64;
  const int nv = valid_rows - row0 < C::BT ? valid_rows - row0 : C::BT;
  // The clamp is computed on the VALU, so the descriptor lands in VGPRs and each load gets a
  // waterfall loop unless readfirstlane keeps it scalar (SCALAR_DESC). That helps the dq
  // kernels and the hd128 dk/dv kernel (backward hd128 +2% non-causal, +10% causal); the
  // hd256 dk/dv kernel spilled with it (-4% / -12%) and keeps the loop.
  const int nvc = nv > 0 ? nv : 0;
  const uint32_t nrec = (uint32_t)(SCALAR_DESC ? __builtin_amdgcn_readfirstlane(nvc) : nvc) * row_bytes;
  const auto rs = make_rsrc(base + (size_t)row0 * row_bytes, nrec);
#pragma unroll
  for (int n = 0; n < (NI + NW - 1) / NW; ++n) {
    const int I = wave + NW * n;
    if (I < NI) {
      const int slot = 64 * I + lane, row = slot / SL, ch = slot % SL;
      const uint32_t vo = (ch < CPR && row < C::BT) ? (uint32_t)row * row_bytes + ch * 16 : 0x80000000u;
      if (64 * I + 64 <= C::BT * SL || slot < C::BT * SL)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(ldst + 1024 * I), 16, vo, 0, 0, 0);
    }
  }
}

// ------------------------------------------------------------------------------------------
// dq kernel: one workgroup per (b, hq, 128-query tile); K/V tiles of BT keys stream through LDS.
template <int D, bool CAUSAL, class T>
__global__ void __launch_bounds__(BwdCfg<D>::NW * 64)
bwd_dq_kernel(BwdParams p) {
  using x8 = typename T::x8;
  using x2 = typename T::x2;
  using C = BwdCfg<D>;
  constexpr int NW = C::NW, BT = C::BT, BR = NW * 32;
  constexpr int KS1 = D / 16, MT2 = D / 32, KS2 = BT / 16, ROW = C::ROW;
  constexpr int PF1 = BWD_DQ_PF1, PF2 = BWD_DQ_PF2;
  static_assert(BT == 32, "one 32-key score tile per key tile");

  // separate objects per buffer, and a buffer parity that is a literal in the loop: the
  // compiler can then see that the direct-to-LDS loads of the next tile never alias the tile
  // being read (with one [2][TB] array and j & 1 it waited for those loads at the top of
  // every iteration; the dk/dv kernel keeps that form: unrolled the same way it spilled)
  __shared__ __attribute__((aligned(16))) uint8_t k_lds0[C::TB], k_lds1[C::TB], v_lds0[C::TB], v_lds1[C::TB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // causal: the last query tiles see the most keys; they start first (longest-first), with
  // consecutive blocks on consecutive heads
  const unsigned bid = (unsigned)work_item(p.order_mul, p.order_add);
  const int nbh = p.B * p.Hq;
  const int bh = CAUSAL ? (int)(bid % nbh) : (int)(bid / p.ntile);
  const int qt = CAUSAL ? p.ntile - 1 - (int)(bid / nbh) : (int)(bid % p.ntile);
  const int b = bh / p.Hq, hq = bh % p.Hq, kvh = hq / p.group;
  const int Nq = p.Nq, Nk = p.Nk;
  const int q_wg0 = qt * BR, qw0 = q_wg0 + wave * 32, q_lane = qw0 + l32;
  const int q_ld = q_lane < Nq ? q_lane : Nq - 1;
  const int kend = CAUSAL ? min(Nk, min(Nq, q_wg0 + BR)) : Nk;
  const int ntiles = (kend + BT - 1) / BT;
  const int wtiles = CAUSAL ? max(1, min(ntiles, (min(qw0 + 32, Nq) + BT - 1) / BT)) : ntiles;

  // Q and dO of this lane's query as B operands (dims 16t + 8hh .. +7); D = rowsum(dO * O)
  const size_t qrow = (((size_t)b * Nq + q_ld) * p.Hq + hq) * (size_t)(D * 2);
  x8 qf[KS1], df[KS1];
  float dpart = 0.f;
#pragma unroll
  for (int t = 0; t < KS1; ++t) {
    const int off = (16 * t + 8 * hh) * 2;
    qf[t] = __builtin_bit_cast(x8, *(const u32x4*)(p.q + qrow + off));
    df[t] = __builtin_bit_cast(x8, *(const u32x4*)(p.dout + qrow + off));
    const x8 of = __builtin_bit_cast(x8, *(const u32x4*)(p.o + qrow + off));
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart += (float)df[t][e] * (float)of[e];
  }
  if (p.zero_scores) {  // zero scale: S = 0 exactly (masked scores stay -inf)
#pragma unroll
    for (int t = 0; t < KS1; ++t) qf[t] = x8{};
  }
  const float dsum = dpart + other_half(dpart);
  const size_t lrow = ((size_t)b * p.Hq + hq) * Nq + q_ld;
  if (hh == 0 && q_lane < Nq) p.dsum[lrow] = dsum;
  const float lq = p.lse[lrow] * LOG2E;
  const float c = p.c;

  f32x16 acc[MT2];
#pragma unroll
  for (int i = 0; i < MT2; ++i) acc[i] = f32x16{};

  const uint32_t kv_row = (uint32_t)p.Hkv * D * 2;
  const uint8_t* kbase = p.k + ((size_t)b * Nk * p.Hkv + kvh) * (size_t)(D * 2);
  const uint8_t* vbase = p.v + ((size_t)b * Nk * p.Hkv + kvh) * (size_t)(D * 2);
  const int k_rd = l32 * ROW + hh * 16;
  const int grp = lane >> 4, gi = lane & 15;
  const int t_rd = (4 * (grp >> 1) + (gi >> 2)) * ROW + (2 * (grp & 1) + ((gi & 3) >> 1)) * 16 + (gi & 1) * 8;

  bwd_load_rows<D, NW, true>(kbase, kv_row, 0, Nk, k_lds0, wv, lane);
  bwd_load_rows<D, NW, true>(vbase, kv_row, 0, Nk, v_lds0, wv, lane);
  tile_barrier();
  auto iteration = [&](const int j, auto par_tag) {
    constexpr int PAR = decltype(par_tag)::value;  // j & 1
    if (j + 1 < ntiles) {
      bwd_load_rows<D, NW, true>(kbase, kv_row, (j + 1) * BT, Nk, PAR ? k_lds0 : k_lds1, wv, lane);
      bwd_load_rows<D, NW, true>(vbase, kv_row, (j + 1) * BT, Nk, PAR ? v_lds0 : v_lds1, wv, lane);
    }
    if (j < wtiles) {
      const uint8_t* kl = PAR ? k_lds1 : k_lds0;
      const uint8_t* vl = PAR ? v_lds1 : v_lds0;
      // S^T and dP^T: one accumulator each (the two chains alternate, so neither MFMA waits
      // for its predecessor; two alternating accumulators per product cost 32 registers and
      // 32 adds per tile and ran 1-3% slower)
      f32x16 s = f32x16{}, dp = f32x16{};
      {
        // step t: the K and V fragments of head-dim step t, read PF1 steps ahead
        x8 kf_[KS1], vf_[KS1];
        auto rd = [&](const int t) {
          kf_[t] = __builtin_bit_cast(x8, *(const u32x4*)(kl + k_rd + t * 32));
          vf_[t] = __builtin_bit_cast(x8, *(const u32x4*)(vl + k_rd + t * 32));
        };
#pragma unroll
        for (int t = 0; t < PF1; ++t) rd(t);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < KS1; ++t) {
          if (t + PF1 < KS1) rd(t + PF1);
          s = T::mfma(kf_[t], qf[t], s);
          dp = T::mfma(vf_[t], df[t], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // P^T, dS^T; key of register r: j*BT + 8(r/4) + 4hh + r%4; query q_lane
      const int k0 = j * BT;
      const int last = CAUSAL ? min(q_lane, Nk - 1) : Nk - 1;
      const int lim = last - k0 - 4 * hh;
      x8 dsf[KS2];
      auto ds_tile = [&](auto mask_tag) {
        constexpr bool MASKED = decltype(mask_tag)::value;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lq));
          float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], c, -lq));
          if (MASKED && 8 * (r >> 2) + (r & 3) > lim) e0 = 0.f;
          if (MASKED && 8 * (r >> 2) + ((r + 1) & 3) > lim) e1 = 0.f;
          const x2 ds = T::cvt2(e0 * (dp[r] - dsum), e1 * (dp[r + 1] - dsum));
          dsf[r >> 3][r & 7] = ds[0];
          dsf[r >> 3][(r & 7) + 1] = ds[1];
        }
      };
      // the mask only where the tile holds keys past Nk or, causal, keys after a query of this
      // wave (a wave-uniform test): a compare and a select per score on every other tile cost
      // 2-5% of the backward pass at hd128. (The dk/dv kernels keep masking every tile: the
      // second form made them spill.)
      if ((k0 + BT > Nk) || (CAUSAL && k0 + BT - 1 > qw0))
        ds_tile(BoolC<true>{});
      else
        ds_tile(BoolC<false>{});
      // dQ^T += K^T dS^T (K^T read transposed from the K tile), fragments PF2 steps ahead
      {
        constexpr int N = KS2 * MT2;
        x8 tf[N];
        auto rd = [&](const int i) {
          const int u = i / MT2, md = i % MT2;
          tf[i] = bwd_tr_frag<x8>(kl + t_rd + (16 * u) * ROW + md * 64, ROW);
        };
#pragma unroll
        for (int i = 0; i < PF2; ++i) rd(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          if (i + PF2 < N) rd(i + PF2);
          acc[i % MT2] = T::mfma(tf[i], dsf[i / MT2], acc[i % MT2]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    tile_barrier();
  };
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    iteration(j, IntC<0>{});
    iteration(j + 1, IntC<1>{});
  }
  if (j < ntiles) iteration(j, IntC<0>{});

  if (q_lane < Nq) {
    uint8_t* op = p.dq + (((size_t)b * Nq + q_lane) * p.Hq + hq) * (size_t)(D * 2);
    const float sc = p.scale;
#pragma unroll
    for (int md = 0; md < MT2; ++md)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const x2 a = T::cvt2(acc[md][4 * i + 0] * sc, acc[md][4 * i + 1] * sc);
        const x2 bb = T::cvt2(acc[md][4 * i + 2] * sc, acc[md][4 * i + 3] * sc);
        u32x2 w;
        w[0] = __builtin_bit_cast(unsigned, a);
        w[1] = __builtin_bit_cast(unsigned, bb);
        *(u32x2*)(op + (32 * md + 8 * i + 4 * hh) * 2) = w;
      }
  }
}

// ------------------------------------------------------------------------------------------
// dkdv kernel: one workgroup per (b, kvh, 128-key tile); Q/dO tiles of BT queries stream
// through LDS for every query head of the group.
template <int D, bool CAUSAL, class T>
__global__ void __launch_bounds__(BwdCfg<D>::NW * 64, BwdCfg<D>::WPE)
bwd_dkdv_kernel(BwdParams p) {
  using x8 = typename T::x8;
  using x2 = typename T::x2;
  using C = BwdCfg<D>;
  constexpr int NW = C::NW, BT = C::BT, BK = NW * 32;
  constexpr int KS1 = D / 16, MT2 = D / 32, KS2 = BT / 16, ROW = C::ROW;
  constexpr int PF1 = bwd_kv_pf1<D>(), PF2 = bwd_kv_pf2<D>();
  static_assert(BT == 32, "one 32-query score tile per query tile");

  __shared__ __attribute__((aligned(16))) uint8_t q_lds[2][C::TB], d_lds[2][C::TB];
  __shared__ __attribute__((aligned(16))) float l_lds[2][BT], s_lds[2][BT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // causal: the first key tiles are seen by the most queries; they start first
  const unsigned bid = (unsigned)work_item(p.order_mul, p.order_add);
  const int nbk = p.B * p.Hkv;
  const int bk = CAUSAL ? (int)(bid % nbk) : (int)(bid / p.ntile);
  const int kt = CAUSAL ? (int)(bid / nbk) : (int)(bid % p.ntile);
  const int b = bk / p.Hkv, kvh = bk % p.Hkv;
  const int Nq = p.Nq, Nk = p.Nk;
  const int k_wg0 = kt * BK, kw0 = k_wg0 + wave * 32, k_lane = kw0 + l32;
  const int k_ld = k_lane < Nk ? k_lane : Nk - 1;
  // query tiles visited: causal skips those that end before the first key of the workgroup
  const int i0 = CAUSAL ? k_wg0 / BT : 0;
  const int nqt = (Nq + BT - 1) / BT;

  // K and V of this lane's key as B operands (dims 16t + 8hh .. +7)
  const size_t krow = (((size_t)b * Nk + k_ld) * p.Hkv + kvh) * (size_t)(D * 2);
  x8 kf[KS1], vf[KS1];
#pragma unroll
  for (int t = 0; t < KS1; ++t) {
    const int off = (16 * t + 8 * hh) * 2;
    kf[t] = __builtin_bit_cast(x8, *(const u32x4*)(p.k + krow + off));
    vf[t] = __builtin_bit_cast(x8, *(const u32x4*)(p.v + krow + off));
  }
  if (p.zero_scores) {  // zero scale: S = 0 exactly (masked scores stay -inf)
#pragma unroll
    for (int t = 0; t < KS1; ++t) kf[t] = x8{};
  }
  const float c = p.c;
  f32x16 dk[MT2], dv[MT2];
#pragma unroll
  for (int i = 0; i < MT2; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  const uint32_t q_row = (uint32_t)p.Hq * D * 2;
  const int a_rd = l32 * ROW + hh * 16;
  const int grp = lane >> 4, gi = lane & 15;
  const int t_rd = (4 * (grp >> 1) + (gi >> 2)) * ROW + (2 * (grp & 1) + ((gi & 3) >> 1)) * 16 + (gi & 1) * 8;

  const int per_head = nqt - i0;
  const int total = per_head * p.group;
  auto tile_head = [&](int n) { return kvh * p.group + n / per_head; };
  auto tile_q0 = [&](int n) { return (i0 + n % per_head) * BT; };
  auto load_tile = [&](int n, int buf) {
    const int h = tile_head(n), q0 = tile_q0(n);
    const uint8_t* qb = p.q + ((size_t)b * Nq * p.Hq + h) * (size_t)(D * 2);
    const uint8_t* db = p.dout + ((size_t)b * Nq * p.Hq + h) * (size_t)(D * 2);
    bwd_load_rows<D, NW, D == 128>(qb, q_row, q0, Nq, q_lds[buf], wv, lane);
    bwd_load_rows<D, NW, D == 128>(db, q_row, q0, Nq, d_lds[buf], wv, lane);
    if (wv == 0) {  // LSE and D of the tile's BT queries (zeros past Nq)
      const size_t lo = ((size_t)b * p.Hq + h) * Nq;
      const int nv = Nq - q0 < BT ? Nq - q0 : BT;
      const auto rl = make_rsrc((const uint8_t*)(p.lse + lo + q0), (uint32_t)nv * 4);
      const auto rd = make_rsrc((const uint8_t*)(p.dsum + lo + q0), (uint32_t)nv * 4);
      if (lane < BT) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (__attribute__((address_space(3))) void*)l_lds[buf], 4,
                                                 lane * 4, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (__attribute__((address_space(3))) void*)s_lds[buf], 4,
                                                 lane * 4, 0, 0, 0);
      }
    }
  };

  if (total > 0) load_tile(0, 0);
  tile_barrier();
  for (int n = 0; n < total; ++n) {
    const int buf = n & 1;
    if (n + 1 < total) load_tile(n + 1, buf ^ 1);
    const int q0 = tile_q0(n);
    // a wave whose keys all follow every query of the tile has nothing to do (causal)
    const bool active = !CAUSAL || kw0 <= q0 + BT - 1;
    if (active) {
      const uint8_t* ql = q_lds[buf];
      const uint8_t* dl = d_lds[buf];
      // S[q][k] and dP[q][k] (A = Q / dO rows from LDS, B = this lane's K / V). hd128: one
      // accumulator each (with the dq kernel's, +4% non-causal and +1% causal over two
      // alternating ones per product, which cost 32 registers and 32 adds per tile); hd256
      // keeps two each: with one, the compiler's schedule of this kernel ran 10% slower
      // non-causal (3% faster causal)
      constexpr bool TWO_ACC = D == 256;
      f32x16 s0 = f32x16{}, s1_ = f32x16{}, p0 = f32x16{}, p1_ = f32x16{};
      f32x16& s1 = TWO_ACC ? s1_ : s0;
      f32x16& p1 = TWO_ACC ? p1_ : p0;
      if constexpr (PF1 == 0) {
#pragma unroll
        for (int t = 0; t < KS1; t += 2) {
          const x8 qa = __builtin_bit_cast(x8, *(const u32x4*)(ql + a_rd + t * 32));
          const x8 qb = __builtin_bit_cast(x8, *(const u32x4*)(ql + a_rd + (t + 1) * 32));
          const x8 da = __builtin_bit_cast(x8, *(const u32x4*)(dl + a_rd + t * 32));
          const x8 db = __builtin_bit_cast(x8, *(const u32x4*)(dl + a_rd + (t + 1) * 32));
          s0 = T::mfma(qa, kf[t], s0);
          p0 = T::mfma(da, vf[t], p0);
          s1 = T::mfma(qb, kf[t + 1], s1);
          p1 = T::mfma(db, vf[t + 1], p1);
        }
      } else {
        // step t: the Q and dO fragments of head-dim step t, read PF1 steps ahead
        x8 qf_[KS1], df_[KS1];
        auto rd = [&](const int t) {
          qf_[t] = __builtin_bit_cast(x8, *(const u32x4*)(ql + a_rd + t * 32));
          df_[t] = __builtin_bit_cast(x8, *(const u32x4*)(dl + a_rd + t * 32));
        };
#pragma unroll
        for (int t = 0; t < PF1; ++t) rd(t);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < KS1; ++t) {
          if (t + PF1 < KS1) rd(t + PF1);
          if (t & 1) {
            s1 = T::mfma(qf_[t], kf[t], s1);
            p1 = T::mfma(df_[t], vf[t], p1);
          } else {
            s0 = T::mfma(qf_[t], kf[t], s0);
            p0 = T::mfma(df_[t], vf[t], p0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const f32x16 s = TWO_ACC ? s0 + s1_ : s0, dp = TWO_ACC ? p0 + p1_ : p0;
      // register r holds query q0 + 8(r/4) + 4hh + r%4 of this lane's key k_lane
      x8 pf[KS2], dsf[KS2];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int qo = 8 * g4 + 4 * hh;
        const float4 lv = *(const float4*)(&l_lds[buf][qo]);
        const float4 dv4 = *(const float4*)(&s_lds[buf][qo]);
        const float lr[4] = {lv.x, lv.y, lv.z, lv.w};
        const float dr[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
        float pe[4], dse[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          const int qq = q0 + qo + e;
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lr[e] * LOG2E));
          const bool vis = qq < Nq && (!CAUSAL || k_lane <= qq);
          pv = vis ? pv : 0.f;
          pe[e] = pv;
          dse[e] = pv * (dp[r] - dr[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const int r = 4 * g4 + e;
          const x2 pp = T::cvt2(pe[e], pe[e + 1]);
          const x2 dd = T::cvt2(dse[e], dse[e + 1]);
          pf[r >> 3][r & 7] = pp[0];
          pf[r >> 3][(r & 7) + 1] = pp[1];
          dsf[r >> 3][r & 7] = dd[0];
          dsf[r >> 3][(r & 7) + 1] = dd[1];
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T read transposed from the tiles),
      // fragments PF2 steps ahead
      if constexpr (PF2 == 0) {
#pragma unroll
        for (int u = 0; u < KS2; ++u)
#pragma unroll
          for (int md = 0; md < MT2; ++md) {
            const x8 rdo = bwd_tr_frag<x8>(dl + t_rd + (16 * u) * ROW + md * 64, ROW);
            const x8 rq = bwd_tr_frag<x8>(ql + t_rd + (16 * u) * ROW + md * 64, ROW);
            dv[md] = T::mfma(rdo, pf[u], dv[md]);
            dk[md] = T::mfma(rq, dsf[u], dk[md]);
          }
      } else {
        constexpr int N = KS2 * MT2;
        x8 tdf[N], tqf[N];
        auto rd = [&](const int i) {
          const int u = i / MT2, md = i % MT2;
          tdf[i] = bwd_tr_frag<x8>(dl + t_rd + (16 * u) * ROW + md * 64, ROW);
          tqf[i] = bwd_tr_frag<x8>(ql + t_rd + (16 * u) * ROW + md * 64, ROW);
        };
#pragma unroll
        for (int i = 0; i < PF2; ++i) rd(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          if (i + PF2 < N) rd(i + PF2);
          const int u = i / MT2, md = i % MT2;
          dv[md] = T::mfma(tdf[i], pf[u], dv[md]);
          dk[md] = T::mfma(tqf[i], dsf[u], dk[md]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    tile_barrier();
  }

  if (k_lane < Nk) {
    const size_t orow = (((size_t)b * Nk + k_lane) * p.Hkv + kvh) * (size_t)(D * 2);
    const float sc = p.scale;
#pragma unroll
    for (int md = 0; md < MT2; ++md)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * md + 8 * i + 4 * hh;
        u32x2 wk, wvv;
        wk[0] = __builtin_bit_cast(unsigned, T::cvt2(dk[md][4 * i + 0] * sc, dk[md][4 * i + 1] * sc));
        wk[1] = __builtin_bit_cast(unsigned, T::cvt2(dk[md][4 * i + 2] * sc, dk[md][4 * i + 3] * sc));
        wvv[0] = __builtin_bit_cast(unsigned, T::cvt2(dv[md][4 * i + 0], dv[md][4 * i + 1]));
        wvv[1] = __builtin_bit_cast(unsigned, T::cvt2(dv[md][4 * i + 2], dv[md][4 * i + 3]));
        *(u32x2*)(p.dk + orow + d * 2) = wk;
        *(u32x2*)(p.dv + orow + d * 2) = wvv;
      }
  }
}

}  // namespace fa
