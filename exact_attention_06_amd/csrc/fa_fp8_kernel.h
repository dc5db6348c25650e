// fa_fp8_kernel.h - gfx950 exact-attention forward with fp8 (e4m3, OCP) Q, K, V.
//
// The FP8 input path the pages list ("[RFC] FA4 - head_dim=256 & head_dim=512", feature
// table of section "Phase 2": FP8 input on the FP8 tensor-core MMA). The caller passes
// e4m3 tensors and one dequantisation factor per tensor (q_scale, k_scale, v_scale); the
// operation is the dense one of fa_fwd on the dequantised values. Both products run on
// v_mfma_f32_32x32x64_f8f6f4 (fp8 x fp8 -> fp32, twice the bf16 rate): S^T = K Q^T (the
// products are exact; the MFMA sums each group of 64 with fewer bits than fp32, measured at
// up to ~2^-14 of sum |q k|), and O^T += V^T P^T with P rounded to e4m3. The row sum
// that normalises O is the fp32 sum of the rounded P (one extra MFMA against an all-ones
// operand), so P's rounding largely cancels in O; the LSE uses the fp32 sum of unrounded p.
//
// CDNA4 mapping (same transposed form and softmax as the bf16 kernel, 64-key tiles):
//   * hd128 runs the bf16 hd128 kernel's software pipeline: the softmax of tile j is issued
//     between the score MFMAs of tile j+1, and the fp32 row sum of tile j and the row max of
//     tile j+1 between the P.V MFMAs of tile j (two score buffers; 3-6% faster than one tile
//     at a time at N >= 8k, bitwise the same O). hd256 has no registers for a second score
//     buffer and takes one tile at a time;
//   * an MFMA A or B operand is 32 bytes per lane: row (lane % 32), 32 k-values selected by
//     lane / 32. Any k order works as long as A and B use the same one (the product sums
//     over k); GEMM1 takes d = 64t + 32(lane/32) + byte, GEMM2 takes, for byte j = 8w + e of
//     lane half hh, key 32(w/2) + 16(w%2) + 8(e/4) + 4hh + e%4 - exactly the keys the lane
//     holds in the score layout, so P needs no shuffle;
//   * V^T comes from ds_read_b64_tr_b8: in a 16-lane group, output lane i receives byte i%8
//     of the 8-byte rows read by source lanes 2e + i/8 (e = 0..7); source lane 2e + p points
//     at key row e of read w and head-dim column (16 g + 8p) of the 32-wide block, so lane i
//     of group g gets 8 keys of column 16g + i;
//   * K/V rows are stored unpadded (D bytes) with their 16-byte chunks XOR-swizzled per row
//     (chunk c of row r at c ^ f(r)); f makes both the 16-byte K reads of 16 consecutive rows
//     and the transpose reads of V touch every LDS bank once.
#pragma once

#include "fa_kernel.h"

namespace fa {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int D>
struct Fp8Cfg {
  static constexpr int NW = 4, BC = 64, BR = NW * 32;
  static constexpr int ROW = D;               // bytes per K/V row in LDS
  static constexpr int CPR = D / 16;          // 16-byte chunks per row
  static constexpr int TB = BC * ROW;         // bytes per tile
  static constexpr int LPW = TB / 1024 / NW;  // 1 KB direct-to-LDS loads per wave and tile
  static constexpr int LDS = 4 * TB;          // two K and two V buffers
  static_assert(TB % (1024 * NW) == 0, "whole loads per wave");
};

// Chunk swizzle of row r (only its 4 low bits matter): hd128 rows are 8 chunks (half the banks),
// hd256 rows 16 chunks (all banks).
template <int D>
__device__ __forceinline__ int fp8_swz(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
  if constexpr (D == 128) return (r1 << 1) | (r3 << 2) | r2;
  return (r0 << 1) | (r1 << 2) | (r3 << 3) | r2;
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format 0 (e4m3) for both operands, no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(Fp8Cfg<D>::NW * 64, 2)
fwd_fp8_kernel(FwdParams p) {
  using C = Fp8Cfg<D>;
  constexpr int NW = C::NW, BC = C::BC, BR = C::BR, ROW = C::ROW, CPR = C::CPR, LPW = C::LPW;
  constexpr int KS1 = D / 64;   // GEMM1 k-steps (64 head-dim values each)
  constexpr int MT1 = BC / 32;  // score tiles per K/V tile
  constexpr int MT2 = D / 32;   // output tiles
  __shared__ __attribute__((aligned(16))) uint8_t k_lds0[C::TB], k_lds1[C::TB], v_lds0[C::TB], v_lds1[C::TB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  int bh, qt;
  decode_block<CAUSAL, false>(work_item(p.order_mul, p.order_add), p, bh, qt);
  const int b = bh / p.Hq, hq = bh - b * p.Hq, kvh = hq / p.group;
  const int Nq = p.Nq, Nk = p.Nk;
  const int q_wg0 = qt * BR, qw0 = q_wg0 + wave * 32, q_lane = qw0 + l32;
  const int q_ld = q_lane < Nq ? q_lane : Nq - 1;
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(Nq, q_wg0 + BR));
  const int ntiles = (kend + BC - 1) / BC;
  const int wtiles = CAUSAL ? max(1, min(ntiles, (min(qw0 + 32, Nq) + BC - 1) / BC)) : ntiles;
  int nfull = Nk / BC;
  if (CAUSAL) nfull = min(nfull, (q_wg0 + 1) / BC);

  // Q (B operand of GEMM1): lane holds query q_ld, head-dim values 64t + 32hh .. +31
  i32x8 qf[KS1];
  const int sgn8 = p.neg_scores ? (int)0x80808080u : 0;
  {
    const uint8_t* qp = p.q + (((size_t)b * Nq + q_ld) * p.Hq + hq) * (size_t)D;
#pragma unroll
    for (int t = 0; t < KS1; ++t) {
      const u32x4 lo = *(const u32x4*)(qp + 64 * t + 32 * hh);
      const u32x4 hi = *(const u32x4*)(qp + 64 * t + 32 * hh + 16);
      for (int e = 0; e < 4; ++e) {
        qf[t][e] = (int)lo[e];
        qf[t][4 + e] = (int)hi[e];
      }
      // negative scale: -Q (e4m3 sign bit 7 of every byte, exact), as an unconditional xor
      for (int e = 0; e < 8; ++e) qf[t][e] ^= sgn8;
      if (p.zero_scores) qf[t] = i32x8{};
    }
  }
  i32x8 ones;  // e4m3 1.0 in every byte
  for (int e = 0; e < 8; ++e) ones[e] = 0x38383838;

  f32x16 acc[MT2 + 1];  // O^T tiles, and the row sums of the rounded P (all 32 rows alike)
#pragma unroll
  for (int i = 0; i <= MT2; ++i) acc[i] = f32x16{};
  float m_run = -__builtin_inff(), lL = 0.f;
  const float c = p.c;

  // ---- direct-to-LDS tile loads: slot s of a tile is (row s / CPR, physical chunk s % CPR),
  //      which holds logical chunk (s % CPR) ^ f(row); rows past the last key load zeros
  constexpr uint32_t OOB = 0x80000000u;
  const uint32_t kv_row = (uint32_t)p.Hkv * D;
  const uint8_t* kbase = p.k + ((size_t)b * Nk * p.Hkv + kvh) * (size_t)D;
  const uint8_t* vbase = p.v + ((size_t)b * Nk * p.Hkv + kvh) * (size_t)D;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t vo[LPW];
#pragma unroll
  for (int n = 0; n < LPW; ++n) {
    const int slot = 64 * (wv + NW * n) + lane, row = slot / CPR, pc = slot % CPR;
    vo[n] = row < BC ? (uint32_t)row * kv_row + 16 * (pc ^ fp8_swz<D>(row)) : OOB;
  }
  // (the offsets come in as a pointer: a lambda that captures the array keeps the host pass
  // from emitting the kernel's launch stub)
  auto load_tile = [&](int tile, const uint8_t* gbase, uint8_t* ldst, const uint32_t* vop) {
    const int k0 = tile * BC;
    const auto rs = make_rsrc(gbase + (size_t)k0 * kv_row, (uint32_t)min(BC, Nk - k0) * kv_row);
#pragma unroll
    for (int n = 0; n < LPW; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(ldst + 1024 * (wv + NW * n)), 16, vop[n], 0, 0, 0);
  };
  auto load_kv = [&](int tile, int buf) {
    load_tile(tile, kbase, buf ? k_lds1 : k_lds0, vo);
    load_tile(tile, vbase, buf ? v_lds1 : v_lds0, vo);
  };

  // ---- per-lane LDS read offsets
  // GEMM1 (K rows 32mt + l32, logical chunks 4t + 2hh + e): row base and swizzle of row l32
  const int fk = fp8_swz<D>(l32);
  const int k_rd = l32 * ROW;
  // GEMM2 (transpose reads): lane group g = (lane / 16) % 2, source index s = lane % 16
  // (e = s / 2, p = s % 2); row = 32(w/2) + 16(w%2) + 8(e/4) + 4hh + e%4, logical column
  // 32md + 16g + 8p
  const int s16 = lane & 15, g16 = (lane >> 4) & 1, e8 = s16 >> 1, p2 = s16 & 1;
  const int vrow = 8 * (e8 >> 2) + 4 * hh + (e8 & 3);
  const int fv = fp8_swz<D>(vrow);
  const int v_rd = vrow * ROW + 16 * (g16 ^ (fv & 1)) + 8 * p2;  // + 32 (md ^ (fv >> 1))
  const int v_x = 32 * (fv >> 1);

  // hd128: LDS fragments are read PF MFMAs ahead in a fixed order (sched_barrier), so that the
  // read latency hides under the MFMAs before them (+7%). hd256 has no registers to spare for
  // that (the fragments spill and it runs up to 40% slower): there the compiler orders the reads.
  constexpr int PF = D == 128 ? 2 : 0;
  auto gemm1 = [&](const uint8_t* kl, f32x16 (&s)[MT1]) {
    constexpr int N = KS1 * MT1;
    auto frag = [&](const int i) -> i32x8 {
      const int t = i / MT1, mt = i % MT1;
      const int o0 = 16 * ((4 * t + 2 * hh) ^ fk), o1 = 16 * ((4 * t + 2 * hh + 1) ^ fk);
      const uint8_t* rp = kl + k_rd + mt * 32 * ROW;
      const u32x4 lo = *(const u32x4*)(rp + o0);
      const u32x4 hi = *(const u32x4*)(rp + o1);
      i32x8 a;
      for (int e = 0; e < 4; ++e) {
        a[e] = (int)lo[e];
        a[4 + e] = (int)hi[e];
      }
      return a;
    };
    if constexpr (PF == 0) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int t = i / MT1, mt = i % MT1;
        s[mt] = mfma_fp8(frag(i), qf[t], t == 0 ? f32x16{} : s[mt]);
      }
      return;
    }
    i32x8 kf[N];
#pragma unroll
    for (int i = 0; i < PF && i < N; ++i) kf[i] = frag(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + PF < N) kf[i + PF] = frag(i + PF);
      const int t = i / MT1, mt = i % MT1;
      s[mt] = mfma_fp8(kf[i], qf[t], t == 0 ? f32x16{} : s[mt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto gemm2 = [&](const uint8_t* vl, const i32x8& pb) {
    auto frag = [&](const int md) -> i32x8 {
      const uint8_t* base = vl + v_rd + ((32 * md) ^ v_x);
      i32x8 a;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2*)(base + (32 * (w >> 1) + 16 * (w & 1)) * ROW));
        a[2 * w] = r[0];
        a[2 * w + 1] = r[1];
      }
      return a;
    };
    if constexpr (PF == 0) {
#pragma unroll
      for (int md = 0; md < MT2; ++md) acc[md] = mfma_fp8(frag(md), pb, acc[md]);
      acc[MT2] = mfma_fp8(ones, pb, acc[MT2]);
      return;
    }
    i32x8 vf[MT2];
#pragma unroll
    for (int i = 0; i < PF; ++i) vf[i] = frag(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int md = 0; md < MT2; ++md) {
      if (md + PF < MT2) vf[md + PF] = frag(md + PF);
      acc[md] = mfma_fp8(vf[md], pb, acc[md]);
      __builtin_amdgcn_sched_barrier(0);
    }
    acc[MT2] = mfma_fp8(ones, pb, acc[MT2]);
  };
  auto mask = [&](int j, f32x16 (&s)[MT1]) {
    const int k0 = j * BC;
    if ((k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > qw0))) {
      const int last = CAUSAL ? min(q_lane, Nk - 1) : Nk - 1;
      const int lim = last - k0 - 4 * hh;
#pragma unroll
      for (int mt = 0; mt < MT1; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * mt + 8 * (r >> 2) + (r & 3) > lim) s[mt][r] = -__builtin_inff();
    }
  };
  auto rescale = [&](const f32x16 (&s)[MT1]) {
    float mx = s[0][0];
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[mt][r]);
    mx = __builtin_fmaxf(mx, other_half(mx)) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {
      const float mnew = __builtin_fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
#pragma unroll
      for (int i = 0; i <= MT2; ++i) acc[i] *= alpha;
      lL *= alpha;
      m_run = mnew;
    }
  };
  // p = exp2(s*c - m) in fp32 (summed into lL), rounded to e4m3 into the B operand: byte
  // 8w + e is score register 8(w%2) + e of score tile w/2
  auto softmax = [&](const f32x16 (&s)[MT1], i32x8& pb) {
    const float negm = -m_run;
    float sum0, sum1;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int mt = w >> 1, r = 8 * (w & 1) + 4 * h;
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][r + e], c, negm));
        if (w == 0 && h == 0) {
          sum0 = pv[0] + pv[2];
          sum1 = pv[1] + pv[3];
        } else {
          sum0 += pv[0] + pv[2];
          sum1 += pv[1] + pv[3];
        }
        // both halves of the word are written; at hd128 the last tile's word is the merge
        // operand, so no register needs clearing first (hd256 has no registers to keep P live
        // across tiles: its causal kernel spills and runs 11% slower)
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], D == 128 ? pb[2 * w + h] : 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], word, true);
        pb[2 * w + h] = word;
      }
    lL += sum0 + sum1;
  };

  i32x8 pb = {};  // P rounded to e4m3 (B operand of O^T += V^T P^T), rewritten every tile
  using F = BoolC<false>;
  using U = BoolC<true>;
  if constexpr (D == 128) {
  // ---- software pipeline (as the bf16 hd128 loop): iteration j loads K(j+2) and V(j+1);
  //      phase 1 issues the score MFMAs of tile j+1 with the softmax of tile j between them,
  //      phase 2 the P.V MFMAs of tile j with the fp32 row sum of tile j and the row max of
  //      tile j+1 (which decides the next rescale) between them.
  auto load_k = [&](int tile, int buf) { load_tile(tile, kbase, buf ? k_lds1 : k_lds0, vo); };
  auto load_v = [&](int tile, int buf) { load_tile(tile, vbase, buf ? v_lds1 : v_lds0, vo); };
  auto rowmax = [&](const f32x16 (&s)[MT1]) -> float {
    float mx = s[0][0];
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[mt][r]);
    return __builtin_fmaxf(mx, other_half(mx)) * c;
  };
  auto rescale_to = [&](const float mx) {
    if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {
      const float mnew = __builtin_fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
#pragma unroll
      for (int i = 0; i <= MT2; ++i) acc[i] *= alpha;
      lL *= alpha;
      m_run = mnew;
    }
  };
  load_k(0, 0);
  load_v(0, 0);
  if (ntiles > 1) load_k(1, 1);
  tile_barrier();
  f32x16 s_a[MT1], s_b[MT1];
  gemm1(k_lds0, s_a);
  tile_barrier();  // every wave has read K(0) before iteration 0 reloads its buffer
  float mt_cur = 0.f;
  // generic iteration (diagonal and tail tiles, and grids with a single tile)
  auto iteration = [&](const int j, f32x16 (&sc)[MT1], f32x16 (&sn)[MT1], auto mask_tag) {
    constexpr bool MASKED = decltype(mask_tag)::value;
    const int par = j & 1;
    const bool more_k = j + 2 < ntiles, more_v = j + 1 < ntiles;
    if (more_k) load_k(j + 2, par);
    if (more_v) load_v(j + 1, 1 - par);
    const bool active = !MASKED || j < wtiles;
    const bool next_active = MASKED ? (j + 1 < wtiles) : more_v;
    if (active) {
      if (MASKED) mask(j, sc);
      rescale_to(rowmax(sc));
      if (next_active) gemm1(par ? k_lds0 : k_lds1, sn);  // K(j+1): buffer 1 - par
      softmax(sc, pb);
      // keeps the all-ones operand in registers across tiles (the compiler rebuilt it with
      // 7 moves per tile)
      asm volatile("" : "+v"(ones));
      gemm2(par ? v_lds1 : v_lds0, pb);
    }
    tile_barrier();
  };
  constexpr int N1 = KS1 * MT1;  // score MFMAs per tile
  auto main_iteration = [&](const int j, f32x16 (&sc)[MT1], f32x16 (&sn)[MT1], auto par_tag) {
    constexpr int PAR = decltype(par_tag)::value;  // j & 1
    if (j + 2 < ntiles) load_k(j + 2, PAR);
    load_v(j + 1, 1 - PAR);
    rescale_to(mt_cur);
    const float negm = -m_run;
    const uint8_t* kl = PAR ? k_lds0 : k_lds1;  // K(j+1): buffer 1 - PAR
    const uint8_t* vl = PAR ? v_lds1 : v_lds0;  // V(j): buffer PAR
    auto kfrag = [&](const int i) -> i32x8 {
      const int t = i / MT1, mt = i % MT1;
      const int o0 = 16 * ((4 * t + 2 * hh) ^ fk), o1 = 16 * ((4 * t + 2 * hh + 1) ^ fk);
      const uint8_t* rp = kl + k_rd + mt * 32 * ROW;
      const u32x4 lo = *(const u32x4*)(rp + o0);
      const u32x4 hi = *(const u32x4*)(rp + o1);
      i32x8 a;
      for (int e = 0; e < 4; ++e) {
        a[e] = (int)lo[e];
        a[4 + e] = (int)hi[e];
      }
      return a;
    };
    auto vfrag = [&](const int md) -> i32x8 {
      const uint8_t* base = vl + v_rd + ((32 * md) ^ v_x);
      i32x8 a;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2*)(base + (32 * (w >> 1) + 16 * (w & 1)) * ROW));
        a[2 * w] = r[0];
        a[2 * w + 1] = r[1];
      }
      return a;
    };
    i32x8 kf[N1], vf[MT2];
#pragma unroll
    for (int i = 0; i < PF; ++i) kf[i] = kfrag(i);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < N1; ++i) {
      if (i + PF < N1)
        kf[i + PF] = kfrag(i + PF);
      else
        vf[i + PF - N1] = vfrag(i + PF - N1);
      {
        const int t = i / MT1, mt = i % MT1;
        sn[mt] = mfma_fp8(kf[i], qf[t], t == 0 ? f32x16{} : sn[mt]);
      }
      // softmax of two 4-score groups of tile j (words 2w, 2w + 1 of P); p overwrites its score
#pragma unroll
      for (int g = 2 * i; g < 2 * i + 2; ++g) {
        const int w = g >> 1, h = g & 1, mt = w >> 1, r = 8 * (w & 1) + 4 * h;
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mt][r + e], c, negm));
          sc[mt][r + e] = pv[e];
        }
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], pb[g], false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], word, true);
        pb[g] = word;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    asm volatile("" : "+v"(ones));
    float mx = -__builtin_inff(), sum0 = 0.f, sum1 = 0.f;
    constexpr int VPS = 16 * MT1 / MT2;  // p values summed (and next-tile scores maxed) per step
#pragma unroll
    for (int md = 0; md < MT2; ++md) {
      if (md + PF < MT2) vf[md + PF] = vfrag(md + PF);
      acc[md] = mfma_fp8(vf[md], pb, acc[md]);
#pragma unroll
      for (int e = md * VPS; e < (md + 1) * VPS; ++e) {
        if (e & 1)
          sum1 += sc[e / 16][e % 16];
        else
          sum0 += sc[e / 16][e % 16];
        mx = __builtin_fmaxf(mx, sn[e / 16][e % 16]);
      }
      asm volatile("" : "+v"(mx), "+v"(sum0), "+v"(sum1));
      __builtin_amdgcn_sched_barrier(0);
    }
    acc[MT2] = mfma_fp8(ones, pb, acc[MT2]);
    lL += sum0 + sum1;
    mx = __builtin_fmaxf(mx, other_half(mx));
    mt_cur = mx * c;
    tile_barrier();  // the loads of this iteration have landed; LDS reads of it are done
  };
  const int nmain = min(nfull, ntiles - 1);
  int j = 0;
  if (nmain > 0) {
    mt_cur = rowmax(s_a);
    main_iteration(0, s_a, s_b, IntC<0>{});
    j = 1;
    for (; j + 1 < nmain; j += 2) {
      main_iteration(j, s_b, s_a, IntC<1>{});
      main_iteration(j + 1, s_a, s_b, IntC<0>{});
    }
    if (j < nmain) {
      main_iteration(j, s_b, s_a, IntC<1>{});
      ++j;
    }
  }
  // diagonal and tail tiles; the scores of tile j move to s_a first
  if (j < ntiles && (j & 1)) {
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt) s_a[mt] = s_b[mt];
  }
  for (; j < ntiles; ++j) {
    iteration(j, s_a, s_b, U{});
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt) s_a[mt] = s_b[mt];
  }
  } else {
  // ---- hd256: one tile at a time (no registers for a second score buffer); the two
  //      workgroups of a CU overlap each other
  auto iteration = [&](const int j, const int par, auto mask_tag) {
    constexpr bool MASKED = decltype(mask_tag)::value;
    if (j + 1 < ntiles) load_kv(j + 1, 1 - par);
    if (!MASKED || j < wtiles) {
      f32x16 sc[MT1];
      gemm1(par ? k_lds1 : k_lds0, sc);
      if (MASKED) mask(j, sc);
      rescale(sc);
      pb = i32x8{};  // (a fresh value: nothing stays live across tiles)
      softmax(sc, pb);
      gemm2(par ? v_lds1 : v_lds0, pb);
    }
    tile_barrier();  // the loads of this iteration have landed; LDS reads of it are done
  };
  load_kv(0, 0);
  tile_barrier();
  int j = 0;
  for (; j + 1 < nfull; j += 2) {
    iteration(j, 0, F{});
    iteration(j + 1, 1, F{});
  }
  if (j < nfull) {
    iteration(j, j & 1, F{});
    ++j;
  }
  for (; j < ntiles; ++j) iteration(j, j & 1, U{});

  }

  // ---- epilogue: O = v_scale * O_acc / sum(rounded P); LSE from the fp32 sum of p
  lL += other_half(lL);
  const float lO = acc[MT2][0];
  // O leaves through LDS as whole rows (see the bf16 kernel's epilogue): wave w writes its
  // 32 x D bf16 tile into the w-th K/V buffer (a buffer is exactly 32 rows of 2D bytes; every
  // wave is past the last tile's barrier), 16-byte chunk k of row r at chunk k ^ (r mod the
  // chunks per row) so that the 32 rows of a write and the chunks of a read spread over the
  // banks, and reads it back 16 bytes per lane for full-row stores.
  static_assert(32 * D * 2 == C::TB, "a wave's O tile fills one K/V buffer");
  constexpr int CPL = D * 2 / 16, RPI = 64 / CPL;  // 16-byte chunks per row, rows per read
  uint8_t* const ost = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
  const float inv = p.v_scale / lO;
#pragma unroll
  for (int md = 0; md < MT2; ++md)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 a = Bf16::cvt2(acc[md][4 * i + 0] * inv, acc[md][4 * i + 1] * inv);
      const bf16x2 bb = Bf16::cvt2(acc[md][4 * i + 2] * inv, acc[md][4 * i + 3] * inv);
      u32x2 w;
      w[0] = __builtin_bit_cast(unsigned, a);
      w[1] = __builtin_bit_cast(unsigned, bb);
      const int k = 4 * md + i;  // chunk of columns 32md + 8i .. +7; this lane's half at 8hh
      *(u32x2*)(ost + l32 * (D * 2) + ((k ^ (l32 & (CPL - 1))) * 16) + 8 * hh) = w;
    }
  const size_t o_row = (size_t)p.Hq * (D * 2);
  uint8_t* const o0 = p.o + (((size_t)b * Nq + qw0) * p.Hq + hq) * (size_t)(D * 2);
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = it * RPI + lane / CPL, ch = lane % CPL;
    const u32x4 v = *(const u32x4*)(ost + r * (D * 2) + ((ch ^ (r & (CPL - 1))) * 16));
    if (qw0 + r < Nq) *(u32x4*)(o0 + r * o_row + ch * 16) = v;
  }
  if (q_lane < Nq && hh == 0)
    p.lse[((size_t)b * p.Hq + hq) * Nq + q_lane] = (m_run + __builtin_amdgcn_logf(lL)) * LN2;
}

}  // namespace fa
