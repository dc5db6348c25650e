// fa_hd512_kernel.h - gfx950 exact-attention forward for head dim 512 (dense batches).
//
// Head dim 512 is on the pages' list of extended head dims ("[RFC] FA4 - head_dim=256 &
// head_dim=512", table of section "Phase 4": symmetric head_dim=512). The operation is
// fa_fwd's at d = 512: O = softmax(scale * Q K^T [causal]) V and the per-row LSE, with the
// same online softmax, lazy rescale and split row sums as the hd128/hd256 kernel.
//
// Why a kernel of its own: with one wave owning 32 query rows, the fp32 output tile alone
// is 32 x 512 / 64 = 256 registers per lane, a wave's whole budget when two waves share a
// SIMD. Here two waves share each 32-row query block and split the head dim: wave
// (pair, half) keeps Q and O for dims 256*half .. 256*half + 255 (64 + 128 registers, the
// hd256 kernel's budget). Each wave computes the partial scores of its half,
// S_half^T = K[:, half] Q[:, half]^T, and the pair adds the two partials through LDS (in the
// K buffer of the tile, once every wave has finished reading it). Both waves then hold
// bitwise the same S (fp32 addition is commutative), take the same rescale decisions and
// the same P, and each accumulates its half of O^T += V[:, half]^T P^T.
//
// Per 32-key tile the K and V rows are 1 KB each, padded as in the other kernel (K by 16 B,
// V by 64 B) and double buffered: 2 x (33 + 34) KB of LDS, one workgroup of 8 waves (4 pairs,
// 128 query rows) per CU, two waves per SIMD. Three barriers per tile: K reads done (the
// exchange area is free), partials written, and the end of the tile (next loads landed,
// every read of this tile done). The first two do not wait for the tile loads in flight.
#pragma once

#include "fa_kernel.h"

namespace fa {

struct Hd512 {
  static constexpr int D = 512, DH = 256;       // head dim, dims per wave
  static constexpr int NW = 8, BR = 128, BC = 32;  // waves (4 pairs), query rows, keys per tile
  static constexpr int KROW = D * 2 + 16, VROW = D * 2 + 64;  // padded LDS row pitches (bytes)
  static constexpr int KSL = KROW / 16, VSL = VROW / 16;      // 16-byte slots per padded row
  static constexpr int NLK = (BC * KSL + 63) / 64;  // 1 KB direct-to-LDS loads per K tile
  static constexpr int NLV = (BC * VSL + 63) / 64;  // ... per V tile
  static constexpr int KPW = (NLK + NW - 1) / NW, VPW = (NLV + NW - 1) / NW;  // rounds per wave
  static constexpr int KBUF = NLK * 1024, VBUF = NLV * 1024;
  static constexpr int LDS = 2 * KBUF + 2 * VBUF;
  static constexpr int XCH = 4096;  // bytes of partial scores per wave (16 floats x 64 lanes)
  static_assert(NW * XCH <= KBUF, "the score exchange fits in a K buffer");
  static_assert(LDS <= 160 * 1024, "one workgroup per CU");
};

template <bool CAUSAL, class T>
__global__ void __launch_bounds__(Hd512::NW * 64, 2)
fwd_hd512_kernel(FwdParams p) {
  using C = Hd512;
  using x8 = typename T::x8;
  using x2 = typename T::x2;
  constexpr int D = C::D, DH = C::DH, NW = C::NW, BR = C::BR, BC = C::BC;
  constexpr int KROW = C::KROW, VROW = C::VROW, KSL = C::KSL, VSL = C::VSL;
  constexpr int KS1 = DH / 16;  // GEMM1 k-steps over this wave's half of the head dim
  constexpr int MT2 = DH / 32;  // output tiles of this wave
  constexpr int KS2 = BC / 16;  // GEMM2 k-steps over the keys of a tile
  constexpr int CPR = D / 8;    // 16-byte chunks per K/V row
  __shared__ __attribute__((aligned(16))) uint8_t k_lds0[C::KBUF], k_lds1[C::KBUF], v_lds0[C::VBUF],
      v_lds1[C::VBUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int pair = wave >> 1, half = wave & 1;
  int bh, qt;
  decode_block<CAUSAL, false>(work_item(p.order_mul, p.order_add), p, bh, qt);
  const int b = bh / p.Hq, hq = bh - b * p.Hq, kvh = hq / p.group;
  const int Nq = p.Nq, Nk = p.Nk;
  const int q_wg0 = qt * BR, qw0 = q_wg0 + pair * 32, q_lane = qw0 + l32;
  const int q_ld = q_lane < Nq ? q_lane : Nq - 1;
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(Nq, q_wg0 + BR));
  const int ntiles = (kend + BC - 1) / BC;
  // a pair computes on its first wtiles tiles (causal: keys up to its last query); tiles
  // below nfull need no mask for any query of the workgroup
  const int wtiles = CAUSAL ? max(1, min(ntiles, (min(qw0 + 32, Nq) + BC - 1) / BC)) : ntiles;
  int nfull = Nk / BC;
  if (CAUSAL) nfull = min(nfull, (q_wg0 + 1) / BC);

  // ---- Q fragments (B operand of S^T = K Q^T): query q_ld, dims DH*half + 16t + 8hh .. +7
  x8 qf[KS1];
  {
    const uint8_t* qp = p.q + (((size_t)b * Nq + q_ld) * p.Hq + hq) * (size_t)(D * 2) + half * (DH * 2);
#pragma unroll
    for (int t = 0; t < KS1; ++t) qf[t] = __builtin_bit_cast(x8, *(const u32x4*)(qp + (16 * t + 8 * hh) * 2));
    if (p.zero_scores) {  // zero scale: zero Q and use a unit c (masked scores stay -inf)
#pragma unroll
      for (int t = 0; t < KS1; ++t) qf[t] = x8{};
    }
    // negative scale: -Q (exact) with c = |scale| * log2(e)
    const unsigned sgn = p.neg_scores ? 0x80008000u : 0u;
#pragma unroll
    for (int t = 0; t < KS1; ++t) qf[t] = sign16(qf[t], sgn);
  }

  f32x16 acc[MT2];
#pragma unroll
  for (int i = 0; i < MT2; ++i) acc[i] = f32x16{};
  float m_run = -__builtin_inff(), lL = 0.f, lO = 0.f;
  const float c = p.c;
  const x2 one2 = T::ones();

  // ---- K/V tiles: buffer loads straight into LDS. Load n of wave wv fills slots
  //      64 (wv + NW n) .. +63 of the tile (16 bytes each, M0 base + 16 * lane); the last
  //      round covers only part of the tile and is issued by the first waves only (a
  //      wave-uniform test). Pad slots and rows past the last key load zeros.
  constexpr uint32_t OOB = 0x80000000u;
  const uint32_t kv_row = (uint32_t)p.Hkv * D * 2;
  const uint8_t* kbase = p.k + ((size_t)b * Nk * p.Hkv + kvh) * (size_t)(D * 2);
  const uint8_t* vbase = p.v + ((size_t)b * Nk * p.Hkv + kvh) * (size_t)(D * 2);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t k_vo[C::KPW], v_vo[C::VPW];
#pragma unroll
  for (int n = 0; n < C::KPW; ++n) {
    const int slot = 64 * (wv + NW * n) + lane, row = slot / KSL, ch = slot % KSL;
    k_vo[n] = (ch < CPR && row < BC) ? (uint32_t)row * kv_row + ch * 16 : OOB;
  }
#pragma unroll
  for (int n = 0; n < C::VPW; ++n) {
    const int slot = 64 * (wv + NW * n) + lane, row = slot / VSL, ch = slot % VSL;
    v_vo[n] = (ch < CPR && row < BC) ? (uint32_t)row * kv_row + ch * 16 : OOB;
  }
  auto load_tile = [&](int tile, const uint8_t* gbase, uint8_t* ldst, const uint32_t* vo, auto npw_tag,
                       auto nl_tag) {
    constexpr int NPW = decltype(npw_tag)::value, NL = decltype(nl_tag)::value;
    const int k0 = tile * BC;
    const auto rs = make_rsrc(gbase + (size_t)k0 * kv_row, (uint32_t)min(BC, Nk - k0) * kv_row);
#pragma unroll
    for (int n = 0; n < NPW; ++n)
      if (wv + NW * n < NL)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(ldst + 1024 * (wv + NW * n)), 16, vo[n], 0, 0, 0);
  };
  auto load_kv = [&](int tile, int buf) {
    load_tile(tile, kbase, buf ? k_lds1 : k_lds0, k_vo, IntC<C::KPW>{}, IntC<C::NLK>{});
    load_tile(tile, vbase, buf ? v_lds1 : v_lds0, v_vo, IntC<C::VPW>{}, IntC<C::NLV>{});
  };

  // ---- per-lane LDS read bases (the other kernel's, shifted to this wave's half)
  // GEMM1 A operand (K): row l32, dims DH*half + 16t + 8hh .. +7
  const int k_rd = l32 * KROW + hh * 16 + half * (DH * 2);
  // GEMM2 A operand (V^T) via ds_read_b64_tr_b16: k-step u covers keys 16u + {4g + 0..3,
  // 8 + 4g + 0..3}, g = (lane group) / 2 - the order P^T holds them in
  const int grp = lane >> 4, gi = lane & 15;
  const int v_rd = (4 * (grp >> 1) + (gi >> 2)) * VROW + (2 * (grp & 1) + ((gi & 3) >> 1)) * 16 + (gi & 1) * 8 +
                   half * (DH * 2);
  // partial scores of wave w: register group i (4 floats) of lane l at w*XCH + i*1024 + 16l
  const int x_own = wave * C::XCH + lane * 16, x_mate = (wave ^ 1) * C::XCH + lane * 16;

  auto gemm1 = [&](const uint8_t* kbuf, f32x16& s) {
    const uint8_t* kl = kbuf + k_rd;
    s = f32x16{};
#pragma unroll
    for (int t = 0; t < KS1; ++t) s = T::mfma(__builtin_bit_cast(x8, *(const u32x4*)(kl + t * 32)), qf[t], s);
  };
  auto gemm2 = [&](const uint8_t* vbuf, const x8 (&pf)[KS2], const x8* pl) {
    const uint8_t* vl = vbuf + v_rd;
#pragma unroll
    for (int u = 0; u < KS2; ++u)
#pragma unroll
      for (int md = 0; md < MT2; ++md) {
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * u) * VROW + md * 64));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * u + 8) * VROW + md * 64));
        u32x4 raw;
        raw[0] = __builtin_bit_cast(u32x2, lo4)[0];
        raw[1] = __builtin_bit_cast(u32x2, lo4)[1];
        raw[2] = __builtin_bit_cast(u32x2, hi4)[0];
        raw[3] = __builtin_bit_cast(u32x2, hi4)[1];
        const x8 vfrag = __builtin_bit_cast(x8, raw);
        acc[md] = T::mfma(vfrag, pf[u], acc[md]);
        if (pl) acc[md] = T::mfma(vfrag, pl[u], acc[md]);
      }
  };
  // Register r holds key k0 + 8(r/4) + 4hh + r%4 for query q_lane.
  auto mask = [&](int j, f32x16& s) {
    const int k0 = j * BC;
    if ((k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > qw0))) {
      const int last = CAUSAL ? min(q_lane, Nk - 1) : Nk - 1;
      const int lim = last - k0 - 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > lim) s[r] = -__builtin_inff();
    }
  };
  auto rescale = [&](const f32x16& s) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(mx, s[r]);
    mx = __builtin_fmaxf(mx, other_half(mx)) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {
      const float mnew = __builtin_fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);  // 0 on the first tile
#pragma unroll
      for (int i = 0; i < MT2; ++i) acc[i] *= alpha;
      lL *= alpha;
      lO *= alpha;
      m_run = mnew;
    }
  };
  // p = exp2(s*c - m) rounded to the MFMA type; lL += sum p, lO += sum of the rounded p (with
  // pl: also lo = round(p - hi), so hi + lo carries ~16 significant bits)
  auto softmax = [&](const f32x16& s, x8 (&pf)[KS2], x8* pl) {
    const float negm = -m_run;
    float sumL = 0.f, sumO = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, negm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], c, negm));
      sumL += p0 + p1;
      const x2 pb = T::cvt2(p0, p1);
      sumO = T::dot2(pb, one2, sumO);
      const int u = r >> 3;
      pf[u][r & 7] = pb[0];
      pf[u][(r & 7) + 1] = pb[1];
      if (pl) {
        const x2 lo = T::cvt2(p0 - (float)pb[0], p1 - (float)pb[1]);
        sumO = T::dot2(lo, one2, sumO);
        pl[u][r & 7] = lo[0];
        pl[u][(r & 7) + 1] = lo[1];
      }
    }
    lL += sumL;
    lO += sumO;
  };
  // workgroup barrier after this wave's LDS accesses completed; unlike __syncthreads it
  // does not wait for the direct-to-LDS tile loads in flight (they write the other buffers)
  auto lds_barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- tile loop. Iteration j: loads of K(j+1), V(j+1) in flight; partial S of tile j;
  //      exchange; mask (diagonal/tail tiles), rescale, softmax; O += P V(j); barrier.
  auto iteration = [&](const int j, const int par, auto split_tag, auto mask_tag) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    constexpr bool MASKED = decltype(mask_tag)::value;
    if (j + 1 < ntiles) load_kv(j + 1, 1 - par);
    const bool active = !MASKED || j < wtiles;
    uint8_t* kb = par ? k_lds1 : k_lds0;
    f32x16 sc;
    if (active) gemm1(kb, sc);
    lds_barrier();  // every wave has read K(j): its buffer takes the partial scores
    if (active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 w;
        for (int e = 0; e < 4; ++e) w[e] = sc[4 * i + e];
        *(f32x4*)(kb + x_own + i * 1024) = w;
      }
    }
    lds_barrier();
    if (active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 w = *(const f32x4*)(kb + x_mate + i * 1024);
        for (int e = 0; e < 4; ++e) sc[4 * i + e] += w[e];
      }
      if (MASKED) mask(j, sc);
      rescale(sc);
      x8 pf[KS2];
      x8 pl[SPLIT ? KS2 : 1];
      softmax(sc, pf, SPLIT ? pl : nullptr);
      gemm2(par ? v_lds1 : v_lds0, pf, SPLIT ? pl : nullptr);
    }
    tile_barrier();  // the loads of this iteration have landed; LDS reads of it are done
  };
  using F = BoolC<false>;
  using U = BoolC<true>;
  load_kv(0, 0);
  tile_barrier();
  int j = 0;
  if (nfull > 0) {
    iteration(0, 0, U{}, F{});
    j = 1;
    for (; j + 1 < nfull; j += 2) {
      iteration(j, 1, F{}, F{});
      iteration(j + 1, 0, F{}, F{});
    }
    if (j < nfull) {
      iteration(j, 1, F{}, F{});
      ++j;
    }
  } else {
    iteration(0, 0, U{}, U{});
    j = 1;
  }
  for (; j < ntiles; ++j) iteration(j, j & 1, F{}, U{});

  // ---- epilogue: this wave's half of O; the LSE from the first wave of the pair. Causal: O
  //      leaves through LDS as whole half-rows (see the hd128/hd256 kernel's epilogue): wave w
  //      stages its 32 x 256 bf16 tile (16 KB) in half of K/V buffer w/2 (every wave is past
  //      the last tile's barrier), 16-byte chunk k of row r at chunk k ^ (r mod 32), and reads
  //      it back 16 bytes per lane (+1-3% at 8k-32k, +7% at 1k). Non-causal keeps direct
  //      stores: with the staging its tile loop compiled 3-6% slower at 8k-32k.
  lL += other_half(lL);
  lO += other_half(lO);
  if constexpr (!CAUSAL) {
    if (q_lane < Nq) {
      const float inv = 1.0f / lO;
      uint8_t* op = p.o + (((size_t)b * Nq + q_lane) * p.Hq + hq) * (size_t)(D * 2) + half * (DH * 2);
#pragma unroll
      for (int md = 0; md < MT2; ++md)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const x2 a = T::cvt2(acc[md][4 * i + 0] * inv, acc[md][4 * i + 1] * inv);
          const x2 bb = T::cvt2(acc[md][4 * i + 2] * inv, acc[md][4 * i + 3] * inv);
          u32x2 w;
          w[0] = __builtin_bit_cast(unsigned, a);
          w[1] = __builtin_bit_cast(unsigned, bb);
          *(u32x2*)(op + (32 * md + 8 * i + 4 * hh) * 2) = w;
        }
    }
  } else {
    constexpr int RB = DH * 2, CPL = RB / 16, RPI = 64 / CPL;  // bytes, chunks per half-row; rows per read
    static_assert(2 * 32 * RB <= C::KBUF && 2 * 32 * RB <= C::VBUF, "two staged tiles per K/V buffer");
    const int ws = __builtin_amdgcn_readfirstlane(wave), wb = ws >> 1;
    uint8_t* const ost = (wb == 0 ? k_lds0 : wb == 1 ? k_lds1 : wb == 2 ? v_lds0 : v_lds1) + (ws & 1) * (32 * RB);
    const float inv = 1.0f / lO;
#pragma unroll
    for (int md = 0; md < MT2; ++md)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const x2 a = T::cvt2(acc[md][4 * i + 0] * inv, acc[md][4 * i + 1] * inv);
        const x2 bb = T::cvt2(acc[md][4 * i + 2] * inv, acc[md][4 * i + 3] * inv);
        u32x2 w;
        w[0] = __builtin_bit_cast(unsigned, a);
        w[1] = __builtin_bit_cast(unsigned, bb);
        const int k = 4 * md + i;  // chunk of columns 32md + 8i .. +7 of this half; lane half at 8hh
        *(u32x2*)(ost + l32 * RB + ((k ^ (l32 & (CPL - 1))) * 16) + 8 * hh) = w;
      }
    const size_t o_row = (size_t)p.Hq * (D * 2);
    uint8_t* const o0 = p.o + (((size_t)b * Nq + qw0) * p.Hq + hq) * (size_t)(D * 2) + half * RB;
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int r = it * RPI + lane / CPL, ch = lane % CPL;
      const u32x4 v = *(const u32x4*)(ost + r * RB + ((ch ^ (r & (CPL - 1))) * 16));
      if (qw0 + r < Nq) *(u32x4*)(o0 + r * o_row + ch * 16) = v;
    }
  }
  if (q_lane < Nq && hh == 0 && half == 0)
    p.lse[((size_t)b * p.Hq + hq) * Nq + q_lane] = (m_run + __builtin_amdgcn_logf(lL)) * LN2;
}

}  // namespace fa
