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
//   * K/V tiles are double-buffered in LDS; rows are padded (K by 16 B, V by 64 B) so that
//     the 16-byte K reads of 16 consecutive rows and the transpose reads of V (two 16-lane
//     groups, 4 rows x 32 B each) hit distinct banks, and every LDS read address is one
//     per-lane base plus an immediate;
//   * two loop schedules (LoopMode below). PIPE (hd128): a software pipeline inside each
//     wave - while the softmax of tile j runs on the VALU, the score MFMAs of tile j+1 are
//     in flight; then the P.V MFMAs of tile j; K(j+2) and V(j+1) are loaded at the top of
//     iteration j. SEQ (hd256): one tile at a time, two workgroups per CU overlapping each
//     other, LDS fragments read four MFMAs ahead; K(j+1) and V(j+1) are loaded at the top of
//     iteration j. Tile loads are buffer loads that write LDS directly (no staging
//     registers) and whose range check returns zeros past the last key;
//   * softmax in base 2: p = exp2(s*c - m), c = scale*log2(e), on v_exp_f32;
//   * lazy rescale: the running max m (log2 units) is raised only when some row of the
//     wave sees a tile max above m + TAU; until then p <= 2^TAU;
//   * two row sums: lO = sum of the rounded P actually fed to the MFMA (normalises O, so the
//     rounding of P cancels in O = (P_b V) / sum P_b) and lL = fp32 sum of p (feeds the LSE).
//     lO is taken on the matrix cores: a 16x16x32 MFMA of a 0/1 selector and a P fragment
//     gives every lane the 16-key sum of its own row (a VALU dot per pair of p cost as
//     much as three plain VALU ops beside the MFMAs).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Lazy-rescale threshold in log2 units: p = exp2(s*c - m) stays <= 2^TAU between rescales.
constexpr float TAU = 8.0f;
// The first K/V tile of a block feeds P as hi + lo (two bf16 MFMAs, ~16 significant bits):
// for rows that see few keys the bf16 rounding of P is a visible part of the O error. In the
// hd128 loop only when some row of the block sees fewer keys than this in the block's key
// range (rows with more keys average that rounding out), and the first tile otherwise takes
// the scheduled main iteration; the hd256 loop always splits its first tile (a second
// first-tile form in that loop made it slower).
constexpr int P_SPLIT_KEYS = 512;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct Bf16 {
  using x8 = bf16x8;
  using x2 = bf16x2;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ x2 cvt2(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_convertvector(f, x2);  // one v_cvt_pk_bf16_f32, round to nearest even
  }
  static __device__ __forceinline__ f32x4 mfma16(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(x2 a, x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
  static __device__ __forceinline__ x2 ones() {
    x2 r = {(__bf16)1.0f, (__bf16)1.0f};
    return r;
  }
  static __device__ __forceinline__ x8 splat(float v) {
    const __bf16 h = (__bf16)v;
    return x8{h, h, h, h, h, h, h, h};
  }
};

struct F16 {
  using x8 = f16x8;
  using x2 = f16x2;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ x2 cvt2(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_convertvector(f, x2);
  }
  static __device__ __forceinline__ f32x4 mfma16(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(x2 a, x2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
  }
  static __device__ __forceinline__ x2 ones() {
    x2 r = {(_Float16)1.0f, (_Float16)1.0f};
    return r;
  }
  static __device__ __forceinline__ x8 splat(float v) {
    const _Float16 h = (_Float16)v;
    return x8{h, h, h, h, h, h, h, h};
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
  float c;        // |scale| * log2(e); log2(e) when zero_scores is set
  int zero_scores;  // scale is zero (or below the normal range): every score is exactly 0
  int neg_scores;   // scale < 0: Q enters with its sign flipped (exact), so c stays positive
  // variable-length batches (kernel variant VAR): packed q/o rows of sequence b are
  // cu_q[b] .. cu_q[b+1]-1; keys are packed rows cu_k[b] .. cu_k[b+1]-1 or, with a page
  // table, logical key t of sequence b is row t % page_size of page
  // block_table[b * max_pages + t / page_size]; seqused (optional for packed keys) limits
  // the keys of sequence b. Nq is then the longest query length (it sizes the grid).
  const int* cu_q;
  const int* cu_k;
  const int* seqused;
  const int* block_table;
  int total_q, total_k;
  int page_size, max_pages, num_pages;
  // split-KV (kernel variant SPLITK): the key tiles of every query tile are cut into `splits`
  // ranges of `tps` tiles; block (split s, head, query tile) writes its normalised partial
  // output to part_o [splits, B*Hq, Nq, D] and its log-sum-exp to part_lse [splits, B*Hq, Nq]
  // (fp32), which fwd_combine merges.
  float* part_o;
  float* part_lse;
  int splits, tps;
  // fp8 inputs (fwd_fp8_kernel): O is multiplied by v_scale; q and k scales are folded into c
  float v_scale;
  // grid order (a testing hook): with order_mul != 0, workgroup i works on item
  // (i * order_mul + order_add) mod n of a grid of n workgroups; the host keeps order_mul
  // coprime with n, so this permutes the items. 0: item i.
  unsigned order_mul, order_add;
};

// This workgroup's work item: blockIdx.x, or its image under the grid-order permutation. The
// branch is uniform and taken once per workgroup.
__device__ __forceinline__ int work_item(unsigned mul, unsigned add) {
  if (mul == 0) return (int)blockIdx.x;
  return (int)(((unsigned long long)blockIdx.x * mul + add) % gridDim.x);
}

template <bool V> struct BoolC { static constexpr bool value = V; };
template <int V> struct IntC { static constexpr int value = V; };

// Sign of every 16-bit element of a fragment (bf16 / fp16: bit 15) flipped where `mask` has
// it set: mask = 0x80008000 for a negative scale, else 0. Exact, so that |scale| * (-q) . k
// equals scale * q . k bit for bit and c = |scale| * log2(e) stays >= 0, which the row maximum
// relies on (max(s) * c == max(s * c)). An unconditional xor with a uniform mask: a
// conditional flip made the compiler spill Q fragments and reload them inside the tile loop.
template <class X8>
__device__ __forceinline__ X8 sign16(X8 x, unsigned mask) {
  u32x4 u = __builtin_bit_cast(u32x4, x);
  u ^= mask;
  return __builtin_bit_cast(X8, u);
}

// Barrier that publishes K/V tiles loaded straight into LDS: each wave first waits for its own
// buffer loads (vmcnt), then the workgroup meets. The compiler inserts that wait only where the
// same wave reads the data afterwards (gfx950 barriers do not wait by themselves), while every
// wave's share of a tile is read by all waves: only this order makes the whole tile visible.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Lane l and lane l^32 hold the same query row: the value of the other half.
__device__ __forceinline__ float other_half(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  // v_permlane32_swap: r[0] = lanes 0-31 of x in both halves, r[1] = lanes 32-63 of x
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (__lane_id() >> 5) ? r[0] : r[1]);
}

// Block id -> (b*Hq + h, query tile). Workgroups are dispatched round-robin over the 8
// XCDs (bid % 8). Dense batches (all heads carry equal work): when B*Hq is a multiple of 8,
// each XCD gets a contiguous set of heads, so the query heads of a GQA group and all query
// tiles of a head share one XCD's L2 for their K/V. Variable-length batches (SPREAD): head
// bh = bid % (B*Hq), so the heads of one sequence go to different XCDs (a long sequence
// would otherwise occupy one XCD only) while each head keeps one XCD when B*Hq % 8 == 0.
// LONGEST_FIRST (causal, and every variable-length batch, where a high query tile exists
// only in long sequences): highest query tile first.
template <bool LONGEST_FIRST, bool SPREAD>
__device__ __forceinline__ void decode_block(int bid, const FwdParams& p, int& bh, int& qt) {
  const int BH = p.B * p.Hq;
  if (!SPREAD && (BH & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3, hpx = BH >> 3;
    if (LONGEST_FIRST) {
      qt = p.nqt - 1 - slot / hpx;
      bh = xcd * hpx + slot % hpx;
    } else {
      bh = xcd * hpx + slot / p.nqt;
      qt = slot % p.nqt;
    }
  } else {
    if (LONGEST_FIRST) {
      qt = p.nqt - 1 - bid / BH;
      bh = bid % BH;
    } else {
      bh = bid / p.nqt;
      qt = bid % p.nqt;
    }
  }
}

// Variable-length / paged batches of at most 64 sequences go sequence by sequence, longest
// first: lane l of every wave reads sequence l's lengths, ranks the sequences by key count
// (ties by index), and the block's entry e = bid / Hq is found in the ranked prefix sums of the
// query-tile counts. The Hq heads of an entry are consecutive block ids, so head h of all query
// tiles of a sequence lands on one XCD (bid % 8) close together in time and shares its L2 for
// that head's K/V; with Hq a multiple of 8 the heads on one XCD are a contiguous (GQA) range.
// Non-causal, every query tile of a sequence costs the same, and this is the
// longest-processing-time order over the CUs (the order above, highest query tile first, left
// the query tiles 0.. of the longest sequences for the last round). Causal, a sequence's query
// tiles go highest first (the longest blocks of the sequence first).
// Returns false when the block has no entry (the grid is sized for max_seqlen_q).
template <int BR, int BC, bool CAUSAL>
__device__ __forceinline__ bool decode_block_lpt(int bid, const FwdParams& p, int& bh, int& qt) {
  const int l = threadIdx.x & 63;
  int nt = 0, key = -1;
  if (l < p.B) {
    const int q0 = min(max(p.cu_q[l], 0), p.total_q);
    const int q1 = min(max(p.cu_q[l + 1], q0), p.total_q);
    int nk;
    if (p.block_table == nullptr) {
      const int k0 = min(max(p.cu_k[l], 0), p.total_k);
      nk = min(max(p.cu_k[l + 1], k0), p.total_k) - k0;
    } else {
      nk = p.max_pages * p.page_size;
    }
    if (p.seqused != nullptr) nk = min(nk, max(p.seqused[l], 0));
    nt = (q1 - q0 + BR - 1) / BR;
    key = (nk + BC - 1) / BC;
  }
  int rank = 0;
  for (int i = 0; i < p.B; ++i) {
    const int ki = __builtin_amdgcn_readlane(key, i);
    rank += (ki > key || (ki == key && i < l)) ? 1 : 0;
  }
  int start = 0;
  for (int i = 0; i < p.B; ++i) {
    const int ri = __builtin_amdgcn_readlane(rank, i);
    const int ti = __builtin_amdgcn_readlane(nt, i);
    start += ri < rank ? ti : 0;
  }
  const int e = bid / p.Hq, hslot = bid - e * p.Hq;
  const unsigned long long hit = __builtin_amdgcn_ballot_w64(l < p.B && e >= start && e < start + nt);
  if (hit == 0) return false;
  const int b = __builtin_ctzll(hit);
  qt = e - __builtin_amdgcn_readlane(start, b);
  if (CAUSAL) qt = __builtin_amdgcn_readlane(nt, b) - 1 - qt;
  const int h = (p.Hq & 7) == 0 ? (hslot & 7) * (p.Hq >> 3) + (hslot >> 3) : hslot;
  bh = b * p.Hq + h;
  return true;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base, uint32_t bytes) {
  // raw buffer (stride 0): a load whose offset lies past `bytes` returns zeros
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// Tile configuration per head dim: waves per workgroup, keys per K/V tile.
template <int D> struct TileCfg;
// Loop schedules (MODE):
//   PIPE: the scores of the next tile are computed during the softmax of the current one,
//         with an explicit MFMA/VALU interleave inside each wave (one workgroup per CU);
//   SEQ:  one score buffer and a plain per-tile order; two workgroups share a CU and their
//         waves overlap each other (hd256: O alone takes half of a wave's 256 registers, so
//         a second score buffer does not fit at two waves per SIMD).
// WPE: waves per SIMD the register budget is sized for.
enum LoopMode { PIPE = 0, SEQ = 1 };
template <> struct TileCfg<128> { static constexpr int NW = 8, BC = 64, WPE = 2, MODE = PIPE; };
template <> struct TileCfg<256> { static constexpr int NW = 4, BC = 32, WPE = 2, MODE = SEQ; };

// WV: waves per workgroup. hd128 has two forms: 8 waves (256 query rows, one workgroup per
// CU) and 4 waves (128 rows, two workgroups per CU) for grids that do not fill the GPU twice
// over, where twice the workgroups and one workgroup's prologue hidden under the other's
// tiles outweigh the second K/V stream per CU.
template <int D, int WV = TileCfg<D>::NW>
struct Layout {
  static constexpr int NW = WV, BC = TileCfg<D>::BC;
  static constexpr int BR = NW * 32;           // query rows per workgroup
  static constexpr int KROW = D * 2 + 16;      // padded LDS row pitch of K (bytes)
  static constexpr int VROW = D * 2 + 64;      // padded LDS row pitch of V (bytes)
  static constexpr int KT = BC * KROW;         // bytes per K tile
  static constexpr int VT = BC * VROW;         // bytes per V tile
  // A tile is written by 64-slot (1 KB) direct-to-LDS loads spread evenly over the NL
  // loading waves, waves LB .. LB + NL - 1; each buffer is rounded up so that every loading
  // wave issues the same number of whole loads (the slots past the tile receive zeros).
  // hd128 with 8 waves: the four younger waves load (5 loads each per tile and buffers of
  // 20 KB, against 3 per wave for all eight and 24 KB buffers); they are the ones that lag at
  // the tile barriers, and the loads at the top of an iteration let the older waves run on.
  // With 4 waves all of them load (two loading waves were 20-40% slower on causal shapes).
  static constexpr int NL = D == 128 && NW == 8 ? NW / 2 : NW;
  static constexpr int LB = NW - NL;
  static constexpr int KPW = (KT / 16 + 64 * NL - 1) / (64 * NL);  // K loads per loading wave
  static constexpr int VPW = (VT / 16 + 64 * NL - 1) / (64 * NL);  // V loads per loading wave
  static constexpr int KBUF = KPW * NL * 1024, VBUF = VPW * NL * 1024;
  static constexpr int LDS = 2 * KBUF + 2 * VBUF;  // two K and two V buffers
};

// VM: 0 dense batch, 1 variable-length batch (packed or paged K/V), 2 dense batch with the
// key range of each query tile split over several blocks (split-KV), 3 variable-length batch
// with split-KV (every sequence's key tiles cut into chunks of tps tiles).
template <int D, bool CAUSAL, class T, int VM, int WV = TileCfg<D>::NW>
__global__ void __launch_bounds__(WV * 64, TileCfg<D>::WPE)
fwd_kernel(FwdParams p) {
  constexpr bool VAR = VM == 1 || VM == 3, SPLITK = VM == 2 || VM == 3;
  using x8 = typename T::x8;
  using x2 = typename T::x2;
  using L = Layout<D, WV>;
  constexpr int NW = L::NW, BC = L::BC, BR = L::BR;
  constexpr int NT = NW * 64;
  constexpr int KS1 = D / 16;       // GEMM1 k-steps (over head dim)
  constexpr int MT1 = BC / 32;      // score tiles (32 keys each) per K/V tile
  constexpr int MT2 = D / 32;       // output tiles (32 head-dim rows each)
  constexpr int KS2 = BC / 16;      // GEMM2 k-steps (over keys)
  constexpr int CPR = D / 8;        // 16-byte chunks per K/V row
  constexpr int KROW = L::KROW, VROW = L::VROW, KT = L::KT, VT = L::VT;
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");

  // Two K and two V tile buffers as separate LDS objects: the loop's buffer parity is a
  // compile-time value, so the compiler can see that the direct-to-LDS loads of the next
  // tiles never touch the buffers being read and does not wait for them early. The compiler
  // lays the objects out in the order of their names; the V buffers come first so that every
  // V transpose read (the most frequent LDS read) is a base register plus an immediate below
  // 64 KB, with no address add in the loop (hd128: -17 VALU ops per tile, +1.5-4%).
  __shared__ __attribute__((aligned(16))) uint8_t lds0_v[L::VBUF], lds1_v[L::VBUF], lds2_k[L::KBUF],
      lds3_k[L::KBUF];
  uint8_t* const v_lds0 = lds0_v;
  uint8_t* const v_lds1 = lds1_v;
  uint8_t* const k_lds0 = lds2_k;
  uint8_t* const k_lds1 = lds3_k;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int bh, qt, split = 0;
  const int bid = work_item(p.order_mul, p.order_add);
  if constexpr (SPLITK) {
    // all blocks of split 0 first, then split 1, ...; within a split the order without splits
    const int per = p.B * p.Hq * p.nqt;
    split = bid / per;
    decode_block<CAUSAL || VAR, VAR>(bid - split * per, p, bh, qt);
  } else if constexpr (VAR) {
    if (p.B <= 64) {
      if (!decode_block_lpt<L::BR, L::BC, CAUSAL>(bid, p, bh, qt)) return;
    } else {
      decode_block<true, true>(bid, p, bh, qt);
    }
  } else {
    decode_block<CAUSAL || VAR, VAR>(bid, p, bh, qt);
  }
  const int b = bh / p.Hq;
  const int hq = bh - b * p.Hq;
  const int kvh = hq / p.group;

  // ---- this block's sequence: query rows q_row0 .. q_row0 + Nq - 1 of the q/o tensors and
  //      Nk keys. Dense: sequence b of a [B, Nq, H, d] batch. VAR: packed rows (bounds are
  //      clamped to the tensors, so bad offsets cannot reach outside them). Causal: query i
  //      sees keys j <= i + cshift, aligned bottom-right (cshift = 0 when Nq == Nk).
  int Nq, Nk;
  size_t q_row0, lse0;  // first q/o row; LSE index of (this head, row 0)
  const uint8_t* kbase;
  const uint8_t* vbase;
  const size_t head_off = (size_t)kvh * (D * 2);
  if constexpr (!VAR) {
    Nq = p.Nq;
    Nk = p.Nk;
    q_row0 = (size_t)b * Nq;
    lse0 = ((size_t)b * p.Hq + hq) * Nq;
    kbase = p.k + (size_t)b * Nk * p.Hkv * (D * 2) + head_off;
    vbase = p.v + (size_t)b * Nk * p.Hkv * (D * 2) + head_off;
  } else {
    const int q0 = min(max(p.cu_q[b], 0), p.total_q);
    const int q1 = min(max(p.cu_q[b + 1], q0), p.total_q);
    Nq = q1 - q0;
    q_row0 = q0;
    lse0 = (size_t)hq * p.total_q + q0;
    if (p.block_table == nullptr) {
      const int k0 = min(max(p.cu_k[b], 0), p.total_k);
      const int k1 = min(max(p.cu_k[b + 1], k0), p.total_k);
      Nk = k1 - k0;
      kbase = p.k + (size_t)k0 * p.Hkv * (D * 2) + head_off;
      vbase = p.v + (size_t)k0 * p.Hkv * (D * 2) + head_off;
    } else {
      Nk = p.max_pages * p.page_size;  // page bases are added per tile
      kbase = p.k + head_off;
      vbase = p.v + head_off;
    }
    if (p.seqused != nullptr) Nk = min(Nk, max(p.seqused[b], 0));
  }
  const int cshift = CAUSAL ? Nk - Nq : 0;

  const int q_wg0 = qt * BR;
  if (VAR && q_wg0 >= Nq) return;  // a query tile past the end of this sequence
  const int qw0 = q_wg0 + wave * 32;
  const int q_lane = qw0 + l32;
  const int q_ld = q_lane < Nq ? q_lane : Nq - 1;

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(Nq, q_wg0 + BR) + cshift);
  // Key tiles t0 .. t0 + ntiles - 1 are this block's (split-KV: one range of tps tiles; else
  // all). Loop indices below are relative to t0. Tiles below nfull are visible to every query
  // of the block; a wave computes on its first wtiles tiles (causal: keys up to its last
  // query; a wave whose rows see no key of the range has none).
  const int ntiles_all = (kend + BC - 1) / BC;
  const int wtiles_all =
      CAUSAL ? max(VAR || SPLITK ? 0 : 1, min(ntiles_all, (min(qw0 + 32, Nq) + cshift + BC - 1) / BC))
             : ntiles_all;
  int nfull_all = Nk / BC;
  if (CAUSAL) nfull_all = max(0, min(nfull_all, (q_wg0 + 1 + cshift) / BC));
  const int t0 = SPLITK ? split * p.tps : 0;
  const int t1 = SPLITK ? min(ntiles_all, t0 + p.tps) : ntiles_all;
  const int ntiles = max(0, t1 - t0);
  const int wtiles = max(0, min(wtiles_all, t1) - t0);
  const int nfull = max(0, min(nfull_all, t1) - t0);
  const int kfirst = t0 * BC;  // first key of the range
  // fewest keys a row of this block sees in the range: below P_SPLIT_KEYS the first tile of
  // the hd128 loop feeds P as hi + lo
  const bool split_first = min(CAUSAL ? min(Nk, q_wg0 + cshift + 1) : Nk, t1 * BC) - kfirst < P_SPLIT_KEYS;
  // row of (split, this head, query q_lane) in the split-KV partials: dense [splits, B*Hq, Nq],
  // variable-length [splits, Hq, total_q] (packed query rows)
  auto part_row = [&](int ql) -> size_t {
    return VAR ? ((size_t)split * p.Hq + hq) * p.total_q + q_row0 + ql
               : ((size_t)split * p.B * p.Hq + bh) * Nq + ql;
  };
  if (SPLITK && (ntiles == 0 || (VAR && kend <= 0))) {  // no key of this split: empty partial
    if (q_lane < Nq) {
      const size_t row = part_row(q_lane);
      float* po = p.part_o + row * D;
#pragma unroll
      for (int md = 0; md < MT2; ++md)
#pragma unroll
        for (int i = 0; i < 4; ++i) *(f32x4*)(po + 32 * md + 8 * i + 4 * hh) = f32x4{};
      if (hh == 0) p.part_lse[row] = -__builtin_inff();
    }
    return;
  }
  if (VAR && kend <= 0) {  // no row of this block sees a key: O = 0, LSE = -inf
    if (q_lane < Nq) {
      uint8_t* op = p.o + ((q_row0 + q_lane) * p.Hq + hq) * (size_t)(D * 2);
#pragma unroll
      for (int md = 0; md < MT2; ++md)
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x2*)(op + (32 * md + 8 * i + 4 * hh) * 2) = u32x2{0u, 0u};
      if (hh == 0) p.lse[lse0 + q_lane] = -__builtin_inff();
    }
    return;
  }

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query q_ld, dims 16t + 8hh .. +7
  x8 qf[KS1];
  {
    const uint8_t* qp = p.q + ((q_row0 + q_ld) * p.Hq + hq) * (size_t)(D * 2);
#pragma unroll
    for (int t = 0; t < KS1; ++t) {
      u32x4 raw = *(const u32x4*)(qp + (16 * t + 8 * hh) * 2);
      qf[t] = __builtin_bit_cast(x8, raw);
    }
    // zero scale: zero Q (and a unit c), so that masked scores stay -inf instead of -inf * 0;
    // negative scale: -Q with c = |scale| * log2(e)
    if (p.zero_scores) {
#pragma unroll
      for (int t = 0; t < KS1; ++t) qf[t] = x8{};
    }
    const unsigned sgn = p.neg_scores ? 0x80008000u : 0u;
#pragma unroll
    for (int t = 0; t < KS1; ++t) qf[t] = sign16(qf[t], sgn);
  }

  f32x16 acc[MT2];
#pragma unroll
  for (int i = 0; i < MT2; ++i) acc[i] = f32x16{};
  float m_run = -__builtin_inff();
  float lL = 0.f, lO = 0.f;
  // PIPE (hd128) takes lO on the matrix cores; SEQ (hd256) has no registers to spare for the
  // selector and the accumulator and keeps a VALU dot per pair (per lane half, into lO).
  constexpr bool MMA_ROWSUM = TileCfg<D>::MODE == PIPE;
  const x2 one2 = T::ones();
  // lO4 accumulates sel x P fragment (16x16x32 MFMA). B = a P fragment read as 16 columns x
  // 32 k: lanes 16g..16g+15 hold rows 16(g&1)..+15 of the 32-row block, key half g>>1 of the
  // 16-key step. A (row i = lane%16, k-slice g = lane/16) is 1 where g&1 == (i>>2)&1, so
  // output rows 0-3 and 8-11 sum the rows 0-15 of the block and rows 4-7 and 12-15 the rows
  // 16-31; output lane l holds rows 4(l/16)..+3 of column l%16, which is then the sum over
  // all 16 keys of row l%32 - the row the lane owns - in each of its four registers.
  f32x4 lO4 = {};
  const int sel_lane = threadIdx.x & 63;
  const x8 sel = T::splat((((sel_lane >> 4) & 1) == ((sel_lane >> 2) & 1)) ? 1.f : 0.f);
  const float c = p.c;

  // ---- K/V tiles: buffer loads straight into LDS (buffer_load ... lds). One instruction
  //      of a wave fills 64 consecutive 16-byte LDS slots (M0 base + 16 * lane); a padded row
  //      is KROW/16 (VROW/16) slots, so each lane maps its slot to (row, chunk) once, here.
  //      Pad slots, rows past the last key and slots past the tile (in the buffer's rounding)
  //      get an offset beyond the buffer's range, which loads zeros. Every offset is in the
  //      per-lane voffset, which is what the hardware range check covers.
  constexpr int KSL = KROW / 16, VSL = VROW / 16;  // slots per padded row
  constexpr int NL = L::NL, KPW = L::KPW, VPW = L::VPW;  // loading waves, loads per wave and tile
  constexpr uint32_t OOB = 0x80000000u;
  const uint32_t kv_row = (uint32_t)p.Hkv * D * 2;  // bytes between consecutive tokens
  const int wv = __builtin_amdgcn_readfirstlane(wave) - L::LB;  // index among the loading waves
  uint32_t k_vo[KPW], v_vo[VPW];
#pragma unroll
  for (int n = 0; n < KPW; ++n) {
    const int slot = 64 * (wv + NL * n) + lane, row = slot / KSL, ch = slot % KSL;
    k_vo[n] = (ch < CPR && row < BC) ? (uint32_t)row * kv_row + ch * 16 : OOB;
  }
#pragma unroll
  for (int n = 0; n < VPW; ++n) {
    const int slot = 64 * (wv + NL * n) + lane, row = slot / VSL, ch = slot % VSL;
    v_vo[n] = (ch < CPR && row < BC) ? (uint32_t)row * kv_row + ch * 16 : OOB;
  }

  auto load_tile = [&](int tile, const uint8_t* gbase, uint8_t* ldst, const uint32_t* vo,
                       auto nw_tag) {
    constexpr int NPW = decltype(nw_tag)::value;
    if (NL < NW && (wv < 0 || wv >= NL)) return;  // not a loading wave
    const int k0 = (t0 + tile) * BC;
    const uint8_t* tbase = gbase + (size_t)k0 * kv_row;
    int rows = min(BC, Nk - k0);
    if constexpr (VAR) {
      if (p.block_table != nullptr) {  // a tile lies inside one page (page_size % BC == 0)
        const int lp = k0 / p.page_size;
        const int pg = p.block_table[(size_t)b * p.max_pages + lp];
        tbase = gbase + ((size_t)pg * p.page_size + (k0 - lp * p.page_size)) * kv_row;
        if (pg < 0 || pg >= p.num_pages) rows = 0;  // not a page of the cache: zeros, no access
      }
    }
    const auto rs = make_rsrc(tbase, (uint32_t)rows * kv_row);
#pragma unroll
    for (int n = 0; n < NPW; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(ldst + 1024 * (wv + NL * n)), 16, vo[n], 0, 0, 0);
  };
  // `buf` is a literal in the main loop (so buffer addresses are constants) and j & 1 in the
  // diagonal/tail iterations.
  auto load_k = [&](int tile, int buf) {
    load_tile(tile, kbase, buf ? k_lds1 : k_lds0, k_vo, IntC<KPW>{});
  };
  auto load_v = [&](int tile, int buf) {
    load_tile(tile, vbase, buf ? v_lds1 : v_lds0, v_vo, IntC<VPW>{});
  };

  // ---- per-lane LDS read bases
  // GEMM1 A operand (K): lane reads row 32mt + l32, dims 16t + 8hh .. +7
  const int k_rd = l32 * KROW + hh * 16;
  // GEMM2 A operand (V^T) via ds_read_b64_tr_b16: k-step u covers keys
  // 16u + {4g + 0..3, 8 + 4g + 0..3}, g = (lane group) / 2, which is the order P^T holds
  // them in; lane i of a 16-lane group reads row key0 + i/4, dims d0 + 4(i%4) .. +3, and
  // lane c of the group receives V[key0 + 0..3][d0 + c].
  const int grp = lane >> 4, gi = lane & 15;
  const int v_rd = (4 * (grp >> 1) + (gi >> 2)) * VROW + (2 * (grp & 1) + ((gi & 3) >> 1)) * 16 + (gi & 1) * 8;

  // GEMM1 walks the head dim with its score tiles innermost, GEMM2 the keys with its output
  // tiles innermost (a dependent MFMA chain issues at nearly full rate on gfx950, so a single
  // score tile needs no split accumulator).
  // SEQ: LDS fragments are read SPF MFMAs ahead in a fixed order (sched_barrier), so that the
  // read latency hides under the MFMAs before them; left to itself the compiler read them one
  // or two MFMAs ahead.
  // (variable-length causal: 3 ahead; at 4 that kernel spilled and reloaded inside the loop,
  // -8 to -12%; the dense causal kernel is faster at 4)
  constexpr int SPF1 = VAR && CAUSAL ? 3 : 4, SPF2 = VAR && CAUSAL ? 3 : 4;
  auto gemm1 = [&](int buf, f32x16 (&s)[MT1]) {
    const uint8_t* kl = (buf ? k_lds1 : k_lds0) + k_rd;
    if constexpr (TileCfg<D>::MODE == SEQ) {
      constexpr int N = KS1 * MT1;
      auto frag = [&](const int i) -> x8 {
        const int t = i / MT1, mt = i % MT1;
        return __builtin_bit_cast(x8, *(const u32x4*)(kl + mt * 32 * KROW + t * 32));
      };
      x8 kf[N];
#pragma unroll
      for (int i = 0; i < SPF1; ++i) kf[i] = frag(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i + SPF1 < N) kf[i + SPF1] = frag(i + SPF1);
        const int t = i / MT1, mt = i % MT1;
        s[mt] = T::mfma(kf[i], qf[t], t == 0 ? f32x16{} : s[mt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt) s[mt] = f32x16{};
#pragma unroll
    for (int t = 0; t < KS1; ++t)
#pragma unroll
      for (int mt = 0; mt < MT1; ++mt) {
        u32x4 raw = *(const u32x4*)(kl + mt * 32 * KROW + t * 32);
        s[mt] = T::mfma(__builtin_bit_cast(x8, raw), qf[t], s[mt]);
      }
  };

  // V^T fragment i of GEMM2 (k-step i / MT2, output tile i % MT2) from V buffer `buf`
  auto vfrag = [&](int buf, const int i) -> x8 {
    const uint8_t* vl = (buf ? v_lds1 : v_lds0) + v_rd;
    const int u = i / MT2, md = i % MT2;
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * u) * VROW + md * 64));
    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * u + 8) * VROW + md * 64));
    u32x4 raw;
    raw[0] = __builtin_bit_cast(u32x2, lo4)[0];
    raw[1] = __builtin_bit_cast(u32x2, lo4)[1];
    raw[2] = __builtin_bit_cast(u32x2, hi4)[0];
    raw[3] = __builtin_bit_cast(u32x2, hi4)[1];
    return __builtin_bit_cast(x8, raw);
  };
  auto gemm2 = [&](int buf, const x8 (&pf)[KS2], const x8* pl) {
    const uint8_t* vl = (buf ? v_lds1 : v_lds0) + v_rd;
    if constexpr (TileCfg<D>::MODE == SEQ) {
      constexpr int N = KS2 * MT2;
      auto frag = [&](const int i) -> x8 { return vfrag(buf, i); };
      x8 vf[N];
#pragma unroll
      for (int i = 0; i < SPF2; ++i) vf[i] = frag(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i + SPF2 < N) vf[i + SPF2] = frag(i + SPF2);
        const int u = i / MT2, md = i % MT2;
        acc[md] = T::mfma(vf[i], pf[u], acc[md]);
        if (pl) acc[md] = T::mfma(vf[i], pl[u], acc[md]);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < KS2; ++u)
#pragma unroll
      for (int md = 0; md < MT2; ++md) {
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vl + (16 * u) * VROW + md * 64));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vl + (16 * u + 8) * VROW + md * 64));
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

  // Mask scores of tile j: causal (key > query) and tail (key >= Nk). Register r of score
  // tile mt holds key k0 + 32mt + 8(r/4) + 4hh + r%4 for the lane's query q_lane, so a key
  // is visible iff its compile-time offset 32mt + 8(r/4) + r%4 is <= one per-lane limit.
  auto mask = [&](int j, f32x16 (&s)[MT1]) {
    const int k0 = (t0 + j) * BC;
    const bool need = (k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > qw0 + cshift));
    if (need) {
      const int last = CAUSAL ? min(q_lane + cshift, Nk - 1) : Nk - 1;  // last visible key
      const int lim = last - k0 - 4 * hh;
#pragma unroll
      for (int mt = 0; mt < MT1; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * mt + 8 * (r >> 2) + (r & 3) > lim) s[mt][r] = -__builtin_inff();
    }
  };

  // Row max of a tile in log2 units (c >= 0 always: a negative scale flips the sign of Q
  // instead, so max(s)*c == max(s*c)), over both lane halves.
  auto rowmax = [&](const f32x16 (&s)[MT1]) -> float {
    float mx = s[0][0];
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[mt][r]);
    mx = __builtin_fmaxf(mx, other_half(mx));
    return mx * c;
  };
  // Lazy rescale of O and the sums, decided per wave: only when some row's tile max exceeds
  // its running max by more than TAU.
  auto rescale_to = [&](const float mtile) {
    const bool grow = mtile > m_run + TAU;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = __builtin_fmaxf(m_run, mtile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);  // 0 on the first tile
#pragma unroll
      for (int i = 0; i < MT2; ++i) acc[i] *= alpha;
      lL *= alpha;
      if constexpr (MMA_ROWSUM)
        lO4 *= alpha;
      else
        lO *= alpha;
      m_run = mnew;
    }
  };

  // p = exp2(s*c - m), rounded to the MFMA type; lL += sum p (fp32), lO += sum of rounded p.
  // With pl, also lo = round(p - hi), so hi + lo carries ~16 significant bits.
  auto softmax = [&](const f32x16 (&s)[MT1], x8 (&pf)[KS2], x8* pl) {
    // With the row-sum MFMA, a row that sees no key so far (m = -inf, all scores -inf) gets
    // p = 0, not NaN: that MFMA reads two rows through one B column, and 0 * NaN would reach
    // the other. (The per-lane dots keep such a NaN in its own row, which is then stored as
    // empty: O = 0, LSE = -inf.)
    const float negm = MMA_ROWSUM && m_run == -__builtin_inff() ? 0.f : -m_run;
    float sumL = 0.f, sumO = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][r], c, negm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][r + 1], c, negm));
        sumL += p0 + p1;
        const x2 pb = T::cvt2(p0, p1);
        if constexpr (!MMA_ROWSUM) sumO = T::dot2(pb, one2, sumO);
        const int u = mt * 2 + (r >> 3);
        pf[u][(r & 7)] = pb[0];
        pf[u][(r & 7) + 1] = pb[1];
        if (pl) {
          const x2 lo = T::cvt2(p0 - (float)pb[0], p1 - (float)pb[1]);
          if constexpr (!MMA_ROWSUM) sumO = T::dot2(lo, one2, sumO);
          pl[u][(r & 7)] = lo[0];
          pl[u][(r & 7) + 1] = lo[1];
        }
      }
    lL += sumL;
    if constexpr (MMA_ROWSUM) {
#pragma unroll
      for (int u = 0; u < KS2; ++u) {
        lO4 = T::mfma16(sel, pf[u], lO4);
        if (pl) lO4 = T::mfma16(sel, pl[u], lO4);
      }
    } else {
      lO += sumO;
    }
  };

  if constexpr (TileCfg<D>::MODE == SEQ) {
  // ---- sequential tile loop. Iteration j: loads of K(j+1), V(j+1) in flight; S = Q K(j)^T;
  //      mask (diagonal/tail tiles); rescale; softmax; O += P V(j); barrier.
  auto seq_iteration = [&](const int j, const int par, auto split_tag, auto mask_tag) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    constexpr bool MASKED = decltype(mask_tag)::value;
    if (j + 1 < ntiles) {
      load_k(j + 1, 1 - par);
      load_v(j + 1, 1 - par);
    }
    if (!MASKED || j < wtiles) {
      f32x16 sc[MT1];
      gemm1(par, sc);
      if (MASKED) mask(j, sc);
      rescale_to(rowmax(sc));
      x8 pf[KS2];
      x8 pl[SPLIT ? KS2 : 1];
      softmax(sc, pf, SPLIT ? pl : nullptr);
      gemm2(par, pf, SPLIT ? pl : nullptr);
    }
    tile_barrier();  // the loads of this iteration have landed; LDS reads of it are done
  };
  using F = BoolC<false>;
  using U = BoolC<true>;
  load_k(0, 0);
  load_v(0, 0);
  tile_barrier();
  int j = 0;
  if (nfull > 0) {
    seq_iteration(0, 0, U{}, F{});
    j = 1;
    for (; j + 1 < nfull; j += 2) {
      seq_iteration(j, 1, F{}, F{});
      seq_iteration(j + 1, 0, F{}, F{});
    }
    if (j < nfull) {
      seq_iteration(j, 1, F{}, F{});
      ++j;
    }
  } else {
    seq_iteration(0, 0, U{}, U{});
    j = 1;
  }
  for (; j < ntiles; ++j) seq_iteration(j, j & 1, F{}, U{});
  } else {
  // ---- prologue: K(0), V(0), K(1) into LDS, scores of tile 0
  load_k(0, 0);
  load_v(0, 0);
  if (ntiles > 1) load_k(1, 1);
  tile_barrier();  // waits for the loads (vmcnt) before the barrier

  f32x16 s_a[MT1], s_b[MT1];
  gemm1(0, s_a);
  tile_barrier();  // every wave has read K(0) before iteration 0 reloads its buffer

  // ---- tile loop. Iteration j: loads of K(j+2), V(j+1) in flight; softmax(j) with the
  //      MFMAs of GEMM1(j+1); GEMM2(j); barrier. Scores of tile j are in `sc`, those of
  //      tile j+1 go to `sn`.
  //      Tiles below `nfull` are visible to every query of the workgroup and inside Nk, so
  //      their iterations carry no masking code; the rest (diagonal and tail tiles) mask,
  //      and a wave whose queries all precede a tile skips that tile's math.
  // main iterations: unmasked and followed by a next tile
  const int nmain = min(nfull, ntiles - 1);

  // Scaled row max of the scores of the next tile, computed at the end of each iteration
  // for the main iterations (whose tiles need no mask).
  float mt_cur = 0.f;

  // Generic iteration (first tile, diagonal and tail tiles): straightforward order.
  auto iteration = [&](const int j, f32x16 (&sc)[MT1], f32x16 (&sn)[MT1], auto split_tag,
                       auto mask_tag) {
    constexpr bool SPLIT = decltype(split_tag)::value;
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
      x8 pf[KS2];
      x8 pl[SPLIT ? KS2 : 1];
      if (next_active) gemm1(1 - par, sn);
      softmax(sc, pf, SPLIT ? pl : nullptr);
      gemm2(par, pf, SPLIT ? pl : nullptr);
      if (next_active) mt_cur = rowmax(sn);
    }
    tile_barrier();  // the loads of this iteration have landed; LDS reads of it are done
  };

  // Main iteration (unmasked tile j, tile j+1 exists), with an explicit instruction order:
  //   phase 1: each GEMM1(j+1) MFMA is issued with the LDS read PF steps ahead and with one
  //            slice of the softmax VALU work of tile j (fma, exp and pack of a pair);
  //            the last steps start reading the V fragments of GEMM2;
  //   phase 2: each GEMM2(j) MFMA with the V read PF steps ahead, one slice of the fp32 row
  //            sum of tile j and of the row max of tile j+1 (which the next iteration's
  //            rescale decision needs); after the last MFMA of each 16-key step, the row-sum
  //            MFMA of that step's rounded P.
  // sched_barrier fences keep each step's instructions together.
  constexpr int PF = D == 256 ? 2 : 4;  // LDS fragment reads issued this many MFMAs ahead
  constexpr int N1 = MT1 * KS1, N2 = MT2 * KS2;
  constexpr int NPAIR = 8 * MT1;  // score pairs per lane per tile
  auto main_iteration = [&](const int j, f32x16 (&sc)[MT1], f32x16 (&sn)[MT1], auto par_tag) {
    constexpr int PAR = decltype(par_tag)::value;  // j & 1
    if (j + 2 < ntiles) load_k(j + 2, PAR);
    load_v(j + 1, 1 - PAR);
    rescale_to(mt_cur);
    const float negm = -m_run;
    const uint8_t* kl = (PAR ? k_lds0 : k_lds1) + k_rd;  // K(j+1): buffer 1 - PAR
    const uint8_t* vl = (PAR ? v_lds1 : v_lds0) + v_rd;  // V(j): buffer PAR
    auto kfrag = [&](const int i) -> x8 {
      const int t = i / MT1, mt = i % MT1;
      return __builtin_bit_cast(x8, *(const u32x4*)(kl + mt * 32 * KROW + t * 32));
    };
    auto vfrag = [&](const int i) -> x8 {
      const int u = i / MT2, md = i % MT2;
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * u) * VROW + md * 64));
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * u + 8) * VROW + md * 64));
      u32x4 raw;
      raw[0] = __builtin_bit_cast(u32x2, lo4)[0];
      raw[1] = __builtin_bit_cast(u32x2, lo4)[1];
      raw[2] = __builtin_bit_cast(u32x2, hi4)[0];
      raw[3] = __builtin_bit_cast(u32x2, hi4)[1];
      return __builtin_bit_cast(x8, raw);
    };
    x8 kf[N1], vf[N2], pf[KS2];
    float sumL0 = 0.f, sumL1 = 0.f;
#pragma unroll
    for (int i = 0; i < PF; ++i) kf[i] = kfrag(i);
    __builtin_amdgcn_sched_barrier(0);
    // Wave priority by progress: the two waves that share a SIMD meet at every tile barrier,
    // and the issue arbiter otherwise favours the older one, which then waits at the barrier
    // while the younger finishes alone. A wave in phase 1 outranks one already in phase 2.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < N1; ++i) {
      if (i + PF < N1)
        kf[i + PF] = kfrag(i + PF);
      else
        vf[i + PF - N1] = vfrag(i + PF - N1);
      {
        const int t = i / MT1, mt = i % MT1;
        sn[mt] = T::mfma(kf[i], qf[t], t == 0 ? f32x16{} : sn[mt]);
      }
      if ((i * NPAIR) % N1 == 0) {
        // softmax of one pair: p overwrites its score (the sums are taken in phase 2)
        const int pi = i * NPAIR / N1, mt = pi / 8, r = (pi % 8) * 2;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mt][r], c, negm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mt][r + 1], c, negm));
        sc[mt][r] = p0;
        sc[mt][r + 1] = p1;
        const x2 pb = T::cvt2(p0, p1);
        const int u = mt * 2 + (r >> 3);
        pf[u][(r & 7)] = pb[0];
        pf[u][(r & 7) + 1] = pb[1];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float mx = -__builtin_inff();
    constexpr int VPS = (16 * MT1) / N2;  // p values summed (and next-tile scores maxed) per step
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < N2; ++i) {
      if (i + PF < N2) vf[i + PF] = vfrag(i + PF);
      const int u = i / MT2, md = i % MT2;
      acc[md] = T::mfma(vf[i], pf[u], acc[md]);
#pragma unroll
      for (int e = i * VPS; e < (i + 1) * VPS; ++e) {
        if (e & 1)
          sumL1 += sc[e / 16][e % 16];
        else
          sumL0 += sc[e / 16][e % 16];
        mx = __builtin_fmaxf(mx, sn[e / 16][e % 16]);
      }
      if (md == MT2 - 1) lO4 = T::mfma16(sel, pf[u], lO4);  // sum of the rounded P of step u
      // keep this slice in this step (otherwise the reductions are sunk past the interleave)
      asm volatile("" : "+v"(mx), "+v"(sumL0), "+v"(sumL1));
      __builtin_amdgcn_sched_barrier(0);
    }
    lL += sumL0 + sumL1;
    mx = __builtin_fmaxf(mx, other_half(mx));
    mt_cur = mx * c;
    tile_barrier();  // the loads of this iteration have landed; LDS reads of it are done
  };

  using T0 = BoolC<false>;
  using T1 = BoolC<true>;
  int j = 0;
  if (nmain > 0) {
    if (split_first) {
      iteration(0, s_a, s_b, T1{}, T0{});
    } else {
      mt_cur = rowmax(s_a);
      main_iteration(0, s_a, s_b, IntC<0>{});
    }
    j = 1;
    for (; j + 1 < nmain; j += 2) {
      main_iteration(j, s_b, s_a, IntC<1>{});
      main_iteration(j + 1, s_a, s_b, IntC<0>{});
    }
    if (j < nmain) {
      main_iteration(j, s_b, s_a, IntC<1>{});
      ++j;
    }
  } else {
    iteration(0, s_a, s_b, T1{}, T1{});
    j = 1;
  }
  // diagonal and tail tiles; scores of tile j move to s_a first
  if (j < ntiles && (j & 1)) {
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt) s_a[mt] = s_b[mt];
  }
  for (; j < ntiles; ++j) {
    iteration(j, s_a, s_b, T0{}, T1{});
#pragma unroll
    for (int mt = 0; mt < MT1; ++mt) s_a[mt] = s_b[mt];
  }
  }

  // ---- epilogue: combine the two lane halves' sums, normalise, store O and LSE
  lL += other_half(lL);
  if constexpr (MMA_ROWSUM)
    lO = lO4[0];  // already the sum over both lane halves
  else
    lO += other_half(lO);
  // causal: a row that sees no key of this block's range (VAR: q_lane + cshift < 0; split-KV:
  // a range that starts past the row's last key) stores O = 0, LSE = -inf
  const bool empty = (VAR || SPLITK) && CAUSAL && q_lane + cshift < kfirst;
  if (empty) {
    lO = 1.f;
#pragma unroll
    for (int md = 0; md < MT2; ++md) acc[md] = f32x16{};
  }
  if constexpr (!SPLITK) {
    // O leaves through LDS: a lane holds 8-byte pieces of one row (lanes 0-31 = 32 rows, so a
    // direct store writes 32 rows 4 KB apart per instruction, and the workgroup's slot stays
    // busy until those scattered stores drain). The wave writes its 32 x D tile into its own
    // part of the K/V buffers (free: every wave is past the last tile's barrier) and reads it
    // back as whole rows, 16 bytes per lane, so each store instruction covers complete rows.
    constexpr int RS = D * 2 + 16;  // LDS row pitch of the staged tile (bytes)
    constexpr int WB = 32 * RS;     // bytes per wave
    constexpr int OBJ = L::KBUF < L::VBUF ? L::KBUF : L::VBUF;
    constexpr int WPO = OBJ / WB;   // waves per K/V buffer
    static_assert(WPO >= 1 && (NW + WPO - 1) / WPO <= 4, "the staged O tiles fit in the K/V buffers");
    const int wo = wave / WPO;
    uint8_t* const ost = (wo == 0 ? lds0_v : wo == 1 ? lds1_v : wo == 2 ? lds2_k : lds3_k) + (wave % WPO) * WB;
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
        *(u32x2*)(ost + l32 * RS + (32 * md + 8 * i + 4 * hh) * 2) = w;
      }
    constexpr int CPL = D * 2 / 16, RPI = 64 / CPL;  // 16-byte chunks per row, rows per read
    const size_t o_row = (size_t)p.Hq * (D * 2);
    uint8_t* const o0 = p.o + ((q_row0 + qw0) * p.Hq + hq) * (size_t)(D * 2);
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int r = it * RPI + lane / CPL, ch = lane % CPL;
      const u32x4 v = *(const u32x4*)(ost + r * RS + ch * 16);
      if (qw0 + r < Nq) *(u32x4*)(o0 + r * o_row + ch * 16) = v;
    }
    if (q_lane < Nq && hh == 0)
      p.lse[lse0 + q_lane] = empty ? -__builtin_inff() : (m_run + __builtin_amdgcn_logf(lL)) * LN2;
    return;
  }
  if (q_lane < Nq) {  // split-KV: the normalised fp32 partial and its log-sum-exp
    const float inv = 1.0f / lO;
    const size_t row = part_row(q_lane);
    float* po = p.part_o + row * D;
#pragma unroll
    for (int md = 0; md < MT2; ++md)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 w;
        for (int e = 0; e < 4; ++e) w[e] = acc[md][4 * i + e] * inv;
        *(f32x4*)(po + 32 * md + 8 * i + 4 * hh) = w;
      }
    if (hh == 0) p.part_lse[row] = empty ? -__builtin_inff() : (m_run + __builtin_amdgcn_logf(lL)) * LN2;
  }
}

// Merge of the split-KV partials (exact): for each row, LSE = ln sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) * O_s, where O_s is split s's normalised output. A split that
// saw no key of the row has LSE_s = -inf and weight 0. One thread per (row, 8 head-dim
// values). NS > 0: the split count is NS, known at compile time, and every split's LSE and
// partial loads are issued before the first use (a loop over a run-time count issued them one
// split after the other, each behind the previous one's wait: the merge was latency-bound);
// NS = 0: any count. Both sum in split order, so they agree bit for bit.
template <int D, int NS>
__device__ __forceinline__ void merge_row(const FwdParams& p, size_t r, int g, size_t plane, float (&acc)[8],
                                          float& m, float& sum) {
  m = -__builtin_inff();
  sum = 0.f;
  if constexpr (NS > 0) {
    float ls[NS];
    f32x4 a[NS], bq[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      ls[s] = p.part_lse[s * plane + r];
      const f32x4* po = (const f32x4*)(p.part_o + (s * plane + r) * D + 8 * g);
      a[s] = po[0];
      bq[s] = po[1];
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) m = __builtin_fmaxf(m, ls[s]);
    // no branch on m (the loads above would sink behind it): with every LSE_s = -inf the
    // weights are exp2(-inf) = 0 and the row stays empty, as in the loop below
    const float mm = m == -__builtin_inff() ? 0.f : m;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float w = __builtin_amdgcn_exp2f((ls[s] - mm) * LOG2E);
      sum += w;
      for (int e = 0; e < 4; ++e) {
        acc[e] += w * a[s][e];
        acc[4 + e] += w * bq[s][e];
      }
    }
  } else {
    for (int s = 0; s < p.splits; ++s) m = __builtin_fmaxf(m, p.part_lse[s * plane + r]);
    if (m != -__builtin_inff()) {
      for (int s = 0; s < p.splits; ++s) {
        const float w = __builtin_amdgcn_exp2f((p.part_lse[s * plane + r] - m) * LOG2E);
        sum += w;
        const f32x4* po = (const f32x4*)(p.part_o + (s * plane + r) * D + 8 * g);
        const f32x4 a = po[0], bq = po[1];
        for (int e = 0; e < 4; ++e) {
          acc[e] += w * a[e];
          acc[4 + e] += w * bq[e];
        }
      }
    }
  }
}

// Dense batches: partials [splits, B*Hq, Nq, D] and [splits, B*Hq, Nq]; the result goes to
// o [B, Nq, Hq, D] (T) and lse [B, Hq, Nq].
template <int D, class T, int NS>
__global__ void __launch_bounds__(256) fwd_combine(FwdParams p) {
  constexpr int G = D / 8;
  const size_t rows = (size_t)p.B * p.Hq * p.Nq;
  const size_t idx = (size_t)work_item(p.order_mul, p.order_add) * 256 + threadIdx.x;
  if (idx >= rows * G) return;
  const size_t r = idx / G;  // (b*Hq + h) * Nq + i
  const int g = (int)(idx - r * G);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float m, sum;
  merge_row<D, NS>(p, r, g, rows, acc, m, sum);
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  const size_t bhq = r / p.Nq;
  const int i = (int)(r - bhq * p.Nq);
  const int b = (int)(bhq / p.Hq), h = (int)(bhq - (size_t)b * p.Hq);
  uint8_t* op = p.o + (((size_t)b * p.Nq + i) * p.Hq + h) * (size_t)(D * 2) + 16 * g;
  u32x4 w;
  for (int e = 0; e < 4; ++e)
    w[e] = __builtin_bit_cast(unsigned, T::cvt2(acc[2 * e] * inv, acc[2 * e + 1] * inv));
  *(u32x4*)op = w;
  if (g == 0) p.lse[r] = sum > 0.f ? m + __builtin_amdgcn_logf(sum) * LN2 : -__builtin_inff();
}

// The same merge for variable-length batches: partials [splits, Hq, total_q, D] and
// [splits, Hq, total_q]; the result goes to o [total_q, Hq, D] (T) and lse [Hq, total_q].
// A row whose splits all saw no key keeps O = 0 and LSE = -inf.
template <int D, class T, int NS>
__global__ void __launch_bounds__(256) fwd_combine_var(FwdParams p) {
  constexpr int G = D / 8;
  const size_t rows = (size_t)p.Hq * p.total_q;
  const size_t idx = (size_t)work_item(p.order_mul, p.order_add) * 256 + threadIdx.x;
  if (idx >= rows * G) return;
  const size_t r = idx / G;  // h * total_q + i
  const int g = (int)(idx - r * G);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float m, sum;
  merge_row<D, NS>(p, r, g, rows, acc, m, sum);
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  const int h = (int)(r / p.total_q);
  const size_t i = r - (size_t)h * p.total_q;
  uint8_t* op = p.o + (i * p.Hq + h) * (size_t)(D * 2) + 16 * g;
  u32x4 w;
  for (int e = 0; e < 4; ++e)
    w[e] = __builtin_bit_cast(unsigned, T::cvt2(acc[2 * e] * inv, acc[2 * e + 1] * inv));
  *(u32x4*)op = w;
  if (g == 0) p.lse[r] = sum > 0.f ? m + __builtin_amdgcn_logf(sum) * LN2 : -__builtin_inff();
}

}  // namespace fa
