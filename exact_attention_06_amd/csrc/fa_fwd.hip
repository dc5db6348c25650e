// fa_fwd.hip - host side of the C ABI declared in include/fa_fwd.h: argument checks,
// compile-time kernel selection (head dim x causal x element type) and the launch.
// Every check runs before the first HIP call; there is no fallback kernel.
#include <hip/hip_runtime.h>

#include <climits>
#include <algorithm>
#include <atomic>
#include <numeric>
#include <mutex>
#include <cfloat>
#include <cmath>
#include <cstdint>

#include "fa_fwd.h"
#include "fa_kernel.h"
#include "fa_bwd_kernel.h"
#include "fa_fp8_kernel.h"
#include "fa_hd512_kernel.h"

// Device scratch of the allocation-free backward entry point: D = rowsum(dO * O) for up to
// FA_BWD_NOALLOC_MAX_ROWS rows. In host code this name is only a handle for the runtime; the
// device address of each GPU's copy comes from hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) float scratch[FA_BWD_NOALLOC_MAX_ROWS];

namespace {

// Per-device address of `scratch`, resolved once per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// 0 and the address of the current device's scratch, or FA_ERR_LAUNCH.
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return FA_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

// Grid order set by fa_set_grid_order (0: natural), read at each launch.
std::atomic<unsigned> g_order_mul{0}, g_order_add{0};

// The grid-order parameters of one launch of n workgroups: workgroup i takes item
// (i * mul + add) mod n, with mul the first value >= the requested one (mod n; 1 for 0) that is
// coprime with n, so that the map is a permutation. (0, 0) in the natural order.
template <class P>
P ordered(P prm, unsigned n) {
  prm.order_mul = prm.order_add = 0;
  const unsigned m = g_order_mul.load(std::memory_order_relaxed);
  if (m == 0 || n == 0) return prm;
  unsigned s = std::max(m % n, 1u);
  while (std::gcd(s, n) != 1u) s = s + 1 < n ? s + 1 : 1u;  // ends at the latest at 1
  prm.order_mul = s;
  prm.order_add = g_order_add.load(std::memory_order_relaxed) % n;
  return prm;
}

// The merge kernel with the split count as a compile-time constant (2-8: all loads issued
// together) or read at run time (any other count).
template <int D, class T, bool VAR, int NS>
void launch_combine_ns(const fa::FwdParams& prm, unsigned g, hipStream_t stream) {
  if (VAR)
    hipLaunchKernelGGL((fa::fwd_combine_var<D, T, NS>), dim3(g), dim3(256), 0, stream, ordered(prm, g));
  else
    hipLaunchKernelGGL((fa::fwd_combine<D, T, NS>), dim3(g), dim3(256), 0, stream, ordered(prm, g));
}
template <int D, class T, bool VAR>
void launch_combine(const fa::FwdParams& prm, unsigned g, hipStream_t stream) {
  switch (prm.splits) {
    case 2: launch_combine_ns<D, T, VAR, 2>(prm, g, stream); break;
    case 3: launch_combine_ns<D, T, VAR, 3>(prm, g, stream); break;
    case 4: launch_combine_ns<D, T, VAR, 4>(prm, g, stream); break;
    case 5: launch_combine_ns<D, T, VAR, 5>(prm, g, stream); break;
    case 6: launch_combine_ns<D, T, VAR, 6>(prm, g, stream); break;
    case 7: launch_combine_ns<D, T, VAR, 7>(prm, g, stream); break;
    case 8: launch_combine_ns<D, T, VAR, 8>(prm, g, stream); break;
    default: launch_combine_ns<D, T, VAR, 0>(prm, g, stream); break;
  }
}

template <int D, bool CAUSAL, class T, int VM, int WV = fa::TileCfg<D>::NW>
int launch(const fa::FwdParams& prm, int grid, hipStream_t stream) {
  using L = fa::Layout<D, WV>;
  // the kernel's K/V buffers are static LDS (L::LDS bytes, within gfx950's 160 KB per CU)
  hipLaunchKernelGGL((fa::fwd_kernel<D, CAUSAL, T, VM, WV>), dim3(grid), dim3(L::NW * 64), 0, stream,
                     ordered(prm, (unsigned)grid));
  if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
  if (VM == 2) {  // split-KV: merge the partials
    const size_t threads = (size_t)prm.B * prm.Hq * prm.Nq * (D / 8);
    const unsigned g = (unsigned)((threads + 255) / 256);
    launch_combine<D, T, false>(prm, g, stream);
    if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
  }
  if (VM == 3) {  // variable-length split-KV: merge the partials of the packed rows
    const size_t threads = (size_t)prm.Hq * prm.total_q * (D / 8);
    const unsigned g = (unsigned)((threads + 255) / 256);
    launch_combine<D, T, true>(prm, g, stream);
    if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
  }
  return FA_OK;
}

// Scale: the kernels take c = |scale| * log2(e) > 0 (the row maximum relies on c >= 0). A
// negative scale flips the sign of Q instead (exact: |scale| (-q).k == scale q.k bit for bit).
// A zero (or subnormal) scale makes every visible score exactly 0; the kernel then zeroes Q
// and uses c = log2(e), since -inf * 0 would turn masked scores into NaN.
template <class P>
void set_scale(P& prm, float scale) {
  const float a = std::fabs(scale) * fa::LOG2E;
  prm.zero_scores = !(a >= FLT_MIN);
  prm.neg_scores = scale < 0.f && !prm.zero_scores;
  prm.c = prm.zero_scores ? fa::LOG2E : a;
}

// hd128 takes the 4-wave workgroup when the 8-wave grid (without splits; for
// variable-length batches the grid sized by the longest query sequence) has at most this many
// workgroups, one per CU (measured on MI355X: +14-30% on causal shapes with 64-256
// workgroups, 1-4% slower on full grids), and for causal GQA batches (query heads sharing a
// K/V head) of at most kGqaCausalN4 query rows (measured: +6-12% at N = 1k and 2k with 2 and 4
// query heads per K/V head, where the second K/V stream per CU stays in L2; the same form lost
// 3-8% on causal batches without GQA), and for non-causal batches of at most kNonCausalN4
// query rows (measured: +2-4% at N = 512 and 1k, 8-64 batches of 16 heads, with and without
// GQA; no change at N = 1k with 56 heads; at N = 2k the 8-wave form stays 1% ahead). Every
// form decides alike, so that one sequence through the variable-length path and the dense
// path, or one split and none, take the same kernel configuration and agree bit for bit.
constexpr int kSmallGrid128 = 256;
constexpr int kGqaCausalN4 = 2048;
constexpr int kNonCausalN4 = 1024;

bool use_4wave(const fa::FwdParams& prm, int d, int causal) {
  const int64_t BR8 = fa::Layout<128>::BR;
  if (d != 128) return false;
  if ((int64_t)prm.B * prm.Hq * ((prm.Nq + BR8 - 1) / BR8) <= kSmallGrid128) return true;
  if (!causal) return prm.Nq <= kNonCausalN4;
  return prm.group >= 2 && prm.Nq <= kGqaCausalN4;
}

template <int VM, class T>
int dispatch(fa::FwdParams& prm, int d, int causal, hipStream_t s) {
  const int splits = VM >= 2 ? prm.splits : 1;
  if (use_4wave(prm, d, causal)) {
    constexpr int BR = fa::Layout<128, 4>::BR;
    prm.nqt = (prm.Nq + BR - 1) / BR;
    const int grid = prm.B * prm.Hq * prm.nqt * splits;
    return causal ? launch<128, true, T, VM, 4>(prm, grid, s) : launch<128, false, T, VM, 4>(prm, grid, s);
  }
  const int BR = d == 128 ? fa::Layout<128>::BR : fa::Layout<256>::BR;
  prm.nqt = (prm.Nq + BR - 1) / BR;
  const int grid = prm.B * prm.Hq * prm.nqt * splits;
  if (d == 128)
    return causal ? launch<128, true, T, VM>(prm, grid, s) : launch<128, false, T, VM>(prm, grid, s);
  return causal ? launch<256, true, T, VM>(prm, grid, s) : launch<256, false, T, VM>(prm, grid, s);
}

void clear_extras(fa::FwdParams& prm) {
  prm.cu_q = prm.cu_k = prm.seqused = prm.block_table = nullptr;
  prm.total_q = prm.total_k = prm.page_size = prm.max_pages = prm.num_pages = 0;
  prm.part_o = prm.part_lse = nullptr;
  prm.splits = prm.tps = 0;
  prm.v_scale = 1.f;
}

// ---- fp8 (e4m3) forward
template <int D, bool CAUSAL>
int launch_fp8(const fa::FwdParams& prm, hipStream_t stream) {
  const int grid = prm.B * prm.Hq * prm.nqt;
  hipLaunchKernelGGL((fa::fwd_fp8_kernel<D, CAUSAL>), dim3(grid), dim3(fa::Fp8Cfg<D>::NW * 64), 0, stream,
                     ordered(prm, (unsigned)grid));
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int run_fp8(const void* q, const void* k, const void* v, void* o, float* lse, float q_scale, float k_scale,
            float v_scale, int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || Nq <= 0 || Nk <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (causal && Nq != Nk) return FA_ERR_CAUSAL_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  for (float x : {q_scale, k_scale, v_scale})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;
  const int64_t BR = fa::Fp8Cfg<128>::BR;
  if ((int64_t)B * Hq * ((Nq + BR - 1) / BR) > INT_MAX || (int64_t)Nq + BR > INT_MAX ||
      (int64_t)Nk + 256 > INT_MAX)
    return FA_ERR_TOO_LARGE;
  fa::FwdParams prm;
  prm.q = (const uint8_t*)q;
  prm.k = (const uint8_t*)k;
  prm.v = (const uint8_t*)v;
  prm.o = (uint8_t*)o;
  prm.lse = lse;
  prm.B = B;
  prm.Nq = Nq;
  prm.Nk = Nk;
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.group = Hq / Hkv;
  clear_extras(prm);
  set_scale(prm, scale * q_scale * k_scale);
  prm.v_scale = v_scale;
  prm.nqt = (Nq + (int)BR - 1) / (int)BR;
  hipStream_t s = (hipStream_t)stream;
  if (d == 128) return causal ? launch_fp8<128, true>(prm, s) : launch_fp8<128, false>(prm, s);
  return causal ? launch_fp8<256, true>(prm, s) : launch_fp8<256, false>(prm, s);
}

template <int D> int br() { return fa::Layout<D>::BR; }

// hd512: head dim 512 is accepted (the dense forward pass only)
int check(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
          int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale, bool hd512 = false) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || Nq <= 0 || Nk <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (d != 128 && d != 256 && !(hd512 && d == 512)) return FA_ERR_HEADDIM;
  if (causal && Nq != Nk) return FA_ERR_CAUSAL_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;
  const int64_t BR = d == 128 ? br<128>() : d == 256 ? br<256>() : fa::Hd512::BR;
  const int64_t nqt = (Nq + BR - 1) / BR;
  const int64_t grid = (int64_t)B * Hq * nqt;
  if (grid > INT_MAX || (int64_t)Nq + BR > INT_MAX || (int64_t)Nk + 256 > INT_MAX) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

template <bool CAUSAL, class T>
int launch_hd512(fa::FwdParams& prm, hipStream_t stream) {
  prm.nqt = (prm.Nq + fa::Hd512::BR - 1) / fa::Hd512::BR;
  const unsigned grid = (unsigned)(prm.B * prm.Hq * prm.nqt);
  hipLaunchKernelGGL((fa::fwd_hd512_kernel<CAUSAL, T>), dim3(grid), dim3(fa::Hd512::NW * 64), 0, stream,
                     ordered(prm, grid));
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <class T>
int run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Nq, int Nk,
        int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  const int st = check(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, causal, scale, true);
  if (st != FA_OK) return st;
  fa::FwdParams prm;
  prm.q = (const uint8_t*)q;
  prm.k = (const uint8_t*)k;
  prm.v = (const uint8_t*)v;
  prm.o = (uint8_t*)o;
  prm.lse = lse;
  prm.B = B;
  prm.Nq = Nq;
  prm.Nk = Nk;
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.group = Hq / Hkv;
  clear_extras(prm);
  set_scale(prm, scale);
  if (d == 512)
    return causal ? launch_hd512<true, T>(prm, (hipStream_t)stream) : launch_hd512<false, T>(prm, (hipStream_t)stream);
  return dispatch<0, T>(prm, d, causal, (hipStream_t)stream);
}

// ---- split-KV forward: the key tiles of each query tile are cut into num_splits ranges
int key_tile(int d) { return d == 128 ? fa::Layout<128>::BC : fa::Layout<256>::BC; }

size_t splitkv_ws_bytes(int B, int Nq, int Hq, int d, int splits) {
  if (B <= 0 || Nq <= 0 || Hq <= 0 || (d != 128 && d != 256) || splits < 1) return 0;
  return (size_t)splits * B * Hq * Nq * (size_t)(d + 1) * sizeof(float);
}

// Split count from a sweep on MI355X (plain grid against 1, 2, 3, 4, 6 and 8 splits; 1..4
// batches of 1k..4k tokens, 8 or 16 heads, hd128 and hd256, causal and not, best of 3 x 40
// launches): splitting pays only on a nearly empty GPU (at most 128 workgroups; 256 for long
// causal hd256 ranges) with enough key tiles per split, because a split costs its partials'
// fp32 traffic, the merge kernel and a workgroup's fixed work (prologue, first tile, stores).
// One split through the split-KV path ran 15-35% slower than the plain grid at these sizes.
// Rules, first match wins: {most workgroups of the 8-wave (hd128) or 4-wave (hd256) grid,
// fewest key tiles, splits}.
struct SplitRule {
  int max_blocks, min_tiles, splits;
};
// (hd128 measured with its 4-wave form on these small grids, which already doubles the
// workgroups: non-causal splits no longer pay there)
constexpr SplitRule kSplit128[] = {{-1, 0, 1}};
constexpr SplitRule kSplit128Causal[] = {{64, 32, 2}, {128, 64, 3}};
constexpr SplitRule kSplit256[] = {{64, 24, 3}, {128, 48, 3}};
constexpr SplitRule kSplit256Causal[] = {{64, 32, 4}, {128, 32, 2}, {256, 128, 3}};

int num_splits(int B, int Nq, int Nk, int Hq, int d, int causal) {
  if (B <= 0 || Nq <= 0 || Nk <= 0 || Hq <= 0 || (d != 128 && d != 256)) return 1;
  const int BR = d == 128 ? fa::Layout<128>::BR : fa::Layout<256>::BR;
  const int64_t blocks = (int64_t)B * Hq * ((Nq + BR - 1) / BR);
  const int64_t tiles = ((int64_t)Nk + key_tile(d) - 1) / key_tile(d);
  auto pick = [&](const auto& rules) {
    for (const SplitRule& r : rules)
      if (blocks <= r.max_blocks && tiles >= r.min_tiles) return r.splits;
    return 1;
  };
  if (d == 128) return causal ? pick(kSplit128Causal) : pick(kSplit128);
  return causal ? pick(kSplit256Causal) : pick(kSplit256);
}

template <class T>
int run_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* ws, size_t ws_bytes,
                int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale, int splits,
                void* stream) {
  const int st = check(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, causal, scale);
  if (st != FA_OK) return st;
  if (splits < 1 || splits > 256) return FA_ERR_SHAPE;
  const size_t need = splitkv_ws_bytes(B, Nq, Hq, d, splits);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 15)) return FA_ERR_WORKSPACE;
  if ((int64_t)B * Hq * ((Nq + 127) / 128) * splits > INT_MAX) return FA_ERR_TOO_LARGE;
  fa::FwdParams prm;
  prm.q = (const uint8_t*)q;
  prm.k = (const uint8_t*)k;
  prm.v = (const uint8_t*)v;
  prm.o = (uint8_t*)o;
  prm.lse = lse;
  prm.B = B;
  prm.Nq = Nq;
  prm.Nk = Nk;
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.group = Hq / Hkv;
  clear_extras(prm);
  const int ntiles = (Nk + key_tile(d) - 1) / key_tile(d);
  prm.tps = (ntiles + splits - 1) / splits;
  prm.splits = splits;
  prm.part_o = (float*)ws;
  prm.part_lse = (float*)ws + (size_t)splits * B * Hq * Nq * d;
  set_scale(prm, scale);
  return dispatch<2, T>(prm, d, causal, (hipStream_t)stream);
}

// Variable-length forward (packed K/V when block_table is NULL, else paged K/V).
int check_var(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const int* cu_q, const int* cu_k, const int* seqused, const int* block_table, int B,
              int max_seqlen_q, int total_q, int total_k, int num_pages, int page_size, int max_pages,
              int Hq, int Hkv, int d, float scale, bool paged) {
  if (!q || !k || !v || !o || !lse || !cu_q) return FA_ERR_NULL;
  if (paged ? (!seqused || !block_table) : !cu_k) return FA_ERR_NULL;
  if (B <= 0 || max_seqlen_q <= 0 || total_q <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return FA_ERR_SHAPE;
  if (!paged && total_k < 0) return FA_ERR_SHAPE;
  if (paged && (page_size <= 0 || page_size % 64 != 0 || num_pages <= 0 || max_pages <= 0 ||
                (int64_t)max_pages * page_size > INT_MAX || (int64_t)num_pages * page_size > INT_MAX))
    return FA_ERR_PAGE;
  if (d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)cu_q | (uintptr_t)cu_k | (uintptr_t)seqused | (uintptr_t)block_table) & 3)
    return FA_ERR_ALIGN;
  const int64_t BR = d == 128 ? br<128>() : br<256>();
  const int64_t grid = (int64_t)B * Hq * ((max_seqlen_q + BR - 1) / BR);
  if (grid > INT_MAX || (int64_t)max_seqlen_q + BR > INT_MAX || (int64_t)B * Hq > INT_MAX)
    return FA_ERR_TOO_LARGE;
  return FA_OK;
}

size_t var_splitkv_ws_bytes(int total_q, int Hq, int d, int splits) {
  if (total_q <= 0 || Hq <= 0 || (d != 128 && d != 256) || splits < 1) return 0;
  return (size_t)splits * Hq * total_q * (size_t)(d + 1) * sizeof(float);
}

// Split count for variable-length / paged batches, measured on MI355X (128 paged sequences of
// 1k..32k keys, 1..16 queries each, hd256: 4.2 TB/s of K/V without splits, 5.5-5.8 TB/s with
// 2..16, best at 8; packed and paged prefill of 32k tokens only get slower, by the partials'
// traffic): split decode-shaped batches (at most 64 query rows per sequence) whose key bound
// spans many tiles.
int var_num_splits(int B, int max_seqlen_q, int key_bound, int Hq, int d) {
  if (B <= 0 || max_seqlen_q <= 0 || key_bound <= 0 || Hq <= 0 || (d != 128 && d != 256)) return 0;
  if (max_seqlen_q > 64) return 0;
  const int tiles = (key_bound + key_tile(d) - 1) / key_tile(d);
  if (tiles < 32) return 0;
  return tiles >= 128 ? 8 : std::max(2, tiles / 16);
}

// splits = 0: no split. Otherwise every sequence's key tiles are cut into chunks of tps tiles,
// tps = ceil(ceil(K / BC) / splits) for K a bound on any sequence's key count (paged:
// max_pages * page_size; packed: total_k), so that the splits cover every sequence's keys.
template <class T>
int run_var(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_q,
            const int* cu_k, const int* seqused, const int* block_table, int B, int max_seqlen_q,
            int total_q, int total_k, int num_pages, int page_size, int max_pages, int Hq, int Hkv,
            int d, int causal, float scale, void* stream, bool paged, int splits = 0, void* ws = nullptr,
            size_t ws_bytes = 0) {
  const int st = check_var(q, k, v, o, lse, cu_q, cu_k, seqused, block_table, B, max_seqlen_q, total_q,
                           total_k, num_pages, page_size, max_pages, Hq, Hkv, d, scale, paged);
  if (st != FA_OK) return st;
  int tps = 0;
  if (splits != 0) {
    if (splits < 1 || splits > 256) return FA_ERR_SHAPE;
    if (!ws || ws_bytes < var_splitkv_ws_bytes(total_q, Hq, d, splits) || ((uintptr_t)ws & 15))
      return FA_ERR_WORKSPACE;
    const int64_t BR = d == 128 ? br<128>() : br<256>();
    if ((int64_t)B * Hq * ((max_seqlen_q + BR - 1) / BR) * splits > INT_MAX) return FA_ERR_TOO_LARGE;
    const int64_t bound = paged ? (int64_t)max_pages * page_size : (int64_t)total_k;
    const int64_t tiles = (bound + key_tile(d) - 1) / key_tile(d);
    tps = (int)std::max<int64_t>(1, (tiles + splits - 1) / splits);
  }
  fa::FwdParams prm;
  prm.q = (const uint8_t*)q;
  prm.k = (const uint8_t*)k;
  prm.v = (const uint8_t*)v;
  prm.o = (uint8_t*)o;
  prm.lse = lse;
  prm.B = B;
  prm.Nq = max_seqlen_q;  // sizes the grid; each block reads its own sequence's length
  prm.Nk = 0;
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.group = Hq / Hkv;
  prm.cu_q = cu_q;
  prm.cu_k = paged ? nullptr : cu_k;
  prm.seqused = seqused;
  prm.block_table = paged ? block_table : nullptr;
  prm.total_q = total_q;
  prm.total_k = paged ? 0 : total_k;
  prm.page_size = paged ? page_size : 0;
  prm.max_pages = paged ? max_pages : 0;
  prm.num_pages = paged ? num_pages : 0;
  prm.part_o = prm.part_lse = nullptr;
  prm.splits = prm.tps = 0;
  prm.v_scale = 1.f;
  set_scale(prm, scale);
  if (splits == 0) return dispatch<1, T>(prm, d, causal, (hipStream_t)stream);
  prm.splits = splits;
  prm.tps = tps;
  prm.part_o = (float*)ws;
  prm.part_lse = (float*)ws + (size_t)splits * Hq * total_q * d;
  return dispatch<3, T>(prm, d, causal, (hipStream_t)stream);
}

size_t bwd_ws_bytes(int B, int Nq, int Hq) {
  if (B <= 0 || Nq <= 0 || Hq <= 0) return 0;
  return (size_t)B * Hq * Nq * sizeof(float);
}

template <int D, bool CAUSAL, class T>
int launch_bwd(const fa::BwdParams& base, hipStream_t stream) {
  constexpr int NW = fa::BwdCfg<D>::NW, BR = NW * 32;
  fa::BwdParams prm = base;
  prm.ntile = (prm.Nq + BR - 1) / BR;
  const unsigned gq = (unsigned)(prm.B * prm.Hq * prm.ntile);
  hipLaunchKernelGGL((fa::bwd_dq_kernel<D, CAUSAL, T>), dim3(gq), dim3(NW * 64), 0, stream, ordered(prm, gq));
  if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
  prm.ntile = (prm.Nk + BR - 1) / BR;
  const unsigned gk = (unsigned)(prm.B * prm.Hkv * prm.ntile);
  hipLaunchKernelGGL((fa::bwd_dkdv_kernel<D, CAUSAL, T>), dim3(gk), dim3(NW * 64), 0, stream, ordered(prm, gk));
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// every host check of the backward pass except the workspace
int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              const void* dq, const void* dk, const void* dv, int B, int Nq, int Nk, int Hq, int Hkv, int d,
              int causal, float scale) {
  int st = check(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, causal, scale);
  if (st != FA_OK) return st;
  if (!dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (((uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15) return FA_ERR_ALIGN;
  const int64_t BR = fa::BwdCfg<128>::NW * 32;
  if ((int64_t)B * Hq * ((Nq + BR - 1) / BR) > INT_MAX || (int64_t)B * Hkv * ((Nk + BR - 1) / BR) > INT_MAX)
    return FA_ERR_TOO_LARGE;
  return FA_OK;
}

template <class T>
int run_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
            void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, int B, int Nq, int Nk, int Hq, int Hkv,
            int d, int causal, float scale, void* stream) {
  const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Nq, Nk, Hq, Hkv, d, causal, scale);
  if (st != FA_OK) return st;
  if (!ws || ws_bytes < bwd_ws_bytes(B, Nq, Hq) || ((uintptr_t)ws & 3)) return FA_ERR_WORKSPACE;
  fa::BwdParams prm;
  prm.q = (const uint8_t*)q;
  prm.k = (const uint8_t*)k;
  prm.v = (const uint8_t*)v;
  prm.o = (const uint8_t*)o;
  prm.lse = lse;
  prm.dout = (const uint8_t*)dout;
  prm.dq = (uint8_t*)dq;
  prm.dk = (uint8_t*)dk;
  prm.dv = (uint8_t*)dv;
  prm.dsum = (float*)ws;
  prm.B = B;
  prm.Nq = Nq;
  prm.Nk = Nk;
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.group = Hq / Hkv;
  prm.ntile = 0;
  // zero (or subnormal) scale as in the forward pass; otherwise the signed c
  prm.zero_scores = !(std::fabs(scale) * fa::LOG2E >= FLT_MIN);
  prm.c = prm.zero_scores ? fa::LOG2E : scale * fa::LOG2E;
  prm.scale = scale;
  hipStream_t s = (hipStream_t)stream;
  if (d == 128)
    return causal ? launch_bwd<128, true, T>(prm, s) : launch_bwd<128, false, T>(prm, s);
  return causal ? launch_bwd<256, true, T>(prm, s) : launch_bwd<256, false, T>(prm, s);
}

}  // namespace

extern "C" {

int fa_fwd_check(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                 int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale) {
  return check(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, causal, scale, true);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Nq, int Nk,
           int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  return run<fa::Bf16>(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, causal, scale, stream);
}

int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Nq,
               int Nk, int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  return run<fa::F16>(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, causal, scale, stream);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, const int* seqused_k, int B, int max_seqlen_q, int total_q,
                  int total_k, int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  return run_var<fa::Bf16>(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, seqused_k, nullptr, B, max_seqlen_q,
                           total_q, total_k, 0, 0, 0, Hq, Hkv, d, causal, scale, stream, false);
}

int fa_fwd_varlen_f16(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens_q,
                      const int* cu_seqlens_k, const int* seqused_k, int B, int max_seqlen_q, int total_q,
                      int total_k, int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  return run_var<fa::F16>(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, seqused_k, nullptr, B, max_seqlen_q,
                          total_q, total_k, 0, 0, 0, Hq, Hkv, d, causal, scale, stream, false);
}

int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                 const int* cu_seqlens_q, const int* seqused_k, const int* block_table, int B, int max_seqlen_q,
                 int total_q, int num_pages, int page_size, int max_pages, int Hq, int Hkv, int d, int causal,
                 float scale, void* stream) {
  return run_var<fa::Bf16>(q, k_cache, v_cache, o, lse, cu_seqlens_q, nullptr, seqused_k, block_table, B,
                           max_seqlen_q, total_q, 0, num_pages, page_size, max_pages, Hq, Hkv, d, causal, scale,
                           stream, true);
}

int fa_fwd_paged_f16(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                     const int* cu_seqlens_q, const int* seqused_k, const int* block_table, int B,
                     int max_seqlen_q, int total_q, int num_pages, int page_size, int max_pages, int Hq, int Hkv,
                     int d, int causal, float scale, void* stream) {
  return run_var<fa::F16>(q, k_cache, v_cache, o, lse, cu_seqlens_q, nullptr, seqused_k, block_table, B,
                          max_seqlen_q, total_q, 0, num_pages, page_size, max_pages, Hq, Hkv, d, causal, scale,
                          stream, true);
}

size_t fa_fwd_var_splitkv_workspace_bytes(int total_q, int Hq, int d, int num_splits) {
  return var_splitkv_ws_bytes(total_q, Hq, d, num_splits);
}

int fa_fwd_var_num_splits(int B, int max_seqlen_q, int key_bound, int Hq, int d) {
  return var_num_splits(B, max_seqlen_q, key_bound, Hq, d);
}

int fa_fwd_varlen_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                          size_t workspace_bytes, const int* cu_seqlens_q, const int* cu_seqlens_k,
                          const int* seqused_k, int B, int max_seqlen_q, int total_q, int total_k, int Hq, int Hkv,
                          int d, int causal, float scale, int num_splits, void* stream) {
  if (num_splits < 1) return FA_ERR_SHAPE;
  return run_var<fa::Bf16>(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, seqused_k, nullptr, B, max_seqlen_q,
                           total_q, total_k, 0, 0, 0, Hq, Hkv, d, causal, scale, stream, false, num_splits, workspace,
                           workspace_bytes);
}

int fa_fwd_varlen_splitkv_f16(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                              size_t workspace_bytes, const int* cu_seqlens_q, const int* cu_seqlens_k,
                              const int* seqused_k, int B, int max_seqlen_q, int total_q, int total_k, int Hq,
                              int Hkv, int d, int causal, float scale, int num_splits, void* stream) {
  if (num_splits < 1) return FA_ERR_SHAPE;
  return run_var<fa::F16>(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, seqused_k, nullptr, B, max_seqlen_q,
                          total_q, total_k, 0, 0, 0, Hq, Hkv, d, causal, scale, stream, false, num_splits, workspace,
                          workspace_bytes);
}

int fa_fwd_paged_splitkv(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, const int* cu_seqlens_q, const int* seqused_k,
                         const int* block_table, int B, int max_seqlen_q, int total_q, int num_pages, int page_size,
                         int max_pages, int Hq, int Hkv, int d, int causal, float scale, int num_splits,
                         void* stream) {
  if (num_splits < 1) return FA_ERR_SHAPE;
  return run_var<fa::Bf16>(q, k_cache, v_cache, o, lse, cu_seqlens_q, nullptr, seqused_k, block_table, B,
                           max_seqlen_q, total_q, 0, num_pages, page_size, max_pages, Hq, Hkv, d, causal, scale,
                           stream, true, num_splits, workspace, workspace_bytes);
}

int fa_fwd_paged_splitkv_f16(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                             void* workspace, size_t workspace_bytes, const int* cu_seqlens_q,
                             const int* seqused_k, const int* block_table, int B, int max_seqlen_q, int total_q,
                             int num_pages, int page_size, int max_pages, int Hq, int Hkv, int d, int causal,
                             float scale, int num_splits, void* stream) {
  if (num_splits < 1) return FA_ERR_SHAPE;
  return run_var<fa::F16>(q, k_cache, v_cache, o, lse, cu_seqlens_q, nullptr, seqused_k, block_table, B,
                          max_seqlen_q, total_q, 0, num_pages, page_size, max_pages, Hq, Hkv, d, causal, scale,
                          stream, true, num_splits, workspace, workspace_bytes);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, float q_scale, float k_scale,
               float v_scale, int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale,
               void* stream) {
  return run_fp8(q, k, v, o, lse, q_scale, k_scale, v_scale, B, Nq, Nk, Hq, Hkv, d, causal, scale, stream);
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int Nq, int Hq, int d, int num_splits) {
  return splitkv_ws_bytes(B, Nq, Hq, d, num_splits);
}

int fa_fwd_num_splits(int B, int Nq, int Nk, int Hq, int d, int causal) {
  return num_splits(B, Nq, Nk, Hq, d, causal);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                   size_t workspace_bytes, int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale,
                   int num_splits, void* stream) {
  return run_splitkv<fa::Bf16>(q, k, v, o, lse, workspace, workspace_bytes, B, Nq, Nk, Hq, Hkv, d, causal, scale,
                               num_splits, stream);
}

int fa_fwd_splitkv_f16(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                       size_t workspace_bytes, int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal,
                       float scale, int num_splits, void* stream) {
  return run_splitkv<fa::F16>(q, k, v, o, lse, workspace, workspace_bytes, B, Nq, Nk, Hq, Hkv, d, causal, scale,
                              num_splits, stream);
}

size_t fa_bwd_workspace_bytes(int B, int Nq, int Hq) { return bwd_ws_bytes(B, Nq, Hq); }

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Nq, int Nk,
           int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  return run_bwd<fa::Bf16>(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Nq, Nk, Hq, Hkv, d,
                           causal, scale, stream);
}

int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Nq, int Nk,
               int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  return run_bwd<fa::F16>(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Nq, Nk, Hq, Hkv, d,
                          causal, scale, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal,
                   float scale, void* stream) {
  // every host check of fa_bwd, then the scratch limit, then the device address: no HIP call
  // before the arguments are known good
  int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Nq, Nk, Hq, Hkv, d, causal, scale);
  if (st != FA_OK) return st;
  if ((int64_t)B * Hq * Nq > (int64_t)FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != FA_OK) return st;
  return run_bwd<fa::Bf16>(q, k, v, o, lse, dout, dq, dk, dv, ws, sizeof(scratch), B, Nq, Nk, Hq, Hkv, d, causal,
                           scale, stream);
}

int fa_set_grid_order(unsigned mul, unsigned add) {
  g_order_add.store(add, std::memory_order_relaxed);
  g_order_mul.store(mul, std::memory_order_relaxed);
  return FA_OK;
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a pointer argument is NULL";
    case FA_ERR_SHAPE: return "B, Nq, Nk, Hq and Hkv must be positive and Hq a multiple of Hkv";
    case FA_ERR_HEADDIM: return "head dim must be 128 or 256 (or 512 for fa_fwd / fa_fwd_f16)";
    case FA_ERR_CAUSAL_SHAPE: return "causal attention needs Nq == Nk";
    case FA_ERR_SCALE: return "scale must be finite (fp8 dequantisation factors finite and positive)";
    case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_TOO_LARGE: return "problem too large for 32-bit grid or sequence indexing";
    case FA_ERR_LAUNCH: return "HIP kernel launch failed";
    case FA_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than the *_workspace_bytes size";
    case FA_ERR_PAGE: return "paged K/V: page_size must be a positive multiple of 64, num_pages and max_pages positive";
    case FA_ERR_SCRATCH: return "fa_bwd_noalloc: B * Hq * Nq exceeds the fixed device scratch (FA_BWD_NOALLOC_MAX_ROWS rows)";
    default: return "unknown fa status code";
  }
}

}  // extern "C"
