/*
 * fa_fwd.h - C ABI of the MI355X (gfx950) exact-attention forward library (libfa.so).
 *
 * The operation (softmax attention, computed tile by tile with an online softmax so the
 * Nq x Nk score matrix never reaches device memory):
 *
 *   for every batch b and query head h, with kv head  kvh = h / (Hq / Hkv):
 *     S[i][j]  = scale * dot(Q[b,i,h,:], K[b,j,kvh,:])
 *     causal:  S[i][j] = -inf for j > i   (query i sees keys 0..i)
 *     O[b,i,h,:]  = sum_j softmax_j(S[i][:]) * V[b,j,kvh,:]
 *     LSE[b,h,i]  = ln( sum_j exp(S[i][j]) )
 *
 * Where each part is stated:
 *   - the attention product and its tile-by-tile, running-max/running-sum evaluation:
 *     "FlashAttention 4: Snellere, Geheugenefficiente Aandacht voor LLM's", sections
 *     "Inleiding" and "Waarom aandachtkernels nog steeds de kosten van LLM's domineren";
 *   - the native [batch, sequence, heads, head_dim] layout with matching FP16/BF16 Q/K/V
 *     and an error (never a silent kernel change) on any contract violation:
 *     "h3-blackwell-runtime/FLASH4.md", section "API";
 *   - head_dim 256 next to 128, causal and non-causal variants: "[RFC] FA4 - head_dim=256 &
 *     head_dim=512", sections "Overview" and "Performance Snapshot"; head_dim 512 (fa_fwd
 *     and fa_fwd_f16 only): the same page, table of section "Phase 4";
 *   - grouped-query heads sharing one K/V head: the Dutch page's compatibility section.
 *   The pages never define the LSE output; it is the natural-log log-sum-exp of the scaled
 *   scores over the visible keys, in fp32.
 *
 * Layouts (all row-major, contiguous, element type bf16 for fa_fwd and fp16 for fa_fwd_f16):
 *   q   [B, Nq, Hq,  d]        k, v  [B, Nk, Hkv, d]        o  [B, Nq, Hq, d]
 *   lse [B, Hq, Nq] float32
 *
 * Ownership: every pointer is device memory owned by the caller. The library allocates
 * nothing, keeps no state between calls and is re-entrant; concurrent calls on different
 * streams are independent.
 *
 * Execution: asynchronous on `stream` (a hipStream_t; NULL means the default stream). The
 * call never synchronises. Kernel faults surface at the caller's next synchronisation.
 *
 * Errors: 0 (FA_OK) or a negative FA_ERR_* code. Every argument check runs on the host
 * before any HIP call, so invalid arguments never reach the GPU. There is no fallback path.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,         /* a pointer argument is NULL                                  */
  FA_ERR_SHAPE = -2,        /* B, Nq, Nk, Hq or Hkv <= 0, or Hq % Hkv != 0                 */
  FA_ERR_HEADDIM = -3,      /* d is not 128 or 256 (fa_fwd and fa_fwd_f16: or 512)         */
  FA_ERR_CAUSAL_SHAPE = -4, /* causal with Nq != Nk (the causal alignment is defined for
                               square problems only)                                       */
  FA_ERR_SCALE = -5,        /* scale is NaN or infinite                                    */
  FA_ERR_ALIGN = -6,        /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
  FA_ERR_TOO_LARGE = -7,    /* the work grid or a per-head extent exceeds 2^31 - 1         */
  FA_ERR_LAUNCH = -8,       /* the HIP launch reported an error                            */
  FA_ERR_WORKSPACE = -9,    /* workspace NULL, not 16-byte aligned (split-KV) or smaller
                               than fa_bwd_workspace_bytes / fa_fwd_splitkv_workspace_bytes */
  FA_ERR_PAGE = -10,        /* paged K/V: page_size not a positive multiple of 64, or
                               num_pages / max_pages not positive, or a page extent
                               (pages x page_size) above 2^31 - 1                          */
  FA_ERR_SCRATCH = -11      /* fa_bwd_noalloc: the problem needs more than the library's
                               fixed device scratch (FA_BWD_NOALLOC_MAX_ROWS rows)          */
};

/* Forward pass, bf16 q/k/v/o, fp32 LSE. Arguments as described above; `scale` multiplies
 * the q.k dot products (1/sqrt(d) is the usual choice; any finite value is accepted: zero
 * gives uniform weights over the visible keys, a negative scale scores of the opposite
 * sign). d is 128, 256 or 512. Returns an fa_status. */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale,
           void* stream);

/* Same as fa_fwd with fp16 q/k/v/o. */
int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale,
               void* stream);

/* ---- FP8 inputs: q, k, v in e4m3 (OCP FP8, 1 byte per element), o in bf16.
 *
 * The FP8 input path of the pages ("[RFC] FA4 - head_dim=256 & head_dim=512", feature
 * table of section "Phase 2": FP8 input on the FP8 tensor-core MMA). Layouts, shapes,
 * causal mask and LSE are those of fa_fwd; the operation is fa_fwd's on the dequantised
 * inputs q_scale*Q, k_scale*K, v_scale*V (one positive factor per tensor). In Q K^T the
 * e4m3 products are exact, but the fp8 matrix cores sum each group of 64 of them with fewer
 * bits than fp32 (measured on MI355X: at most about 2^-14 of sum |q k| for operands spread
 * like quantised normal data), so a score can be off by that much; the softmax weights P are
 * rounded to e4m3 for P V
 * (3 mantissa bits: up to 2^-4 relative, 2^-10 absolute below 2^-6) and O is normalised
 * by the fp32 sum of those rounded weights; the LSE uses the fp32 sum of the unrounded
 * ones. Errors: as fa_fwd; FA_ERR_SCALE also for a dequantisation factor that is not
 * finite and positive. */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               float q_scale, float k_scale, float v_scale,
               int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale,
               void* stream);

/* ---- Split-KV forward: more parallel work for short sequences and few heads.
 *
 * The pages gain 10-25% at 8 query heads and 1k tokens from a persistent, cluster-aware
 * tile scheduler ("[RFC] FA4 - head_dim=256 & head_dim=512", feature table of section
 * "Phase 2": the persistent scheduler gated on short key lengths; "short-sequence perf"
 * in the same table). On the 256 CUs of an MI355X such shapes leave most CUs idle, so here
 * the key range of every query tile is cut into num_splits ranges computed by separate
 * workgroups; each writes its normalised output O_s and log-sum-exp LSE_s (fp32) to the
 * workspace, and a second kernel merges them exactly:
 *     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) * O_s
 * The result is the operation of fa_fwd (same layouts, same causal mask, same errors);
 * only the rounding order of the sums differs.
 *
 * workspace: caller-owned device memory of at least
 *   fa_fwd_splitkv_workspace_bytes(B, Nq, Hq, d, num_splits) = num_splits*B*Hq*Nq*(d+1)*4
 * bytes, 16-byte aligned; its contents on entry do not matter. num_splits: 1..256 (splits
 * past the keys of a query tile are empty). fa_fwd_num_splits returns the library's
 * choice for a shape (1 when the plain grid already fills the GPU). */
size_t fa_fwd_splitkv_workspace_bytes(int B, int Nq, int Hq, int d, int num_splits);

int fa_fwd_num_splits(int B, int Nq, int Nk, int Hq, int d, int causal);

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes,
                   int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale,
                   int num_splits, void* stream);

/* Same as fa_fwd_splitkv with fp16 q/k/v/o. */
int fa_fwd_splitkv_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                       void* workspace, size_t workspace_bytes,
                       int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale,
                       int num_splits, void* stream);

/* ---- Variable-length batches, per-sequence key counts and a paged K/V cache.
 *
 * The serving variants the pages list beside the dense pass ("[RFC] FA4 - head_dim=256 &
 * head_dim=512", feature table of section "Phase 2": paged KV with the page size equal to
 * the key tile, seqused_k with an early exit for sequences without keys, varlen; the Dutch
 * page, section "Compatibiliteit en huidige status": variable-length batches through
 * cu_seqlens). Each sequence b is computed exactly as the dense operation above, on its
 * own rows, with these readings (the pages do not fix them):
 *   - causal alignment is bottom-right: query i of a sequence with Lq queries and Lk keys
 *     sees keys j <= i + (Lk - Lq) (the dense pass's mask when Lq == Lk; a decode row sees
 *     every key); a query row that sees no key gets O = 0 and LSE = -inf;
 *   - q and o are packed [total_q, Hq, d]; lse is [Hq, total_q] float32; sequence b owns
 *     rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1;
 *   - seqused_k[b] (when given) is the number of keys of sequence b that are used (the
 *     first ones); 0 gives O = 0 and LSE = -inf for the whole sequence.
 *
 * cu_seqlens_q, cu_seqlens_k, seqused_k and block_table are int32 device arrays owned by
 * the caller. Their contents are read on the GPU and are not validated on the host: offsets
 * must be non-decreasing, cu_seqlens_q[B] <= total_q, every query length <= max_seqlen_q
 * (rows beyond it are not written). Offsets are clamped to the tensors and page numbers
 * outside [0, num_pages) read as zero pages, so bad contents give wrong numbers but no
 * access outside the buffers. Everything else is as for fa_fwd (ownership, stream,
 * error codes, alignment; the four int arrays must be 4-byte aligned).
 */

/* Packed K/V: k, v are [total_k, Hkv, d]; sequence b owns key rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 (B+1 entries). seqused_k: NULL or B entries. */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, const int* seqused_k,
                  int B, int max_seqlen_q, int total_q, int total_k,
                  int Hq, int Hkv, int d, int causal, float scale, void* stream);

/* Same as fa_fwd_varlen with fp16 q/k/v/o. */
int fa_fwd_varlen_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int* cu_seqlens_q, const int* cu_seqlens_k, const int* seqused_k,
                      int B, int max_seqlen_q, int total_q, int total_k,
                      int Hq, int Hkv, int d, int causal, float scale, void* stream);

/* Paged K/V: k_cache, v_cache are [num_pages, page_size, Hkv, d]; block_table is
 * [B, max_pages] int32; logical key t of sequence b is row t % page_size of page
 * block_table[b * max_pages + t / page_size]; seqused_k (B entries, required) gives the
 * key count of each sequence (at most max_pages * page_size). page_size is a multiple of
 * 64, so a key tile never straddles two pages. */
int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                 const int* cu_seqlens_q, const int* seqused_k, const int* block_table,
                 int B, int max_seqlen_q, int total_q, int num_pages, int page_size, int max_pages,
                 int Hq, int Hkv, int d, int causal, float scale, void* stream);

/* Same as fa_fwd_paged with fp16 q/k/v/o. */
int fa_fwd_paged_f16(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                     const int* cu_seqlens_q, const int* seqused_k, const int* block_table,
                     int B, int max_seqlen_q, int total_q, int num_pages, int page_size,
                     int max_pages, int Hq, int Hkv, int d, int causal, float scale, void* stream);

/* Split-KV forms of the two calls above, for batches whose sequences have few query rows and
 * many keys (decoding): the key tiles of every sequence are cut into chunks of tps tiles,
 * tps = ceil(ceil(Kmax / key_tile) / num_splits), where Kmax bounds every sequence's key count
 * (fa_fwd_paged_splitkv: max_pages * page_size; fa_fwd_varlen_splitkv: total_k) and key_tile
 * is 64 keys (d = 128) or 32 (d = 256). Chunk s of a sequence is computed by its own
 * workgroups, which write their normalised output O_s and LSE_s (fp32) to the workspace; a
 * second kernel merges them exactly, LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s
 * (the merge of the dense split-KV call above). The result is the operation of
 * fa_fwd_varlen / fa_fwd_paged (same layouts, masks, empty-row convention and errors); only
 * the rounding order differs. Packed query rows that belong to no sequence receive
 * unspecified values (the calls without splits leave them untouched).
 *
 * workspace: caller-owned device memory of at least
 *   fa_fwd_var_splitkv_workspace_bytes(total_q, Hq, d, num_splits) = num_splits*Hq*total_q*(d+1)*4
 * bytes, 16-byte aligned (FA_ERR_WORKSPACE otherwise); contents on entry do not matter.
 * num_splits: 1..256 (FA_ERR_SHAPE otherwise). */
size_t fa_fwd_var_splitkv_workspace_bytes(int total_q, int Hq, int d, int num_splits);

/* The library's split count for such a batch (0: call the form without splits). key_bound is
 * the Kmax above. Measured on MI355X: decode-shaped batches (at most 64 query rows per
 * sequence) over long caches gain about a third in K/V bandwidth; prefill batches only lose
 * (the partials' traffic), so they get 0. */
int fa_fwd_var_num_splits(int B, int max_seqlen_q, int key_bound, int Hq, int d);

int fa_fwd_varlen_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes,
                          const int* cu_seqlens_q, const int* cu_seqlens_k, const int* seqused_k,
                          int B, int max_seqlen_q, int total_q, int total_k,
                          int Hq, int Hkv, int d, int causal, float scale, int num_splits, void* stream);

/* Same as fa_fwd_varlen_splitkv with fp16 q/k/v/o. */
int fa_fwd_varlen_splitkv_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                              void* workspace, size_t workspace_bytes,
                              const int* cu_seqlens_q, const int* cu_seqlens_k, const int* seqused_k,
                              int B, int max_seqlen_q, int total_q, int total_k,
                              int Hq, int Hkv, int d, int causal, float scale, int num_splits,
                              void* stream);

int fa_fwd_paged_splitkv(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                         void* workspace, size_t workspace_bytes,
                         const int* cu_seqlens_q, const int* seqused_k, const int* block_table,
                         int B, int max_seqlen_q, int total_q, int num_pages, int page_size,
                         int max_pages, int Hq, int Hkv, int d, int causal, float scale, int num_splits,
                         void* stream);

/* Same as fa_fwd_paged_splitkv with fp16 q/k/v/o. */
int fa_fwd_paged_splitkv_f16(const void* q, const void* k_cache, const void* v_cache, void* o,
                             float* lse, void* workspace, size_t workspace_bytes,
                             const int* cu_seqlens_q, const int* seqused_k, const int* block_table,
                             int B, int max_seqlen_q, int total_q, int num_pages, int page_size,
                             int max_pages, int Hq, int Hkv, int d, int causal, float scale,
                             int num_splits, void* stream);

/* Grid order, for tests that look for races between workgroups (a scheduling race shows up as
 * a result that depends on the order in which workgroups run). After fa_set_grid_order(mul,
 * add) with mul != 0, every later launch of this library in the process (forward, split-KV
 * merge, fp8, head dim 512, backward) maps workgroup i of a grid of n workgroups to work item
 * (i * m + add mod n) mod n, where m is the first value >= max(mul mod n, 1) coprime with n: a
 * permutation of the work items, under which every result must stay bitwise the same.
 * fa_set_grid_order(0, 0) restores the natural order (item i), which is the default. The
 * setting is process-wide and read at launch; no HIP call is made. Returns FA_OK. */
int fa_set_grid_order(unsigned mul, unsigned add);

/* Static, NUL-terminated description of an fa_status code (never NULL). */
const char* fa_strerror(int code);

/* Host-only argument check shared by both entry points: returns the fa_status that
 * fa_fwd would return for these arguments before launching anything (FA_OK when the
 * launch would proceed). Makes no HIP call. */
int fa_fwd_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale);

/*
 * Backward pass: gradients of sum(O * dout) with respect to q, k and v, for the forward
 * above ("[RFC] FA4 - head_dim=256 & head_dim=512", Phase 1 "Backward kernel").
 *
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D) with D_i = sum_d dO_id O_id,
 *   dQ = scale * dS K,  dK = scale * dS^T Q,  P = exp(scale * Q K^T - LSE) (causal-masked).
 * For grouped-query heads dK/dV of a KV head sum over its query heads.
 *
 * Inputs: q, k, v as for fa_fwd; o and lse as produced by fa_fwd with the same arguments;
 * dout [B, Nq, Hq, d] (same element type). Outputs: dq [B, Nq, Hq, d], dk and dv
 * [B, Nk, Hkv, d] (element type of the inputs; fully overwritten). workspace: caller-owned
 * device memory of at least fa_bwd_workspace_bytes(B, Nq, Hq) bytes, 4-byte aligned; it
 * receives D (fp32 [B, Hq, Nq]) and holds no state between calls. Same execution and error
 * rules as fa_fwd (FA_ERR_WORKSPACE for a missing or short workspace); two kernels run in
 * order on `stream`.
 */
size_t fa_bwd_workspace_bytes(int B, int Nq, int Hq);

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, void* workspace,
           size_t workspace_bytes, int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal,
           float scale, void* stream);

/* Same as fa_bwd with fp16 tensors. */
int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, int B, int Nq, int Nk, int Hq, int Hkv, int d,
               int causal, float scale, void* stream);

/*
 * Allocation-free backward pass, for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): fa_bwd's operation, layouts and kernels (bf16), with D kept in a device array
 * of the library itself (32 MiB per GPU, FA_BWD_NOALLOC_MAX_ROWS fp32 rows, allocated when
 * the library's code object is loaded on that GPU and held until the process ends). The
 * call allocates nothing. The first call on a GPU resolves that GPU's copy of the array
 * once (hipGetSymbolAddress, with the GPU current); a failure there returns FA_ERR_LAUNCH.
 * Limit: B * Hq * Nq <= FA_BWD_NOALLOC_MAX_ROWS, else FA_ERR_SCRATCH (checked on the host
 * before any HIP call). All calls on one GPU share its array: calls that overlap in time on
 * one GPU (different streams, or threads) race on it and give wrong gradients; serialise
 * them. Nothing needs clearing between calls (every launch writes all of D before reading it).
 */
#define FA_BWD_NOALLOC_MAX_ROWS (8u << 20)

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq,
                   int Hkv, int d, int causal, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
