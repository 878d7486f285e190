/*
 * mla.h -- C ABI of the MI355X (gfx950) paged MLA decode library, libmla.so.
 *
 * Operation.  Multi-head latent attention decode over a paged latent cache, in
 * "MQA mode": every cache token is one row of d_qk bf16 values (576 = 512 NoPE
 * + 64 RoPE, or 512), the value is the first d_v = 512 columns of that same
 * row, and all query heads share the single KV head (upstream FlashMLA README
 * embedded in the DeepLink-org/flashmla-optimization page: "Support matrix" and
 * its footnote on MQA mode; "FP8 KV Cache" for the row split).  Rows sit in
 * 64-token pages reached through a block table (FlashMLA summary page on
 * sourcepulse.org, "How It Works"; deepep.org usage page, "Block Table
 * Manager").  The call sequence is the pages' one: metadata once per decode
 * step from the sequence lengths and head configuration, then one decode call
 * per layer that reuses it (deepep.org usage example; upstream README "Usage /
 * MLA Decoding").  Sparse decode replaces the block table by per-query token
 * indices (upstream README, "Sparse Attention (indices tensor)").
 *
 * For every request b, query token i < s_q and head h, with L = cache_seqlens[b]
 * and n = L (or, when causal, min(L, max(0, L - s_q + i + 1))):
 *     s_t  = softmax_scale * <q[b,i,h,:], K_t>              t < n
 *     lse  = ln sum_t exp(s_t)                              (-inf when n == 0)
 *     out  = sum_t exp(s_t - lse) * K_t[0:d_v]              (0 when n == 0)
 * where K_t is cache row t of request b.  LSE is natural-log; the sparse-prefill
 * equations of the upstream README use base 2 with log2(e)-scaled scores, which
 * is the same value divided by ln 2.
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are device memory owned by the caller; "host" is
 *    host memory owned by the caller.  The library keeps no pointer after it
 *    returns, allocates nothing, and holds no global state other than a
 *    thread-local message for the last error and the static device array of
 *    mla_decode_paged_noalloc (one per GPU, with its address).
 *  - Tensors are dense and row-major (C-contiguous) in the layout stated.
 *  - Decode calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  They neither synchronise nor allocate.
 *  - Return value: MLA_OK (0), a positive warning, or a negative error code.
 *    Errors are detected before any work is enqueued; nothing is written on
 *    error.  mla_strerror() names a code, mla_last_error() gives details.
 *  - Supported by the kernels: h_kv == 1, page_block_size == 64, d_qk in
 *    {576, 512}, d_v == 512 (<= d_qk); q/kvcache/out bf16, or fp16 through the
 *    *_f16 entry points, or a bf16 q with an FP8-with-scale cache through the
 *    *_fp8 entry points.  Anything else returns MLA_E_NOTSUP.
 */
#ifndef MLA_PAGED_KV_MLA_H
#define MLA_PAGED_KV_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MLA_OK = 0,
  /* active_h_q was not in [1, h_q] or not a multiple of 8: all h_q heads are
   * scheduled instead (the fail-closed rule of the DeepLink-org fork's
   * runtime-switch section). */
  MLA_W_ACTIVE_FALLBACK = 1,
  MLA_E_INVAL = -1,  /* bad shape, stride, pointer or argument */
  MLA_E_NOTSUP = -2, /* valid per the pages but not built here (h_kv != 1, ...) */
  MLA_E_NOSPC = -3,  /* metadata array or workspace too small */
  MLA_E_HIP = -4,    /* a HIP launch or query failed */
};

/* Metadata header; identical to the first 16 int32 of the metadata array. */
typedef struct mla_sched_info {
  int32_t num_parts;       /* parts holding >= 1 segment (workgroup columns) */
  int32_t num_segments;    /* (unit, block range, slot) work items */
  int32_t total_slots;     /* fp32 partial-result slots the workspace needs */
  int32_t num_split_units; /* units cut into >= 2 segments (combine work) */
  int32_t max_splits;      /* most segments of any one unit */
  int32_t num_units;       /* dense: batch; sparse: batch * s_q */
  int32_t quota;           /* per-part budget, in 64-token blocks */
  int32_t total_cost;      /* sum over units of blocks + per-segment overhead */
  int32_t target_parts;    /* part count the schedule was built for */
  int32_t overhead;        /* per-segment overhead in blocks (5) */
  int32_t row_blocks;      /* workgroups per part: ceil(rows / G), G = 128 if rows > 64 else 64 */
  int32_t rows;            /* query rows per unit: dense s_q*heads, sparse heads */
  int32_t off_segs;        /* int offset of segs[num_segments][4] = (u, blk0, blk1, slot) */
  int32_t off_num_splits;  /* int offset of num_splits[num_units + 1] (cumulative) */
  int32_t off_split_list;  /* int offset of split_list[num_split_units][2] = (u, slot0) */
  int32_t total_ints;      /* metadata length in int32 */
} mla_sched_info;

/* Library version, e.g. 0x00010000 for 1.0.0. */
int32_t mla_version(void);

/* Short name of a return code (static string). */
const char* mla_strerror(int code);

/* Details of the last non-OK return on the calling thread (static per thread). */
const char* mla_last_error(void);

/* Default part count for `rows` query rows per unit on a device with `num_cus`
 * compute units: max(1, num_cus / ceil(rows / G)), G = 128 if rows > 64 else
 * 64, i.e. one part per workgroup slot (G rows per workgroup, one resident
 * workgroup per CU). */
int32_t mla_default_num_parts(int32_t rows, int32_t num_cus);

/* Upper bound, in int32, of the metadata for `num_units` units and at most
 * `target_parts` parts: 18 + 5 * target_parts + 7 * num_units. */
size_t mla_metadata_capacity(int32_t num_units, int32_t target_parts);

/*
 * mla_get_metadata -- tile scheduler (the pages' get_mla_metadata: deepep.org
 * usage example; upstream README "Usage / MLA Decoding", six-argument form
 * with h_q and topk).  Host only: no HIP call, no device memory.
 *
 *   cache_seqlens_host [batch] int32, host.  Dense mode only (topk == 0);
 *                      may be NULL in sparse mode.  Values must be >= 0.
 *   batch, s_q, h_q, h_kv   shapes of the decode call this metadata serves.
 *   topk               0 = dense paged decode; > 0 = sparse decode with topk
 *                      indices per query token (units are query tokens).
 *   active_h_q         heads actually computed (the first active_h_q); 0 = h_q.
 *                      Must be in [1, h_q] and a multiple of 8 (or equal to
 *                      h_q); otherwise h_q is used and MLA_W_ACTIVE_FALLBACK is
 *                      returned (DeepLink-org fork, runtime-switch section).
 *   num_cus            compute units of the target device (used when
 *                      num_parts == 0).
 *   num_parts          target part count; 0 = mla_default_num_parts(rows, num_cus).
 *   meta_host          [meta_capacity_ints] int32, host: receives the metadata
 *                      array (header, part_ptr, segs, num_splits, split_list).
 *                      The caller copies info->total_ints of it to the device
 *                      for the decode calls.
 *   info               receives the header.
 *
 * Schedule: units of nb = ceil(len / 64) blocks; total = sum(nb + 5);
 * quota = ceil(total / P) + 5; parts are filled greedily in unit order, a unit
 * is cut only when more than the 5-block overhead of budget is left, and a cut
 * unit's segments get consecutive workspace slots.  At most P parts are used.
 * Errors: MLA_E_INVAL (negative/zero shapes, h_q % h_kv, negative length,
 * num_cus and num_parts both 0), MLA_E_NOSPC (meta_capacity_ints too small).
 */
int mla_get_metadata(const int32_t* cache_seqlens_host, int32_t batch, int32_t s_q,
                     int32_t h_q, int32_t h_kv, int32_t topk, int32_t active_h_q,
                     int32_t num_cus, int32_t num_parts, int32_t* meta_host,
                     size_t meta_capacity_ints, mla_sched_info* info);

/*
 * mla_get_metadata_device -- the same tile scheduler run on the GPU, for
 * sequence lengths that are already in device memory (the pages call
 * get_mla_metadata on the device tensor of cache lengths once per decode step:
 * deepep.org usage example).  It enqueues one single-workgroup kernel on
 * `stream` and returns without synchronising, so a decode step needs no host
 * round trip and can be captured in a HIP graph.  The device array it writes
 * is bit-identical to mla_get_metadata's output for the same lengths.
 *
 *   cache_seqlens_dev  [batch] int32, device.  Dense mode only (topk == 0);
 *                      may be NULL in sparse mode.  Read when the kernel runs.
 *   batch ... num_parts  as for mla_get_metadata.
 *   meta_dev           [meta_capacity_ints] int32, device: receives the
 *                      metadata array.  meta_capacity_ints must be at least
 *                      mla_metadata_capacity(units, parts).
 *   info               host: receives a header of upper bounds, which is what
 *                      the decode calls and mla_workspace_bytes need: num_parts
 *                      = the target part count P, num_segments = U + P - 1,
 *                      total_slots = min(U + P - 1, 2(P - 1)), num_split_units
 *                      = min(U, P - 1), max_splits = P; quota and total_cost
 *                      are -1; off_segs, off_num_splits and off_split_list are
 *                      -1, which tells the kernels to read the exact counts
 *                      and offsets from the device header; total_ints = the
 *                      capacity.  Pass this info with meta_dev to the decode
 *                      calls, which then size their grids by the bounds.
 *   stream             hipStream_t (NULL = the null stream).
 *
 * Limits: at most 4096 units and 1024 parts (MLA_E_NOTSUP beyond).  A length
 * below 0 or above 2^24 cannot be reported to the host without a round trip:
 * the kernel then writes an empty schedule (num_parts = num_split_units = 0,
 * total_ints = -1 in the device header, the unit and row counts kept) and a
 * decode call with it writes O = 0 and LSE = NaN (max_logits NaN) into every
 * output row.  Other errors as for mla_get_metadata, plus MLA_E_HIP.
 */
int mla_get_metadata_device(const int32_t* cache_seqlens_dev, int32_t batch, int32_t s_q,
                            int32_t h_q, int32_t h_kv, int32_t topk, int32_t active_h_q,
                            int32_t num_cus, int32_t num_parts, int32_t* meta_dev,
                            size_t meta_capacity_ints, mla_sched_info* info, void* stream);

/* Workspace bytes a decode call with this metadata needs (0 if nothing is
 * split): fp32 partial outputs [total_slots, rows, d_v] then, each 256-byte
 * aligned, fp32 partial log-sum-exps [total_slots, rows] and fp32 partial row
 * maxima [total_slots, rows] (used by mla_sparse_prefill). */
size_t mla_workspace_bytes(const mla_sched_info* info, int32_t d_v);

/*
 * mla_decode_paged -- dense paged MLA decode (the pages' flash_mla_with_kvcache
 * without indices: deepep.org usage example; upstream README "Usage / MLA
 * Decoding").
 *
 *   q              [batch, s_q, h_q, d_qk] bf16, device.
 *   kvcache        [num_blocks, page_block_size, h_kv, d_qk] bf16, device.
 *   block_table    [batch, bt_stride] int32, device.  Entries for logical
 *                  blocks below ceil(cache_seqlens[b] / 64) must be in
 *                  [0, num_blocks); other entries are never read.  Any
 *                  size: a table of 2 GiB or more runs units of more than 64
 *                  query rows on the 64-row kernel (slower, same results).
 *   cache_seqlens  [batch] int32, device; the same values the metadata was
 *                  built from.  Must be <= bt_stride * 64.
 *   dv             value width (first dv columns of each cache row).
 *   causal         0/1; bottom-right aligned (query i sees positions
 *                  <= L - s_q + i).
 *   softmax_scale  multiplies q.k (commonly d_qk^-0.5); must be > 0.
 *   meta_dev, info metadata (device copy) and header from mla_get_metadata
 *                  in dense mode with the same batch, s_q, h_q.
 *   workspace      device, >= mla_workspace_bytes(info, dv) bytes (may be
 *                  NULL when that is 0).
 *   out            [batch, s_q, h_q, dv] bf16, device.
 *   lse            [batch, s_q, h_q] fp32, device.
 * Heads >= the metadata's active head count are not written.
 */
int mla_decode_paged(const void* q, const void* kvcache, const int32_t* block_table,
                     const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                     int32_t h_kv, int32_t d_qk, int32_t dv, int32_t num_blocks,
                     int32_t page_block_size, int32_t bt_stride, int32_t causal,
                     float softmax_scale, const int32_t* meta_dev, const mla_sched_info* info,
                     void* workspace, size_t workspace_bytes, void* out, float* lse,
                     void* stream);

/*
 * mla_decode_sparse -- token-level top-k sparse MLA decode (upstream README,
 * "Sparse Attention (indices tensor)"; the DeepLink-org fork's active-head
 * split/combine kernels).
 *
 *   q              [batch, s_q, h_q, d_qk] bf16, device.
 *   kvcache        [num_blocks, page_block_size, h_kv, d_qk] bf16, device,
 *                  addressed as [num_blocks * page_block_size, h_kv, d_qk].
 *   indices        [batch, s_q, topk] int32, device: block * 64 + offset.  An
 *                  entry < 0 or >= num_blocks * 64 is invalid and skipped; no
 *                  block table is needed.  Any size, as for the block table
 *                  of mla_decode_paged.
 *   meta_dev, info from mla_get_metadata in sparse mode (topk > 0) with the
 *                  same batch, s_q, h_q, topk; its active head count decides
 *                  which heads are computed (the first ones).
 *   out, lse       as for mla_decode_paged; heads >= active are not written.
 */
int mla_decode_sparse(const void* q, const void* kvcache, const int32_t* indices,
                      int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                      int32_t dv, int32_t num_blocks, int32_t page_block_size, int32_t topk,
                      float softmax_scale, const int32_t* meta_dev,
                      const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                      void* out, float* lse, void* stream);

/*
 * The two stages of a decode call, for callers that schedule them separately
 * (the pages name the split-KV and combine kernels as the two hot kernels of
 * sparse decode: DeepLink-org fork, background section).  A decode call is
 * exactly mla_splitkv_* followed by mla_combine on the same stream, with the
 * same metadata, workspace, out and lse.
 *
 * mla_splitkv_paged / mla_splitkv_sparse: same arguments and checks as
 *   mla_decode_paged / mla_decode_sparse.  Writes out/lse of every unit that
 *   the metadata does not split, and the fp32 partials of split units into
 *   the workspace.
 * mla_combine: LSE-merges the workspace partials of every split unit into
 *   out/lse, for the active rows only (the fork's active-head combine).
 *   sparse = 0/1 says which mode the metadata was built for; batch, s_q, h_q
 *   as in the decode call.  Nothing is launched when no unit is split.
 */
int mla_splitkv_paged(const void* q, const void* kvcache, const int32_t* block_table,
                      const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                      int32_t h_kv, int32_t d_qk, int32_t dv, int32_t num_blocks,
                      int32_t page_block_size, int32_t bt_stride, int32_t causal,
                      float softmax_scale, const int32_t* meta_dev, const mla_sched_info* info,
                      void* workspace, size_t workspace_bytes, void* out, float* lse,
                      void* stream);

int mla_splitkv_sparse(const void* q, const void* kvcache, const int32_t* indices,
                       int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                       int32_t dv, int32_t num_blocks, int32_t page_block_size, int32_t topk,
                       float softmax_scale, const int32_t* meta_dev,
                       const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                       void* out, float* lse, void* stream);

int mla_combine(const int32_t* meta_dev, const mla_sched_info* info, int32_t batch, int32_t s_q,
                int32_t h_q, int32_t dv, int32_t sparse, const void* workspace,
                size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * mla_decode_paged_noalloc -- mla_decode_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks and results as
 * mla_decode_paged (bf16), without workspace/workspace_bytes: the fp32 split
 * partials go to a static device array of MLA_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  The call
 * allocates nothing (no hipMalloc, no allocating library routine); the first
 * call on a device looks up that device's array address.
 *
 *   Limit: mla_workspace_bytes(info, dv) must be <= MLA_NOALLOC_SCRATCH_BYTES
 *   (128 MiB: every bundled schedule of up to 256 rows per unit and 256
 *   parts fits), else MLA_E_NOSPC and nothing is enqueued.
 *   Sharing: every call on one GPU uses the same array.  Calls that overlap
 *   on one GPU (different streams, or host threads, with no ordering between
 *   them) race on it; calls ordered on one stream do not.  Nothing in it needs
 *   to start at zero: each call writes every partial its combine reads.
 *   Errors: those of mla_decode_paged, MLA_E_NOSPC as above, MLA_E_HIP if the
 *   device or the array's address cannot be queried.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int mla_decode_paged_noalloc(const void* q, const void* kvcache, const int32_t* block_table,
                             const int32_t* cache_seqlens, int32_t batch, int32_t s_q,
                             int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t dv,
                             int32_t num_blocks, int32_t page_block_size, int32_t bt_stride,
                             int32_t causal, float softmax_scale, const int32_t* meta_dev,
                             const mla_sched_info* info, void* out, float* lse, void* stream);

/*
 * mla_sparse_prefill -- sparse MLA prefill (the pages' flash_mla_sparse_fwd:
 * upstream FlashMLA README, "Sparse MLA Prefill").  For query token i and
 * head h, over the valid entries t of indices[i] (0 <= t < s_kv; -1 or
 * >= s_kv is invalid and skipped):
 *     P_t        = sm_scale * log2(e) * <q[i,h,:], kv[t,:]>
 *     max_logits = max_t P_t                       (-inf if no valid entry)
 *     lse        = log2 sum_t 2^P_t                (base 2; -inf if none)
 *     out        = sum_t 2^(P_t - lse) * kv[t, 0:dv]   (0 if none)
 *
 *   q           [s_q, h_q, d_qk] bf16, device.
 *   kv          [s_kv, h_kv, d_qk] bf16, device (h_kv must be 1).
 *   indices     [s_q, h_kv, topk] int32, device.
 *   sm_scale    > 0.
 *   meta_dev, info  from mla_get_metadata in sparse mode with batch = s_q,
 *               s_q = 1, the same h_q, h_kv and topk (each query token is a
 *               unit); its active head count decides which heads are
 *               computed (the first ones).
 *   workspace   >= mla_workspace_bytes(info, dv) bytes.
 *   out         [s_q, h_q, dv] bf16; max_logits [s_q, h_q] fp32 (may be NULL:
 *               not written); lse [s_q, h_q] fp32, base 2.  Device.
 * d_qk in {576, 512}, dv = 512.  Errors as for mla_decode_sparse.
 */
int mla_sparse_prefill(const void* q, const void* kv, const int32_t* indices, int32_t s_q,
                       int32_t s_kv, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t dv,
                       int32_t topk, float sm_scale, const int32_t* meta_dev,
                       const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                       void* out, float* max_logits, float* lse, void* stream);

/*
 * fp16 inputs (the pages list BF16 and FP16: sourcepulse.org FlashMLA
 * summary, "How It Works" and "Highlighted Details").  Same arguments,
 * checks, metadata and workspace as the entry point without the suffix, with
 * q, kvcache (kv) and out in IEEE fp16 instead of bf16: the products run on
 * the fp16 matrix cores, P is rounded to fp16 before the PV product and the
 * output to fp16 (nearest even); lse (and max_logits) stay fp32.
 */
int mla_decode_paged_f16(const void* q, const void* kvcache, const int32_t* block_table,
                         const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                         int32_t h_kv, int32_t d_qk, int32_t dv, int32_t num_blocks,
                         int32_t page_block_size, int32_t bt_stride, int32_t causal,
                         float softmax_scale, const int32_t* meta_dev,
                         const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                         void* out, float* lse, void* stream);
int mla_splitkv_paged_f16(const void* q, const void* kvcache, const int32_t* block_table,
                          const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                          int32_t h_kv, int32_t d_qk, int32_t dv, int32_t num_blocks,
                          int32_t page_block_size, int32_t bt_stride, int32_t causal,
                          float softmax_scale, const int32_t* meta_dev,
                          const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                          void* out, float* lse, void* stream);
int mla_decode_sparse_f16(const void* q, const void* kvcache, const int32_t* indices,
                          int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                          int32_t dv, int32_t num_blocks, int32_t page_block_size, int32_t topk,
                          float softmax_scale, const int32_t* meta_dev,
                          const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                          void* out, float* lse, void* stream);
int mla_splitkv_sparse_f16(const void* q, const void* kvcache, const int32_t* indices,
                           int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                           int32_t dv, int32_t num_blocks, int32_t page_block_size, int32_t topk,
                           float softmax_scale, const int32_t* meta_dev,
                           const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                           void* out, float* lse, void* stream);
int mla_combine_f16(const int32_t* meta_dev, const mla_sched_info* info, int32_t batch,
                    int32_t s_q, int32_t h_q, int32_t dv, int32_t sparse, const void* workspace,
                    size_t workspace_bytes, void* out, float* lse, void* stream);
int mla_sparse_prefill_f16(const void* q, const void* kv, const int32_t* indices, int32_t s_q,
                           int32_t s_kv, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t dv,
                           int32_t topk, float sm_scale, const int32_t* meta_dev,
                           const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                           void* out, float* max_logits, float* lse, void* stream);

/*
 * FP8 KV cache ("FP8 with scale": upstream FlashMLA README, "FP8 KV Cache";
 * the pages' is_fp8_kvcache flag).  Every cache row is 656 bytes:
 *   bytes   0..511  512 float8 e4m3 values (OCP E4M3FN: bias 7, no infinity,
 *                   S.1111.111 is NaN) -- the NoPE part,
 *   bytes 512..527  4 fp32 scales; scale g applies to values 128g..128g+127,
 *   bytes 528..655  64 bf16 values -- the RoPE part, not quantized.
 * The kernel dequantizes each NoPE value to bf16 as bf16(fp32(v) * scale)
 * (the product rounded to fp32, then to bf16, to nearest even), keeps the
 * RoPE values, and computes exactly as for a bf16 cache whose rows are these
 * 576 values (V = the first 512).  q, out and lse are as for bf16.
 *
 * Same arguments and checks as the bf16 entry points, except:
 *   kvcache   [num_blocks, page_block_size, h_kv, 656] bytes, device,
 *             16-byte aligned (rows are 16-byte aligned since 656 = 41 * 16).
 *   d_qk      must be 576 (MLA_E_NOTSUP otherwise), d_v 512.
 * The metadata and workspace are the same as for a bf16 cache.
 */
int mla_decode_paged_fp8(const void* q, const void* kvcache, const int32_t* block_table,
                         const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                         int32_t h_kv, int32_t d_qk, int32_t dv, int32_t num_blocks,
                         int32_t page_block_size, int32_t bt_stride, int32_t causal,
                         float softmax_scale, const int32_t* meta_dev,
                         const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                         void* out, float* lse, void* stream);

int mla_decode_sparse_fp8(const void* q, const void* kvcache, const int32_t* indices,
                          int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                          int32_t dv, int32_t num_blocks, int32_t page_block_size, int32_t topk,
                          float softmax_scale, const int32_t* meta_dev,
                          const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                          void* out, float* lse, void* stream);

/* The split-KV stage alone for an FP8 cache (then mla_combine), as above. */
int mla_splitkv_paged_fp8(const void* q, const void* kvcache, const int32_t* block_table,
                          const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                          int32_t h_kv, int32_t d_qk, int32_t dv, int32_t num_blocks,
                          int32_t page_block_size, int32_t bt_stride, int32_t causal,
                          float softmax_scale, const int32_t* meta_dev,
                          const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                          void* out, float* lse, void* stream);

int mla_splitkv_sparse_fp8(const void* q, const void* kvcache, const int32_t* indices,
                           int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                           int32_t dv, int32_t num_blocks, int32_t page_block_size, int32_t topk,
                           float softmax_scale, const int32_t* meta_dev,
                           const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                           void* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_KV_MLA_H */
