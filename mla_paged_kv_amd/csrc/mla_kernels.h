// Kernel parameter blocks and launchers of libmla.so (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mla {

constexpr int kMetaHeaderInts = 16;  // int32 header ahead of part_ptr in the metadata
// "FP8 with scale" cache row: 512 e4m3 values, 4 fp32 scales (one per 128
// values), 64 bf16 RoPE values (upstream FlashMLA README, "FP8 KV Cache").
constexpr int kFp8RowBytes = 656;

struct SplitKVParams {
  const uint16_t* q;           // [batch, s_q, h_q, d_qk] bf16 (fp16 for the fp16 kernels)
  const uint16_t* kv;          // [num_blocks * 64] rows: d_qk bf16, or 656-byte FP8 rows (h_kv = 1)
  const int32_t* block_table;  // dense: [batch, bt_stride]
  const int32_t* seqlens;      // dense: [batch]
  const int32_t* indices;      // sparse: [batch * s_q, topk]
  const int32_t* meta;         // device copy of the scheduler metadata
  uint16_t* out;               // [batch, s_q, h_q, 512] bf16
  float* lse;                  // [batch, s_q, h_q] fp32 (natural log)
  float* ws_o;                 // [slots, rows, 512] fp32 partial outputs
  float* ws_lse;               // [slots, rows] fp32 partial LSE (base 2)
  float* max_logits;           // optional [batch, s_q, h_q] fp32 row maxima of the scaled
                               // logits (base 2); null = not written
  float* ws_max;               // [slots, rows] fp32 partial maxima (with max_logits)
  int32_t lse_base2;           // 1: lse is written in base 2, 0: natural log
  int32_t s_q, h_q;
  int32_t heads;      // active heads (first `heads` of h_q)
  int32_t rows;       // query rows per unit
  int32_t bt_stride;
  int32_t num_rows;   // num_blocks * 64 (sparse index bound)
  int32_t topk;
  int32_t causal;
  int32_t num_parts, row_blocks;
  float scale_log2;   // softmax_scale * log2(e)
};

struct CombineParams {
  const int32_t* meta;
  const float* ws_o;
  const float* ws_lse;
  const float* ws_max;  // partial maxima (read when max_logits is set)
  uint16_t* out;
  float* lse;
  float* max_logits;    // optional row maxima output
  int32_t lse_base2;
  int32_t off_split_list, num_split_units;
  int32_t max_splits;  // most splits of any unit (picks the combine layout)
  int32_t out_f16;     // 1: out is fp16, 0: bf16
  int32_t rows, s_q, h_q, heads;
  int32_t sparse;
};

// bf16 / fp16 caches (mla_decode_kernel.h), one launcher per (d_qk, type)
template <int D_QK, bool F16>
hipError_t launch_decode_d(const SplitKVParams& p, bool sparse, hipStream_t stream);
hipError_t launch_decode(const SplitKVParams& p, int d_qk, bool sparse, bool f16, hipStream_t stream);
// The pair kernel (mla_splitkv_kernel.h; wavefront pairs share 32 query rows,
// 64 rows per workgroup): FP8-with-scale caches, and bf16 / fp16 caches for
// units of at most 64 query rows.
hipError_t launch_pairs(const SplitKVParams& p, int d_qk, bool sparse, bool fp8, bool f16,
                        hipStream_t stream);
hipError_t launch_pairs_f16(const SplitKVParams& p, int d_qk, bool sparse, hipStream_t stream);
// The narrow kernel (mla_narrow_kernel.h; units of at most 16 query rows,
// one 16-row MFMA block per workgroup): bf16 / fp16 / FP8-with-scale caches,
// sparse pools whose byte size fits 32-bit offsets.
hipError_t launch_narrow(const SplitKVParams& p, int d_qk, bool sparse, bool fp8, bool f16,
                         hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);

}  // namespace mla
