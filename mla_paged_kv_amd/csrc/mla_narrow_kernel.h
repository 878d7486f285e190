// Split-KV kernel of the paged MLA decode library for units of at most 16
// query rows, written for gfx950 (CDNA4).
//
// A unit of few rows -- the 8 or 16 heads a rank actually computes out of a
// padded head set (DeepLink-org "FlashMLA vLLM Optimization" page,
// background), one query token each -- fills one 16-row column block of
// v_mfma_f32_16x16x32 exactly, so no MFMA work goes to rows that do not
// exist.  With the matrix cores this lightly loaded, a tile's time is its
// gather's latency, so the kernel is built to keep many rows in flight.
//
// One workgroup = one part of the tile-scheduler metadata: 4 wavefronts, one
// per SIMD.  The part's segments (unit, block range, slot) are walked as one
// stream of 64-token tiles (a page of the block table, or 64 entries of the
// index list).  Wavefront w owns tile rows (tokens) 16w..16w+15 of every tile
// and runs its own online softmax over them:
//   gather            each lane loads 16-byte chunks 4k + g (g = lane / 16) of
//                     tile row lane % 16 straight into registers -- exactly
//                     the A operand of the QK product -- DEPTH tiles ahead,
//                     so 4 x DEPTH x 16 rows are in flight per workgroup;
//   S^T = K . Q^T     v_mfma_f32_16x16x32: K from those registers, Q^T (all 16
//                     query rows) resident for the segment;
//   softmax           fp32, base 2; each lane holds 4 tokens of one query row,
//                     the row maximum over the wavefront's 16 tokens takes two
//                     lane exchanges; the reference maximum moves only when it
//                     grows by more than 2^8 (the result does not depend on it);
//   O^T += V^T . P^T  v_mfma_f32_16x16x16 over the wavefront's 16 tokens and
//                     all 512 value columns: the score registers are already
//                     the P^T operand, and V^T comes from the wavefront's own
//                     rows written to LDS and read back with the transpose read.
// The wavefronts never exchange data inside a segment (no workgroup barrier
// per tile).  At a segment's end they merge their (maximum, sum, O) states
// through LDS -- the LSE merge of split-KV decode, inside the workgroup -- and
// each wavefront writes 128 of the 512 output columns: 16-bit O and the LSE
// for a segment covering its whole unit, fp32 O and a base-2 LSE into the
// workspace slot of a split segment (merged later by the combine kernel).
// This follows the structure of the deepep.org usage page (tile scheduler,
// block-table manager; QK^T, scaled softmax, output stages); sparse gathering
// follows the upstream FlashMLA README ("Sparse Attention (indices tensor)").
//
// All memory reads are buffer loads into registers that the compiler sees and
// orders itself; rows past a request's length (dense) or behind an invalid
// index (sparse) are read past the end of their buffer resource, which
// returns zeros, and are masked out of the softmax.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "mla_kernels.h"

namespace mla {

namespace nk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Uniform metadata reads go through the constant address space (scalar loads).
typedef const __attribute__((address_space(4))) int32_t cint;
// a segment record (unit, first block, end block, slot), read as one scalar load
typedef int32_t i32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef const __attribute__((address_space(4))) i32x4a cseg;
__device__ __forceinline__ cint* as_const(const int32_t* ptr) { return (cint*)(uintptr_t)ptr; }

constexpr int kRows = 16;                 // query rows per workgroup
constexpr int kPage = 64;                 // tokens per tile (the scheduler's block)
constexpr int kWaves = 4;                 // wavefronts per workgroup
constexpr int kWaveRows = kPage / kWaves;  // tile rows per wavefront (16)
constexpr int kDV = 512;                  // value width
constexpr int kCB = kDV / 16;             // 16-column output blocks (32)
constexpr int kOwn = kCB / kWaves;        // blocks each wavefront writes out (8)
constexpr int kVRow = kDV * 2;            // bytes of one staged V row
constexpr int kVStage = kWaveRows * kVRow;  // staged V rows of one wavefront (16 KB)
// segment-end merge: each wavefront hands the 24 blocks it does not write to
// their writers (owner, source, block, lane) -> 16 bytes
constexpr int kXBytes = kWaves * (kWaves - 1) * kOwn * 64 * 16;  // 96 KB
static_assert(kWaves * kVStage <= kXBytes, "the V stages live inside the merge area");
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference maximum may lag
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
template <bool F16>
__device__ __forceinline__ unsigned short f2e(float x) {
  if constexpr (F16)
    return __builtin_bit_cast(unsigned short, (_Float16)x);
  else
    return __builtin_bit_cast(unsigned short, (__bf16)x);
}
// Workgroup barrier for LDS traffic: waits for this wavefront's LDS accesses
// only (not for the tile loads in flight), then the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// the four lanes of a query row (lane % 16 equal) combined
__device__ __forceinline__ float row_max4(float v) {
  v = smax(v, __shfl_xor(v, 16));
  return smax(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float row_sum4(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// v_mfma_f32_16x16x32 (QK): A (16 x 32) lane l holds row l % 16, k = 8 (l / 16)
// .. +7; B (32 x 16) lane l holds column l % 16, k = 8 (l / 16) .. +7; C (16 x
// 16) register j of lane l is row 4 (l / 16) + j, column l % 16.
// v_mfma_f32_16x16x16 (PV): the same with k = 4 (l / 16) .. +3.
//
// The matrix-core instructions are inline assembly so that their register
// classes are the kernel's: the tile rows in flight, Q^T and the scores in
// VGPRs, the output accumulator in AGPRs (the compiler gives every MFMA
// result of a function one class, and together they exceed either file).  The
// wait states the compiler cannot see are written out: each MFMA statement
// starts with 4 (a VALU instruction -- a P conversion, an accumulator clear,
// or a register the compiler moves back from an AGPR -- may write one of its
// operands right before it), and 16 come before a VALU read of an MFMA result
// (at least 11 are needed), tied to the result registers so that no read is
// scheduled above them.
__device__ __forceinline__ void mfma_wait_result() { asm volatile("s_nop 7\n\ts_nop 7" ::: "memory"); }
__device__ __forceinline__ void mfma_wait_result(f32x4& c) { asm volatile("s_nop 7\n\ts_nop 7" : "+v"(c)); }
// Keeps a value in AGPRs.
__device__ __forceinline__ void pin_agpr(f32x4& x) { asm volatile("" : "+a"(x)); }
// c (VGPRs) = a . b (+ c unless first); a: K rows, b: Q^T (VGPRs)
template <bool F16>
__device__ __forceinline__ void mfma_qk(f32x4& c, const bf16x8& a, const bf16x8& b, bool first) {
  if constexpr (F16) {
    if (first)
      asm volatile("s_nop 3\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else
      asm volatile("s_nop 3\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  } else {
    if (first)
      asm volatile("s_nop 3\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else
      asm volatile("s_nop 3\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  }
}
// c (AGPRs) += a . b; a: V^T, b: P^T (VGPRs).  (One form only: a second,
// from-zero form on a segment's first tile would make the compiler keep two
// copies of the accumulator; it is cleared at the segment start instead.)
template <bool F16>
__device__ __forceinline__ void mfma_pv(f32x4& c, const s16x4& a, const s16x4& b) {
  if constexpr (F16)
    asm volatile("s_nop 3\n\tv_mfma_f32_16x16x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 3\n\tv_mfma_f32_16x16x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Staged V rows: 16-byte chunk k of row t (t < 16) sits at chunk k ^ vsw(t).
// The transpose read of a 16-column block takes 8 rows x 2 chunks per half
// wavefront, and the row writes 16 rows x 1 chunk per quarter: vsw maps both
// onto distinct bank groups.
__host__ __device__ constexpr int vsw(int t) { return ((t & 7) << 1) | (t >> 3); }

// 8 e4m3 values (byte i of x = value i) times their group's scale, each
// product rounded to fp32 and then to bf16 (nearest even): the dequantized
// values of the upstream FlashMLA README's "FP8 KV Cache" format.
__device__ __forceinline__ bf16x8 dequant8(u32x2 x, float sc) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(x[e], false) * sc;
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(x[e], true) * sc;
    w[2 * e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
    w[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
  }
  return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}

// Workgroups are dispatched to the 8 XCDs round-robin; each XCD gets a
// contiguous run of parts, so neighbouring parts (often the pieces of one
// request, with the same queries) share an L2.
__device__ __forceinline__ int logical_group(int id, int total) {
  constexpr int kXcd = 8;
  const int xcd = id % kXcd, k = id / kXcd;
  const int per = total / kXcd, rem = total % kXcd;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + k;
}

}  // namespace nk

// D_QK: cache row width (576 or 512); SPARSE: rows through top-k index lists
// (pools whose byte size fits 32-bit offsets); F16: fp16 q, cache and output;
// FP8: 656-byte "FP8 with scale" cache rows (d_qk 576, bf16 q), dequantized in
// the registers they are loaded into, by the wavefront that owns their token;
// DEPTH: tiles in flight per wavefront.
template <int D_QK, bool SPARSE, bool F16, bool FP8, int DEPTH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_narrow(SplitKVParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using namespace nk;
  constexpr int NK = D_QK / 32;   // QK k-steps
  constexpr int NV = kDV / 32;    // k-steps holding the value columns
  constexpr int ROWB = FP8 ? kFp8RowBytes : D_QK * 2;  // bytes of one cache row
  static_assert(DEPTH >= 2 && DEPTH <= 4, "tiles in flight");
  static_assert(!FP8 || (D_QK == 576 && !F16), "FP8 rows: 512 e4m3 + 64 bf16 RoPE values, bf16 q");
  constexpr int NE = FP8 ? kDV / 32 : 1;  // FP8: k-steps held as e4m3 bytes (the value columns)
  // FP8: the dot product over d_qk does not depend on the order of its terms,
  // so k-step ks (< NE) of lane group g takes value columns 8 fp8_chunk(ks, g)
  // .. +7 -- for K and Q alike -- and a lane's e4m3 bytes of two k-steps are
  // 16 consecutive bytes, one load.  (bf16: chunk 4 ks + g.)
  auto fp8_chunk = [](int ks, int gg) { return 8 * (ks >> 1) + 2 * gg + (ks & 1); };
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kXBytes];
  __shared__ float xstat[3][kWaves][kRows];  // per-wavefront row maxima, sums, exact maxima

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int r = lane & 15;  // query row (QK B / C column), tile row (QK A row)
  const int g = lane >> 4;  // k-group of the MFMA operands

  // the metadata pointer, the shape words and the output pointers are
  // requested with the launch's part count, so the header reads below do not
  // wait for further rounds of argument loads
  asm volatile("" ::"s"(p.meta), "s"(p.num_parts), "s"(p.row_blocks), "s"(p.rows), "s"(p.s_q),
               "s"(p.h_q), "s"(p.heads), "s"(p.lse_base2), "s"(p.topk), "s"(p.num_rows), "s"(p.out),
               "s"(p.lse), "s"(p.ws_o), "s"(p.ws_lse), "s"(p.max_logits), "s"(p.ws_max));
  const int part = logical_group(blockIdx.x, p.num_parts);
  cint* meta = as_const(p.meta);
  // the grid covers p.num_parts parts, the device header says how many exist
  // (fewer only when the metadata was built on the device; header word 15 is
  // -1 when the device scheduler rejected the lengths).  The header words and
  // the part's segment range are independent reads, requested together before
  // anything branches on them (one memory round trip, not three).
  const int h_parts = meta[0], h_segs = meta[12], h_status = meta[15];
  const int seg_begin = meta[kMetaHeaderInts + part];
  const int seg_end = meta[kMetaHeaderInts + part + 1];
  asm volatile("" ::"s"(h_parts), "s"(h_segs), "s"(h_status), "s"(seg_begin), "s"(seg_end));
  const bool meta_bad = h_status == -1;
  if (part >= h_parts && !meta_bad) return;
  cint* segs = meta + h_segs;
  auto seg_u = [&](int s) __attribute__((always_inline)) { return segs[4 * s + 0]; };
  auto seg_slot = [&](int s) __attribute__((always_inline)) { return segs[4 * s + 3]; };
  auto seg_rec = [&](int s) __attribute__((always_inline)) { return *(cseg*)(segs + 4 * s); };

  const bool row_ok = r < p.rows;
  const int qr = row_ok ? r : p.rows - 1;  // rows past the unit's last read it (never written)
  // output row of query row rr of unit u: dense rows are (query token, head)
  // pairs of a request, sparse units are single query tokens
  auto row_index = [&](int u, int rr) __attribute__((always_inline)) -> size_t {
    int b, iq, h;
    if constexpr (SPARSE) {
      b = u / p.s_q;
      iq = u - b * p.s_q;
      h = rr;
    } else {
      b = u;
      iq = rr / p.heads;
      h = rr - iq * p.heads;
    }
    return (size_t(b) * p.s_q + iq) * p.h_q + h;
  };
  // cache positions this lane's row may see (bottom-right causal alignment)
  auto visible = [&](int L) __attribute__((always_inline)) -> int {
    if (!p.causal) return L;
    const int n = L - p.s_q + qr / p.heads + 1;
    return n < 0 ? 0 : (n > L ? L : n);
  };

  // ---- output ----
  // Wavefront w writes column blocks 8w..8w+7 (columns 16 cb + 4 g + j of
  // row r); wavefront 0's lanes 0..15 write the row statistics.
  auto store_block = [&](size_t orow, int slot, int cb, const f32x4& v) __attribute__((always_inline)) {
    if (slot < 0) {
      uint16_t* o = p.out + orow * kDV + 16 * cb + 4 * g;
      const uint32_t lo = uint32_t(f2e<F16>(v[0])) | (uint32_t(f2e<F16>(v[1])) << 16);
      const uint32_t hi = uint32_t(f2e<F16>(v[2])) | (uint32_t(f2e<F16>(v[3])) << 16);
      *reinterpret_cast<uint2*>(o) = uint2{lo, hi};
    } else {
      float* o = p.ws_o + (size_t(slot) * p.rows + r) * kDV + 16 * cb + 4 * g;
      *reinterpret_cast<f32x4*>(o) = v;
    }
  };
  auto store_stats = [&](size_t orow, int slot, float lse2, float mx) __attribute__((always_inline)) {
    if (wave != 0 || g != 0) return;
    if (slot < 0) {
      p.lse[orow] = p.lse_base2 ? lse2 : lse2 * kLn2;
      if (p.max_logits) p.max_logits[orow] = mx;
    } else {
      const size_t wrow = size_t(slot) * p.rows + r;
      p.ws_lse[wrow] = lse2;
      if (p.max_logits) p.ws_max[wrow] = mx;
    }
  };
  // a segment without tokens: O = 0, LSE = -inf
  auto write_empty = [&](int u, int slot) __attribute__((always_inline)) {
    if (!row_ok) return;
    const size_t orow = row_index(u, r);
#pragma unroll
    for (int k = 0; k < kOwn; ++k) store_block(orow, slot, kOwn * wave + k, f32x4{0.f, 0.f, 0.f, 0.f});
    store_stats(orow, slot, -__builtin_inff(), -__builtin_inff());
  };

  // Lengths the device scheduler rejected: every output row of the call gets
  // O = 0 and LSE = NaN (and max_logits = NaN); part k takes units k, k + grid
  // parts, ...
  if (meta_bad) {
    if (!row_ok) return;
    for (int u = part; u < meta[5]; u += p.num_parts) {
      const size_t orow = row_index(u, r);
      uint16_t* o = p.out + orow * kDV + 128 * wave + 32 * g;
#pragma unroll
      for (int c = 0; c < 32; c += 8) *reinterpret_cast<uint4*>(o + c) = uint4{0, 0, 0, 0};
      if (wave == 0 && g == 0) {
        p.lse[orow] = __builtin_nanf("");
        if (p.max_logits) p.max_logits[orow] = __builtin_nanf("");
      }
    }
    return;
  }

  // ---- tile stream of the part ----
  struct Tile {
    int s, blk, u;
    bool last;
  };
  int la_b1 = 0, la_u = 0;  // cached segment of the furthest tile looked up
  auto first_tile_from = [&](int s2) __attribute__((always_inline)) -> Tile {
    // segments without tiles are passed over; each record is one load
    i32x4a rec = s2 < seg_end ? seg_rec(s2) : i32x4a{0, 0, 0, 0};
    while (s2 < seg_end && rec[1] == rec[2]) {
      ++s2;
      if (s2 < seg_end) rec = seg_rec(s2);
    }
    if (s2 >= seg_end) return Tile{seg_end, 0, 0, true};
    la_u = rec[0];
    la_b1 = rec[2];
    return Tile{s2, rec[1], la_u, rec[1] + 1 >= la_b1};
  };
  auto next_tile = [&](const Tile& t) __attribute__((always_inline)) -> Tile {
    if (t.s >= seg_end) return t;
    if (!t.last) return Tile{t.s, t.blk + 1, t.u, t.blk + 2 >= la_b1};
    return first_tile_from(t.s + 1);
  };

  // What a tile's gather needs, read one tile ahead of it.  Sparse: this
  // lane's index (tile row 16 w + r); dense: the page and the request length.
  // The reads are unconditional (a tile past the stream's end reads unit 0's
  // first entries), so every step issues the same memory operations.
  // The loaded index is not used here (only where the tile is issued, a step
  // later): any use waits for the load, and with it for every older one.
  struct Meta {
    int idx, phys, len;
    bool in_list;  // sparse: the lane's position is inside the index list
  };
  auto fetch_meta = [&](const Tile& t) __attribute__((always_inline)) -> Meta {
    Meta m{-1, 0, 0, false};
    if constexpr (SPARSE) {
      const int pos = t.blk * kPage + kWaveRows * wave + r;
      m.in_list = pos < p.topk;
      m.idx = p.indices[size_t(t.u) * p.topk + (m.in_list ? pos : p.topk - 1)];
    } else {
      m.phys = as_const(p.block_table)[size_t(t.u) * p.bt_stride + t.blk];
      m.len = as_const(p.seqlens)[t.u];
    }
    return m;
  };

  // ---- registers ----
  // tile rows in flight (row r of the wavefront's 16): bf16 chunk 4 ks + g;
  // FP8 rows: e4m3 bytes 64 j + 16 g .. +15 of the value columns (kq, the
  // values of k-steps 2 j and 2 j + 1, see fp8_chunk), the row's 4 group
  // scales (ksc) and the RoPE chunks 4 j + g (kr, j = ks - 16)
  bf16x8 kr[DEPTH][FP8 ? NK - NE : NK];
  u32x4 kq[DEPTH][NE / 2 > 0 ? NE / 2 : 1];
  f32x4 ksc[DEPTH];
  Tile sl_t[DEPTH];      // the tile each slot holds
  bool sl_ok[DEPTH];     // the slot holds a tile of the stream
  uint32_t sl_vm[DEPTH];  // sparse: valid rows of the wavefront's 16 (bit t)
  bf16x8 qf[NK];         // Q^T (B operand of QK): chunk 4 ks + g of query row qr
  f32x4 acc[kCB];        // O^T: register j of block cb = column 16 cb + 4 g + j, row r
  float m_run = -__builtin_inff(), m_exact = -__builtin_inff(), l_part = 0.f;
  bool seg_first = true;
  int n_vis = 0;

  auto load_q = [&](int u) __attribute__((always_inline)) {
    const uint16_t* qrow = p.q + row_index(u, qr) * D_QK;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int c = FP8 && ks < NE ? fp8_chunk(ks, g) : 4 * ks + g;
      qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 8 * c);
    }
  };
  auto reset_state = [&]() __attribute__((always_inline)) {
    seg_first = true;
    m_run = -__builtin_inff();
    m_exact = -__builtin_inff();
    l_part = 0.f;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      pin_agpr(acc[cb]);
    }
  };

  // Issues the loads of tile t into slot S (ok = t is a tile of the stream;
  // otherwise every load reads past the end of an empty resource: zeros, no
  // memory traffic).
  auto issue = [&](auto S, const Tile& t, const Meta& m, bool ok) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t off;
    if constexpr (SPARSE) {
      const bool v = ok && m.in_list && m.idx >= 0 && m.idx < p.num_rows;
      sl_vm[s] = uint32_t(__ballot(v)) & 0xFFFFu;  // lanes 0..15 are rows 0..15
      // the pool, with 32-bit byte offsets; an invalid index reads row num_rows
      rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.kv), 0,
                                             int(uint32_t(p.num_rows) * uint32_t(ROWB)), kBufferWord3);
      off = uint32_t(v ? m.idx : p.num_rows) * uint32_t(ROWB);
    } else {
      // the page, ending after the request's last cached row
      // (uniform values, said so: a resource the compiler believes divergent
      // costs a loop over the lanes around every load)
      const int vt = ok ? m.len - t.blk * kPage : 0;
      const int nrow = __builtin_amdgcn_readfirstlane(vt < 0 ? 0 : (vt > kPage ? kPage : vt));
      const int phys = __builtin_amdgcn_readfirstlane(m.phys);
      const uint8_t* pg = reinterpret_cast<const uint8_t*>(p.kv) + size_t(phys) * kPage * ROWB;
      rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pg), 0, nrow * ROWB, kBufferWord3);
      off = uint32_t((kWaveRows * wave + r) * ROWB);
    }
    if constexpr (FP8) {
      // the scales first: the first k-step's dequant then waits for two loads
      ksc[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + kDV, 0, 0));
#pragma unroll
      for (int j = 0; j < NE / 2; ++j)
        kq[s][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * j + 16 * g, 0, 0));
#pragma unroll
      for (int j = 0; j < NK - NE; ++j)
        kr[s][j] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off + kDV + 16 + 16 * (4 * j + g), 0, 0));
    } else {
#pragma unroll
      for (int ks = 0; ks < NK; ++ks)
        kr[s][ks] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * ks + 16 * g, 0, 0));
    }
    sl_t[s] = t;
    sl_ok[s] = ok;
  };

  // LDS addresses of this lane's staged V (wavefront w's 16 rows at w x 16 KB)
  uint8_t* const vst = lds + wave * kVStage;
  // row writes: chunk 4 ks + g of row r -> (4 ks + g) ^ vsw(r); the XOR only
  // touches the low 4 bits, so 4 per-lane bases (ks % 4) plus a compile-time
  // 64 ks bytes cover every k-step
  int vw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vw[j] = r * kVRow + 16 * (((4 * j + g) ^ vsw(r)) - 4 * j);
  // FP8: chunk fp8_chunk(ks, g) = 16 (ks / 4) + fp8_chunk(ks % 4, g), so again
  // 4 bases (ks % 4) plus a compile-time 256 (ks / 4) bytes
  int vw8[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vw8[j] = r * kVRow + 16 * (fp8_chunk(j, g) ^ vsw(r));
  // transpose reads of block cb: rows 4 g + rr (rr = (lane & 15) / 4), columns
  // 16 cb + 4 c .. +3 (c = lane & 3) = chunk 2 cb + c / 2, byte 8 (c & 1);
  // 8 per-lane bases (cb % 8) plus a compile-time 32 cb bytes
  int vr[8];
  {
    const int t = 4 * g + ((lane & 15) >> 2), c = lane & 3;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      vr[j] = t * kVRow + 16 * (((2 * j + (c >> 1)) ^ vsw(t)) - 2 * j) + 8 * (c & 1);
  }

  // ---- segment end: merge the 4 wavefronts' states, write the result ----
  float* const xm = &xstat[0][0][0];
  float* const xl = &xstat[1][0][0];
  float* const xe = &xstat[2][0][0];
  auto finish_segment = [&](int u, int slot) __attribute__((always_inline)) {
    mfma_wait_result();  // the last PV product has landed before it is read out
    const float l_w = row_sum4(l_part);
    if (g == 0) {
      xm[kRows * wave + r] = m_run;
      xl[kRows * wave + r] = l_w;
      xe[kRows * wave + r] = m_exact;
    }
    lds_barrier();  // every wavefront's PV is done: the V stages are free
    float M = -__builtin_inff(), E = -__builtin_inff();
    float mw[kWaves], lw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = xm[kRows * w + r];
      lw[w] = xl[kRows * w + r];
      M = smax(M, mw[w]);
      E = smax(E, xe[kRows * w + r]);
    }
    float L = 0.f, a_me = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float a = mw[w] == -__builtin_inff() ? 0.f : fast_exp2(mw[w] - M);
      L += a * lw[w];
      if (w == wave) a_me = a;
    }
    const bool empty = !(L > 0.f) || seg_first;
    const float f = empty ? 0.f : a_me / L;
    const float lse2 = empty ? -__builtin_inff() : M + fast_log2(L);
    // hand the blocks other wavefronts write to them
    f32x4* const xo = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int o = cb / kOwn;
      if (o == wave) continue;
      const int src = wave < o ? wave : wave - 1;
      pin_agpr(acc[cb]);
      xo[((o * (kWaves - 1) + src) * kOwn + cb % kOwn) * 64 + lane] = acc[cb] * f;
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
    const size_t orow = row_index(u, r);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      if (cb / kOwn != wave) continue;  // acc is indexed by compile-time blocks only
      pin_agpr(acc[cb]);
      f32x4 v = acc[cb] * f;
#pragma unroll
      for (int src = 0; src < kWaves - 1; ++src)
        v += xo[((wave * (kWaves - 1) + src) * kOwn + cb % kOwn) * 64 + lane];
      if (row_ok) store_block(orow, slot, cb, v);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (row_ok) store_stats(orow, slot, lse2, E);
    lds_barrier();  // the merge area is read before the next tile's V is staged
  };

  // ---- one tile: QK^T, softmax, PV ----
  auto compute = [&](auto S) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    // S^T of the wavefront's 16 tokens x 16 query rows, one accumulation chain
    f32x4 st;  // st[j]: token 16 w + 4 g + j, query row r
    if constexpr (FP8) {
      // dequantized k-step by k-step; the value columns go to the V stage
      // at their own columns (chunk fp8_chunk(ks, g))
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        bf16x8 a;
        if (ks < NE) {
          const u32x4 w = kq[s][ks < NE ? ks >> 1 : 0];
          a = dequant8((ks & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]}, ksc[s][(ks < NE ? ks : 0) / 4]);
        } else {
          a = kr[s][ks < NE ? 0 : ks - NE];
        }
        mfma_qk<F16>(st, a, qf[ks], ks == 0);
        if (ks < NV) *reinterpret_cast<bf16x8*>(vst + vw8[ks & 3] + 256 * (ks >> 2)) = a;
      }
      mfma_wait_result(st);
    } else {
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) mfma_qk<F16>(st, kr[s][ks], qf[ks], ks == 0);
      mfma_wait_result(st);
      // the value columns into the wavefront's V stage
#pragma unroll
      for (int ks = 0; ks < NV; ++ks)
        *reinterpret_cast<bf16x8*>(vst + vw[ks & 3] + 64 * ks) = kr[s][ks];
    }
    // the slot's registers are free from here: its refill must not be
    // scheduled above these reads of it (both would be live at once)
    __builtin_amdgcn_sched_barrier(0);
    return st;
  };

  auto softmax_pv = [&](const Tile& t, uint32_t vmask, f32x4 st) __attribute__((always_inline)) {
    float mloc = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bool vis;
      if constexpr (SPARSE)
        vis = (vmask >> (4 * g + j)) & 1u;
      else
        vis = t.blk * kPage + kWaveRows * wave + 4 * g + j < n_vis;
      st[j] = vis ? st[j] : -__builtin_inff();
      mloc = smax(mloc, st[j]);
    }
    mloc = row_max4(mloc) * p.scale_log2;
    m_exact = smax(m_exact, mloc);
    const bool grow = mloc > m_run + kRescaleSlack;
    if (__any(grow)) {
      const float m_new = grow ? mloc : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
      m_run = m_new;
      l_part *= alpha;
      if (!seg_first) {  // (before the first tile the accumulator is zero)
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          pin_agpr(acc[cb]);  // read out of the AGPRs here, not earlier
          acc[cb] *= alpha;
          pin_agpr(acc[cb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    const float neg_m = m_run == -__builtin_inff() ? 0.f : -m_run;
    s16x4 pb;  // P^T operand: tokens 4 g + j of query row r
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = fast_exp2(__builtin_fmaf(st[j], p.scale_log2, neg_m));
      lsum += e;
      pb[j] = (short)f2e<F16>(e);
    }
    l_part += lsum;
    // O^T += V^T . P^T over the wavefront's 16 tokens
    constexpr int VD = 4;  // V^T fragments read this many blocks ahead
    {
      s16x4 vf[VD + 1];
      auto load_v = [&](int cb) __attribute__((always_inline)) {
        vf[cb % (VD + 1)] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vst + vr[cb & 7] + 32 * cb));
      };
#pragma unroll
      for (int cb = 0; cb < VD; ++cb) load_v(cb);
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        if (cb + VD < kCB) load_v(cb + VD);
        mfma_pv<F16>(acc[cb], vf[cb % (VD + 1)], pb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    seg_first = false;
  };

  // leading segments without tiles (one scalar load per segment record)
  int cs0 = seg_begin;
  i32x4a rec0 = cs0 < seg_end ? seg_rec(cs0) : i32x4a{0, 0, 0, 0};
  while (cs0 < seg_end && rec0[1] == rec0[2]) {
    write_empty(rec0[0], rec0[3]);
    ++cs0;
    if (cs0 < seg_end) rec0 = seg_rec(cs0);
  }
  if (cs0 >= seg_end) return;

  // prologue: the first segment's queries, the first DEPTH tiles
  la_u = rec0[0];
  la_b1 = rec0[2];
  Tile nt{cs0, rec0[1], la_u, rec0[1] + 1 >= la_b1};
  Meta nmeta = fetch_meta(nt);
  load_q(nt.u);
  if constexpr (!SPARSE) n_vis = visible(nmeta.len);
  reset_state();
  // The metadata of the tile after is requested before a tile's row loads:
  // the vector-memory counter completes in order, so waiting for metadata
  // requested after a tile's loads would wait for those loads too.
  auto fill = [&](auto S) __attribute__((always_inline)) {
    const Tile t_in = nt;
    const Meta m_in = nmeta;
    nt = next_tile(nt);
    nmeta = fetch_meta(nt);
    __builtin_amdgcn_sched_barrier(0);
    issue(S, t_in, m_in, t_in.s < seg_end);
  };
  fill(std::integral_constant<int, 0>{});
  if constexpr (DEPTH > 1) fill(std::integral_constant<int, 1>{});
  if constexpr (DEPTH > 2) fill(std::integral_constant<int, 2>{});
  if constexpr (DEPTH > 3) fill(std::integral_constant<int, 3>{});

  // One step computes the tile in slot S and refills S with the tile DEPTH
  // ahead, in two halves: the QK product, then (rest) the query reload at a
  // segment change, the refill, the softmax, PV and the segment end; rest
  // returns whether the stream goes on.  The loop is rotated so that its head
  // sits right after a refill: on every path into it the newest loads are
  // those of one slot, so the compiler's count of the loads in flight stays
  // exact there and each QK product waits only for its own tile.
  auto rest = [&](auto S, const f32x4& st) __attribute__((always_inline)) -> bool {
    constexpr int s = decltype(S)::value;
    constexpr int sn = (s + 1) % DEPTH;
    const Tile t = sl_t[s];
    const uint32_t vmask = sl_vm[s];
    const bool more = sl_ok[sn];
    // the next segment's queries, once this segment's last QK product is done
    if (t.last && more) load_q(sl_t[sn].u);
    fill(S);
    __builtin_amdgcn_sched_barrier(0);
    softmax_pv(t, vmask, st);
    if (t.last) {
      finish_segment(t.u, seg_slot(t.s));
      const int e_end = more ? sl_t[sn].s : seg_end;
      for (int e = t.s + 1; e < e_end; ++e) write_empty(seg_u(e), seg_slot(e));
      if (more) {
        const int un = sl_t[sn].u;
        if constexpr (!SPARSE) n_vis = visible(as_const(p.seqlens)[un]);
        reset_state();
      }
      // A segment change adds query loads and output stores to the memory
      // operations in flight; draining them here (a wait the compiler sees)
      // keeps its count exact at the loop head.
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    return more;
  };
  static_assert(DEPTH == 2 || DEPTH == 3, "the rotated loop below");
  f32x4 st = compute(std::integral_constant<int, 0>{});
  for (;;) {
    if (!rest(std::integral_constant<int, 0>{}, st)) break;
    st = compute(std::integral_constant<int, 1>{});
    if (!rest(std::integral_constant<int, 1>{}, st)) break;
    if constexpr (DEPTH == 3) {
      st = compute(std::integral_constant<int, 2>{});
      if (!rest(std::integral_constant<int, 2 % DEPTH>{}, st)) break;
    }
    st = compute(std::integral_constant<int, 0>{});
  }
#endif
}

// Launches the narrow kernel (one 4-wavefront workgroup per part) for units of
// at most 16 query rows.
template <bool F16>
hipError_t launch_narrow_t(const SplitKVParams& p, int d_qk, bool sparse, bool fp8, hipStream_t stream) {
  if (p.num_parts <= 0) return hipSuccess;
  const dim3 grid(p.num_parts), block(256);
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, block, 0, stream, p); };
  if constexpr (!F16) {
    if (fp8) {
      // (a lighter ring -- 44 registers per tile -- leaves room for 3 tiles)
      if (sparse) go(mla_narrow<576, true, false, true, 3>);
      else go(mla_narrow<576, false, false, true, 3>);
      return hipGetLastError();
    }
  }
  if (d_qk == 576) {
    if (sparse) go(mla_narrow<576, true, F16, false, 2>);
    else go(mla_narrow<576, false, F16, false, 2>);
  } else {
    if (sparse) go(mla_narrow<512, true, F16, false, 2>);
    else go(mla_narrow<512, false, F16, false, 2>);
  }
  return hipGetLastError();
}

}  // namespace mla
