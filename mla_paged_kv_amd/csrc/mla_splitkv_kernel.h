// Split-KV kernel of the paged MLA decode library, written for gfx950 (CDNA4).
//
// One workgroup = (part, block of 64 query rows) of the tile-scheduler
// metadata: 4 wavefronts, one per SIMD.  The workgroup walks its part's
// segments (unit, block range, slot) as one stream of 64-token tiles.  Each
// tile is gathered into LDS with direct-to-LDS loads -- a contiguous 64-row
// page reached through the block table for dense decode, 64 scattered rows
// reached through the index list for sparse decode -- into one of two buffers,
// so the next tile streams in while the current one is computed.
//
// Wavefronts 2r and 2r+1 form a pair that owns query rows 32r..32r+31.  Each
// wavefront of a pair computes
//   S^T = K . Q^T      for its half of the tile's tokens, over all d_qk
//                      (v_mfma_f32_32x32x16_bf16; K from LDS, Q^T resident in
//                      registers for the whole segment),
//   online softmax     fp32, base 2, one query row per lane pair; the pair
//                      exchanges row maxima, row sums and its bf16 P half
//                      through LDS; the reference maximum moves only when it
//                      grows by more than 2^8, so the accumulator is rarely
//                      rescaled (the result does not depend on it),
//   O^T += V^T . P^T   for its half of the 512 value columns over all 64
//                      tokens; V^T is read with the LDS transpose read from the
//                      first 512 columns of the same tile.
// Every K and V element read from LDS thus feeds 32 query rows.
//
// The gather of the next tile is issued in slices between the QK MFMAs, so
// its address arithmetic runs in the shadow of the matrix cores.  The
// metadata of the tile after next is read at the end of each step, and the
// next segment's
// queries are loaded as soon as the current segment's last QK product is
// done.  A segment covering its whole unit writes bf16 O and fp32 LSE; a split
// segment writes fp32 O and a base-2 LSE into its workspace slot for the
// combine kernel.  This is the structure the deepep.org usage page describes
// (tile scheduler, block-table manager, memory manager; QK^T, scaled softmax,
// output stages); sparse gathering follows the upstream FlashMLA README
// ("Sparse Attention (indices tensor)").  Only active heads are computed.
//
// LDS tile layout: cache row t of a tile occupies 16-byte chunks
// [t*CPR, (t+1)*CPR), with its chunk c stored at position c ^ f(t).  The
// swizzle f spreads the operand reads over all banks; it is applied on the
// source side of the gather, and since f depends only on the low bits of t,
// every operand address is one of a few per-lane bases plus a compile-time
// offset.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_kernels.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Read-only metadata (scheduler output, block table, sequence lengths) is
// read through the constant address space so uniform reads become scalar
// loads instead of vector loads that would share the vector memory counter
// with the in-flight tile gathers.
typedef const __attribute__((address_space(4))) int32_t cint;
// a segment record (unit, first block, end block, slot), read as one scalar load
typedef int32_t i32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef const __attribute__((address_space(4))) i32x4a cseg;
__device__ __forceinline__ cint* as_const(const int32_t* ptr) { return (cint*)(uintptr_t)ptr; }

constexpr int kPage = 64;          // tokens per tile (one page, or 64 sparse indices)
constexpr int kWaves = 4;          // wavefronts per workgroup
constexpr int kDV = 512;           // value width
constexpr int kRowsPerGroup = 64;  // query rows per workgroup
constexpr int kRows = 32;          // query rows per wavefront pair
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference max may lag
// Word 3 of a raw (untyped, unswizzled) buffer resource on gfx9-family parts:
// a valid 32-bit data format, everything else zero.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ unsigned short f2bf(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);
}
// 16-bit element of the output / P operand: bf16 or fp16, rounded to nearest even
template <bool F16>
__device__ __forceinline__ unsigned short f2e(float x) {
  if constexpr (F16)
    return __builtin_bit_cast(unsigned short, (_Float16)x);
  else
    return f2bf(x);
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// waits until at most N of this wave's vector memory operations are in flight
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier for LDS traffic only: waits for this wave's LDS (and
// scalar) accesses, not for the tile gathers still in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Reductions over lanes l and l ^ 32 (the two k-groups that share a query
// row) with v_permlane32_swap, which exchanges the upper 32 lanes of its
// first operand with the lower 32 lanes of its second: swapping a value with
// a copy of itself leaves its lower half broadcast in one register and its
// upper half in the other.  It is written out (with the wait states the
// instruction needs after a VALU write of its operands) because the compiler
// folds the builtin's two results into one when both operands are equal.
__device__ __forceinline__ void swap_halves(float v, float& lo, float& hi) {
  lo = v;
  hi = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}
// Maximum of scores.  The NaN-propagating form maps to v_maximum3_f32 with no
// operand quieting, where fmaxf would first canonicalize operands that the
// compiler cannot prove are quiet.  Masked scores are -inf, never NaN; a NaN
// among the visible scores makes the row's output NaN with either form.
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float xor32_max(float v) {
  float lo, hi;
  swap_halves(v, lo, hi);
  return smax(lo, hi);
}
__device__ __forceinline__ float xor32_sum(float v) {
  float lo, hi;
  swap_halves(v, lo, hi);
  return lo + hi;
}
// Register-class pin: an empty asm statement that takes the value in AGPRs.
// It emits no instruction; it keeps the long-lived accumulators in the
// accumulation registers, so the vector registers stay free for the per-tile
// working set and no copies are hoisted into the tile loop.
__device__ __forceinline__ void pin_agpr(f32x16& x) { asm volatile("" : "+a"(x)); }

// Workgroups are dispatched to the 8 XCDs round-robin; give each XCD a
// contiguous run of logical groups so the row blocks of a part (and nearby
// parts) share one L2.
__device__ __forceinline__ int logical_group(int id, int total) {
  constexpr int kXcd = 8;
  const int xcd = id % kXcd, k = id / kXcd;
  const int per = total / kXcd, rem = total % kXcd;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + k;
}

// ---- v_mfma_f32_32x32x16_bf16 operand layouts ----
// A (32 x 16): lane l holds row l % 32, k = 8 (l / 32) .. +7.  B (16 x 32):
// lane l holds column l % 32, k = 8 (l / 32) .. +7.  C (32 x 32): register j
// of lane l is row 8 (j / 4) + 4 (l / 32) + j % 4, column l % 32.
template <bool F16>
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// token (within the pair half's 32) of score register v of k-group g
__device__ __forceinline__ int tok(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }
// output column of O^T register j of column tile ct, k-group g
__device__ __forceinline__ int col(int ct, int j, int g) {
  return 32 * ct + 8 * (j >> 2) + 4 * g + (j & 3);
}
// V^T transpose read h of PV k-step kc: the tile row (token) this lane
// addresses, and the 16-byte chunk of column tile 0 it addresses
__device__ __forceinline__ int vrow(int kc, int h, int lane) {
  return 16 * kc + 8 * h + 4 * (lane >> 5) + ((lane & 15) >> 2);
}
__device__ __forceinline__ int vchunk(int lane) { return 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1); }
// chunk swizzle f(t) for 72- and 64-chunk rows; f(t) < 8 (resp. < 16), so it
// permutes chunks inside aligned groups of 8 (resp. 16), and it depends only
// on bits 1..3 (resp. 0..3) of t
template <int CPR>
__host__ __device__ constexpr int swz(int t) {
  if constexpr (CPR == 72) return 4 * ((t >> 1) & 1) + ((t >> 2) & 3);
  else return ((t & 3) << 2) | ((t >> 2) & 3);
}

struct TileMeta {
  int phys;  // dense: physical page of the tile
  int len;   // dense: cache length of the tile's request
  int idx;   // sparse: this lane's index (tile token = lane)
};

// what a tile gather needs
struct Gather {
  int phys;        // dense: the physical page
  int tmax;        // dense: last valid row of the tile
  int idx;         // sparse: this lane's (substituted) index
  uint64_t vmask;  // sparse: valid tokens of the tile
};

}  // namespace

// WIDE (sparse only): the cache pool is 4 GiB or larger, so rows are reached
// with 64-bit addresses instead of 32-bit offsets into one buffer resource.
// FP8 (D_QK = 576 only): the cache holds 656-byte "FP8 with scale" rows, which
// are staged in LDS as they are and dequantized to the bf16 tile layout
// before the tile is computed.  F16: q, cache and output are fp16 instead of
// bf16 (the fp16 MFMA, P and O rounded to fp16); not with FP8.
template <int D_QK, bool SPARSE, bool WIDE, bool FP8, bool F16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_splitkv(SplitKVParams p) {
  // The body is compiled for the GPU only; the host pass needs just the
  // kernel's launch stub (and would otherwise drop it for this body).
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int CPR = D_QK / 8;           // 16-byte chunks per cache row
  constexpr int RSB = CPR * 16;           // LDS row stride in bytes
  constexpr int NLD = CPR;                // 1 KB gather loads per tile
  constexpr int NLW = NLD / kWaves;       // ... per wavefront (18 or 16)
  constexpr int BUF = NLD * 1024;         // bytes per tile buffer
  constexpr int KK = D_QK / 16;           // QK k-steps
  constexpr int NCT = kDV / 2 / 32;       // output column tiles per wavefront (8)
  constexpr int NSTEP = 4 * NCT;          // PV steps: 4 k-steps of 16 tokens x NCT
  constexpr int FMAX = CPR == 72 ? 8 : 16;  // swizzle values are below this
  constexpr int NKB = FMAX / 2;           // K-read bases (kk mod NKB)
  constexpr int NVB = FMAX / 4;           // V-read bases (ct mod NVB)
  static_assert(NLD % kWaves == 0 && (16 * CPR) % 64 == 0, "16 whole rows per wavefront");
  static_assert(2 * NLW <= KK + 1, "gather slices fit the QK loop");
  static_assert(!FP8 || D_QK == 576, "the FP8 row format carries 512 + 64 values");
  static_assert(!(FP8 && F16), "an FP8 cache dequantizes to bf16");
  constexpr int SROW = kFp8RowBytes;      // FP8 cache row: 512 e4m3, 4 fp32 scales, 64 bf16
  constexpr int SBUF = kPage * SROW;      // staged FP8 tile (41 KB)
  constexpr int SNL = SBUF / 1024;        // 1 KB gather loads per FP8 tile (41)
  static_assert(SBUF % 1024 == 0, "whole 1 KB loads");
  // bf16 tiles: two buffers, the next tile streams into one while the other is
  // computed.  FP8 tiles: the raw rows stream into two staging buffers and
  // one bf16 buffer holds the dequantized tile being computed; the pair
  // exchange area then lives in the staging buffer just dequantized.
  constexpr int XP_BYTES = kWaves * 2 * 64 * 16, XM_BYTES = kWaves * 32 * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t buf_a[BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t buf_b[FP8 ? 16 : BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t stg_a[FP8 ? SBUF : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t stg_b[FP8 ? SBUF : 16];
  __shared__ __attribute__((aligned(16))) uint8_t x_own[FP8 ? 16 : XP_BYTES + 2 * XM_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int rgrp = wave >> 1;  // row group (pair) of the wavefront
  const int half = wave & 1;   // pair half: token half (QK) and column half (PV)
  const int lrow = lane & 31;  // query row owned within the pair
  const int lgrp = lane >> 5;  // k-group of the MFMA operands

  // the metadata pointer, the shape words and the output pointers are
  // requested with the launch's part count, so the header reads below do not
  // wait for further rounds of argument loads
  asm volatile("" ::"s"(p.meta), "s"(p.num_parts), "s"(p.row_blocks), "s"(p.rows), "s"(p.s_q),
               "s"(p.h_q), "s"(p.heads), "s"(p.lse_base2), "s"(p.topk), "s"(p.num_rows), "s"(p.out),
               "s"(p.lse), "s"(p.ws_o), "s"(p.ws_lse), "s"(p.max_logits), "s"(p.ws_max));
  const int total = p.num_parts * p.row_blocks;
  const int lg = logical_group(blockIdx.x, total);
  const int part = lg / p.row_blocks;
  const int rb = lg - part * p.row_blocks;
  if (part >= p.num_parts) return;

  cint* meta = as_const(p.meta);
  // the grid covers p.num_parts parts, the device header says how many exist
  // (fewer only when the metadata was built on the device; header word 15 is
  // -1 when the device scheduler rejected the lengths)
  // The header words and the part's segment range are independent reads,
  // requested together before anything branches on them (one memory round
  // trip, not three).
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

  const int row0 = rb * kRowsPerGroup + rgrp * kRows;
  const int row = row0 + lrow;
  const bool row_ok = row < p.rows;

  // Per-lane LDS operand bases.  Chunk c of tile row t is stored at position
  // c ^ f(t), and f depends only on low bits of t that are fixed per lane, so
  //  K  (A of QK): row 32*half + lrow, chunk 2*kk + lgrp, stored at
  //     2*(kk ^ (f/2)) + (lgrp ^ (f%2)) -> kbase[kk % NKB] + 32*kk;
  //  V^T (A of PV, transpose read h): row vrow(kc, h), chunk 4*ct + y of this
  //     half's columns, stored at 4*(ct ^ (f/4)) + (y ^ (f%4)) ->
  //     vbase[h][ct % NVB] + 64*ct (the column-half offset is in the base).
  int kbase[NKB], vbase[2][NVB];
  {
    const int fk = swz<CPR>(lrow);
#pragma unroll
    for (int j = 0; j < NKB; ++j)
      kbase[j] = (32 * half + lrow) * RSB + 16 * (lgrp ^ (fk % 2)) + 32 * ((j ^ (fk / 2)) - j);
    const int y = vchunk(lane);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int vr = vrow(0, h, lane);
      const int fv = swz<CPR>(vr);
#pragma unroll
      for (int j = 0; j < NVB; ++j)
        vbase[h][j] = vr * RSB + 16 * (y ^ (fv % 4)) + 64 * ((j ^ (fv / 4)) - j) + 8 * (lane & 1) +
                      64 * NCT * half;
    }
  }

  // output row of this lane for unit u: dense rows are (query token, head)
  // pairs of a request, sparse units are single query tokens
  auto row_index = [&](int u, int r) __attribute__((always_inline)) -> size_t {
    int b, iq, h;
    if constexpr (SPARSE) {
      b = u / p.s_q;
      iq = u - b * p.s_q;
      h = r;
    } else {
      b = u;
      iq = r / p.heads;
      h = r - iq * p.heads;
    }
    return (size_t(b) * p.s_q + iq) * p.h_q + h;
  };
  // cache positions this lane's row may see (bottom-right causal alignment)
  auto visible = [&](int L) __attribute__((always_inline)) -> int {
    if (!p.causal) return L;
    const int n = L - p.s_q + row / p.heads + 1;
    return n < 0 ? 0 : (n > L ? L : n);
  };

  // ---- tile metadata, fetched ahead of the tile's gather ----
  auto fetch_meta = [&](int u, int blk) __attribute__((always_inline)) -> TileMeta {
    TileMeta m{0, 0, -1};
    if constexpr (SPARSE) {
      const int pos = blk * kPage + lane;
      m.idx = pos < p.topk ? p.indices[size_t(u) * p.topk + pos] : -1;
    } else {
      m.phys = as_const(p.block_table)[size_t(u) * p.bt_stride + blk];
      m.len = as_const(p.seqlens)[u];
    }
    return m;
  };

  // ---- tile gather ----
  // Wavefront w fills LDS rows 16w..16w+15 (1 KB loads n = NLW*w + i), so the
  // tile row of every lane of load i, its swizzle and the row boundary inside
  // the load are compile-time constants; only the tail clamp depends on the
  // tile.  Every lane fetches an in-bounds row: the tail of a request's last
  // page repeats its last cached token (masked out of the softmax, so it
  // contributes exactly zero), and an invalid sparse index is replaced by the
  // tile's first valid one (also masked).  A sparse tile without any valid
  // index is neither loaded nor computed.
  constexpr int ROWB = FP8 ? SROW : RSB;  // bytes of one cache row in memory
  auto page_rsrc = [&](int phys) __attribute__((always_inline)) {
    const uint8_t* pg = reinterpret_cast<const uint8_t*>(p.kv) + size_t(phys) * kPage * ROWB;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pg), 0, kPage * ROWB,
                                            kBufferWord3);
  };
  // the whole pool (sparse rows, pools below 4 GiB)
  auto pool_rsrc = [&]() __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.kv), 0,
                                            int(uint32_t(p.num_rows) * uint32_t(ROWB)), kBufferWord3);
  };
  auto plan_gather = [&](int blk, const TileMeta& m) __attribute__((always_inline)) -> Gather {
    Gather g;
    g.phys = SPARSE ? 0 : m.phys;
    g.tmax = kPage - 1;
    g.idx = 0;
    g.vmask = ~0ull;
    if constexpr (SPARSE) {
      const bool ok = m.idx >= 0 && m.idx < p.num_rows;
      g.vmask = __ballot(ok);
      // a tile without any valid index: through one buffer resource (pools
      // below 4 GiB) every lane reads row num_rows, past the end of the
      // resource, which returns zeros -- the tile is then computed like any
      // other, fully masked, and adds exactly nothing; with 64-bit addressing
      // the tile is skipped instead
      const int sub = g.vmask ? __shfl(m.idx, __builtin_ctzll(g.vmask)) : (WIDE ? 0 : p.num_rows);
      g.idx = ok ? m.idx : sub;
    } else {
      const int vt = m.len - blk * kPage;
      g.tmax = vt < 1 ? 0 : (vt > kPage ? kPage - 1 : vt - 1);
    }
    return g;
  };
  // load i of this wavefront: LDS chunks q = 64 n + lane (n = NLW*wave + i),
  // rows t0 (lanes below `bnd`) and t0 + 1; the source chunk of LDS chunk q
  // of row t is q ^ f(t) (t*CPR is a multiple of the swizzle group).  `ln` is
  // the lane id, passed through an opaque copy per tile so the compiler
  // recomputes these few operations instead of keeping 18 offsets alive.
  auto gather_one = [&](const Gather& g, uint8_t* dst, int i, int ln) __attribute__((always_inline)) {
    const int q0 = 64 * i;  // first chunk of the load within the wavefront's rows
    const int tl = q0 / CPR;
    const int bnd = (tl + 1) * CPR - q0;  // first lane of row tl + 1 (>= 64: none)
    const bool second = bnd < 64 && ln >= bnd;
    const int f16 = 16 * (second ? swz<CPR>(tl + 1) : swz<CPR>(tl));
    const int n = NLW * wave + i;
    lds_void* to = (lds_void*)(dst + n * 1024);
    const int t = 16 * wave + tl + (second ? 1 : 0);  // tile row of this lane
    if constexpr (SPARSE) {
      // the load covers two tile rows, so two uniform index reads suffice
      const int r0 = __builtin_amdgcn_readlane(g.idx, 16 * wave + tl);
      const int r1 = bnd < 64 ? __builtin_amdgcn_readlane(g.idx, 16 * wave + tl + 1) : r0;
      const int r = second ? r1 : r0;
      const int in_row = ((q0 + ln) * 16 - (tl + (second ? 1 : 0)) * RSB) ^ f16;
      if constexpr (WIDE) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(p.kv) + size_t(r) * RSB + in_row;
        __builtin_amdgcn_global_load_lds(src, to, 16, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pool_rsrc(), to, 16,
                                                 uint32_t(r) * uint32_t(RSB) + uint32_t(in_row), 0, 0, 0);
      }
    } else {
      // in-page offset of source chunk q ^ f(t), moved down to row tmax for
      // rows past it
      int off = (n * 1024 + ln * 16) ^ f16;
      if (t > g.tmax) off -= (t - g.tmax) * RSB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(page_rsrc(g.phys), to, 16, off, 0, 0, 0);
    }
  };
  auto gather_all = [&](const Gather& g, uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NLW; ++i) gather_one(g, dst, i, lane);
  };
  // The workgroup's 64 query rows, when they are consecutive rows of q,
  // gathered like a dense tile (same LDS layout and swizzle; rows past the
  // last one repeat it): 1 KB per load instead of 32-byte pieces of 32 rows
  // per wavefront load, and each row fetched once rather than by both
  // wavefronts of its pair.
  auto gather_q = [&](int u, uint8_t* dst) __attribute__((always_inline)) {
    const int r0 = rb * kRowsPerGroup;
    const int tmax = p.rows - 1 - r0 < kRowsPerGroup - 1 ? p.rows - 1 - r0 : kRowsPerGroup - 1;
    const uint16_t* base = p.q + row_index(u, r0) * D_QK;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0,
                                                      kRowsPerGroup * RSB, kBufferWord3);
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int q0 = 64 * i;
      const int tl = q0 / CPR;
      const int bnd = (tl + 1) * CPR - q0;
      const bool second = bnd < 64 && lane >= bnd;
      const int f16 = 16 * (second ? swz<CPR>(tl + 1) : swz<CPR>(tl));
      const int n = NLW * wave + i;
      const int t = 16 * wave + tl + (second ? 1 : 0);
      int off = (n * 1024 + lane * 16) ^ f16;
      if (t > tmax) off -= (t - tmax) * RSB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + n * 1024), 16, off, 0, 0, 0);
    }
  };
  // FP8 tile: the 64 raw rows, back to back, in 41 loads of 1 KB; wavefront w
  // issues loads w, w + 4, ...  Lane chunk q of the tile is chunk q % 41 of
  // tile row q / 41.  Rows are clamped / substituted as for bf16 tiles.  The
  // lane id goes through an opaque copy so the per-lane offsets are
  // recomputed for every tile rather than kept live (or spilled) across it.
  auto gather_fp8 = [&](const Gather& g, uint8_t* dst) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < (SNL + kWaves - 1) / kWaves; ++i) {
      const int n = wave + kWaves * i;
      if (n < SNL) {
        const int q = 64 * n + ln;
        int t = q / (SROW / 16);
        const int cb = 16 * (q - t * (SROW / 16));  // byte of the chunk in its row
        lds_void* to = (lds_void*)(dst + n * 1024);
        if constexpr (SPARSE) {
          const int r = __shfl(g.idx, t);
          if constexpr (WIDE) {
            const uint8_t* src = reinterpret_cast<const uint8_t*>(p.kv) + size_t(r) * SROW + cb;
            __builtin_amdgcn_global_load_lds(src, to, 16, 0, 0);
          } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(pool_rsrc(), to, 16,
                                                     uint32_t(r) * uint32_t(SROW) + uint32_t(cb), 0, 0, 0);
          }
        } else {
          if (t > g.tmax) t = g.tmax;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(page_rsrc(g.phys), to, 16, t * SROW + cb, 0, 0,
                                                  0);
        }
      }
    }
  };
  // Dequantizes a staged FP8 tile into the bf16 tile layout (upstream
  // FlashMLA README, "FP8 KV Cache": value * scale of its group of 128, then
  // bf16; the RoPE part is bf16 already).  Wavefront w takes tile rows
  // w, w + 4, ..., and lane l makes bf16 chunk l of the row from 8 e4m3
  // values (scale group l / 16): 16 lanes read one contiguous 128 bytes and
  // write 8 distinct chunks of a swizzle group, so neither side conflicts.
  // The product is rounded to fp32, then to bf16 (nearest even).
  auto dequant = [&](const uint8_t* stg, uint8_t* dst) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed per tile (see gather_fp8)
    const int fw = 4 * ((wave >> 1) & 1);  // swizzle bit of row w + 4i from the wave
    const uint8_t* src = stg + wave * SROW;
    uint8_t* drow = dst + wave * RSB;
    // rows in groups of 4; the reads of group g + 1 are in flight while
    // group g is converted
    constexpr int GR = 4, NG = kPage / kWaves / GR;
    u32x2 raw[2][GR];
    float sc[2][GR];
    auto read_group = [&](int g) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        const uint8_t* sr = src + 4 * (GR * g + r) * SROW;
        raw[g & 1][r] = *reinterpret_cast<const u32x2*>(sr + 8 * ln);
        sc[g & 1][r] = *reinterpret_cast<const float*>(sr + 512 + 4 * (ln >> 4));
      }
    };
    read_group(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) read_group(g + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        const int i = GR * g + r;
        const int f = fw + (i & 3);  // swz<72>(wave + 4 i)
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const u32x2 x = raw[g & 1][r];
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(x[e], false) * sc[g & 1][r];
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(x[e], true) * sc[g & 1][r];
          w[2 * e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
          w[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
        }
        *reinterpret_cast<u32x4*>(drow + 4 * i * RSB + 16 * (ln ^ f)) =
            u32x4{w[0], w[1], w[2], w[3]};
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // RoPE: 8 chunks per row, 8 rows per pass (rows w + 4 (8 k + ln / 8))
#pragma unroll
    for (int k = 0; k < kPage / kWaves / 8; ++k) {
      const int i = 8 * k + (ln >> 3);
      const int c = ln & 7;
      const int f = fw + (i & 3);
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + 4 * i * SROW + 528 + 16 * c);
      *reinterpret_cast<u32x4*>(drow + 4 * i * RSB + 16 * ((64 + c) ^ f)) = v;
    }
  };

  // ---- per-segment state ----
  // m_run: reference maximum (base 2, scaled) of the lane's row, identical in
  // both halves of a pair.  l_part: the row's sum of softmax numerators.
  bf16x8 qf[KK];
  f32x16 acc[NCT];
  float m_run = -__builtin_inff();
  float m_exact = -__builtin_inff();  // exact row maximum of the scaled logits (base 2)
  float l_part = 0.f;
  size_t qrow = 0;
  int n_vis = 0;

  // rows past the unit's last row read that last row (never written back)
  auto load_q = [&](int u) __attribute__((always_inline)) {
    const uint16_t* qp = p.q + row_index(u, row_ok ? row : p.rows - 1) * D_QK + 8 * lgrp;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
  };
  // this wavefront's query fragments (rows 32 rgrp + lrow, the B operand of
  // QK) from a gathered query tile: the K-operand addressing moved to the
  // pair's rows
  auto read_q = [&](const uint8_t* src) __attribute__((always_inline)) {
    const int dq = (rgrp - half) * kRows * RSB;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(src + kbase[kk % NKB] + dq + kk * 32);
  };
  // The accumulator is not cleared here: the segment's first computed tile
  // starts its PV product from zero instead, so acc is only ever touched by
  // MFMAs in the tile loop (and by the rare rescale).
  bool seg_first = true;
  auto reset_state = [&]() __attribute__((always_inline)) {
    seg_first = true;
    m_run = -__builtin_inff();
    m_exact = -__builtin_inff();
    l_part = 0.f;
  };

  // Writes the segment result of this lane's row (each pair half its own value
  // columns); a segment without tokens (empty_seg) writes O = 0 and LSE = -inf.
  auto write_segment = [&](size_t orow, int slot, bool empty_seg) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) pin_agpr(acc[ct]);
    const float l_tot = empty_seg ? 0.f : l_part;
    const bool empty = !(l_tot > 0.f) || seg_first;
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse2 = empty ? -__builtin_inff() : m_run + fast_log2(l_tot);
    if (!row_ok) return;
    const int ct0 = NCT * half;  // first value column tile of this wavefront
    const bool lse_lane = lgrp == 0 && half == 0;
    if (slot < 0) {
      uint16_t* o = p.out + orow * kDV;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = empty ? 0.f : acc[ct][j + e] * inv;
          const uint32_t lo = uint32_t(f2e<F16>(v[0])) | (uint32_t(f2e<F16>(v[1])) << 16);
          const uint32_t hi = uint32_t(f2e<F16>(v[2])) | (uint32_t(f2e<F16>(v[3])) << 16);
          *reinterpret_cast<uint2*>(o + col(ct0 + ct, j, lgrp)) = uint2{lo, hi};
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (lse_lane) {
        p.lse[orow] = p.lse_base2 ? lse2 : lse2 * kLn2;
        if (p.max_logits) p.max_logits[orow] = m_exact;
      }
    } else {
      const size_t wrow = size_t(slot) * p.rows + row;
      float* o = p.ws_o + wrow * kDV;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = empty ? 0.f : acc[ct][j + e] * inv;
          *reinterpret_cast<f32x4*>(o + col(ct0 + ct, j, lgrp)) = v;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (lse_lane) {
        p.ws_lse[wrow] = lse2;
        if (p.max_logits) p.ws_max[wrow] = m_exact;
      }
    }
  };

  // The next tile's gather, issued in slices from inside the tile
  // computation; the step sets it up.
  Gather nx_plan{0, 0, 0, 0};
  uint8_t* nx_dst = buf_b;
  int nx_ln = 0;
  auto gather_slice = [&](int i) __attribute__((always_inline)) {
    gather_one(nx_plan, nx_dst, i, nx_ln);
  };

  // ---- one 64-token tile: QK^T, softmax, PV ----
  // `next_q_unit` >= 0: this is the segment's last tile and the next segment's
  // queries are loaded once the QK product no longer needs the current ones.
  // gather_slice(i) issues slice i of the next tile's gather (between QK
  // k-steps).
  // `xb`: the LDS area of the pair exchanges (P halves, row maxima and sums).
  // A row group whose 32 rows all lie past the unit's rows (units of at most
  // 32 rows, e.g. 16 active heads) has nothing to compute: it issues its share
  // of the next gather and meets the two workgroup barriers of the tile.
  const bool idle_rows = row0 >= p.rows;
  auto compute_tile = [&](const uint8_t* buf, int blk, uint64_t vmask, int next_q_unit,
                          uint8_t* xb) __attribute__((always_inline)) {
    if (idle_rows) {
      if constexpr (!FP8) {
#pragma unroll
        for (int i = 0; i < NLW; ++i) gather_slice(i);
      }
      lds_barrier();  // the row maxima exchange
      lds_barrier();  // the P exchange
      return;
    }
    s16x8* x_p = reinterpret_cast<s16x8*>(xb);                     // [wave][2][64]
    float* x_max = reinterpret_cast<float*>(xb + XP_BYTES);           // [wave][32]
    float* x_sum = reinterpret_cast<float*>(xb + XP_BYTES + XM_BYTES);  // [wave][32]
    // FP8: the exchange area moves between the two staging buffers, so its
    // lane offsets are recomputed per tile rather than kept live for both
    int xl = lane;
    if constexpr (FP8) asm volatile("" : "+v"(xl));
    // S^T of this half's 32 tokens, one accumulation chain over the k-steps
    // (the matrix core accumulates back-to-back into the same registers, so a
    // second chain would only add its read-out and 16 additions)
    constexpr int QD = 4;  // K fragments prefetched this many k-steps ahead
    f32x16 st[1];
    bf16x8 kf[QD + 1];
    auto load_k = [&](int kk) __attribute__((always_inline)) {
      kf[kk % (QD + 1)] = *reinterpret_cast<const bf16x8*>(buf + kbase[kk % NKB] + kk * 32);
    };
#pragma unroll
    for (int kk = 0; kk < QD; ++kk) {
      load_k(kk);
      __builtin_amdgcn_sched_barrier(0);  // keep the ring in k-step order
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + QD < KK) load_k(kk + QD);
      st[0] = mfma<F16>(kf[kk % (QD + 1)], qf[kk], kk < 1 ? f32x16{} : st[0]);
      // the next tile's gather, one slice every other k-step
      if constexpr (!FP8)
        if ((kk & 1) == 0 && kk / 2 < NLW) gather_slice(kk / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (next_q_unit >= 0) load_q(next_q_unit);

    // V^T fragments, prefetched PD (k-step, column-tile) steps ahead; the
    // first PD are issued before the softmax so their latency hides behind it.
    // PV runs its k-steps in the order e = 0..3 where e = 0, 1 cover this
    // half's own 32 tokens (P on hand after the softmax) and e = 2, 3 the
    // partner's (P read after the exchange): token block 16 e + 32 half for
    // e < 2, 16 (e - 2) + 32 (1 - half) after.
    constexpr int PD = 6;
    s16x4 vf[PD + 1][2];
    const int vsh_own = half * 32 * RSB, vsh_oth = (1 - half) * 32 * RSB;
    auto load_v = [&](int i) __attribute__((always_inline)) {
      const int e = i / NCT, ct = i % NCT;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint8_t* a = buf + vbase[h][ct % NVB] + (e < 2 ? vsh_own : vsh_oth) +
                           (e & 1) * 16 * RSB + ct * 64;
        vf[i % (PD + 1)][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
      }
    };
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      load_v(i);
      __builtin_amdgcn_sched_barrier(0);
    }

    // mask + online softmax (base 2), 16 raw scores per lane.  The scale is
    // folded into the exponent: p = 2^(s * scale_log2 - m).
    bool full;  // every token of the tile is visible to every row of the wave
    if constexpr (SPARSE) {
      full = vmask == ~0ull;
    } else {
      full = __all(blk * kPage + kPage <= n_vis);
    }
    float mloc = -__builtin_inff();
    if (full) {
#pragma unroll
      for (int v = 0; v < 16; v += 2) mloc = smax(smax(mloc, st[0][v]), st[0][v + 1]);
    } else {
      // sparse: the lane's tokens are 32 half + 4 lgrp + c, c = tok(v, 0) <= 27,
      // so one shift of the tile mask leaves a 32-bit word tested at
      // compile-time bit positions
      uint32_t vm = 0;
      if constexpr (SPARSE) vm = uint32_t(vmask >> (32 * half + 4 * lgrp));
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = 32 * half + tok(v, lgrp);
        bool vis;
        if constexpr (SPARSE) {
          vis = (vm >> tok(v, 0)) & 1;
        } else {
          vis = blk * kPage + t < n_vis;
        }
        const float x = vis ? st[0][v] : -__builtin_inff();
        st[0][v] = x;
        mloc = smax(mloc, x);
      }
    }
    mloc = xor32_max(mloc);
    if (lane < 32) x_max[32 * wave + xl] = mloc;  // maximum over both token halves
    lds_barrier();
    mloc = smax(mloc, x_max[32 * (wave ^ 1) + (xl & 31)]) * p.scale_log2;
    m_exact = smax(m_exact, mloc);
    const bool grow = mloc > m_run + kRescaleSlack;
    if (__any(grow)) {
      const float m_new = grow ? mloc : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
      m_run = m_new;
      l_part *= alpha;
      if (!seg_first) {
        // one column tile at a time, each back in its AGPRs before the next
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          pin_agpr(acc[ct]);  // read out of the AGPRs here, not earlier
          acc[ct] *= alpha;
          pin_agpr(acc[ct]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) pin_agpr(acc[ct]);
    const float neg_m = m_run == -__builtin_inff() ? 0.f : -m_run;
    s16x8 pk[2];  // this lane's P^T operand: scores 8c .. 8c+7
    float pe[16];
    // the score goes through an opaque copy: the two copies of the PV loop
    // (first tile of a segment or not) would otherwise share their
    // exponentials, hoisted out of both loops ahead of the MFMAs
    auto expo = [&](int v) __attribute__((always_inline)) {
      float sv = st[0][v];
      asm volatile("" : "+v"(sv));
      pe[v] = fast_exp2(__builtin_fmaf(sv, p.scale_log2, neg_m));
      pk[v >> 3][v & 7] = (short)f2e<F16>(pe[v]);
    };
#pragma unroll
    for (int v = 0; v < 8; ++v) expo(v);
    x_p[128 * wave + xl] = pk[0];
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T . P^T.  Between the MFMAs of the own k-steps go the other
    // half of the exponentials, the row sum (a pairwise tree, short
    // dependency chain) and the exchange writes; the exchange barrier comes
    // two MFMAs before the partner's P is needed.
    auto pv = [&](bool from_zero) __attribute__((always_inline)) {
      s16x8 pp[2];
      float own = 0.f, other = 0.f;
#pragma unroll
      for (int i = 0; i < NSTEP; ++i) {
        if (i + PD < NSTEP) load_v(i + PD);
        const int e = i / NCT, ct = i % NCT;
        const s16x4 lo = vf[i % (PD + 1)][0], hi = vf[i % (PD + 1)][1];
        const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const s16x8 pb = e < 2 ? pk[e] : pp[e - 2];
        const f32x16 c_in = (from_zero && e == 0) ? f32x16{} : acc[ct];
        acc[ct] = mfma<F16>(__builtin_bit_cast(bf16x8, vv), __builtin_bit_cast(bf16x8, pb), c_in);
        static_assert(NCT == 8, "one exponential per MFMA of the first k-step");
        if (i < NCT) expo(8 + i);
        if (i == NCT - 1) x_p[128 * wave + 64 + xl] = pk[1];
        if (i == NCT) {
#pragma unroll
          for (int v = 0; v < 8; ++v) pe[v] += pe[v + 8];
        }
        if (i == NCT + 1) {
#pragma unroll
          for (int v = 0; v < 4; ++v) pe[v] += pe[v + 4];
        }
        if (i == NCT + 2) {
#pragma unroll
          for (int v = 0; v < 2; ++v) pe[v] += pe[v + 2];
          own = xor32_sum(pe[0] + pe[1]);
        }
        if (i == NCT + 3 && lane < 32) x_sum[32 * wave + xl] = own;
        if (i == 2 * NCT - 3) {
          // exchange P halves and row sums with the pair partner
          lds_barrier();
          pp[0] = x_p[128 * (wave ^ 1) + xl];
          pp[1] = x_p[128 * (wave ^ 1) + 64 + xl];
          other = x_sum[32 * (wave ^ 1) + (xl & 31)];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      l_part += half == 0 ? own + other : other + own;  // same sum in both halves
    };
    if (seg_first) {
      pv(true);
      seg_first = false;
    } else {
      pv(false);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) pin_agpr(acc[ct]);
  };

  // ---- tile stream of the part ----
  // A tile of the stream: its segment, block, unit, and whether it is the
  // segment's last.  The segment of the furthest tile looked up is cached
  // (la_*), so stepping within a segment reads no metadata, and a step issues
  // one independent scalar load (the block-table entry) that nothing waits
  // for until two steps later.
  struct Tile {
    int s, blk, u;
    bool last;
  };
  int la_u = 0, la_b1 = 0;  // cached segment
  // first tile at or after segment s2 (whose record is rec, when s2 is a
  // segment), skipping segments without tiles; each record is one load
  auto first_tile_rec = [&](int s2, i32x4a rec) __attribute__((always_inline)) -> Tile {
    while (s2 < seg_end && rec[1] == rec[2]) {
      ++s2;
      if (s2 < seg_end) rec = seg_rec(s2);
    }
    if (s2 >= seg_end) return Tile{seg_end, 0, 0, true};
    la_u = rec[0];
    la_b1 = rec[2];
    return Tile{s2, rec[1], la_u, rec[1] + 1 >= la_b1};
  };
  auto first_tile_from = [&](int s2) __attribute__((always_inline)) -> Tile {
    return first_tile_rec(s2, s2 < seg_end ? seg_rec(s2) : i32x4a{0, 0, 0, 0});
  };
  // the tile after t (t is in the cached segment)
  auto next_tile = [&](const Tile& t) __attribute__((always_inline)) -> Tile {
    if (t.s >= seg_end) return t;
    if (!t.last) return Tile{t.s, t.blk + 1, t.u, t.blk + 2 >= la_b1};
    return first_tile_from(t.s + 1);
  };

  // Lengths the device scheduler rejected: every output row of the call gets
  // O = 0 and LSE = NaN (and max_logits = NaN), rather than whatever the
  // buffers held; workgroup (part, row block) takes units part, part + grid
  // parts, ...
  if (meta_bad) {
    if (!row_ok) return;
    for (int u = part; u < meta[5]; u += p.num_parts) {
      const size_t orow = row_index(u, row);
      uint16_t* o = p.out + orow * kDV + 256 * half + 4 * lgrp;
      for (int c = 0; c < 256; c += 8) *reinterpret_cast<uint2*>(o + c) = uint2{0, 0};
      if (lgrp == 0 && half == 0) {
        p.lse[orow] = __builtin_nanf("");
        if (p.max_logits) p.max_logits[orow] = __builtin_nanf("");
      }
    }
    return;
  }

  // leading segments without tiles
  int cs0 = seg_begin;
  i32x4a rec0 = cs0 < seg_end ? seg_rec(cs0) : i32x4a{0, 0, 0, 0};
  while (cs0 < seg_end && rec0[1] == rec0[2]) {
    write_segment(row_index(rec0[0], row), rec0[3], true);
    ++cs0;
    if (cs0 < seg_end) rec0 = seg_rec(cs0);
  }
  if (cs0 >= seg_end) return;

  // first tile: gathered into buf_a before the stream starts
  Tile ct = first_tile_rec(cs0, rec0);
  uint64_t cmask;
  const TileMeta m0 = fetch_meta(ct.u, ct.blk);
  {
    qrow = row_index(ct.u, row);
    // The first segment's queries go through LDS when the workgroup's rows
    // are consecutive rows of q (always, except for a dense call with fewer
    // heads than h_q and several query tokens), staged in the buffer the
    // first step gathers into (bf16) or dequantizes into (FP8).
    const bool q_lds = SPARSE || p.heads == p.h_q || p.s_q == 1;
    uint8_t* const q_stage = FP8 ? buf_a : buf_b;
    if (q_lds)
      gather_q(ct.u, q_stage);
    else
      load_q(ct.u);
    if (!SPARSE) n_vis = visible(m0.len);
    reset_state();
    const Gather g0 = plan_gather(ct.blk, m0);
    cmask = g0.vmask;
    const bool g0_issued = !SPARSE || !WIDE || cmask != 0;
    if (g0_issued) {
      if constexpr (FP8)
        gather_fp8(g0, stg_a);
      else
        gather_all(g0, buf_a);
    }
    if (q_lds) {
      // the query loads were issued before the tile's, which stay in flight
      // (an FP8 tile is 10 or 11 loads per wavefront)
      if (g0_issued)
        wait_vmem_n<FP8 ? SNL / kWaves : NLW>();
      else
        wait_vmem();
      lds_barrier();
      read_q(q_stage);
      lds_barrier();  // every wavefront has its queries before the buffer is reused
    }
  }
  // Tile j+1 is gathered during step j; metadata runs two tiles ahead of the
  // gathers (that of tile j+3 is read at the end of step j).  All scalar
  // metadata reads of a step happen after its compute: a scalar load in
  // flight shares the LDS wait counter and would turn every LDS operand wait
  // of the tile into a full drain.
  Tile nt = next_tile(ct);
  Tile n2t = next_tile(nt);
  // Past the last tile the metadata repeats the last real tile's, so the
  // unused loads of the last step read a page this workgroup just read
  // (rather than every workgroup reading page 0 at once).
  TileMeta nmeta = m0, n2meta = m0;
  if (nt.s < seg_end) nmeta = fetch_meta(nt.u, nt.blk);
  n2meta = nmeta;
  if (n2t.s < seg_end) n2meta = fetch_meta(n2t.u, n2t.blk);

  // One step computes the tile in `cur_buf` while the next one streams into
  // `nxt_buf`.  The two buffers are distinct LDS objects named statically at
  // every call site, so the compiler can tell reads of one from the
  // asynchronous writes into the other and does not wait for those writes.
  // FP8: the buffers are the staging buffers; the next tile's gather is issued
  // whole at the start of the step, then the current tile is dequantized into
  // buf_a and computed, with the pair exchanges in its (consumed) staging
  // buffer.
  auto step = [&](uint8_t* cur_buf, uint8_t* nxt_buf) __attribute__((always_inline)) -> bool {
#pragma unroll
    for (int ct_ = 0; ct_ < NCT; ++ct_) pin_agpr(acc[ct_]);  // loop-carried in AGPRs
    wait_vmem();
    __syncthreads();
    const bool has_next = nt.s < seg_end;
    // Without a next tile the slices load page 0 (or, sparse, the zero row)
    // instead: harmless, in bounds and branch-free (a branch per slice costs
    // the QK loop its schedule).
    nx_plan = plan_gather(nt.blk, nmeta);
    const uint64_t nmask = has_next ? nx_plan.vmask : 0;
    nx_dst = nxt_buf;
    nx_ln = lane;
    asm volatile("" : "+v"(nx_ln));
    const int next_q_unit = (ct.last && has_next) ? nt.u : -1;
    if constexpr (FP8) {
      if (has_next && (!SPARSE || !WIDE || nmask != 0)) gather_fp8(nx_plan, nxt_buf);
      if (!SPARSE || !WIDE || cmask != 0) {
        dequant(cur_buf, buf_a);
        lds_barrier();
        compute_tile(buf_a, ct.blk, cmask, next_q_unit, cur_buf);
      } else if (next_q_unit >= 0) {
        load_q(next_q_unit);
      }
    } else if (!SPARSE || !WIDE || cmask != 0) {
      compute_tile(cur_buf, ct.blk, cmask, next_q_unit, x_own);
    } else {
      if (next_q_unit >= 0) load_q(next_q_unit);
#pragma unroll
      for (int i = 0; i < NLW; ++i) gather_slice(i);
    }
    // The last step: its (unused) tile loads finished during the compute;
    // waiting for them here, before the output stores, lets the workgroup end
    // without waiting for those stores (no load into LDS outlives it).
    if (!has_next) wait_vmem();
    if (ct.last) {
      write_segment(qrow, seg_slot(ct.s), false);
      const int e_end = has_next ? nt.s : seg_end;
      for (int e = ct.s + 1; e < e_end; ++e)  // segments without tiles passed over
        write_segment(row_index(seg_u(e), row), seg_slot(e), true);
      if (has_next) {
        qrow = row_index(nt.u, row);
        if (!SPARSE) n_vis = visible(nmeta.len);
        reset_state();
      }
    }
    if (!has_next) return false;
    const Tile n3t = next_tile(n2t);
    TileMeta n3meta = n2meta;
    if (n3t.s < seg_end) n3meta = fetch_meta(n3t.u, n3t.blk);
    ct = nt;
    cmask = nmask;
    nt = n2t;
    nmeta = n2meta;
    n2t = n3t;
    n2meta = n3meta;
    return true;
  };
  if constexpr (FP8) {
    for (;;) {
      if (!step(stg_a, stg_b)) break;
      if (!step(stg_b, stg_a)) break;
    }
  } else {
    for (;;) {
      if (!step(buf_a, buf_b)) break;
      if (!step(buf_b, buf_a)) break;
    }
  }
  // (the last step waited for its tile loads before its output stores)
#endif
}

// Launches the pair kernel (64 query rows per workgroup, whatever the rows per
// workgroup the schedule was sized for: a part then spans ceil(rows / 64)
// workgroups) for one element type: the FP8-with-scale cache (bf16 only) or
// bf16 / fp16 caches of 576- or 512-wide rows.
template <bool F16>
hipError_t launch_pairs_t(const SplitKVParams& p, int d_qk, bool sparse, bool fp8, hipStream_t stream) {
  const int row_blocks = (p.rows + kRowsPerGroup - 1) / kRowsPerGroup;
  const int groups = p.num_parts * row_blocks;
  if (groups <= 0) return hipSuccess;
  SplitKVParams q = p;
  q.row_blocks = row_blocks;
  const dim3 grid(groups), block(256);
  // Sparse rows are addressed with 32-bit byte offsets while the pool (plus
  // the past-the-end row an all-invalid tile reads) fits in 32 bits.
  const uint64_t row_bytes = fp8 ? kFp8RowBytes : uint64_t(d_qk) * 2;
  const bool wide = (uint64_t(p.num_rows) + 2) * row_bytes > 0xFFFFFFFFull;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, block, 0, stream, q); };
  if constexpr (F16) {
    if (d_qk == 576) {
      if (!sparse) go(mla_splitkv<576, false, false, false, true>);
      else if (!wide) go(mla_splitkv<576, true, false, false, true>);
      else go(mla_splitkv<576, true, true, false, true>);
    } else {
      if (!sparse) go(mla_splitkv<512, false, false, false, true>);
      else if (!wide) go(mla_splitkv<512, true, false, false, true>);
      else go(mla_splitkv<512, true, true, false, true>);
    }
  } else {
    if (fp8) {
      if (!sparse) go(mla_splitkv<576, false, false, true, false>);
      else if (!wide) go(mla_splitkv<576, true, false, true, false>);
      else go(mla_splitkv<576, true, true, true, false>);
    } else if (d_qk == 576) {
      if (!sparse) go(mla_splitkv<576, false, false, false, false>);
      else if (!wide) go(mla_splitkv<576, true, false, false, false>);
      else go(mla_splitkv<576, true, true, false, false>);
    } else {
      if (!sparse) go(mla_splitkv<512, false, false, false, false>);
      else if (!wide) go(mla_splitkv<512, true, false, false, false>);
      else go(mla_splitkv<512, true, true, false, false>);
    }
  }
  return hipGetLastError();
}

}  // namespace mla
