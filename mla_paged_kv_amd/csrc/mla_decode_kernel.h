// Split-KV decode kernel of the paged MLA library for bf16 / fp16 caches,
// written for gfx950 (CDNA4).
//
// One workgroup = (part, row block) of the tile-scheduler metadata: 4
// wavefronts, one per SIMD.  Every wavefront owns 32 query rows outright: it
// computes their scores, their softmax and their output columns with no
// exchange with the other wavefronts, so the only workgroup barrier of a tile
// is the one that hands a tile buffer from the gathers to the readers.  With
// NCOL = 512 each wavefront holds all 512 output columns of its rows (the
// accumulator fills the 256 AGPRs) and a workgroup covers 128 rows; with NCOL
// = 256 or 128, two or four wavefronts share 32 rows, each computing the
// scores in full and its own quarter or half of the output columns, and a
// workgroup covers 64 or 32 rows (for units with few rows).
//
// The part's segments (unit, block range, slot) are walked as one stream of
// 32-token tiles, two per 64-token page (or per 64-index chunk).  Tiles stream
// HBM -> LDS through direct-to-LDS loads into 4 buffers: while tile t is
// computed, tiles t+1 and t+2 are in flight or landed and the gather of tile
// t+3 is issued in slices between the matrix-core instructions of tile t.
// Per tile and wavefront:
//   S^T = K . Q^T     v_mfma_f32_32x32x16_{bf16,f16}, K from LDS, Q^T resident
//                     in registers for the whole segment;
//   softmax           fp32, base 2, one query row per lane pair; the running
//                     reference maximum moves only when a tile's maximum
//                     exceeds it by more than 2^8, so the accumulator is
//                     rarely rescaled (the result does not depend on it);
//   O^T += V^T . P^T  V^T read with the LDS transpose read from the first 512
//                     columns of the same tile.
// A segment covering its whole unit writes 16-bit O and the LSE; a split
// segment writes fp32 O and a base-2 LSE into its workspace slot for the
// combine kernel.  This is the structure the deepep.org usage page describes
// (tile scheduler, block-table manager; QK^T, scaled softmax, output stages);
// sparse gathering follows the upstream FlashMLA README ("Sparse Attention
// (indices tensor)").  Only active heads are computed.
//
// LDS tile layout: cache row t of a tile occupies 16-byte chunks
// [t*CPR, (t+1)*CPR), with its chunk c stored at position c ^ f(t); f depends
// on bits 0..3 of t only, spreads the operand reads over all banks, and is
// applied on the source side of the gather.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "mla_internal.h"
#include "mla_kernels.h"

namespace mla {

namespace dk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Read-only metadata (scheduler output, block table, sequence lengths) is read
// through the constant address space, so uniform reads become scalar loads
// that do not share the vector-memory counter with the tile gathers.
typedef const __attribute__((address_space(4))) int32_t cint;
// a segment record (unit, first block, end block, slot), read as one scalar load
typedef int32_t i32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef const __attribute__((address_space(4))) i32x4a cseg;
__device__ __forceinline__ cint* as_const(const int32_t* ptr) { return (cint*)(uintptr_t)ptr; }

constexpr int kTile = 32;      // tokens per tile (half a page / index chunk)
constexpr int kPage = 64;      // tokens per page (the scheduler's block)
constexpr int kBufs = 4;       // LDS tile buffers
constexpr int kWaves = 4;      // wavefronts per workgroup
constexpr int kDV = 512;       // value width
constexpr int kRowsWave = 32;  // query rows per wavefront
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference maximum may lag
// Word 3 of a raw (untyped) buffer resource on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
template <bool F16>
__device__ __forceinline__ unsigned short f2e(float x) {
  if constexpr (F16)
    return __builtin_bit_cast(unsigned short, (_Float16)x);
  else
    return __builtin_bit_cast(unsigned short, (__bf16)x);
}
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier for LDS traffic: waits for this wavefront's LDS and scalar
// accesses (not for the gathers still in flight), then the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// lanes l and l ^ 32 hold the two k-groups of a query row: v_permlane32_swap
// of a value with a copy of itself leaves the lower half broadcast in one
// register and the upper half in the other (written out because the compiler
// folds the builtin's two results when both operands are equal)
__device__ __forceinline__ void swap_halves(float v, float& lo, float& hi) {
  lo = v;
  hi = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}
// NaN-propagating maximum (v_maximum3_f32; no operand quieting).  Masked
// scores are -inf, never NaN.
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
// Register-class pin: keeps the long-lived accumulators in AGPRs.
__device__ __forceinline__ void pin_agpr(f32x16& x) { asm volatile("" : "+a"(x)); }
// A VGPR copy of an accumulator tile: the accumulator itself is only ever an
// AGPR operand, so the register allocator never gives it a VGPR home.
__device__ __forceinline__ f32x16 read_acc(const f32x16& x) {
  f32x16 t = x;
  asm volatile("" : "+v"(t));
  return t;
}

// Direct-to-LDS loads written as inline assembly.  Each lane copies 16 (or 4)
// bytes to LDS address m0 + 16 * lane (4 * lane).  The compiler does not see
// them as loads into LDS: it would otherwise make every LDS read of the tile
// being computed wait for all of them, because the tile buffers are picked at
// run time.  The kernel's own waits order them (s_waitcnt vmcnt with the
// exact count of loads issued after, then a barrier).  They write no
// register, so nothing of the compiler's register use can overlap them.
// The compiler cannot see the hazards of an instruction inside asm either, so
// the nops are written out: a buffer resource that a VALU instruction has just
// written (v_readlane_b32, where the compiler keeps SGPRs in VGPR lanes) needs
// 5 wait states before a memory instruction reads it, and an M0 write needs 1
// before an LDS DMA.
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds_addr)
               : "memory");
}
__device__ __forceinline__ void dma_b32(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds_addr)
               : "memory");
}
// N query fragments of 16 bytes at a 32-byte stride, loaded and waited for
// in one statement: the registers are written before the statement ends, so
// no load into a register is ever in flight outside it (early-clobber
// outputs keep the address register apart from them).  Compiler-visible
// loads instead would be waited for by counts that leave out the
// direct-to-LDS loads issued after them, and the compiler would drain every
// gather in flight before the QK product of every tile.  The closing
// vmcnt(0) also waits for every older load: the tile gathers in flight at a
// segment change land before the next segment starts.
#define QO(i) "=&v"(d[i])
template <int N>
__device__ __forceinline__ void load_q_half(bf16x8* d, const uint16_t* src) {
  static_assert(N == 18 || N == 16, "18 (d_qk 576) or 16 (d_qk 512) fragments");
  if constexpr (N == 18) {
    asm volatile(
        "global_load_dwordx4 %0, %18, off offset:0\n\tglobal_load_dwordx4 %1, %18, off offset:32\n\t"
        "global_load_dwordx4 %2, %18, off offset:64\n\tglobal_load_dwordx4 %3, %18, off offset:96\n\t"
        "global_load_dwordx4 %4, %18, off offset:128\n\tglobal_load_dwordx4 %5, %18, off offset:160\n\t"
        "global_load_dwordx4 %6, %18, off offset:192\n\tglobal_load_dwordx4 %7, %18, off offset:224\n\t"
        "global_load_dwordx4 %8, %18, off offset:256\n\tglobal_load_dwordx4 %9, %18, off offset:288\n\t"
        "global_load_dwordx4 %10, %18, off offset:320\n\tglobal_load_dwordx4 %11, %18, off offset:352\n\t"
        "global_load_dwordx4 %12, %18, off offset:384\n\tglobal_load_dwordx4 %13, %18, off offset:416\n\t"
        "global_load_dwordx4 %14, %18, off offset:448\n\tglobal_load_dwordx4 %15, %18, off offset:480\n\t"
        "global_load_dwordx4 %16, %18, off offset:512\n\tglobal_load_dwordx4 %17, %18, off offset:544\n\t"
        "s_waitcnt vmcnt(0)"
        : QO(0), QO(1), QO(2), QO(3), QO(4), QO(5), QO(6), QO(7), QO(8), QO(9), QO(10), QO(11),
          QO(12), QO(13), QO(14), QO(15), QO(16), QO(17)
        : "v"(src) : "memory");
  } else {
    asm volatile(
        "global_load_dwordx4 %0, %16, off offset:0\n\tglobal_load_dwordx4 %1, %16, off offset:32\n\t"
        "global_load_dwordx4 %2, %16, off offset:64\n\tglobal_load_dwordx4 %3, %16, off offset:96\n\t"
        "global_load_dwordx4 %4, %16, off offset:128\n\tglobal_load_dwordx4 %5, %16, off offset:160\n\t"
        "global_load_dwordx4 %6, %16, off offset:192\n\tglobal_load_dwordx4 %7, %16, off offset:224\n\t"
        "global_load_dwordx4 %8, %16, off offset:256\n\tglobal_load_dwordx4 %9, %16, off offset:288\n\t"
        "global_load_dwordx4 %10, %16, off offset:320\n\tglobal_load_dwordx4 %11, %16, off offset:352\n\t"
        "global_load_dwordx4 %12, %16, off offset:384\n\tglobal_load_dwordx4 %13, %16, off offset:416\n\t"
        "global_load_dwordx4 %14, %16, off offset:448\n\tglobal_load_dwordx4 %15, %16, off offset:480\n\t"
        "s_waitcnt vmcnt(0)"
        : QO(0), QO(1), QO(2), QO(3), QO(4), QO(5), QO(6), QO(7), QO(8), QO(9), QO(10), QO(11),
          QO(12), QO(13), QO(14), QO(15)
        : "v"(src) : "memory");
  }
}
#undef QO
__device__ __forceinline__ void dma_global_b128(const void* src, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_addr) : "memory");
}

// Workgroups go to the 8 XCDs round-robin; each XCD gets a contiguous run of
// logical groups, so the row blocks of a part (and nearby parts) share an L2.
__device__ __forceinline__ int logical_group(int id, int total) {
  constexpr int kXcd = 8;
  const int xcd = id % kXcd, k = id / kXcd;
  const int per = total / kXcd, rem = total % kXcd;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + k;
}

// ---- v_mfma_f32_32x32x16 operand layouts ----
// A (32 x 16): lane l holds row l % 32, k = 8 (l / 32) .. +7.  B (16 x 32):
// lane l holds column l % 32, k = 8 (l / 32) .. +7.  C (32 x 32): register j
// of lane l is row 8 (j / 4) + 4 (l / 32) + j % 4, column l % 32.
//
// The matrix-core instructions are written as inline assembly so that their
// register classes are the kernel's: the output accumulator (up to 256
// registers) in AGPRs, the scores in VGPRs.  (The compiler picks one class
// for every MFMA result of a function, and the two together exceed either
// file.)  The compiler does not see these as MFMAs, so the wait states the
// hardware needs around them are written here:
//   * a VALU (or v_accvgpr_read) read of an MFMA result waits at least 12
//     states after the MFMA is issued: kMfmaResultWait (16) before the scores
//     are read and before the accumulator is read out;
//   * an MFMA reading a VGPR or AGPR that a VALU instruction (or
//     v_accvgpr_write) has just written waits 4 states (the nop in the
//     first instruction of each PV k-step, and after a rescale);
//   * an MFMA accumulating into exactly the registers the previous one wrote
//     needs no wait.
__device__ __forceinline__ void mfma_wait_result() { asm volatile("s_nop 7\n\ts_nop 7" ::: "memory"); }
__device__ __forceinline__ void mfma_wait_operands() { asm volatile("s_nop 3" ::: "memory"); }
// c (VGPRs) = a . b (+ c unless first)
template <bool F16>
__device__ __forceinline__ void mfma_v(f32x16& c, bf16x8 a, bf16x8 b, bool first) {
  if constexpr (F16) {
    if (first)
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  } else {
    if (first)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  }
}
// c (AGPRs) += a . b
template <bool F16>
__device__ __forceinline__ void mfma_a(f32x16& c, bf16x8 a, bf16x8 b) {
  if constexpr (F16)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// c (AGPRs) = 0, through the matrix core (zero operands, zero srcC): the
// accumulator keeps its registers and needs no VALU writes of 256 AGPRs
__device__ __forceinline__ void mfma_zero(f32x16& c, bf16x8 z) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "+a"(c) : "v"(z));
}
// tile token of score register v of k-group g (C layout of S^T)
__device__ __forceinline__ int tok(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }
// output column (within the wavefront's columns) of O^T register j of column
// tile ct, k-group g
__device__ __forceinline__ int col(int ct, int j, int g) {
  return 32 * ct + 8 * (j >> 2) + 4 * g + (j & 3);
}
// V^T transpose read h of PV k-step kc: the tile row (token) this lane
// addresses.  PV k-step kc covers tokens 16 kc + {4g..4g+3, 8+4g..8+4g+3} for
// k-group g, which are exactly the tokens that lane's score registers
// 8 kc .. 8 kc + 7 hold, so P^T comes straight from the lane's own scores.
__device__ __forceinline__ int vrow(int kc, int h, int lane) {
  return 16 * kc + 8 * h + 4 * (lane >> 5) + ((lane & 15) >> 2);
}
__device__ __forceinline__ int vchunk(int lane) { return 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1); }
// chunk swizzle f(t) for 72- and 64-chunk rows; f(t) < 8 (resp. < 16): it
// permutes chunks inside aligned groups of 8 (resp. 16) and depends only on
// bits 0..3 of t.  16 consecutive rows read at one logical chunk hit 16
// distinct 16-byte bank groups.
template <int CPR>
__host__ __device__ constexpr int swz(int t) {
  if constexpr (CPR == 72) return 4 * ((t >> 1) & 1) + ((t >> 2) & 3);
  else return ((t & 3) << 2) | ((t >> 2) & 3);
}

// A tile of the part's stream.  All fields are wavefront-uniform.
struct Tile {
  int s;     // segment (seg_end: past the end of the stream)
  int pos;   // 32-token tile of the unit: block pos / 2, half pos % 2
  int u;     // unit
  int b1;    // end block of the segment
  int len;   // unit length (dense: cache length; sparse: topk)
};

}  // namespace dk

// WIDE (sparse only): the cache pool (plus the past-the-end row) does not fit
// 32-bit byte offsets, so rows are gathered with 64-bit addresses.
template <int D_QK, bool SPARSE, bool WIDE, bool F16, int NCOL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode(SplitKVParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using namespace dk;
  constexpr int CPR = D_QK / 8;            // 16-byte chunks per cache row
  constexpr int RSB = CPR * 16;            // LDS row stride in bytes
  constexpr int TBUF = kTile * RSB;        // bytes per tile buffer
  constexpr int NLW = TBUF / 1024 / kWaves;  // 1 KB gather loads per wavefront and tile
  constexpr int RPW = kTile / kWaves;      // tile rows gathered per wavefront (8)
  constexpr int KK = D_QK / 16;            // QK k-steps
  constexpr int NCT = NCOL / 32;           // output column tiles per wavefront
  constexpr int WPR = kDV / NCOL;          // wavefronts sharing one row group
  constexpr int RB = kRowsWave * kWaves / WPR;  // query rows per workgroup
  constexpr int FMAX = CPR == 72 ? 8 : 16;
  constexpr int NKB = FMAX / 2;            // K-read bases (kk mod NKB)
  constexpr int NVB = FMAX / 4;            // V-read bases (ct mod NVB)
  constexpr int ISLOT = 256;               // LDS bytes of one tile's slot (64 lanes x 4)
  constexpr int NISLOT = 8;                // slots (tile k uses slot k % 8)
  static_assert(TBUF % (1024 * kWaves) == 0 && RPW * RSB == NLW * 1024, "whole loads per wavefront");
  static_assert(NCOL == 512 || NCOL == 256 || NCOL == 128, "column split");
  static_assert(kBufs * TBUF <= 160 * 1024, "tile buffers fit the LDS");
  // the 4 tile buffers, then the slots of the tiles' page numbers (dense) or
  // indices (sparse)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kBufs * TBUF + NISLOT * ISLOT];
  const uint32_t lds_base = uint32_t(uintptr_t((__attribute__((address_space(3))) uint8_t*)lds));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rgrp = wave / WPR;              // row group of the wavefront
  const int cq = wave % WPR;                // column slice of the wavefront
  const int lrow = lane & 31;               // query row owned within the row group
  const int lgrp = lane >> 5;               // k-group of the MFMA operands

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
  // the grid covers p.num_parts parts; the device header says how many exist
  // (header word 15 is -1 when the device scheduler rejected the lengths)
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

  const int row = rb * RB + rgrp * kRowsWave + lrow;
  const bool row_ok = row < p.rows;

  // Per-lane LDS operand bases (chunk c of tile row t is at c ^ f(t), f fixed
  // per lane by the low bits of the lane's rows):
  //  K  (A of QK): row lrow, chunk 2 kk + lgrp -> kbase[kk % NKB] + 32 kk;
  //  V^T (A of PV, transpose read h): row vrow(kc, h), chunk 4 ct + y of the
  //     wavefront's columns -> vbase[h][ct % NVB] + 64 ct + 256 kc RSB / 16.
  int kbase[NKB], vbase[2][NVB];
  {
    const int fk = swz<CPR>(lrow);
#pragma unroll
    for (int j = 0; j < NKB; ++j)
      kbase[j] = lrow * RSB + 16 * (lgrp ^ (fk % 2)) + 32 * ((j ^ (fk / 2)) - j);
    const int y = vchunk(lane);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int vr = vrow(0, h, lane);
      const int fv = swz<CPR>(vr);
#pragma unroll
      for (int j = 0; j < NVB; ++j)
        vbase[h][j] = vr * RSB + 16 * (y ^ (fv % 4)) + 64 * ((j ^ (fv / 4)) - j) + 8 * (lane & 1) +
                      64 * NCT * cq;
    }
  }

  // Dense gathers: this lane's byte offset in the tile for each of its NLW
  // loads (its row and chunk as in gather_one below), computed once.
  int goff[SPARSE ? 1 : NLW];
  if constexpr (!SPARSE) {
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int q0 = 64 * i;
      const int tl = q0 / CPR;
      const int bnd = (tl + 1) * CPR - q0;
      const bool second = bnd < 64 && lane >= bnd;
      const int f16 = 16 * ((second ? swz<CPR>(tl + 1) : swz<CPR>(tl)) ^ (2 * (wave & 1)));
      const int in_row = ((q0 + lane) * 16 - (tl + (second ? 1 : 0)) * RSB) ^ f16;
      goff[i] = (RPW * wave + tl + (second ? 1 : 0)) * RSB + in_row;
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

  // ---- the tile stream ----
  auto seg_u = [&](int s) __attribute__((always_inline)) { return segs[4 * s + 0]; };
  auto seg_slot = [&](int s) __attribute__((always_inline)) { return segs[4 * s + 3]; };
  auto seg_rec = [&](int s) __attribute__((always_inline)) { return *(cseg*)(segs + 4 * s); };
  auto unit_len = [&](int u) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) return p.topk;
    else return as_const(p.seqlens)[u];
  };
  // first tile at or after segment s2 (segments without blocks are skipped;
  // their outputs are written when the stream passes them)
  // first tile at or after segment s2 (whose record is rec, when s2 is a
  // segment), skipping segments without tiles; each record is one load
  auto first_tile_rec = [&](int s2, i32x4a rec) __attribute__((always_inline)) -> Tile {
    while (s2 < seg_end && rec[1] == rec[2]) {
      ++s2;
      if (s2 < seg_end) rec = seg_rec(s2);
    }
    if (s2 >= seg_end) return Tile{seg_end, 0, 0, 0, 1};
    return Tile{s2, 2 * rec[1], rec[0], rec[2], unit_len(rec[0])};
  };
  auto first_tile_from = [&](int s2) __attribute__((always_inline)) -> Tile {
    return first_tile_rec(s2, s2 < seg_end ? seg_rec(s2) : i32x4a{0, 0, 0, 0});
  };
  // a block's second half exists unless the unit ends in its first half
  auto has_next_half = [&](const Tile& t) __attribute__((always_inline)) -> bool {
    return (t.pos & 1) == 0 && t.len - (t.pos >> 1) * kPage > kTile;
  };
  auto is_last = [&](const Tile& t) __attribute__((always_inline)) -> bool {
    return !has_next_half(t) && (t.pos >> 1) + 1 >= t.b1;
  };
  auto next_tile = [&](const Tile& t) __attribute__((always_inline)) -> Tile {
    if (t.s >= seg_end) return t;
    if (has_next_half(t)) return Tile{t.s, t.pos + 1, t.u, t.b1, t.len};
    const int nb = (t.pos >> 1) + 1;
    if (nb < t.b1) return Tile{t.s, 2 * nb, t.u, t.b1, t.len};
    return first_tile_from(t.s + 1);
  };

  // ---- per-tile metadata through LDS ----
  // What a tile's gather needs -- its physical page (dense) or its 32 row
  // indices (sparse) -- is copied into LDS slot (tile number % 8) by one
  // direct-to-LDS load per wavefront three steps ahead of the gather, and read
  // back after the step's barrier.  (A scalar load instead would be waited
  // for wherever the compiler first moves its register.)  Dense: every lane
  // loads the same block-table entry.  Sparse: lanes 0..31 load the tile's
  // 32 indices, lanes 32..63 repeat them; positions past the list read its
  // last entry and are invalid by position.  Every wavefront issues the load,
  // so each step costs exactly one more vector-memory operation per wavefront.
  auto meta_rsrc = [&]() __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(SPARSE ? p.indices : p.block_table), 0, 0x7FFFFFFF, kBufferWord3);
  };
  auto load_slot = [&](const Tile& t, int slot) __attribute__((always_inline)) {
    uint32_t off;
    if constexpr (SPARSE) {
      int pos = t.pos * kTile + lrow;
      pos = pos < t.len ? pos : t.len - 1;
      off = uint32_t((size_t(t.u) * p.topk + pos) * 4);
    } else {
      off = uint32_t((size_t(t.u) * p.bt_stride + (t.pos >> 1)) * 4);
    }
    dma_b32(meta_rsrc(), off, lds_base + kBufs * TBUF + slot * ISLOT);
  };
  // this lane's index of a sparse tile (lanes 0..31: tile token = lane), -1
  // past the list; or the dense tile's page (uniform)
  auto read_slot = [&](const Tile& t, int slot) __attribute__((always_inline)) -> int {
    const int v = *reinterpret_cast<const int*>(lds + kBufs * TBUF + slot * ISLOT + 4 * lrow);
    if constexpr (SPARSE)
      return t.pos * kTile + lrow < t.len ? v : -1;
    else
      return __builtin_amdgcn_readfirstlane(v);
  };

  // ---- tile gathers ----
  // Wavefront w fills LDS rows 8w..8w+7 with NLW direct-to-LDS loads of 1 KB
  // (64 lanes x 16 bytes): load i covers LDS chunks 64 i + lane of those rows,
  // i.e. row tl = (64 i + lane) / CPR at chunk position c = (64 i + lane) %
  // CPR, whose source chunk is c ^ f(row).  Rows past a dense tile's last
  // valid row lie past the end of the tile's buffer resource and read as
  // zeros; invalid sparse indices read row num_rows, past the end of the
  // pool's buffer resource, which also returns zeros (WIDE: the tile's first
  // valid row).  Such tokens are masked out of the softmax, and a zero row
  // adds exactly zero.
  constexpr int ROWB = RSB;
  struct Plan {
    int phys;  // dense: physical page; sparse: unused
    int r0;    // dense: first tile row in the page (0 or 32)
    int tmax;  // dense: last valid row of the tile (rows past it read as zeros)
    int idx;   // sparse: this lane's row index (lanes 0..31; substituted)
    uint32_t vmask;  // sparse: valid tokens of the tile (bit t)
  };
  auto plan_tile = [&](const Tile& t, int sv) __attribute__((always_inline)) -> Plan {
    Plan g{SPARSE ? 0 : sv, (t.pos & 1) * kTile, kTile - 1, 0, 0xFFFFFFFFu};
    const int idx = sv;
    if constexpr (SPARSE) {
      const bool ok = idx >= 0 && idx < p.num_rows;
      g.vmask = uint32_t(__ballot(ok && lane < 32));
      if constexpr (WIDE) {
        const int first = g.vmask ? __builtin_ctz(g.vmask) : 0;
        const int sub = g.vmask ? __shfl(idx, first) : 0;
        g.idx = ok ? idx : sub;
      } else {
        g.idx = ok ? idx : p.num_rows;
      }
    } else {
      const int vt = t.len - t.pos * kTile;
      g.tmax = vt < 1 ? 0 : (vt > kTile ? kTile - 1 : vt - 1);
    }
    return g;
  };
  // a dense tile's valid rows: the resource starts at the tile's first row and
  // ends after its last valid one, so a load of a row past it returns zeros
  // (masked out of the softmax, and zero rows add exactly nothing)
  auto tile_rsrc = [&](const Plan& g) __attribute__((always_inline)) {
    const uint8_t* pg = reinterpret_cast<const uint8_t*>(p.kv) + size_t(g.phys) * kPage * ROWB +
                        size_t(g.r0) * ROWB;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pg), 0, (g.tmax + 1) * ROWB,
                                            kBufferWord3);
  };
  // the whole pool (sparse rows, pools whose byte size plus one row fits 32 bits)
  auto pool_rsrc = [&]() __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.kv), 0,
                                            int(uint32_t(p.num_rows) * uint32_t(ROWB)), kBufferWord3);
  };
  // Load i of this wavefront's share of tile plan g into buffer dst.  Dense:
  // the lane's offset in the tile is fixed (goff, computed once).  Sparse:
  // `ln` is the lane id through an opaque copy, so the few offset operations
  // are recomputed per tile instead of keeping NLW offsets alive.
  auto gather_one = [&](const Plan& g, int dst, int i, int ln) __attribute__((always_inline)) {
    const uint32_t to = lds_base + uint32_t(dst + (NLW * wave + i) * 1024);
    if constexpr (SPARSE) {
      const int q0 = 64 * i;
      const int tl = q0 / CPR;                 // first row of the load (within the wave's 8)
      const int bnd = (tl + 1) * CPR - q0;     // first lane of row tl + 1 (>= 64: none)
      const bool second = bnd < 64 && ln >= bnd;
      // swizzle of the lane's row: the row's bit 3 is wave bit 0 (RPW = 8)
      const int f16 = 16 * ((second ? swz<CPR>(tl + 1) : swz<CPR>(tl)) ^ (2 * (wave & 1)));
      const int in_row = ((q0 + ln) * 16 - (tl + (second ? 1 : 0)) * RSB) ^ f16;  // byte in the row
      const int r0 = __builtin_amdgcn_readlane(g.idx, RPW * wave + tl);
      const int r1 = bnd < 64 ? __builtin_amdgcn_readlane(g.idx, RPW * wave + tl + 1) : r0;
      const int r = second ? r1 : r0;
      if constexpr (WIDE) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(p.kv) + size_t(uint32_t(r)) * RSB + in_row;
        dma_global_b128(src, to);
      } else {
        dma_b128(pool_rsrc(), uint32_t(r) * uint32_t(RSB) + uint32_t(in_row), to);
      }
    } else {
      (void)ln;
      dma_b128(tile_rsrc(g), uint32_t(goff[i]), to);
    }
  };

  // ---- per-segment state ----
  bf16x8 qf[KK] = {};      // Q^T fragments of the wavefront's 32 rows
  f32x16 acc[NCT];         // O^T accumulator (AGPRs)
  float m_run = -__builtin_inff();    // reference maximum (base 2, scaled) of the lane's row
  float m_exact = -__builtin_inff();  // exact row maximum of the scaled logits (base 2)
  float l_run = 0.f;                  // the row's sum of softmax numerators
  bool seg_first = true;
  int n_vis = 0;
  // the accumulator starts every segment at zero
  auto zero_acc = [&]() __attribute__((always_inline)) {
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
    asm volatile("" : "+v"(z));
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) mfma_zero(acc[ct], z);
  };
  auto reset_state = [&]() __attribute__((always_inline)) {
    zero_acc();
    seg_first = true;
    m_run = -__builtin_inff();
    m_exact = -__builtin_inff();
    l_run = 0.f;
  };
  // rows past the unit's last row read that last row (never written back).
  // WIDE kernels spill registers, so their loads are the compiler's own (they
  // wait for everything at every step anyway).
  auto load_q = [&](int u) __attribute__((always_inline)) {
    const uint16_t* qp = p.q + row_index(u, row_ok ? row : p.rows - 1) * D_QK + 8 * lgrp;
    if constexpr (WIDE) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
    } else {
      static_assert(KK % 2 == 0, "two halves");
#pragma unroll
      for (int h = 0; h < 2; ++h) load_q_half<KK / 2>(qf + h * (KK / 2), qp + h * (KK / 2) * 16);
    }
  };

  // The first segment's queries, when the workgroup's rows are consecutive
  // rows of q (always, except for a dense call with fewer heads than h_q and
  // several query tokens): wavefront w copies the 32 rows of its row group
  // into tile buffer w with 1 KB direct-to-LDS loads laid out like a tile
  // (chunk c of row t at c ^ f(t); rows past the unit's last one read zeros),
  // and after the wait reads its fragments back with the K-read addresses.
  // Each load fetches 1 KB of consecutive bytes, where the register loads of
  // a segment change fetch 32 bytes from each of 32 rows: the prologue's
  // burst of query loads from every workgroup at once takes several times
  // longer that way.
  static_assert(kWaves / WPR <= kBufs && kRowsWave == kTile, "a row group's queries fill one tile buffer");
  auto gather_q_block = [&](int u) __attribute__((always_inline)) {
    const int r0 = rb * RB + rgrp * kRowsWave;  // first row of the wavefront's block
    const int nvalid = p.rows - r0 < 0 ? 0 : (p.rows - r0 > kRowsWave ? kRowsWave : p.rows - r0);
    const uint16_t* base = p.q + row_index(u, r0 < p.rows ? r0 : p.rows - 1) * D_QK;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, nvalid * RSB,
                                                      kBufferWord3);
#pragma unroll
    for (int i = 0; i < kWaves * NLW; ++i) {
      const int q = 64 * i + lane;
      const int t = q / CPR;
      const int c = q - t * CPR;
      dma_b128(rs, uint32_t(t * RSB + 16 * (c ^ swz<CPR>(t))),
               lds_base + uint32_t(rgrp * TBUF + i * 1024));
    }
  };
  auto read_q_block = [&]() __attribute__((always_inline)) {
    const uint8_t* buf = lds + rgrp * TBUF;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(buf + kbase[kk % NKB] + kk * 32);
  };

  // Writes the segment result of this lane's row (its NCOL columns): 16-bit O
  // and the LSE when the segment covers its unit (slot < 0), else fp32 O and
  // the base-2 LSE into workspace slot `slot`.  A row without any visible
  // token gets O = 0 and LSE = -inf.  Every store of a lane goes through one
  // base pointer with immediate offsets.
  auto write_segment = [&](int u, int slot) __attribute__((always_inline)) {
    mfma_wait_result();  // the last PV product has landed before it is read out
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) pin_agpr(acc[ct]);
    const bool empty = !(l_run > 0.f) || seg_first;
    const float inv = empty ? 0.f : 1.f / l_run;
    const float lse2 = empty ? -__builtin_inff() : m_run + fast_log2(l_run);
    if (!row_ok) return;
    const int c0 = NCOL * cq + 4 * lgrp;  // first output column of this lane
    const bool lse_lane = lgrp == 0 && cq == 0;
    if (slot < 0) {
      const size_t orow = row_index(u, row);
      uint16_t* o = p.out + orow * kDV + c0;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const f32x16 a = read_acc(acc[ct]);
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = a[j + e] * inv;
          const uint32_t lo = uint32_t(f2e<F16>(v[0])) | (uint32_t(f2e<F16>(v[1])) << 16);
          const uint32_t hi = uint32_t(f2e<F16>(v[2])) | (uint32_t(f2e<F16>(v[3])) << 16);
          *reinterpret_cast<uint2*>(o + 32 * ct + 8 * (j >> 2)) = uint2{lo, hi};
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (lse_lane) {
        p.lse[orow] = p.lse_base2 ? lse2 : lse2 * kLn2;
        if (p.max_logits) p.max_logits[orow] = m_exact;
      }
    } else {
      const size_t wrow = size_t(slot) * p.rows + row;
      float* o = p.ws_o + wrow * kDV + c0;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const f32x16 a = read_acc(acc[ct]);
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = a[j + e] * inv;
          *reinterpret_cast<f32x4*>(o + 32 * ct + 8 * (j >> 2)) = v;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (lse_lane) {
        p.ws_lse[wrow] = lse2;
        if (p.max_logits) p.ws_max[wrow] = m_exact;
      }
    }
  };
  // the result of a segment without tokens: O = 0, LSE = -inf
  auto write_empty = [&](int u, int slot) __attribute__((always_inline)) {
    if (!row_ok) return;
    const int c0 = NCOL * cq + 4 * lgrp;
    const bool lse_lane = lgrp == 0 && cq == 0;
    if (slot < 0) {
      const size_t orow = row_index(u, row);
      uint16_t* o = p.out + orow * kDV + c0;
      for (int ct = 0; ct < NCT; ++ct)
        for (int j = 0; j < 16; j += 4) *reinterpret_cast<uint2*>(o + 32 * ct + 8 * (j >> 2)) = uint2{0, 0};
      if (lse_lane) {
        p.lse[orow] = -__builtin_inff();
        if (p.max_logits) p.max_logits[orow] = -__builtin_inff();
      }
    } else {
      const size_t wrow = size_t(slot) * p.rows + row;
      float* o = p.ws_o + wrow * kDV + c0;
      for (int ct = 0; ct < NCT; ++ct)
        for (int j = 0; j < 16; j += 4) *reinterpret_cast<f32x4*>(o + 32 * ct + 8 * (j >> 2)) = f32x4{0, 0, 0, 0};
      if (lse_lane) {
        p.ws_lse[wrow] = -__builtin_inff();
        if (p.max_logits) p.ws_max[wrow] = -__builtin_inff();
      }
    }
  };

  // ---- one 32-token tile: QK^T, softmax, PV ----
  // gslice(i) issues slice i of the next gather (NLW slices spread over the
  // tile's matrix-core instructions).  next_q_unit >= 0: this is the
  // segment's last tile and the next segment's queries are loaded once the QK
  // product no longer needs the current ones.
  constexpr int NMF = KK + 2 * NCT;  // matrix-core instructions per tile
  auto compute_tile = [&](int buf_off, int tok0, uint32_t vmask, int next_q_unit,
                          auto&& gslice) __attribute__((always_inline)) {
    const uint8_t* buf = lds + buf_off;
    // S^T over all d_qk: one accumulation chain, K fragments read 4 ahead
    constexpr int QD = 3;
    f32x16 st;
    bf16x8 kf[QD + 1];
    auto load_k = [&](int kk) __attribute__((always_inline)) {
      kf[kk % (QD + 1)] = *reinterpret_cast<const bf16x8*>(buf + kbase[kk % NKB] + kk * 32);
    };
#pragma unroll
    for (int kk = 0; kk < QD; ++kk) {
      load_k(kk);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + QD < KK) load_k(kk + QD);
      mfma_v<F16>(st, kf[kk % (QD + 1)], qf[kk], kk < 1);
      // gather slices: one every ~NMF/NLW matrix-core instructions
#pragma unroll
      for (int i = 0; i < NLW; ++i)
        if ((i * NMF) / NLW + 1 == kk) gslice(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (next_q_unit >= 0) load_q(next_q_unit);
    mfma_wait_result();  // before the softmax reads the scores

    // V^T fragments, prefetched PD MFMAs ahead (issued before the softmax so
    // their latency hides behind it)
    constexpr int PD = 3;
    constexpr int NSTEP = 2 * NCT;  // PV MFMAs: 2 k-steps x NCT column tiles
    s16x4 vf[PD + 1][2];
    auto load_v = [&](int i) __attribute__((always_inline)) {
      const int kc = i / NCT, ct = i % NCT;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint8_t* a = buf + vbase[h][ct % NVB] + kc * 16 * RSB + ct * 64;
        vf[i % (PD + 1)][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
      }
    };
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      load_v(i);
      __builtin_amdgcn_sched_barrier(0);
    }

    // mask + softmax (base 2), 16 raw scores per lane; the scale is folded
    // into the exponent: p = 2^(s * scale_log2 - m)
    bool full;
    if constexpr (SPARSE)
      full = vmask == 0xFFFFFFFFu;
    else
      full = __all(tok0 + kTile <= n_vis);
    float mloc = -__builtin_inff();
    if (full) {
#pragma unroll
      for (int v = 0; v < 16; v += 2) mloc = smax(smax(mloc, st[v]), st[v + 1]);
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = tok(v, lgrp);
        bool vis;
        if constexpr (SPARSE)
          vis = (vmask >> t) & 1;
        else
          vis = tok0 + t < n_vis;
        const float x = vis ? st[v] : -__builtin_inff();
        st[v] = x;
        mloc = smax(mloc, x);
      }
    }
    mloc = xor32_max(mloc) * p.scale_log2;  // row maximum over the tile, scaled
    m_exact = smax(m_exact, mloc);
    const bool grow = mloc > m_run + kRescaleSlack;
    if (__any(grow)) {
      const float m_new = grow ? mloc : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
      m_run = m_new;
      l_run *= alpha;
      if (!seg_first) {
        // one column tile at a time, each back in its AGPRs before the next
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          f32x16 t = read_acc(acc[ct]);
          t *= alpha;
          acc[ct] = t;
          pin_agpr(acc[ct]);
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_wait_operands();  // v_accvgpr_write -> MFMA srcC
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) pin_agpr(acc[ct]);
    const float neg_m = m_run == -__builtin_inff() ? 0.f : -m_run;
    s16x8 pk[2];  // P^T operands of the two PV k-steps
    float psum[2] = {0.f, 0.f};  // the lane's partial row sums (two chains)
    // the score goes through an opaque copy: the two copies of the PV loop
    // (first tile of a segment or not) would otherwise share the exponentials
    auto expo = [&](int v) __attribute__((always_inline)) {
      float sv = st[v];
      asm volatile("" : "+v"(sv));
      const float e = fast_exp2(__builtin_fmaf(sv, p.scale_log2, neg_m));
      psum[v & 1] += e;
      pk[v >> 3][v & 7] = (short)f2e<F16>(e);
    };
#pragma unroll
    for (int v = 0; v < 8; ++v) expo(v);
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T . P^T.  The second k-step's exponentials and the row sum go
    // between the first k-step's MFMAs.
    auto pv = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NSTEP; ++i) {
        if (i + PD < NSTEP) load_v(i + PD);
        const int kc = i / NCT, ct = i % NCT;
        const s16x4 lo = vf[i % (PD + 1)][0], hi = vf[i % (PD + 1)][1];
        const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (ct == 0) mfma_wait_operands();  // P^T was just written by VALU instructions
        mfma_a<F16>(acc[ct], __builtin_bit_cast(bf16x8, vv), __builtin_bit_cast(bf16x8, pk[kc]));
        // the second k-step's eight exponentials, spread over the first
        // k-step's MFMAs
        if (i < NCT) {
#pragma unroll
          for (int v = 8; v < 16; ++v)
            if ((v - 8) * NCT / 8 == i) expo(v);
        }
        if (i == NCT) l_run += xor32_sum(psum[0] + psum[1]);
#pragma unroll
        for (int s = 0; s < NLW; ++s)
          if ((s * NMF) / NLW + 1 == KK + i) gslice(s);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    pv();
    seg_first = false;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) pin_agpr(acc[ct]);
  };

  // ---- lengths the device scheduler rejected ----
  // Every output row of the call gets O = 0 and LSE = NaN (and max_logits =
  // NaN), rather than whatever the buffers held: workgroup (part, row block)
  // takes units part, part + grid parts, ...
  if (meta_bad) {
    if (!row_ok) return;
    for (int u = part; u < meta[5]; u += p.num_parts) {
      const size_t orow = row_index(u, row);
      uint16_t* o = p.out + orow * kDV + NCOL * cq + 4 * lgrp;
      for (int c = 0; c < NCOL; c += 8) *reinterpret_cast<uint2*>(o + c) = uint2{0, 0};
      if (lgrp == 0 && cq == 0) {
        p.lse[orow] = __builtin_nanf("");
        if (p.max_logits) p.max_logits[orow] = __builtin_nanf("");
      }
    }
    return;
  }

  // ---- the stream of the part ----
  // leading segments without tiles
  int cs0 = seg_begin;
  i32x4a rec0 = cs0 < seg_end ? seg_rec(cs0) : i32x4a{0, 0, 0, 0};
  while (cs0 < seg_end && rec0[1] == rec0[2]) {
    write_empty(rec0[0], rec0[3]);
    ++cs0;
    if (cs0 < seg_end) rec0 = seg_rec(cs0);
  }
  if (cs0 >= seg_end) return;

  // Tiles t .. t+5 are tracked: t is computed, t+1 and t+2 are in flight or
  // landed, t+3 is gathered during step t (its plan needs its slot, loaded
  // three steps earlier), t+4 and t+5 are looked up ahead, and the end of
  // step t looks up t+6 and loads its slot.
  // All metadata lookups of a step come after its compute: a scalar load in
  // flight shares the LDS wait counter and would make every operand wait of
  // the tile a full drain.  Past the end of the stream a tile repeats the
  // last real one, so its (unused) loads are in bounds and every step issues
  // the same number of vector-memory operations, which the waits count on:
  //   step t: NLW gather loads of tile t+3, then the slot load of tile t+6.
  auto clamp_end = [&](const Tile& n, const Tile& prev) __attribute__((always_inline)) -> Tile {
    return n.s < seg_end ? n : Tile{seg_end, prev.pos, prev.u, prev.b1, prev.len};
  };
  Tile t0 = first_tile_rec(cs0, rec0);
  Tile t1 = clamp_end(next_tile(t0), t0);
  Tile t2 = clamp_end(next_tile(t1), t1);
  Tile t3 = clamp_end(next_tile(t2), t2);
  Tile t4 = clamp_end(next_tile(t3), t3);
  Tile t5 = clamp_end(next_tile(t4), t4);
  uint32_t vm0, vm1, vm2;
  {
    // The slots of tiles 0..2 and the first queries are loaded together (one
    // round trip for both); the slots of 3..5 follow the gathers of 0..2 in
    // the steady-state order.
    const bool q_lds = !WIDE && (SPARSE || p.heads == p.h_q || p.s_q == 1);
    load_slot(t0, 0);
    load_slot(t1, 1);
    load_slot(t2, 2);
    if (q_lds)
      gather_q_block(t0.u);
    else
      load_q(t0.u);
    zero_acc();
    n_vis = SPARSE ? 0 : visible(t0.len);
    wait_vmem_n<0>();
    lds_barrier();
    if (q_lds) {
      read_q_block();
      lds_barrier();  // every wavefront has its queries before the buffers are refilled
    }
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const Plan g0 = plan_tile(t0, read_slot(t0, 0));
    vm0 = g0.vmask;
#pragma unroll
    for (int i = 0; i < NLW; ++i) gather_one(g0, 0 * TBUF, i, ln);
    load_slot(t3, 3);
    const Plan g1 = plan_tile(t1, read_slot(t1, 1));
    vm1 = g1.vmask;
#pragma unroll
    for (int i = 0; i < NLW; ++i) gather_one(g1, 1 * TBUF, i, ln);
    load_slot(t4, 4);
    const Plan g2 = plan_tile(t2, read_slot(t2, 2));
    vm2 = g2.vmask;
#pragma unroll
    for (int i = 0; i < NLW; ++i) gather_one(g2, 2 * TBUF, i, ln);
    load_slot(t5, 5);
  }
  // outstanding now (oldest first): q, g0, s3, g1, s4, g2, s5
  bool seg_start = false;  // first step of a segment after the first one
  int tnum = 0;            // stream position of t0 (buffer tnum % 4, index slot tnum % 8)

  // One step computes tile t0 and gathers tile t3 into the buffer of the tile
  // computed one step earlier.
  for (;;) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) pin_agpr(acc[ct]);
    // Tile t0's loads (and the indices of t3) have landed; the loads of t1,
    // t2 (and the indices of t4, t5) may still be in flight.  At a segment
    // start the queries were loaded during the previous step, after its QK
    // product, by a statement that waited for every older load (tile t0's
    // and t3's indices among them); waiting until at most 63 operations are
    // in flight then leaves the previous segment's output stores alone.
    // (WIDE kernels spill registers to scratch, whose accesses share the
    // counter, so they always wait for everything.)
    if (WIDE)
      wait_vmem_n<0>();
    else if (seg_start)
      wait_vmem_n<63>();
    else
      wait_vmem_n<2 * NLW + 2>();
    lds_barrier();
    const bool has_next = t1.s < seg_end;
    const Plan g3 = plan_tile(t3, read_slot(t3, (tnum + 3) % NISLOT));
    const uint32_t vm3 = g3.vmask;
    const bool last = is_last(t0);
    const int next_q_unit = (last && has_next) ? t1.u : -1;
    const int tok0 = t0.pos * kTile;
    const int cur = (tnum % kBufs) * TBUF;
    const int nxt = ((tnum + 3) % kBufs) * TBUF;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    auto gslice = [&](int i) __attribute__((always_inline)) { gather_one(g3, nxt, i, ln); };
    if (!SPARSE || !WIDE || vm0 != 0) {
      compute_tile(cur, tok0, vm0, next_q_unit, gslice);
    } else {
      if (next_q_unit >= 0) load_q(next_q_unit);
#pragma unroll
      for (int i = 0; i < NLW; ++i) gslice(i);
    }
    if (last) {
      write_segment(t0.u, seg_slot(t0.s));
      const int e_end = has_next ? t1.s : seg_end;
      for (int e = t0.s + 1; e < e_end; ++e)  // segments without tiles passed over
        write_empty(seg_u(e), seg_slot(e));
      if (has_next) {
        if constexpr (!SPARSE) n_vis = visible(t1.len);
        reset_state();
      }
    }
    seg_start = last && has_next;
    const Tile t6 = clamp_end(next_tile(t5), t5);
    load_slot(t6, (tnum + 6) % NISLOT);
    if (!has_next) break;
    t0 = t1;
    t1 = t2;
    t2 = t3;
    t3 = t4;
    t4 = t5;
    t5 = t6;
    vm0 = vm1;
    vm1 = vm2;
    vm2 = vm3;
    ++tnum;
  }
  // no load into LDS may outlive the workgroup
  wait_vmem_n<0>();
#endif
}

// Launches the decode kernel for one (d_qk, element type); the column split
// follows the rows per workgroup chosen for the unit's row count.
template <int D_QK, bool F16>
hipError_t launch_decode_d(const SplitKVParams& p, bool sparse, hipStream_t stream) {
  const int rbk = rows_per_group(p.rows);
  const int row_blocks = (p.rows + rbk - 1) / rbk;
  const int groups = p.num_parts * row_blocks;
  if (groups <= 0) return hipSuccess;
  SplitKVParams q = p;
  q.row_blocks = row_blocks;
  const dim3 grid(groups), block(256);
  // Sparse rows are addressed with 32-bit byte offsets while the pool plus
  // the past-the-end row an invalid index reads fits in 32 bits.
  const uint64_t row_bytes = uint64_t(D_QK) * 2;
  const bool wide = (uint64_t(p.num_rows) + 2) * row_bytes > 0xFFFFFFFFull;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, block, 0, stream, q); };
  auto cases = [&](auto ncol) {
    constexpr int NC = decltype(ncol)::value;
    if (!sparse) go(mla_decode<D_QK, false, false, F16, NC>);
    else if (!wide) go(mla_decode<D_QK, true, false, F16, NC>);
    else go(mla_decode<D_QK, true, true, F16, NC>);
  };
  // (units of more than 64 rows only: 128 rows per workgroup, each wavefront
  // holding all 512 output columns of its rows; the column splits of the
  // template are not instantiated)
  if (rbk != 128) return hipErrorInvalidValue;
  cases(std::integral_constant<int, 512>{});
  return hipGetLastError();
}

}  // namespace mla
