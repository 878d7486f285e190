// Split-KV kernel of the paged MLA decode library, written for gfx950 (CDNA4).
//
// One workgroup = (part, row block of 64 query rows) of the tile-scheduler
// metadata: 4 wavefronts, one per SIMD.  The workgroup walks its part's
// segments (unit, block range, slot) as one stream of 64-token tiles.  Each
// tile is gathered into LDS with direct global->LDS loads -- a contiguous
// 64-row page reached through the block table for dense decode, 64 scattered
// rows reached through the index list for sparse decode -- into one of two
// buffers, so the next tile streams in while the current one is computed:
//
//   S^T = K . Q^T      bf16 MFMA; K from LDS, Q^T resident in registers for
//                      the whole segment
//   online softmax     fp32, base 2, one query row per lane (reduced over the
//                      lanes sharing it); the reference maximum is moved only
//                      when it grows by more than 2^8, so the accumulator is
//                      rarely rescaled (the result does not depend on it)
//   O^T += V^T . P^T   bf16 MFMA; P^T straight from registers, V^T read with
//                      the LDS transpose read from the first 512 columns of
//                      the same tile
//
// Two layouts of the four wavefronts:
//  * pairs (more than 16 rows): wavefronts 2r and 2r+1 share query rows
//    32r..32r+31.  Each computes S^T for its half of the tile's tokens over all
//    d_qk and O^T for its half of the 512 value columns with 32x32x16 MFMAs;
//    the two exchange their row maxima, row sums and bf16 P halves through
//    LDS.  Every K and V element read from LDS then feeds 32 query rows.
//  * single wavefronts (16 rows or fewer): each owns 16 rows and the whole
//    tile with 16x16x32 MFMAs.
//
// The metadata of the tile after next (block-table entry and sequence length,
// or the sparse index list) is fetched one step ahead, and the next segment's
// queries are loaded as soon as the current segment's last QK product is done,
// so neither sits on the critical path.  A segment covering its whole unit
// writes bf16 O and fp32 LSE; a split segment writes fp32 O and a base-2 LSE
// into its workspace slot for the combine kernel.  This is the structure the
// deepep.org usage page describes (tile scheduler, block-table manager, memory
// manager; QK^T, scaled softmax, output stages); sparse gathering follows the
// upstream FlashMLA README ("Sparse Attention (indices tensor)").  Only active
// heads are ever computed.
//
// LDS tile layout: cache row t of a tile occupies 16-byte chunks
// [t*CPR, (t+1)*CPR), with its chunk c stored at position c ^ f(t).  The
// swizzle f spreads both operand reads over all banks.  It is applied on the
// source side of the global->LDS gather, and since f depends only on the low
// bits of t, every operand address is one of a few per-lane bases plus a
// compile-time offset.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_kernels.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Read-only metadata (scheduler output, block table, sequence lengths) is
// read through the constant address space so uniform reads become scalar
// loads instead of vector loads that would share the vector memory counter
// with the in-flight tile gathers.
typedef const __attribute__((address_space(4))) int32_t cint;
__device__ __forceinline__ cint* as_const(const int32_t* ptr) { return (cint*)(uintptr_t)ptr; }

constexpr int kPage = 64;       // tokens per tile (one page, or 64 sparse indices)
constexpr int kWaves = 4;       // wavefronts per workgroup
constexpr int kDV = 512;        // value width
constexpr int kRowsPerGroup = 64;  // query rows per workgroup
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
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier for LDS traffic only: waits for this wave's LDS (and
// scalar) accesses, not for the tile gathers still in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Register-class pins: an empty asm statement that takes the value in an AGPR.
// It emits no instruction; it keeps the long-lived accumulators and query
// fragments in the accumulation registers, so the vector registers stay free
// for the per-tile working set and no copies are hoisted into the tile loop.
__device__ __forceinline__ void pin_agpr(f32x4& x) { asm volatile("" : "+a"(x)); }
__device__ __forceinline__ void pin_agpr(f32x16& x) { asm volatile("" : "+a"(x)); }
__device__ __forceinline__ void pin_agpr(bf16x8& x) { asm volatile("" : "+a"(x)); }

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

// MFMA shapes.  Each wavefront owns RW query rows; lane l owns row l % RW of
// every S^T and O^T tile (the B operand's column), so a query row's softmax
// state lives in the RW/16... lanes sharing it.
//
// RW = 16, v_mfma_f32_16x16x32_bf16: S^T tiles of 16 tokens, k-steps of 32
//   d; O^T tiles of 16 columns, PV k-steps of 32 tokens.
// RW = 32, v_mfma_f32_32x32x16_bf16: S^T tiles of 32 tokens, k-steps of 16
//   d; O^T tiles of 32 columns, PV k-steps of 16 tokens.
// Score v of a lane (v < NV) is register v % CREG of S^T tile v / CREG; the
// P^T operand of PV k-step kc is scores 8kc..8kc+7, whose tokens match the
// V^T rows the two transpose reads of that k-step deliver.
template <int RW>
struct Shape;

template <>
struct Shape<16> {
  using C = f32x4;
  static constexpr int CREG = 4, TT = 4, TW = 16, KD = 32, NCT = 32, CW = 16, KC = 2, NV = 16;
  static constexpr int HROW = 16;  // row offset between the two transpose reads
  __device__ static C mfma(bf16x8 a, bf16x8 b, C c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static int tok(int v, int g) { return 16 * (v >> 2) + 4 * g + (v & 3); }
  __device__ static int col(int ct, int j, int g) { return 16 * ct + 4 * g + j; }
  // V^T transpose read h of PV k-step kc: row (token), 16-byte chunk
  __device__ static int vrow(int kc, int h, int lane) {
    return 32 * kc + 16 * h + 4 * (lane >> 4) + ((lane & 15) >> 2);
  }
  __device__ static int vchunk(int ct, int lane) { return 2 * ct + ((lane & 3) >> 1); }
  // chunk swizzle f(t) of the LDS tile for 72- and 64-chunk rows
  template <int CPR>
  __device__ static int swz(int t) {
    if constexpr (CPR == 72) return (2 * ((t >> 1) & 3)) | ((t >> 3) & 1);
    else return ((t & 7) << 1) | ((t >> 3) & 1);
  }
};

template <>
struct Shape<32> {
  using C = f32x16;
  static constexpr int CREG = 16, TT = 2, TW = 32, KD = 16, NCT = 16, CW = 32, KC = 4, NV = 32;
  static constexpr int HROW = 8;
  __device__ static C mfma(bf16x8 a, bf16x8 b, C c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static int tok(int v, int g) {
    return 32 * (v >> 4) + 8 * ((v & 15) >> 2) + 4 * g + (v & 3);
  }
  __device__ static int col(int ct, int j, int g) { return 32 * ct + 8 * (j >> 2) + 4 * g + (j & 3); }
  __device__ static int vrow(int kc, int h, int lane) {
    return 16 * kc + 8 * h + 4 * (lane >> 5) + ((lane & 15) >> 2);
  }
  __device__ static int vchunk(int ct, int lane) {
    return 4 * ct + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  }
  template <int CPR>
  __device__ static int swz(int t) {
    if constexpr (CPR == 72) return 4 * ((t >> 1) & 1) + ((t >> 2) & 3);
    else return ((t & 3) << 2) | ((t >> 2) & 3);
  }
};

struct TileMeta {
  int phys;  // dense: physical page of the tile
  int len;   // dense: cache length of the tile's request
  int idx;   // sparse: this lane's index (tile token = lane)
};

}  // namespace

// PAIR = false: each wavefront owns 16 query rows and the whole tile (16x16x32
// MFMAs).  PAIR = true: the two wavefronts of a pair share 32 query rows; each
// computes S^T for its half of the tile's tokens over all d_qk and O^T for its
// half of the 512 value columns (32x32x16 MFMAs), and the pair exchanges its
// row maxima, row sums and bf16 P halves through LDS.  A pair reads each K and
// V element from LDS once per 32 rows instead of once per 16.
template <int D_QK, bool SPARSE, bool PAIR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_splitkv(SplitKVParams p) {
  constexpr int RW = PAIR ? 32 : 16;  // query rows per wavefront (pair)
  using S = Shape<RW>;
  using C = typename S::C;
  constexpr int CPR = D_QK / 8;    // 16-byte chunks per cache row
  constexpr int RSB = CPR * 16;    // LDS row stride in bytes
  constexpr int NLD = CPR;         // 64-chunk load instructions per tile
  constexpr int BUF = NLD * 1024;  // bytes per tile buffer
  constexpr int KK = D_QK / S::KD; // QK k-steps
  constexpr int CK = S::KD / 8;    // 16-byte chunks per QK k-step
  constexpr int CV = S::CW / 8;    // 16-byte chunks per output column tile
  constexpr int KT = kPage / S::KC;  // tokens per PV k-step
  constexpr int FMAX = CPR == 72 ? 8 : 16;  // swizzle values are below this
  constexpr int NKB = FMAX / CK;   // K-read bases (kk mod NKB)
  constexpr int NVB = FMAX / CV;   // V-read bases (ct mod NVB)
  constexpr int NCT = PAIR ? S::NCT / 2 : S::NCT;  // output column tiles per wavefront
  constexpr int NX = PAIR ? kWaves : 1;             // pair exchange slots
  static_assert(NLD % kWaves == 0, "whole load instructions per wave");
  static_assert(S::NV == 16 || PAIR, "16 scores per lane");
  __shared__ __attribute__((aligned(1024))) uint8_t buf_a[BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t buf_b[BUF];
  __shared__ __attribute__((aligned(16))) uint32_t l2_sink[kWaves * 64];  // written, never read
  __shared__ __attribute__((aligned(16))) s16x8 x_p[NX][2][64];  // bf16 P of a pair half
  __shared__ float x_max[NX][32];                                 // row maxima of a half
  __shared__ float x_sum[NX][32];                                 // row sums of a half

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rgrp = PAIR ? wave >> 1 : wave;  // row group of the wavefront
  const int half = PAIR ? wave & 1 : 0;      // pair half: token half and column half
  const int lrow = lane % RW;  // query row owned within the row group
  const int lgrp = lane / RW;  // k-group of the MFMA operands

  const int total = p.num_parts * p.row_blocks;
  const int lg = logical_group(blockIdx.x, total);
  const int part = lg / p.row_blocks;
  const int rb = lg - part * p.row_blocks;
  if (part >= p.num_parts) return;

  cint* meta = as_const(p.meta);
  const int seg_begin = meta[kMetaHeaderInts + part];
  const int seg_end = meta[kMetaHeaderInts + part + 1];
  cint* segs = meta + meta[12];
  auto seg_u = [&](int s) __attribute__((always_inline)) { return segs[4 * s + 0]; };
  auto seg_b0 = [&](int s) __attribute__((always_inline)) { return segs[4 * s + 1]; };
  auto seg_b1 = [&](int s) __attribute__((always_inline)) { return segs[4 * s + 2]; };
  auto seg_slot = [&](int s) __attribute__((always_inline)) { return segs[4 * s + 3]; };

  const int row0 = rb * kRowsPerGroup + rgrp * RW;
  const bool wave_active = row0 < p.rows;
  const int row = row0 + lrow;
  const bool row_ok = row < p.rows;

  // Per-lane LDS operand bases.  Chunk c of tile row t is stored at position
  // c ^ f(t), and f depends only on low bits of t that are fixed per lane, so
  //  K  (A of QK): row TW*tt + lrow, chunk CK*kk + lgrp, stored at
  //     CK*(kk ^ (f/CK)) + (lgrp ^ (f%CK)) -> kbase[kk % NKB] + 16*CK*kk;
  //  V^T (A of PV, transpose read h): row vrow(kc, h), chunk CV*ct + y, stored
  //     at CV*(ct ^ (f/CV)) + (y ^ (f%CV)) -> vbase[h][ct % NVB] + 16*CV*ct.
  // With 16 rows per wave the two transpose reads of a V^T fragment are 16
  // rows apart, which leaves the swizzle unchanged: one set of V bases serves
  // both (the second read adds an immediate row offset).
  constexpr int NVH = RW == 16 ? 1 : 2;
  int kbase[NKB], vbase[NVH][NVB];
  {
    const int fk = S::template swz<CPR>(lrow);
#pragma unroll
    for (int j = 0; j < NKB; ++j)
      kbase[j] = (32 * half + lrow) * RSB + 16 * (lgrp ^ (fk % CK)) + 16 * CK * ((j ^ (fk / CK)) - j);
    const int y = S::vchunk(0, lane);
#pragma unroll
    for (int h = 0; h < NVH; ++h) {
      const int vr = S::vrow(0, h, lane);
      const int fv = S::template swz<CPR>(vr);
#pragma unroll
      for (int j = 0; j < NVB; ++j)
        vbase[h][j] = vr * RSB + 16 * (y ^ (fv % CV)) + 16 * CV * ((j ^ (fv / CV)) - j) + 8 * (lane & 1) +
                      16 * CV * NCT * half;
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
  auto fetch_meta = [&](int s, int blk) __attribute__((always_inline)) -> TileMeta {
    TileMeta m{0, 0, -1};
    const int u = seg_u(s);
    if constexpr (SPARSE) {
      const int pos = blk * kPage + lane;
      m.idx = pos < p.topk ? p.indices[size_t(u) * p.topk + pos] : -1;
    } else {
      m.phys = as_const(p.block_table)[size_t(u) * p.bt_stride + blk];
      m.len = as_const(p.seqlens)[u];
    }
    return m;
  };

  // Buffer resource of one physical page (dense decode).  Page gathers and
  // warm-ups use buffer loads: unlike global (flat-encoded) loads into LDS,
  // they leave the LDS wait counter to LDS reads, so the operand waits of the
  // tile being computed stay exact while the next tile streams in.
  auto page_rsrc = [&](int phys) __attribute__((always_inline)) {
    const uint8_t* pg = reinterpret_cast<const uint8_t*>(p.kv) + size_t(phys) * kPage * D_QK * 2;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pg), 0, kPage * D_QK * 2,
                                            kBufferWord3);
  };

  // ---- tile gather into `dst`; returns the sparse validity mask ----
  // Every lane of every load fetches an in-bounds row: the tail of a
  // request's last page repeats its last cached token (masked out of the
  // softmax, so it contributes exactly zero), and an invalid sparse index is
  // replaced by the tile's first valid one (also masked).  A sparse tile
  // without any valid index is neither loaded nor computed.
  auto load_tile = [&](uint8_t* dst, int blk, const TileMeta& m) __attribute__((always_inline)) -> uint64_t {
    uint64_t vmask = ~0ull;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(p.kv);
    int tmax = kPage - 1;
    int idx_lane = 0;
    const __amdgpu_buffer_rsrc_t page = page_rsrc(SPARSE ? 0 : m.phys);  // dense only
    if constexpr (SPARSE) {
      const bool ok = m.idx >= 0 && m.idx < p.num_rows;
      vmask = __ballot(ok);
      if (vmask == 0) return 0;
      const int sub = __shfl(m.idx, __builtin_ctzll(vmask));
      idx_lane = ok ? m.idx : sub;
    } else {
      const int vt = m.len - blk * kPage;
      tmax = vt < 1 ? 0 : (vt > kPage ? kPage - 1 : vt - 1);
    }
    // LDS chunk q = 64 n + lane of load n holds row t = q / CPR at position
    // q % CPR, i.e. source chunk (q % CPR) ^ f(t); successive loads of a wave
    // are 64 * kWaves = 256 chunks apart
    constexpr int kStep = 64 * kWaves;
    // recomputed per tile from an opaque copy of the thread id, so the
    // compiler does not keep 18 per-lane source offsets alive across the loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    int t = tid / CPR;
    int c = tid - t * CPR;
#pragma unroll
    for (int i = 0; i < NLD / kWaves; ++i) {
      const int n = wave + i * kWaves;
      const int cc = c ^ S::template swz<CPR>(t);
      if constexpr (SPARSE) {
        const uint8_t* src = base + size_t(__shfl(idx_lane, t)) * D_QK * 2 + cc * 16;
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + n * 1024), 16, 0, 0);
      } else {
        const int off = (t < tmax ? t : tmax) * (D_QK * 2) + cc * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(page, (lds_void*)(dst + n * 1024), 16, off, 0, 0, 0);
      }
      t += kStep / CPR;
      c += kStep % CPR;
      if (c >= CPR) {
        c -= CPR;
        t += 1;
      }
    }
    return vmask;
  };

  // ---- L2 warm-up of the tile after next ----
  // One dword of every 128-byte line of the tile is loaded into a scratch LDS
  // slot that is never read: the lines are then in L2 when the tile's gather
  // is issued one step later, so that gather waits for L2 instead of HBM and
  // two tiles' worth of HBM reads are in flight per workgroup.
  auto warm_tile = [&](const TileMeta& m) __attribute__((always_inline)) {
    constexpr int kLine = 128;
    constexpr int kRowLines = D_QK * 2 / kLine;  // 9 (576) or 8 (512)
    lds_void* dst = (lds_void*)(l2_sink + wave * 64);
    const uint8_t* kv = reinterpret_cast<const uint8_t*>(p.kv);
    if constexpr (SPARSE) {
      const bool ok = m.idx >= 0 && m.idx < p.num_rows;
      const uint8_t* row_ptr = kv + size_t(ok ? m.idx : 0) * D_QK * 2;
#pragma unroll
      for (int k = wave; k < kRowLines; k += kWaves)
        __builtin_amdgcn_global_load_lds(row_ptr + k * kLine, dst, 4, 0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t page = page_rsrc(m.phys);
      constexpr int kLines = kPage * kRowLines;
#pragma unroll
      for (int k = 0; k < (kLines + 255) / 256; ++k) {
        const int line = k * 256 + wave * 64 + lane;
        if (k * 256 + wave * 64 < kLines)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(page, dst, 4, line * kLine, 0, 0, 0);
      }
    }
  };

  // ---- per-segment state ----
  // m_run: reference maximum (base 2) of the lane's row, identical in both
  // halves of a pair.  l_part: sum of the softmax numerators; per lane for
  // 16-row wavefronts (reduced over the row's lanes at the end), the row total
  // for pairs.
  bf16x8 qf[KK];
  C acc[NCT];
  float m_run = -__builtin_inff();
  float l_part = 0.f;
  size_t qrow = 0;
  int n_vis = 0;

  // rows past the unit's last row read that last row (never written back)
  auto load_q = [&](int u) __attribute__((always_inline)) {
    const uint16_t* qp = p.q + row_index(u, row_ok ? row : p.rows - 1) * D_QK + 8 * lgrp;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * S::KD);
    if constexpr (!PAIR) {  // with 16 rows per wave the queries fit beside acc
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) pin_agpr(qf[kk]);
    }
  };
  // The accumulator is not cleared here: the segment's first computed tile
  // starts its PV product from zero instead, so acc is only ever touched by
  // MFMAs in the tile loop (and by the rare rescale).
  bool seg_first = true;
  auto reset_state = [&]() __attribute__((always_inline)) {
    seg_first = true;
    m_run = -__builtin_inff();
    l_part = 0.f;
  };

  // reduction over the lanes of one wavefront that share a query row
  auto row_sum = [&](float x) __attribute__((always_inline)) {
    if constexpr (!PAIR) x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
  };
  auto row_max = [&](float x) __attribute__((always_inline)) {
    if constexpr (!PAIR) x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
  };

  // Writes the segment result of this lane's row (a pair half writes its own
  // value columns); a segment without tokens (empty_seg) writes O = 0 and
  // LSE = -inf.
  auto write_segment = [&](size_t orow, int slot, bool empty_seg) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) pin_agpr(acc[ct]);
    const float l_tot = empty_seg ? 0.f : (PAIR ? l_part : row_sum(l_part));
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
        for (int j = 0; j < S::CREG; j += 4) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = empty ? 0.f : acc[ct][j + e] * inv;
          const uint32_t lo = uint32_t(f2bf(v[0])) | (uint32_t(f2bf(v[1])) << 16);
          const uint32_t hi = uint32_t(f2bf(v[2])) | (uint32_t(f2bf(v[3])) << 16);
          *reinterpret_cast<uint2*>(o + S::col(ct0 + ct, j, lgrp)) = uint2{lo, hi};
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (lse_lane) p.lse[orow] = lse2 * kLn2;
    } else {
      const size_t wrow = size_t(slot) * p.rows + row;
      float* o = p.ws_o + wrow * kDV;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int j = 0; j < S::CREG; j += 4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = empty ? 0.f : acc[ct][j + e] * inv;
          *reinterpret_cast<f32x4*>(o + S::col(ct0 + ct, j, lgrp)) = v;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (lse_lane) p.ws_lse[wrow] = lse2;
    }
  };

  // ---- one 64-token tile: QK^T, softmax, PV ----
  // `next_q_unit` >= 0: this is the segment's last tile and the next segment's
  // queries are loaded once the QK product no longer needs the current ones.
  auto compute_tile = [&](const uint8_t* buf, int blk, uint64_t vmask,
                          int next_q_unit) __attribute__((always_inline)) {
    // S^T accumulators: 16-row wavefronts hold TT token tiles of 16; a pair
    // half holds its 32 tokens as two accumulation chains (even and odd
    // k-steps) that are added at the end.
    constexpr int NST = PAIR ? 2 : S::TT;
    constexpr int QD = PAIR ? 4 : 2;  // K fragments prefetched this many k-steps ahead
    constexpr int NTT = PAIR ? 1 : S::TT;  // token tiles read per k-step
    C st[NST];
    bf16x8 kf[QD + 1][NTT];
    auto load_k = [&](int kk) __attribute__((always_inline)) {
      const uint8_t* kb = buf + kbase[kk % NKB];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
        kf[kk % (QD + 1)][tt] =
            *reinterpret_cast<const bf16x8*>(kb + tt * S::TW * RSB + kk * 16 * CK);
    };
#pragma unroll
    for (int kk = 0; kk < QD; ++kk) {
      load_k(kk);
      __builtin_amdgcn_sched_barrier(0);  // keep the ring in k-step order
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + QD < KK) load_k(kk + QD);
      if constexpr (PAIR) {
        const int c = kk & 1;
        st[c] = S::mfma(kf[kk % (QD + 1)][0], qf[kk], kk < 2 ? C{} : st[c]);
      } else {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
          st[tt] = S::mfma(kf[kk % (QD + 1)][tt], qf[kk], kk == 0 ? C{} : st[tt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (PAIR) st[0] += st[1];
    if (next_q_unit >= 0) load_q(next_q_unit);

    // V^T fragments, prefetched PD (k-step, column-tile) steps ahead; the
    // first PD are issued before the softmax so their latency hides behind it
    constexpr int PD = PAIR ? 6 : 8;
    constexpr int NSTEP = S::KC * NCT;
    s16x4 vf[PD + 1][2];
    auto load_v = [&](int i) __attribute__((always_inline)) {
      const int kc = i / NCT, ct = i % NCT;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        constexpr int hoff = NVH == 2 ? 0 : S::HROW * RSB;
        const uint8_t* a = buf + vbase[NVH == 2 ? h : 0][ct % NVB] + h * hoff + kc * KT * RSB + ct * 16 * CV;
        vf[i % (PD + 1)][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
      }
    };
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      load_v(i);
      __builtin_amdgcn_sched_barrier(0);
    }

    // mask + online softmax (base 2), 16 scores per lane, in place
    auto score = [&](int v) __attribute__((always_inline)) -> float {
      if constexpr (PAIR) return st[0][v];
      else return st[v / S::CREG][v % S::CREG];
    };
    auto set_score = [&](int v, float x) __attribute__((always_inline)) {
      if constexpr (PAIR) st[0][v] = x;
      else st[v / S::CREG][v % S::CREG] = x;
    };
    float mloc = -__builtin_inff();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = 32 * half + S::tok(v, lgrp);
      bool vis;
      if constexpr (SPARSE) {
        vis = (vmask >> t) & 1;
      } else {
        vis = blk * kPage + t < n_vis;
      }
      const float x = vis ? score(v) * p.scale_log2 : -__builtin_inff();
      set_score(v, x);
      mloc = fmaxf(mloc, x);
    }
    mloc = row_max(mloc);
    if constexpr (PAIR) {  // maximum over both token halves
      if (lane < 32) x_max[wave][lane] = mloc;
      lds_barrier();
      mloc = fmaxf(mloc, x_max[wave ^ 1][lane & 31]);
    }
    const bool grow = mloc > m_run + kRescaleSlack;
    const bool rescale = __any(grow);
    if (rescale) {
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
    const float m_use = m_run == -__builtin_inff() ? 0.f : m_run;
    float psum = 0.f;
    s16x8 pk[2];  // this lane's P^T operand: scores 8c .. 8c+7
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float pe = fast_exp2(score(v) - m_use);
      psum += pe;
      pk[v >> 3][v & 7] = (short)f2bf(pe);
    }
    s16x8 pp[2];  // the partner half's P^T operand (pairs)
    if constexpr (PAIR) {
      const float own = row_sum(psum);
      x_p[wave][0][lane] = pk[0];
      x_p[wave][1][lane] = pk[1];
      if (lane < 32) x_sum[wave][lane] = own;
      lds_barrier();
      pp[0] = x_p[wave ^ 1][0][lane];
      pp[1] = x_p[wave ^ 1][1][lane];
      const float other = x_sum[wave ^ 1][lane & 31];
      l_part += half == 0 ? own + other : other + own;  // same sum in both halves
    } else {
      l_part += psum;
    }
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T . P^T; a pair's PV k-steps 0,1 cover tokens 0..31 (half 0's
    // scores) and 2,3 tokens 32..63 (half 1's)
    auto pv = [&](bool from_zero) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NSTEP; ++i) {
        if (i + PD < NSTEP) load_v(i + PD);
        const int kc = i / NCT, ct = i % NCT;
        const s16x4 lo = vf[i % (PD + 1)][0], hi = vf[i % (PD + 1)][1];
        const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        s16x8 pb;
        if constexpr (PAIR) pb = (kc >> 1) == half ? pk[kc & 1] : pp[kc & 1];
        else pb = pk[kc];
        const C c_in = (from_zero && kc == 0) ? C{} : acc[ct];
        acc[ct] = S::mfma(__builtin_bit_cast(bf16x8, vv), __builtin_bit_cast(bf16x8, pb), c_in);
        __builtin_amdgcn_sched_barrier(0);
      }
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
  // next tile after (s, blk), skipping segments without tiles
  auto advance = [&](int s, int blk, int& s2, int& blk2) __attribute__((always_inline)) {
    if (blk + 1 < seg_b1(s)) {
      s2 = s;
      blk2 = blk + 1;
      return;
    }
    s2 = s + 1;
    while (s2 < seg_end && seg_b0(s2) == seg_b1(s2)) ++s2;
    blk2 = s2 < seg_end ? seg_b0(s2) : 0;
  };

  // leading segments without tiles
  int cs = seg_begin;
  while (cs < seg_end && seg_b0(cs) == seg_b1(cs)) {
    if (wave_active) write_segment(row_index(seg_u(cs), row), seg_slot(cs), true);
    ++cs;
  }
  if (cs >= seg_end) return;

  // first tile: gathered into buf_a before the stream starts
  int cblk = seg_b0(cs);
  uint64_t cmask;
  {
    const TileMeta m0 = fetch_meta(cs, cblk);
    if (!SPARSE) n_vis = visible(m0.len);
    qrow = row_index(seg_u(cs), row);
    load_q(seg_u(cs));
    reset_state();
    cmask = load_tile(buf_a, cblk, m0);
  }
  // tiles j+1 (gathered at the next step) and j+2 (warmed into L2 at the next
  // step); the metadata of tile j+3 is read at the end of the step.  All
  // scalar metadata reads of a step happen after its compute: a scalar load in
  // flight shares the LDS wait counter and would turn every LDS operand wait of
  // the tile into a full drain.
  int ns, nblk, n2s, n2blk;
  advance(cs, cblk, ns, nblk);
  TileMeta nmeta{0, 0, -1}, n2meta{0, 0, -1};
  n2s = seg_end;
  n2blk = 0;
  if (ns < seg_end) {
    nmeta = fetch_meta(ns, nblk);
    advance(ns, nblk, n2s, n2blk);
    if (n2s < seg_end) n2meta = fetch_meta(n2s, n2blk);
    warm_tile(nmeta);
  }
  // the current tile ends its segment / the unit whose queries follow it
  bool seg_last = cblk + 1 >= seg_b1(cs);
  int next_q_unit = (seg_last && ns < seg_end) ? seg_u(ns) : -1;

  // One step computes the tile in `cur_buf` while the next one streams into
  // `nxt_buf`.  The two buffers are distinct LDS objects named statically at
  // every call site, so the compiler can tell reads of one from the
  // asynchronous writes into the other and does not wait for those writes.
  auto step = [&](const uint8_t* cur_buf, uint8_t* nxt_buf) __attribute__((always_inline)) -> bool {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) pin_agpr(acc[ct]);  // loop-carried in AGPRs
    wait_vmem();
    __syncthreads();
    uint64_t nmask = 0;
    if (ns < seg_end) nmask = load_tile(nxt_buf, nblk, nmeta);
    if (n2s < seg_end) warm_tile(n2meta);
    if (PAIR || wave_active) {  // a pair's exchange barriers need all four wavefronts
      if (!SPARSE || cmask != 0) {
        compute_tile(cur_buf, cblk, cmask, next_q_unit);
      } else if (next_q_unit >= 0) {
        load_q(next_q_unit);
      }
    }
    if (seg_last) {
      if (wave_active) {
        write_segment(qrow, seg_slot(cs), false);
        for (int e = cs + 1; e < ns; ++e)  // segments without tiles passed over
          write_segment(row_index(seg_u(e), row), seg_slot(e), true);
      }
      if (ns < seg_end) {
        qrow = row_index(seg_u(ns), row);
        if (!SPARSE) n_vis = visible(nmeta.len);
        reset_state();
      }
    }
    if (ns >= seg_end) return false;
    int n3s = seg_end, n3blk = 0;
    TileMeta n3meta{0, 0, -1};
    if (n2s < seg_end) {
      advance(n2s, n2blk, n3s, n3blk);
      if (n3s < seg_end) n3meta = fetch_meta(n3s, n3blk);
    }
    cs = ns;
    cblk = nblk;
    cmask = nmask;
    ns = n2s;
    nblk = n2blk;
    nmeta = n2meta;
    n2s = n3s;
    n2blk = n3blk;
    n2meta = n3meta;
    seg_last = cblk + 1 >= seg_b1(cs);
    next_q_unit = (seg_last && ns < seg_end) ? seg_u(ns) : -1;
    return true;
  };
  for (;;) {
    if (!step(buf_a, buf_b)) break;
    if (!step(buf_b, buf_a)) break;
  }
}

hipError_t launch_splitkv(const SplitKVParams& p, int d_qk, bool sparse, hipStream_t stream) {
  const int groups = p.num_parts * p.row_blocks;
  if (groups <= 0) return hipSuccess;
  const dim3 grid(groups), block(256);
  const bool pair = true;
#define MLA_LAUNCH(D, SP)                                                             \
  do {                                                                                \
    if (pair)                                                                         \
      hipLaunchKernelGGL((mla_splitkv<D, SP, true>), grid, block, 0, stream, p);      \
    else                                                                              \
      hipLaunchKernelGGL((mla_splitkv<D, SP, false>), grid, block, 0, stream, p);     \
  } while (0)
  if (d_qk == 576) {
    if (sparse) MLA_LAUNCH(576, true); else MLA_LAUNCH(576, false);
  } else {
    if (sparse) MLA_LAUNCH(512, true); else MLA_LAUNCH(512, false);
  }
#undef MLA_LAUNCH
  return hipGetLastError();
}

}  // namespace mla
