// HIP kernels of the paged MLA decode library, written for gfx950 (CDNA4).
//
//  * mla_splitkv<D_QK, SPARSE>: one workgroup = (part, row block).  It walks
//    its part's segments (unit, block range, slot) from the tile-scheduler
//    metadata.  For each 64-token tile it gathers the cache rows into LDS with
//    direct global->LDS loads (one contiguous 73,728-byte page for dense decode,
//    64 scattered rows for sparse decode), computes S^T = K.Q^T with bf16
//    MFMA 16x16x32, runs the online softmax in fp32 (base 2), and accumulates
//    O^T += V^T.P^T on MFMA, V being the first 512 columns of the same LDS
//    tile.  A segment that covers its whole unit writes bf16 O and fp32 LSE;
//    a split segment writes fp32 O and a base-2 LSE into its workspace slot.
//    The three stages (QK^T, scaled softmax, PV) and the paged addressing are
//    the structure the deepep.org usage page describes ("Block Table Manager",
//    "three stages"); sparse gathering follows the upstream FlashMLA README
//    ("Sparse Attention (indices tensor)"); only active heads are ever
//    computed (the DeepLink-org fork's padded-head changes, taken further:
//    padded heads cost nothing here because MFMA tiles are 16 rows).
//  * mla_combine: LSE merge of the split partials, one wavefront per
//    (split unit, active row); up to 64 splits per pass of a wavefront, more in
//    further passes (the fork's "exact fast combine path" idea on wave64).
//
// Wave layout of the split-KV kernel (4 waves, 16 query rows each):
//  MFMA 16x16x32 bf16: lane l holds A[l%16][8(l/16)..+7], B[8(l/16)..+7][l%16]
//  and C[4(l/16)+i][l%16].  With A = K (rows = tokens) and B = Q^T (columns =
//  query rows), lane l owns query row l%16 in every output tile, so the
//  softmax row state is per lane (reduced over the 4 lanes l, l^16, l^32,
//  l^48), P feeds the PV MFMA as its B operand straight from registers, and
//  the O^T accumulator is row l%16 again.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_kernels.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPage = 64;      // tokens per tile (page size / index chunk)
constexpr int kWaves = 4;      // waves per workgroup
constexpr int kRowsPerWave = 16;
constexpr int kDV = 512;       // value width handled by the kernels
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ unsigned short f2bf(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);  // v_cvt_pk_bf16_f32, RNE
}

// LDS tile layout: cache row t of the tile occupies chunks [t*RS, t*RS + CPR)
// of 16 bytes, RS = CPR + 1 (one pad chunk per row).  With RS odd, the 16 rows
// read by one MFMA operand fetch fall in 16 distinct 16-byte bank groups (and
// 8 consecutive rows in 8 distinct groups), and every LDS address is a
// per-lane base plus a compile-time offset that fits the DS immediate.
// XCD-aware mapping of the linear workgroup id: workgroups are dispatched to
// the 8 XCDs round-robin, so consecutive logical groups (the row blocks of one
// part, then neighbouring parts) are placed on the same XCD and share its L2.
__device__ __forceinline__ int logical_group(int id, int total) {
  constexpr int kXcd = 8;
  const int xcd = id % kXcd, k = id / kXcd;
  const int per = total / kXcd, rem = total % kXcd;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + k;
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace

template <int D_QK, bool SPARSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_splitkv(SplitKVParams p) {
  constexpr int CPR = D_QK / 8;   // 16-byte chunks per cache row
  constexpr int RS = CPR + 1;     // LDS row stride in chunks (one pad chunk)
  constexpr int RSB = RS * 16;    // LDS row stride in bytes
  constexpr int NLD = (kPage * RS + 63) / 64;  // 64-chunk load instructions per tile
  constexpr int KK = D_QK / 32;   // k-steps of the QK MFMA
  constexpr int NCT = kDV / 16;   // output column tiles
  __shared__ __attribute__((aligned(1024))) uint8_t tile[NLD * 1024];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lrow = lane & 15;  // query row within the wave / token within a 16-tile
  const int lgrp = lane >> 4;  // k-group of the MFMA operands

  const int total = p.num_parts * p.row_blocks;
  const int lg = logical_group(blockIdx.x, total);
  const int part = lg / p.row_blocks;
  const int rb = lg - part * p.row_blocks;
  if (part >= p.num_parts) return;

  const int32_t* meta = p.meta;
  const int seg_begin = meta[kMetaHeaderInts + part];
  const int seg_end = meta[kMetaHeaderInts + part + 1];
  const int off_segs = meta[12];

  const int row0 = rb * (kWaves * kRowsPerWave) + wave * kRowsPerWave;  // first row of this wave
  const bool wave_active = row0 < p.rows;
  const int row = row0 + lrow;  // this lane's query row (softmax/accumulator owner)
  const bool row_ok = row < p.rows;

  for (int s = seg_begin; s < seg_end; ++s) {
    const int u = meta[off_segs + 4 * s + 0];
    const int blk0 = meta[off_segs + 4 * s + 1];
    const int blk1 = meta[off_segs + 4 * s + 2];
    const int slot = meta[off_segs + 4 * s + 3];

    // unit -> request / query token / head of this lane's row
    int b, iq, h;
    if constexpr (SPARSE) {
      b = u / p.s_q;
      iq = u - b * p.s_q;
      h = row;
    } else {
      b = u;
      iq = row / p.heads;
      h = row - iq * p.heads;
    }
    const int L = SPARSE ? 0 : p.seqlens[b];
    int n_vis = L;  // positions this row may see (dense)
    if (!SPARSE && p.causal) {
      n_vis = L - p.s_q + iq + 1;
      n_vis = n_vis < 0 ? 0 : (n_vis > L ? L : n_vis);
    }
    const size_t qrow = (size_t(b) * p.s_q + iq) * p.h_q + h;

    // Q^T operand, resident for the whole segment: lane holds row lrow,
    // columns 32kk + 8*lgrp .. +7.
    bf16x8 qf[KK];
    {
      const uint16_t* qp = p.q + qrow * D_QK + 8 * lgrp;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (row_ok) {
          qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 32 * kk);
        } else {
          qf[kk] = __builtin_bit_cast(bf16x8, s16x8{0, 0, 0, 0, 0, 0, 0, 0});
        }
      }
    }

    f32x4 acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff();
    float l_part = 0.f;  // this lane's share of the row's sum of weights

    for (int blk = blk0; blk < blk1; ++blk) {
      // ---- gather the tile into LDS (all four waves) ----
      const uint8_t* page_base = nullptr;
      int valid_tokens = kPage;
      if constexpr (!SPARSE) {
        const int phys = p.block_table[size_t(b) * p.bt_stride + blk];
        page_base = reinterpret_cast<const uint8_t*>(p.kv) + size_t(phys) * kPage * D_QK * 2;
        valid_tokens = L - blk * kPage;
        valid_tokens = valid_tokens > kPage ? kPage : valid_tokens;
      }
      const int32_t* idx_row = nullptr;
      if constexpr (SPARSE) idx_row = p.indices + size_t(u) * p.topk + size_t(blk) * kPage;
#pragma unroll 2
      for (int n = wave; n < NLD; n += kWaves) {
        const int q = n * 64 + lane;  // LDS chunk written by this lane
        const int t = q / RS;
        const int c = q - t * RS;
        if (t >= kPage || c >= CPR) continue;  // pad chunk / past the tile
        const uint8_t* src;
        bool ok;
        if constexpr (SPARSE) {
          const int pos = blk * kPage + t;
          const int idx = pos < p.topk ? idx_row[t] : -1;
          ok = idx >= 0 && idx < p.num_rows;
          src = reinterpret_cast<const uint8_t*>(p.kv) + size_t(ok ? idx : 0) * D_QK * 2 + c * 16;
        } else {
          ok = t < valid_tokens;
          src = page_base + size_t(t) * D_QK * 2 + c * 16;
        }
        if (ok) {
          __builtin_amdgcn_global_load_lds(src, (lds_void*)(tile + n * 1024), 16, 0, 0);
        } else {
          *reinterpret_cast<u32x4*>(tile + q * 16) = u32x4{0u, 0u, 0u, 0u};
        }
      }
      wait_vmem();
      __syncthreads();

      if (wave_active) {
        // ---- S^T = K . Q^T over d_qk ----
        f32x4 st[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) st[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint8_t* kbase = tile + lrow * RSB + lgrp * 16;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const bf16x8 kf =
                *reinterpret_cast<const bf16x8*>(kbase + tt * 16 * RSB + kk * 64);
            st[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], st[tt], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }

        // ---- mask + online softmax (base 2), row = lrow ----
        float sv[16];
        float mloc = -__builtin_inff();
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = tt * 16 + lgrp * 4 + i;  // token within the tile
            bool vis;
            if constexpr (SPARSE) {
              const int pos = blk * kPage + t;
              const int idx = pos < p.topk ? idx_row[t] : -1;
              vis = idx >= 0 && idx < p.num_rows;
            } else {
              vis = blk * kPage + t < n_vis;
            }
            const float x = vis ? st[tt][i] * p.scale_log2 : -__builtin_inff();
            sv[tt * 4 + i] = x;
            mloc = fmaxf(mloc, x);
          }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run, mloc);
        const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
        s16x8 pk[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pe = fast_exp2(sv[e] - m_use);
          psum += pe;
          pk[e >> 3][e & 7] = (short)f2bf(pe);
        }
        l_part = l_part * alpha + psum;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] *= alpha;

        // ---- O^T += V^T . P^T ----
        // lane reads V[token][column] with token = 32kc + 4*lgrp + {0..3, 16..19}
        // and column = 16ct + lrow
        const uint8_t* vbase = tile + lgrp * 4 * RSB + lrow * 2;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[kc]);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            s16x8 vv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int tj = kc * 32 + (j < 4 ? j : 12 + j);
              vv[j] = *reinterpret_cast<const short*>(vbase + tj * RSB + ct * 32);
            }
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pb,
                                                              acc[ct], 0, 0, 0);
            if (ct & 1) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __syncthreads();
    }

    // ---- segment epilogue ----
    if (wave_active) {
      float l_tot = l_part + __shfl_xor(l_part, 16);
      l_tot += __shfl_xor(l_tot, 32);
      const bool empty = !(l_tot > 0.f);
      const float inv = empty ? 0.f : 1.f / l_tot;
      const float lse2 = empty ? -__builtin_inff() : m_run + fast_log2(l_tot);
      if (row_ok) {
        if (slot < 0) {
          uint16_t* o = p.out + qrow * kDV + 4 * lgrp;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const f32x4 v = acc[ct] * inv;
            const uint32_t lo = uint32_t(f2bf(v[0])) | (uint32_t(f2bf(v[1])) << 16);
            const uint32_t hi = uint32_t(f2bf(v[2])) | (uint32_t(f2bf(v[3])) << 16);
            *reinterpret_cast<uint2*>(o + ct * 16) = uint2{lo, hi};
          }
          if (lgrp == 0) p.lse[qrow] = lse2 * kLn2;
        } else {
          const size_t wrow = size_t(slot) * p.rows + row;
          float* o = p.ws_o + wrow * kDV + 4 * lgrp;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            *reinterpret_cast<f32x4*>(o + ct * 16) = acc[ct] * inv;
          }
          if (lgrp == 0) p.ws_lse[wrow] = lse2;
        }
      }
    }
  }
}

// One wavefront per (split unit, row); lane k holds splits k, k+64, ...
__global__ __launch_bounds__(256) void mla_combine(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row_groups = (p.rows + 3) / 4;
  const int k = blockIdx.x / row_groups;
  const int row = (blockIdx.x - k * row_groups) * 4 + wave;
  if (k >= p.num_split_units || row >= p.rows) return;

  const int32_t* meta = p.meta;
  const int u = meta[p.off_split_list + 2 * k];
  const int slot0 = meta[p.off_split_list + 2 * k + 1];
  const int nsplit = meta[p.off_num_splits + u + 1] - meta[p.off_num_splits + u];

  // pass 1: max and sum of 2^lse over the splits
  float mx = -__builtin_inff();
  for (int s = lane; s < nsplit; s += 64) mx = fmaxf(mx, p.ws_lse[size_t(slot0 + s) * p.rows + row]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float m_use = mx == -__builtin_inff() ? 0.f : mx;
  float sum = 0.f;
  for (int s = lane; s < nsplit; s += 64)
    sum += fast_exp2(p.ws_lse[size_t(slot0 + s) * p.rows + row] - m_use);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  const bool empty = !(sum > 0.f);
  const float lse2 = empty ? -__builtin_inff() : m_use + fast_log2(sum);

  // pass 2: weighted sum of the partial outputs; lane owns columns 8*lane..+7
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  if (!empty) {
    for (int base = 0; base < nsplit; base += 64) {
      const int s_l = base + lane;
      const float w_l =
          s_l < nsplit ? fast_exp2(p.ws_lse[size_t(slot0 + s_l) * p.rows + row] - lse2) : 0.f;
      const int cnt = nsplit - base < 64 ? nsplit - base : 64;
      for (int j = 0; j < cnt; ++j) {
        const float w = __shfl(w_l, j);
        const f32x4* src =
            reinterpret_cast<const f32x4*>(p.ws_o + (size_t(slot0 + base + j) * p.rows + row) * kDV) +
            2 * lane;
        a0 += w * src[0];
        a1 += w * src[1];
      }
    }
  }
  int b, iq, h;
  if (p.sparse) {
    b = u / p.s_q;
    iq = u - b * p.s_q;
    h = row;
  } else {
    b = u;
    iq = row / p.heads;
    h = row - iq * p.heads;
  }
  const size_t qrow = (size_t(b) * p.s_q + iq) * p.h_q + h;
  uint32_t w4[4];
  w4[0] = uint32_t(f2bf(a0[0])) | (uint32_t(f2bf(a0[1])) << 16);
  w4[1] = uint32_t(f2bf(a0[2])) | (uint32_t(f2bf(a0[3])) << 16);
  w4[2] = uint32_t(f2bf(a1[0])) | (uint32_t(f2bf(a1[1])) << 16);
  w4[3] = uint32_t(f2bf(a1[2])) | (uint32_t(f2bf(a1[3])) << 16);
  *reinterpret_cast<u32x4*>(p.out + qrow * kDV + 8 * lane) = u32x4{w4[0], w4[1], w4[2], w4[3]};
  if (lane == 0) p.lse[qrow] = lse2 * kLn2;
}

hipError_t launch_splitkv(const SplitKVParams& p, int d_qk, bool sparse, hipStream_t stream) {
  const int groups = p.num_parts * p.row_blocks;
  if (groups <= 0) return hipSuccess;
  const dim3 grid(groups), block(256);
  if (d_qk == 576) {
    if (sparse)
      hipLaunchKernelGGL((mla_splitkv<576, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((mla_splitkv<576, false>), grid, block, 0, stream, p);
  } else {
    if (sparse)
      hipLaunchKernelGGL((mla_splitkv<512, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((mla_splitkv<512, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.num_split_units <= 0) return hipSuccess;
  const dim3 grid(p.num_split_units * ((p.rows + 3) / 4)), block(256);
  hipLaunchKernelGGL(mla_combine, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
