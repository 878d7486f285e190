// LSE combine kernel of the paged MLA decode library, written for gfx950.
//
// mla_combine merges the fp32 partial outputs of a split unit by their base-2
// log-sum-exps, over active rows only (the DeepLink-org fork's active-head
// combine).  Every split count is merged exactly in one kernel (the fork
// special-cases small split counts; here the loop simply runs once for up to
// 32 splits).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_kernels.h"

namespace mla {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDV = 512;       // value width handled by the kernels
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ unsigned short f2bf(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);  // v_cvt_pk_bf16_f32, RNE
}

}  // namespace

// Two layouts, picked per launch from the largest split count:
//  * ROW_WAVES = true (many splits): one workgroup per (split unit, row);
//    wavefront w merges splits w, w+4, ... and the four results are merged
//    through LDS;
//  * ROW_WAVES = false (at most a few splits): one wavefront per (split unit,
//    row), four rows per workgroup, no LDS.  With at most 5 splits per unit
//    the loads of 4 splits are issued at a time (UNROLL = 4): 56 instead of
//    93 registers, so 8 wavefronts per SIMD instead of 5, which matters when
//    the grid has many rows (h_q = 128: thousands of wavefronts).
// A wavefront merges its splits against its own running maximum, issuing the
// loads of up to kUnroll splits (their LSE and 8 partial-output columns per
// lane) before using any, so the partial outputs are read in one round trip
// per kUnroll splits with no separate pass over the LSEs.  Base-2
// log-sum-exp throughout:
//   lse = m + log2 sum_s 2^(lse_s - m),  O = sum_s 2^(lse_s - lse) O_s.
template <bool ROW_WAVES, int UNROLL>
__global__ __launch_bounds__(256) void mla_combine(CombineParams p) {
  constexpr int kWaves = 4, kUnroll = UNROLL;
  constexpr int kStride = ROW_WAVES ? kWaves : 1;  // split stride of a wavefront
  __shared__ f32x4 red[ROW_WAVES ? kWaves : 1][64][2];  // per-wavefront weighted sums
  __shared__ float red_m[kWaves], red_l[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int k, row;
  if constexpr (ROW_WAVES) {
    k = blockIdx.x / p.rows;
    row = blockIdx.x - k * p.rows;
  } else {
    const int groups = (p.rows + kWaves - 1) / kWaves;
    k = blockIdx.x / groups;
    row = (blockIdx.x - k * groups) * kWaves + wave;
    if (row >= p.rows) return;
  }

  const int32_t* meta = p.meta;
  // offsets and the split-unit count come from the host when it built the
  // metadata, else (negative offsets) from the device header, and the grid
  // then covers an upper bound of the split units
  int off_sl = p.off_split_list, nsu = p.num_split_units;
  if (off_sl < 0) {
    nsu = meta[3];
    if (k >= nsu) return;
    off_sl = meta[14];
  }
  // Split units own consecutive workspace slots, numbered in unit order, so
  // unit k's split count is the next unit's first slot (or, for the last,
  // the total slot count in header word 2) minus its own: read in the same
  // round trip as the unit, not after it.
  const int u = meta[off_sl + 2 * k];
  const int slot0 = meta[off_sl + 2 * k + 1];
  const int nsplit = meta[k + 1 < nsu ? off_sl + 2 * k + 3 : 2] - slot0;
  const float* lse_col = p.ws_lse + size_t(slot0) * p.rows + row;  // split s at s * rows
  const float* o_col = p.ws_o + (size_t(slot0) * p.rows + row) * kDV + 8 * lane;
  const size_t split_stride = size_t(p.rows) * kDV;

  // this wavefront's splits, merged online: m (running max), l, a0/a1
  float m = -__builtin_inff(), l = 0.f;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = ROW_WAVES ? wave : 0; s0 < nsplit; s0 += kStride * kUnroll) {
    f32x4 v0[kUnroll], v1[kUnroll];
    float ls[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      // only existing splits are read (the test is uniform over the
      // wavefront); the others get weight 0 below
      const int s = s0 + j * kStride;
      ls[j] = -__builtin_inff();
      v0[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      v1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s < nsplit) {
        ls[j] = lse_col[size_t(s) * p.rows];
        const float* src = o_col + size_t(s) * split_stride;
        v0[j] = *reinterpret_cast<const f32x4*>(src);
        v1[j] = *reinterpret_cast<const f32x4*>(src + 4);
      }
    }
    float mb = m;
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
      if (s0 + j * kStride < nsplit) mb = fmaxf(mb, ls[j]);
    if (mb == -__builtin_inff()) continue;  // nothing but empty splits so far
    const float alpha = fast_exp2(m - mb);  // 0 while m is -inf
    l *= alpha;
    a0 *= alpha;
    a1 *= alpha;
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const float w = s0 + j * kStride < nsplit ? fast_exp2(ls[j] - mb) : 0.f;
      l += w;
      a0 += w * v0[j];
      a1 += w * v1[j];
    }
    m = mb;
  }
  if constexpr (ROW_WAVES) {
    red[wave][lane][0] = a0;
    red[wave][lane][1] = a1;
    if (lane == 0) {
      red_m[wave] = m;
      red_l[wave] = l;
    }
    __syncthreads();
    if (wave > 0) return;
    float mt = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mt = fmaxf(mt, red_m[w]);
    float lt = 0.f;
    a0 = f32x4{0.f, 0.f, 0.f, 0.f};
    a1 = f32x4{0.f, 0.f, 0.f, 0.f};
    if (mt != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sc = fast_exp2(red_m[w] - mt);  // 0 for a wavefront without splits
        lt += sc * red_l[w];
        a0 += sc * red[w][lane][0];
        a1 += sc * red[w][lane][1];
      }
    }
    m = mt;
    l = lt;
  }
  // row maximum of the scaled logits over the splits (when asked for); only
  // the wavefront that writes the row reaches this point
  float mx = -__builtin_inff();
  if (p.max_logits) {
    for (int s = lane; s < nsplit; s += 64) mx = fmaxf(mx, p.ws_max[size_t(slot0 + s) * p.rows + row]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
  }
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  const float lse2 = empty ? -__builtin_inff() : m + fast_log2(l);
  a0 *= inv;
  a1 *= inv;

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
  auto cvt = [&](float x) -> uint32_t {  // to the 16-bit output type, nearest even
    return p.out_f16 ? uint32_t(__builtin_bit_cast(unsigned short, (_Float16)x)) : uint32_t(f2bf(x));
  };
  w4[0] = cvt(a0[0]) | (cvt(a0[1]) << 16);
  w4[1] = cvt(a0[2]) | (cvt(a0[3]) << 16);
  w4[2] = cvt(a1[0]) | (cvt(a1[1]) << 16);
  w4[3] = cvt(a1[2]) | (cvt(a1[3]) << 16);
  *reinterpret_cast<u32x4*>(p.out + qrow * kDV + 8 * lane) = u32x4{w4[0], w4[1], w4[2], w4[3]};
  if (lane == 0) {
    p.lse[qrow] = p.lse_base2 ? lse2 : lse2 * kLn2;
    if (p.max_logits) p.max_logits[qrow] = mx;
  }
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.num_split_units <= 0 || p.rows <= 0) return hipSuccess;
  const dim3 block(256);
  const dim3 rows4(p.num_split_units * ((p.rows + 3) / 4));
  if (p.max_splits > 16) {
    hipLaunchKernelGGL((mla_combine<true, 8>), dim3(p.num_split_units * p.rows), block, 0, stream, p);
  } else if (p.max_splits > 5) {
    hipLaunchKernelGGL((mla_combine<false, 8>), rows4, block, 0, stream, p);
  } else {
    hipLaunchKernelGGL((mla_combine<false, 4>), rows4, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
