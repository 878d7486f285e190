// LSE combine kernel of the paged MLA decode library, written for gfx950.
//
// mla_combine merges the fp32 partial outputs of a split unit by their base-2
// log-sum-exps, over active rows only (the DeepLink-org fork's active-head
// combine).  Lane k of a wavefront holds the log-sum-exps of splits k, k+64,
// ..., so up to 64 splits are merged in one pass (the fork's exact small-split
// path, widened to wave64) and more in further passes.
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

// One workgroup per (split unit, row).  Every wavefront derives the merged
// log-sum-exp itself (lane k holds splits k, k+64, ...); the weighted sum of the
// partial outputs is spread over the four wavefronts (wavefront w takes splits
// w, w+4, ..., several loads in flight per lane) and reduced through LDS.
__global__ __launch_bounds__(256) void mla_combine(CombineParams p) {
  constexpr int kWaves = 4, kUnroll = 4;
  __shared__ f32x4 red[kWaves - 1][64][2];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int k = blockIdx.x / p.rows;
  const int row = blockIdx.x - k * p.rows;

  const int32_t* meta = p.meta;
  const int u = meta[p.off_split_list + 2 * k];
  const int slot0 = meta[p.off_split_list + 2 * k + 1];
  const int nsplit = meta[p.off_num_splits + u + 1] - meta[p.off_num_splits + u];
  const float* lse_col = p.ws_lse + size_t(slot0) * p.rows + row;  // split s at s * rows

  // merged LSE (base 2): max, then sum of 2^(lse - max)
  float mx = -__builtin_inff();
  for (int s = lane; s < nsplit; s += 64) mx = fmaxf(mx, lse_col[size_t(s) * p.rows]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float m_use = mx == -__builtin_inff() ? 0.f : mx;
  float sum = 0.f;
  for (int s = lane; s < nsplit; s += 64) sum += fast_exp2(lse_col[size_t(s) * p.rows] - m_use);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  const bool empty = !(sum > 0.f);
  const float lse2 = empty ? -__builtin_inff() : m_use + fast_log2(sum);

  // weighted partial outputs; lane owns columns 8*lane .. 8*lane+7
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  if (!empty) {
    const float* o_col = p.ws_o + (size_t(slot0) * p.rows + row) * kDV + 8 * lane;
    const size_t split_stride = size_t(p.rows) * kDV;
    for (int s0 = wave; s0 < nsplit; s0 += kWaves * kUnroll) {
      f32x4 v0[kUnroll], v1[kUnroll];
      float w[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int s = s0 + j * kWaves;
        const bool ok = s < nsplit;
        const float* src = o_col + size_t(ok ? s : s0) * split_stride;
        v0[j] = *reinterpret_cast<const f32x4*>(src);
        v1[j] = *reinterpret_cast<const f32x4*>(src + 4);
        w[j] = ok ? fast_exp2(lse_col[size_t(ok ? s : s0) * p.rows] - lse2) : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        a0 += w[j] * v0[j];
        a1 += w[j] * v1[j];
      }
    }
  }
  if (wave > 0) {
    red[wave - 1][lane][0] = a0;
    red[wave - 1][lane][1] = a1;
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) {
    a0 += red[w][lane][0];
    a1 += red[w][lane][1];
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

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.num_split_units <= 0 || p.rows <= 0) return hipSuccess;
  const dim3 grid(p.num_split_units * p.rows), block(256);
  hipLaunchKernelGGL(mla_combine, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
