// LSE combine kernel of the paged MLA decode library, written for gfx950.
//
// mla_combine merges the fp32 partial outputs of a split unit by their base-2
// log-sum-exps: one wavefront per (split unit, active row); lane k holds the
// log-sum-exps of splits k, k+64, ... so up to 64 splits are reduced in one
// pass of the wavefront and more in further passes (the DeepLink-org fork's
// exact small-split combine path, widened to wave64), and the combine runs
// over active rows only (the fork's active-head combine).
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

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.num_split_units <= 0) return hipSuccess;
  const dim3 grid(p.num_split_units * ((p.rows + 3) / 4)), block(256);
  hipLaunchKernelGGL(mla_combine, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
