// Device tile scheduler of the paged MLA decode library
// (mla_get_metadata_device).
//
// The pages build the scheduler metadata from the cache sequence lengths once
// per decode step and reuse it in every layer (deepep.org usage page,
// get_mla_metadata example; upstream FlashMLA README embedded in the
// DeepLink-org/flashmla-optimization page, "Usage / MLA Decoding").  This
// variant computes the same specification as the host scheduler in
// mla_sched.cpp, bit for bit, from lengths that already sit in device memory,
// so that a whole decode step (metadata, split-KV, combine) is enqueued without
// a host round trip and can be captured in a HIP graph.
//
// One workgroup of 256 threads, everything in LDS:
//  1. nb[u] = ceil(len[u] / 64) and the exclusive prefix cx of the unit costs
//     nb[u] + F (block-wide scan); quota = ceil(cx[U] / P) + F.
//  2. The greedy walk on wavefront 0.  A part starting at block j0 of unit u0
//     may spend up to lim = cx[u0] + j0 + quota.  If the unit's remaining
//     blocks do not fit (nb - j0 + F > quota), the part and the ones after it
//     each cut quota - F blocks of the unit until the rest fits; that run of
//     parts is written at once.  Otherwise the part takes every unit whose end
//     fits, cx[u + 1] <= lim -- a run of units, since the costs are positive,
//     counted with one ballot per 64 units -- and then cuts the next unit if
//     more than F of the budget is left.  At most 2 min(U, P) + 1 iterations.
//  3. Per-part segment counts -> part_ptr (scan); per-unit segment counts and
//     first part (LDS atomics) -> cumulative counts, slots and the split list
//     (scans); then every part writes its segments in parallel.  The scans are
//     wavefront prefix sums combined across the four wavefronts.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "mla.h"
#include "mla_internal.h"
#include "mla_kernels.h"

namespace mla {

namespace {

constexpr int kThreads = 256;
constexpr int kPage = 64;
constexpr int kOverhead = 5;            // F: per-segment overhead in blocks
constexpr int kMaxLen = 1 << 24;        // longest unit accepted (keeps every sum in int32)

struct SchedDevParams {
  const int32_t* seqlens;  // dense: [units] on the device; sparse: unused
  int32_t* meta;           // output, >= metadata_capacity(units, parts) ints
  int32_t units, parts, topk, sparse, rows, row_blocks;
};

constexpr int kWaves = kThreads / 64;

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ int wave_max(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = max(x, __shfl_xor(x, d));
  return x;
}

// Exclusive scan of a[0..n) in LDS, in place, by the whole block; returns the
// total.  Each thread scans a contiguous run; the run totals are scanned
// within each wavefront and then across the wavefronts.  Every thread of the
// block must call it.
__device__ int block_exclusive_scan(int* a, int n, int* tmp) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int run = 0;
  for (int i = lo; i < hi; ++i) run += a[i];
  const int incl = wave_inclusive_scan(run);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int acc = incl - run, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int v = tmp[w];
    if (w < wave) acc += v;
    total += v;
  }
  for (int i = lo; i < hi; ++i) {
    const int v = a[i];
    a[i] = acc;
    acc += v;
  }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kThreads) void mla_sched_dev(SchedDevParams p) {
  __shared__ int cx[kSchedDevMaxUnits + 1];      // exclusive prefix of unit costs
  __shared__ int nb[kSchedDevMaxUnits];          // blocks per unit
  __shared__ int ucnt[kSchedDevMaxUnits];        // segments per unit
  __shared__ int ufirst[kSchedDevMaxUnits];      // first part holding the unit
  __shared__ int ubase[kSchedDevMaxUnits + 1];   // segments before / slot base
  __shared__ int uidx[kSchedDevMaxUnits];        // split-list index
  __shared__ int pu[kSchedDevMaxParts];          // part: first unit
  __shared__ int pj[kSchedDevMaxParts];          // part: first block of that unit
  __shared__ int pcnt[kSchedDevMaxParts];        // part: units taken whole
  __shared__ int pcut[kSchedDevMaxParts];        // part: blocks of the final cut (0: none)
  __shared__ int pseg[kSchedDevMaxParts + 1];    // part: segments -> first segment
  __shared__ int tmp[kThreads + 1];
  __shared__ int s_np, s_bad;

  const int U = p.units, P = p.parts;
  int32_t* meta = p.meta;
  const int t = threadIdx.x;

  // 1. blocks and costs
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int u = t; u < U; u += kThreads) {
    const int L = p.sparse ? p.topk : p.seqlens[u];
    const bool bad = L < 0 || L > kMaxLen;
    if (bad) s_bad = 1;
    const int n = bad ? 0 : (L + kPage - 1) / kPage;
    nb[u] = n;
    cx[u] = n + kOverhead;
    ucnt[u] = 0;
    ufirst[u] = P;
  }
  __syncthreads();
  const int total = block_exclusive_scan(cx, U, tmp);
  if (t == 0) cx[U] = total;
  const int quota = (total + P - 1) / P + kOverhead;
  __syncthreads();

  // 2. the walk (wavefront 0 only; all its branches are uniform).  A part
  // starting at block j0 of unit u0 whose remaining blocks do not fit in one
  // part (nb - j0 + F > quota) takes just a cut of quota - F blocks, and so do
  // the parts after it until the rest fits: such a run of parts inside one
  // unit is written in one iteration.  Otherwise the part takes at least unit
  // u0 whole, then possibly more units and a cut.
  if (t < 64 && !s_bad) {
    const int lane = t;
    const int step = quota - kOverhead;  // blocks a fresh part cuts (quota > F)
    int u0 = 0, cxu0 = 0, j0 = 0, np = 0;
    while (u0 < U && np < P) {
      const int lim = cxu0 + j0 + quota;
      int v = u0 + 1 + lane <= U ? cx[u0 + 1 + lane] : INT_MAX;  // cx[u0 + 1 + lane]
      const int nbu = __builtin_amdgcn_readfirstlane(v) - cxu0 - kOverhead;
      if (nbu - j0 + kOverhead > quota) {
        int k = (nbu + kOverhead - quota - j0 + step - 1) / step;
        k = min(k, P - np);
        for (int i = lane; i < k; i += 64) {
          pu[np + i] = u0;
          pj[np + i] = j0 + i * step;
          pcnt[np + i] = 0;
          pcut[np + i] = step;
          pseg[np + i] = 1;
        }
        np += k;
        j0 += k * step;
        continue;
      }
      int count = 0, cx_un = cxu0;
      for (int c0 = u0 + 1;; c0 += 64) {
        if (c0 != u0 + 1) v = c0 + lane <= U ? cx[c0 + lane] : INT_MAX;
        const int k = __popcll(__ballot(v <= lim));
        if (k > 0) cx_un = __builtin_amdgcn_readlane(v, k - 1);
        count += k;
        if (k < 64 || c0 + 64 > U) break;
      }
      const int un = u0 + count;  // count >= 1
      const int rem = lim - cx_un;
      const int cut = (un < U && rem > kOverhead) ? rem - kOverhead : 0;
      if (lane == 0) {
        pu[np] = u0;
        pj[np] = j0;
        pcnt[np] = count;
        pcut[np] = cut;
        pseg[np] = count + (cut > 0 ? 1 : 0);
      }
      u0 = un;
      cxu0 = cx_un;
      j0 = cut;
      ++np;
    }
    if (lane == 0) {
      s_np = np;
      if (u0 < U) s_bad = 1;  // cannot happen: the walk needs at most P parts
    }
  }
  __syncthreads();
  if (s_bad) {  // a length out of range: an empty schedule that runs nothing
    // (the unit and row counts stay, so the decode kernels can mark every
    // output row of the call as invalid)
    if (t < kMetaHeaderInts)
      meta[t] = t == kMetaHeaderInts - 1 ? -1 : (t == 5 ? U : (t == 11 ? p.rows : 0));
    return;
  }
  const int NP = s_np;

  // 3. part_ptr; per-unit segment counts and first parts
  if (t == 0) pseg[NP] = 0;
  __syncthreads();
  const int S = block_exclusive_scan(pseg, NP + 1, tmp);
  for (int q = t; q < NP; q += kThreads) {
    const int end = pu[q] + pcnt[q] + (pcut[q] > 0 ? 1 : 0);
    for (int u = pu[q]; u < end; ++u) {
      atomicAdd(&ucnt[u], 1);
      atomicMin(&ufirst[u], q);
    }
  }
  __syncthreads();
  int mx = 0;
  for (int u = t; u < U; u += kThreads) {
    ubase[u] = ucnt[u];
    uidx[u] = ucnt[u] >= 2 ? 1 : 0;
    mx = max(mx, ucnt[u]);
  }
  mx = wave_max(mx);
  if ((t & 63) == 0) tmp[t >> 6] = mx;
  __syncthreads();
  int max_splits = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) max_splits = max(max_splits, tmp[w]);
  __syncthreads();

  const int off_segs = kMetaHeaderInts + NP + 1;
  const int off_ns = off_segs + 4 * S;
  const int off_sl = off_ns + U + 1;
  block_exclusive_scan(ubase, U, tmp);  // segments before each unit
  for (int u = t; u < U; u += kThreads) meta[off_ns + u] = ubase[u];
  if (t == 0) meta[off_ns + U] = S;
  __syncthreads();
  for (int u = t; u < U; u += kThreads) ubase[u] = ucnt[u] >= 2 ? ucnt[u] : 0;
  __syncthreads();
  const int nslots = block_exclusive_scan(ubase, U, tmp);  // slot base of split units
  const int nsu = block_exclusive_scan(uidx, U, tmp);      // split-list index
  for (int u = t; u < U; u += kThreads) {
    if (ucnt[u] >= 2) {
      meta[off_sl + 2 * uidx[u] + 0] = u;
      meta[off_sl + 2 * uidx[u] + 1] = ubase[u];
    }
  }
  for (int q = t; q <= NP; q += kThreads) meta[kMetaHeaderInts + q] = pseg[q];
  // segments: a unit's segments sit in consecutive parts from ufirst[u] on,
  // one per part, so the segment in part q has slot base + (q - ufirst[u])
  auto slot_of = [&](int u, int q) { return ucnt[u] >= 2 ? ubase[u] + (q - ufirst[u]) : -1; };
  for (int q = t; q < NP; q += kThreads) {
    int32_t* sg = meta + off_segs + 4 * pseg[q];
    const int cnt = pcnt[q];
    for (int i = 0; i < cnt; ++i, sg += 4) {
      const int u = pu[q] + i;
      sg[0] = u;
      sg[1] = i == 0 ? pj[q] : 0;
      sg[2] = nb[u];
      sg[3] = slot_of(u, q);
    }
    if (pcut[q] > 0) {
      const int u = pu[q] + cnt;
      const int b0 = cnt == 0 ? pj[q] : 0;
      sg[0] = u;
      sg[1] = b0;
      sg[2] = b0 + pcut[q];
      sg[3] = slot_of(u, q);
    }
  }
  if (t == 0) {
    meta[0] = NP;
    meta[1] = S;
    meta[2] = nslots;
    meta[3] = nsu;
    meta[4] = max_splits;
    meta[5] = U;
    meta[6] = quota;
    meta[7] = total;
    meta[8] = P;
    meta[9] = kOverhead;
    meta[10] = p.row_blocks;
    meta[11] = p.rows;
    meta[12] = off_segs;
    meta[13] = off_ns;
    meta[14] = off_sl;
    meta[15] = off_sl + 2 * nsu;
  }
}

}  // namespace

}  // namespace mla

extern "C" int mla_get_metadata_device(const int32_t* cache_seqlens_dev, int32_t batch,
                                       int32_t s_q, int32_t h_q, int32_t h_kv, int32_t topk,
                                       int32_t active_h_q, int32_t num_cus, int32_t num_parts,
                                       int32_t* meta_dev, size_t meta_capacity_ints,
                                       mla_sched_info* info, void* stream) {
  using namespace mla;
  clear_error();
  if (meta_dev == nullptr || info == nullptr)
    return set_error(MLA_E_INVAL, "get_metadata_device: null meta_dev/info");
  if (topk == 0 && batch > 0 && cache_seqlens_dev == nullptr)
    return set_error(MLA_E_INVAL, "get_metadata_device: dense mode needs cache_seqlens_dev");
  SchedShape sh;
  const int rc = resolve_sched_shape(batch, s_q, h_q, h_kv, topk, active_h_q, num_cus, num_parts,
                                     &sh);
  if (rc < 0) return rc;
  if (sh.units > kSchedDevMaxUnits || sh.parts > kSchedDevMaxParts)
    return set_error(MLA_E_NOTSUP, "get_metadata_device: %d units / %d parts (at most %d / %d)",
                     sh.units, sh.parts, kSchedDevMaxUnits, kSchedDevMaxParts);
  if (topk > kMaxLen) return set_error(MLA_E_INVAL, "get_metadata_device: topk=%d too large", topk);
  const size_t cap = metadata_capacity(sh.units, sh.parts);
  if (meta_capacity_ints < cap)
    return set_error(MLA_E_NOSPC, "get_metadata_device: metadata capacity %zu < %zu ints",
                     meta_capacity_ints, cap);

  SchedDevParams p;
  p.seqlens = cache_seqlens_dev;
  p.meta = meta_dev;
  p.units = sh.units;
  p.parts = sh.parts;
  p.topk = topk;
  p.sparse = topk > 0 ? 1 : 0;
  p.rows = sh.rows;
  p.row_blocks = (sh.rows + rows_per_group(sh.rows) - 1) / rows_per_group(sh.rows);
  hipLaunchKernelGGL(mla_sched_dev, dim3(1), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(MLA_E_HIP, "get_metadata_device launch: %s", hipGetErrorString(e));

  // Host view: the exact values live in the device header; these are bounds.
  const int32_t U = sh.units, P = sh.parts;
  mla_sched_info h;
  h.num_parts = U > 0 ? P : 0;
  h.num_segments = U > 0 ? U + P - 1 : 0;
  h.total_slots = U > 0 ? (U + P - 1 < 2 * (P - 1) ? U + P - 1 : 2 * (P - 1)) : 0;
  h.num_split_units = U < P - 1 ? U : P - 1;
  h.max_splits = U > 0 ? P : 0;
  h.num_units = U;
  h.quota = -1;
  h.total_cost = -1;
  h.target_parts = P;
  h.overhead = kOverhead;
  h.row_blocks = p.row_blocks;
  h.rows = sh.rows;
  h.off_segs = -1;
  h.off_num_splits = -1;
  h.off_split_list = -1;
  h.total_ints = int32_t(cap);
  *info = h;
  if (rc != MLA_OK)
    set_error(rc, "get_metadata_device: active_h_q=%d invalid for h_q=%d, computing all heads",
              active_h_q, h_q);
  return rc;
}
