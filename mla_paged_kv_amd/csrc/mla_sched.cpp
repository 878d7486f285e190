// Host tile scheduler of the paged MLA decode library (mla_get_metadata).
//
// The pages give the scheduler's role -- metadata built once per decode step
// from the cache sequence lengths and the head configuration, reused by every
// layer, spreading variable-length work over the compute units (deepep.org
// usage page, get_mla_metadata example and the "Tile Scheduler" paragraph;
// upstream FlashMLA README embedded in the DeepLink-org/flashmla-optimization
// page, "Usage / MLA Decoding") -- but not its algorithm.  This file implements
// the library's own specification of it (declared in mla.h):
//
//   nb[u] = ceil(len[u] / 64), total = sum(nb[u] + F), quota = ceil(total / P) + F
//
// and a greedy walk that fills part after part in unit order: a unit's
// remaining blocks go whole into the current part when they fit with one
// overhead F, otherwise the part is topped up with a cut of (budget - F) blocks
// if that is positive, and closed.  Because every part boundary costs at most F
// (a cut pays a second overhead, a non-cut close leaves at most F unused), the
// walk never needs more than P parts.
//
// Pure integer host code: no HIP call and no device memory.
#include <climits>
#include <cstdint>
#include <cstring>
#include <new>

#include "mla.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int32_t kPage = 64;
constexpr int32_t kOverhead = 5;      // F, per-segment overhead in blocks
constexpr int32_t kGroupsPerCU = 1;   // resident workgroups per compute unit (LDS-bound)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int32_t default_num_parts(int32_t rows, int32_t num_cus) {
  if (rows <= 0 || num_cus <= 0) return 1;
  const int64_t row_blocks = ceil_div(rows, rows_per_group(rows));
  const int64_t p = (int64_t(kGroupsPerCU) * num_cus) / row_blocks;
  return p < 1 ? 1 : int32_t(p > INT32_MAX ? INT32_MAX : p);
}

size_t metadata_capacity(int32_t num_units, int32_t target_parts) {
  if (num_units < 0 || target_parts < 1) return 0;
  return size_t(kHeaderInts) + 2 + 5 * size_t(target_parts) + 7 * size_t(num_units);
}

// Builds the schedule for unit lengths `len` (n units) into `meta`.
int build_schedule(const int64_t* len, int32_t n, int32_t parts, int32_t rows,
                   int32_t* meta, size_t cap, mla_sched_info* info) {
  if (parts < 1 || rows < 1 || n < 0) return set_error(MLA_E_INVAL, "schedule: bad sizes");
  if (cap < metadata_capacity(n, parts))
    return set_error(MLA_E_NOSPC, "schedule: metadata capacity %zu < %zu ints", cap,
                     metadata_capacity(n, parts));

  int64_t total = 0;
  for (int32_t u = 0; u < n; ++u) total += ceil_div(len[u], kPage) + kOverhead;
  const int64_t quota64 = ceil_div(total, parts) + kOverhead;
  if (total > INT32_MAX / 2 || quota64 > INT32_MAX / 2)
    return set_error(MLA_E_INVAL, "schedule: total work %lld blocks too large", (long long)total);
  const int32_t quota = int32_t(quota64);

  // The walk runs twice: first to count parts and segments (which fixes the
  // array offsets), then to write part_ptr and segs in place.
  int32_t npart = 0, nseg = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int32_t off_segs_now = kHeaderInts + npart + 1;
    int32_t* part_ptr = meta + kHeaderInts;
    int32_t* segs = meta + off_segs_now;
    const bool write = pass == 1;
    int32_t parts_seen = 0, segs_seen = 0;
    if (write) part_ptr[0] = 0;
    int32_t u = 0;
    int64_t j = 0;
    while (u < n) {
      int64_t rem = quota;
      while (u < n) {
        const int64_t nb = ceil_div(len[u], kPage);
        const int64_t need = nb - j + kOverhead;
        int64_t end_blk;
        bool close = false;
        if (need <= rem) {
          end_blk = nb;
          rem -= need;
        } else if (rem > kOverhead) {
          end_blk = j + (rem - kOverhead);
          close = true;
        } else {
          break;
        }
        if (write) {
          segs[4 * segs_seen + 0] = u;
          segs[4 * segs_seen + 1] = int32_t(j);
          segs[4 * segs_seen + 2] = int32_t(end_blk);
          segs[4 * segs_seen + 3] = -1;
        }
        ++segs_seen;
        if (close) {
          j = end_blk;
          break;
        }
        ++u;
        j = 0;
      }
      ++parts_seen;
      if (parts_seen > parts) return set_error(MLA_E_INVAL, "schedule: internal part overflow");
      if (write) part_ptr[parts_seen] = segs_seen;
    }
    npart = parts_seen;
    nseg = segs_seen;
  }

  // Per-unit segment counts (segments are in unit order), cumulative.
  const int32_t off_segs = kHeaderInts + npart + 1;
  const int32_t off_ns = off_segs + 4 * nseg;
  const int32_t off_sl = off_ns + n + 1;
  int32_t* segs = meta + off_segs;
  int32_t* num_splits = meta + off_ns;
  for (int32_t k = 0; k <= n; ++k) num_splits[k] = 0;
  for (int32_t s = 0; s < nseg; ++s) num_splits[segs[4 * s] + 1] += 1;
  int32_t max_splits = 0;
  for (int32_t k = 0; k < n; ++k) {
    if (num_splits[k + 1] > max_splits) max_splits = num_splits[k + 1];
    num_splits[k + 1] += num_splits[k];
  }
  // Slots: the k-th segment of a unit with >= 2 segments gets slot base + k.
  int32_t* split_list = meta + off_sl;
  int32_t nsplit_units = 0, nslots = 0;
  for (int32_t uu = 0; uu < n; ++uu) {
    const int32_t first = num_splits[uu], cnt = num_splits[uu + 1] - num_splits[uu];
    if (cnt >= 2) {
      split_list[2 * nsplit_units + 0] = uu;
      split_list[2 * nsplit_units + 1] = nslots;
      ++nsplit_units;
      for (int32_t k = 0; k < cnt; ++k) segs[4 * (first + k) + 3] = nslots + k;
      nslots += cnt;
    }
  }

  mla_sched_info h;
  h.num_parts = npart;
  h.num_segments = nseg;
  h.total_slots = nslots;
  h.num_split_units = nsplit_units;
  h.max_splits = max_splits;
  h.num_units = n;
  h.quota = quota;
  h.total_cost = int32_t(total);
  h.target_parts = parts;
  h.overhead = kOverhead;
  h.row_blocks = int32_t(ceil_div(rows, rows_per_group(rows)));
  h.rows = rows;
  h.off_segs = off_segs;
  h.off_num_splits = off_ns;
  h.off_split_list = off_sl;
  h.total_ints = off_sl + 2 * nsplit_units;
  static_assert(sizeof(mla_sched_info) == kHeaderInts * sizeof(int32_t), "header size");
  std::memcpy(meta, &h, sizeof(h));
  if (info) *info = h;
  return MLA_OK;
}

int resolve_sched_shape(int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t topk,
                        int32_t active_h_q, int32_t num_cus, int32_t num_parts, SchedShape* out) {
  if (batch < 0 || s_q < 1 || h_q < 1 || h_kv < 1 || topk < 0 || active_h_q < 0 ||
      num_cus < 0 || num_parts < 0)
    return set_error(MLA_E_INVAL, "get_metadata: negative or zero shape");
  if (h_q % h_kv != 0) return set_error(MLA_E_INVAL, "get_metadata: h_q %% h_kv != 0");
  if (num_parts == 0 && num_cus == 0)
    return set_error(MLA_E_INVAL, "get_metadata: give num_cus or num_parts");
  int rc = MLA_OK;
  int32_t heads = h_q;
  if (active_h_q != 0 && active_h_q != h_q) {
    if (active_h_q <= h_q && active_h_q % 8 == 0) {
      heads = active_h_q;
    } else {
      rc = MLA_W_ACTIVE_FALLBACK;  // fail closed: compute every head
    }
  }
  const int32_t per_kv_head = heads / h_kv > 0 ? heads / h_kv : 1;
  const bool sparse = topk > 0;
  const int64_t units64 = sparse ? int64_t(batch) * s_q : int64_t(batch);
  if (units64 > (1 << 24)) return set_error(MLA_E_INVAL, "get_metadata: too many units");
  const int64_t rows64 = sparse ? per_kv_head : int64_t(s_q) * per_kv_head;
  if (rows64 > (1 << 24)) return set_error(MLA_E_INVAL, "get_metadata: too many rows per unit");
  out->units = int32_t(units64);
  out->rows = int32_t(rows64);
  out->parts = num_parts > 0 ? num_parts : default_num_parts(out->rows, num_cus);
  return rc;
}

}  // namespace mla

extern "C" {

int32_t mla_default_num_parts(int32_t rows, int32_t num_cus) {
  return mla::default_num_parts(rows, num_cus);
}

size_t mla_metadata_capacity(int32_t num_units, int32_t target_parts) {
  return mla::metadata_capacity(num_units, target_parts);
}

int mla_get_metadata(const int32_t* cache_seqlens_host, int32_t batch, int32_t s_q,
                     int32_t h_q, int32_t h_kv, int32_t topk, int32_t active_h_q,
                     int32_t num_cus, int32_t num_parts, int32_t* meta_host,
                     size_t meta_capacity_ints, mla_sched_info* info) {
  using namespace mla;
  clear_error();
  if (meta_host == nullptr || info == nullptr)
    return set_error(MLA_E_INVAL, "get_metadata: null meta_host/info");
  if (topk == 0 && batch > 0 && cache_seqlens_host == nullptr)
    return set_error(MLA_E_INVAL, "get_metadata: dense mode needs cache_seqlens_host");
  SchedShape sh;
  const int rc = resolve_sched_shape(batch, s_q, h_q, h_kv, topk, active_h_q, num_cus, num_parts,
                                     &sh);
  if (rc < 0) return rc;
  const int32_t units = sh.units;
  const bool sparse = topk > 0;

  // unit lengths, on the stack for small batches
  constexpr int32_t kStack = 4096;
  int64_t stack_len[kStack];
  int64_t* len = stack_len;
  int64_t* heap_len = nullptr;
  if (units > kStack) {
    heap_len = new (std::nothrow) int64_t[units];
    if (!heap_len) return set_error(MLA_E_NOSPC, "get_metadata: host allocation failed");
    len = heap_len;
  }
  int bad = -1;
  for (int32_t u = 0; u < units; ++u) {
    const int64_t L = sparse ? topk : cache_seqlens_host[u];
    if (L < 0) { bad = u; break; }
    len[u] = L;
  }
  int st;
  if (bad >= 0) {
    st = set_error(MLA_E_INVAL, "get_metadata: cache_seqlens[%d] < 0", bad);
  } else {
    st = build_schedule(len, units, sh.parts, sh.rows, meta_host, meta_capacity_ints, info);
  }
  delete[] heap_len;
  if (st != MLA_OK) return st;
  if (rc != MLA_OK)
    set_error(rc, "get_metadata: active_h_q=%d invalid for h_q=%d, computing all heads",
              active_h_q, h_q);
  return rc;
}

}  // extern "C"
