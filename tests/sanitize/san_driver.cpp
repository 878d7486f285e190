// Host-only driver for the AddressSanitizer / UndefinedBehaviorSanitizer build
// of the library's host code (the tile scheduler and the entry points'
// argument validation), built with g++ by tests/test_sanitize_cpu.py.
//
// Commands on stdin, one per line:
//   S <P> <rows> <n> <len_0> ... <len_n-1>
//       mla_get_metadata in dense mode (batch n, s_q 1, h_q rows, num_parts
//       P) into a heap array of exactly mla_metadata_capacity(n, P) ints, so
//       any write past the capacity is caught; prints "rc total_ints m_0 ...".
//   R
//       every decode entry point with arguments that validation rejects
//       (pointers are never dereferenced); prints "name rc" per call.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "mla.h"

namespace {

const void* const kFake = reinterpret_cast<const void*>(uintptr_t(1) << 20);
void* const kFakeW = reinterpret_cast<void*>(uintptr_t(1) << 20);

void schedule(std::istringstream& in) {
  int32_t P = 0, rows = 0, n = 0;
  in >> P >> rows >> n;
  std::vector<int32_t> lens(size_t(n > 0 ? n : 0));
  for (auto& v : lens) in >> v;
  const size_t cap = mla_metadata_capacity(n, P > 0 ? P : 1);
  int32_t* meta = new int32_t[cap];
  mla_sched_info info;
  std::memset(&info, 0, sizeof(info));
  const int rc = mla_get_metadata(n > 0 ? lens.data() : nullptr, n, 1, rows, 1, 0, 0, 0, P, meta,
                                  cap, &info);
  std::printf("%d %d", rc, rc < 0 ? 0 : info.total_ints);
  if (rc >= 0)
    for (int32_t i = 0; i < info.total_ints; ++i) std::printf(" %d", meta[i]);
  std::printf("\n");
  delete[] meta;
}

struct Paged {
  const void* q = kFake;
  const void* kv = kFake;
  const int32_t* bt = static_cast<const int32_t*>(kFake);
  const int32_t* sl = static_cast<const int32_t*>(kFake);
  int32_t batch = 2, s_q = 1, h_q = 16, h_kv = 1, d_qk = 576, dv = 512, nblk = 8, page = 64,
          bt_stride = 4, causal = 0;
  float scale = 0.04f;
  const int32_t* meta = static_cast<const int32_t*>(kFake);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  void* out = kFakeW;
  float* lse = static_cast<float*>(kFakeW);
  int call(const mla_sched_info* info) const {
    return mla_decode_paged(q, kv, bt, sl, batch, s_q, h_q, h_kv, d_qk, dv, nblk, page, bt_stride,
                            causal, scale, meta, info, ws, ws_bytes, out, lse, nullptr);
  }
};

void rejections() {
  // a valid schedule for two requests of 16 rows, split over many parts
  const int32_t lens[2] = {64, 200};
  const size_t cap = mla_metadata_capacity(2, 512);
  std::vector<int32_t> meta(cap);
  mla_sched_info info;
  std::memset(&info, 0, sizeof(info));
  if (mla_get_metadata(lens, 2, 1, 16, 1, 0, 0, 0, 512, meta.data(), cap, &info) != 0) {
    std::printf("setup_failed 1\n");
    return;
  }
  const size_t ws = mla_workspace_bytes(&info, 512);
  auto run = [&](const char* name, Paged p) { std::printf("%s %d\n", name, p.call(&info)); };
  Paged base;
  base.ws = kFakeW;
  base.ws_bytes = ws;
  Paged p;
  p = base; p.h_kv = 2; run("paged_h_kv", p);
  p = base; p.page = 32; run("paged_page", p);
  p = base; p.d_qk = 192; run("paged_d_qk", p);
  p = base; p.dv = 600; run("paged_dv_gt_dqk", p);
  p = base; p.q = static_cast<const char*>(kFake) + 2; run("paged_misaligned", p);
  p = base; p.ws = nullptr; p.ws_bytes = 0; run("paged_no_workspace", p);
  p = base; p.ws_bytes = 16; run("paged_small_workspace", p);
  p = base; p.batch = 3; run("paged_batch", p);
  p = base; p.s_q = 3; run("paged_s_q", p);
  p = base; p.h_q = 8; run("paged_h_q", p);
  p = base; p.causal = 2; run("paged_causal", p);
  p = base; p.scale = -1.f; run("paged_scale", p);
  p = base; p.bt = nullptr; run("paged_null_table", p);
  p = base; p.bt_stride = 0; run("paged_bt_stride", p);
  p = base; p.nblk = 1 << 26; run("paged_nblk", p);
  p = base; p.batch = -1; run("paged_negative_batch", p);
  {
    mla_sched_info bad = info;
    bad.row_blocks = 7;
    p = base;
    std::printf("paged_bad_header %d\n", p.call(&bad));
    bad = info;
    bad.total_slots = -5;
    std::printf("paged_bad_slots %d\n", p.call(&bad));
  }
  std::printf("paged_null_info %d\n", base.call(nullptr));
  // the other decode entry points share the checks
  std::printf("paged_fp8_d512 %d\n",
              mla_decode_paged_fp8(kFake, kFake, base.bt, base.sl, 2, 1, 16, 1, 512, 512, 8, 64, 4,
                                   0, 0.04f, base.meta, &info, kFakeW, ws, kFakeW, base.lse,
                                   nullptr));
  std::printf("paged_f16_h_kv %d\n",
              mla_decode_paged_f16(kFake, kFake, base.bt, base.sl, 2, 1, 16, 2, 576, 512, 8, 64, 4,
                                   0, 0.04f, base.meta, &info, kFakeW, ws, kFakeW, base.lse,
                                   nullptr));
  std::printf("splitkv_paged_batch %d\n",
              mla_splitkv_paged(kFake, kFake, base.bt, base.sl, 3, 1, 16, 1, 576, 512, 8, 64, 4, 0,
                                0.04f, base.meta, &info, kFakeW, ws, kFakeW, base.lse, nullptr));

  // sparse: 2 query tokens, 64 heads, 16 active, topk 2048
  const size_t scap = mla_metadata_capacity(2, 8);
  std::vector<int32_t> smeta(scap);
  mla_sched_info sinfo;
  std::memset(&sinfo, 0, sizeof(sinfo));
  if (mla_get_metadata(nullptr, 2, 1, 64, 1, 2048, 16, 0, 8, smeta.data(), scap, &sinfo) != 0) {
    std::printf("setup_failed 2\n");
    return;
  }
  const size_t sws = mla_workspace_bytes(&sinfo, 512);
  auto sparse = [&](const char* name, const int32_t* ix, int32_t batch, int32_t h_q, int32_t d_qk,
                    int32_t dv, int32_t nblk, int32_t topk, size_t wsb) {
    std::printf("%s %d\n", name,
                mla_decode_sparse(kFake, kFake, ix, batch, 1, h_q, 1, d_qk, dv, nblk, 64, topk,
                                  0.04f, base.meta, &sinfo, kFakeW, wsb, kFakeW, base.lse,
                                  nullptr));
  };
  const int32_t* ix = static_cast<const int32_t*>(kFake);
  sparse("sparse_null_indices", nullptr, 2, 64, 512, 512, 64, 2048, sws);
  sparse("sparse_topk", ix, 2, 64, 512, 512, 64, 0, sws);
  sparse("sparse_batch", ix, 1, 64, 512, 512, 64, 2048, sws);
  sparse("sparse_h_q", ix, 2, 8, 512, 512, 64, 2048, sws);
  sparse("sparse_dv", ix, 2, 64, 576, 576, 64, 2048, sws);
  sparse("sparse_small_workspace", ix, 2, 64, 512, 512, 64, 2048, sws - 4);
  sparse("sparse_nblk", ix, 2, 64, 512, 512, 1 << 26, 2048, sws);
  // prefill and combine
  std::printf("prefill_s_kv %d\n",
              mla_sparse_prefill(kFake, kFake, ix, 2, 0, 64, 1, 576, 512, 2048, 0.04f, base.meta,
                                 &sinfo, kFakeW, sws, kFakeW, nullptr, base.lse, nullptr));
  std::printf("prefill_topk %d\n",
              mla_sparse_prefill(kFake, kFake, ix, 2, 4096, 64, 1, 576, 512, 0, 0.04f, base.meta,
                                 &sinfo, kFakeW, sws, kFakeW, nullptr, base.lse, nullptr));
  std::printf("combine_null_meta %d\n",
              mla_combine(nullptr, &info, 2, 1, 16, 512, 0, kFakeW, ws, kFakeW, base.lse, nullptr));
  std::printf("combine_small_workspace %d\n",
              mla_combine(base.meta, &info, 2, 1, 16, 512, 0, kFakeW, 16, kFakeW, base.lse,
                          nullptr));
  // error strings of every code
  for (int c : {0, 1, -1, -2, -3, -4, -99})
    std::printf("strerror_%d %d\n", c, int(std::strlen(mla_strerror(c)) > 0));
}

}  // namespace

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    if (!(in >> cmd)) continue;
    if (cmd == "S")
      schedule(in);
    else if (cmd == "R")
      rejections();
    std::fflush(stdout);
  }
  return 0;
}
