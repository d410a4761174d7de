// A client of the C ABI in plain C++: device buffers from hipMalloc, the library's calls on raw pointers, no
// Python and no torch. It runs a few resolve steps and checks, on what the device returns, the properties every
// step must have: each selected id resolves to a slot that holds it, the page table is the slot table's
// inverse, the gathered row is the id's host row, and the miss count is the number of ids that were not
// resident before the step. Then a snapshot through hs_export_state: the steps after it, replayed from the
// imported snapshot, give the same outputs and the same state. Exit status 0 when every check holds.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <set>
#include <vector>

#include "hisparse.h"

#define HS(call)                                                                  \
  do {                                                                            \
    int rc_ = (call);                                                             \
    if (rc_ != HS_OK) {                                                           \
      std::fprintf(stderr, "%s failed (%d): %s\n", #call, rc_, hs_last_error()); \
      return 1;                                                                   \
    }                                                                             \
  } while (0)
#define HIP(call)                                                                                  \
  do {                                                                                             \
    hipError_t e_ = (call);                                                                        \
    if (e_ != hipSuccess) {                                                                        \
      std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));                      \
      return 1;                                                                                    \
    }                                                                                              \
  } while (0)
#define EXPECT(cond, ...)                      \
  do {                                         \
    if (!(cond)) {                             \
      std::fprintf(stderr, __VA_ARGS__);       \
      std::fprintf(stderr, "\n");              \
      return 1;                                \
    }                                          \
  } while (0)

static uint8_t row_byte(int r, int x, int b) { return (uint8_t)((r * 131 + x * 7 + b * 13) & 0xff); }

int main() {
  const int R = 4, k = 64, B = 128, H = 1024, rb = 64, steps = 12;
  hs_config cfg = {R, k, B, 0.0f, rb, H, 0, HS_EVICT_LRU};
  hs_sizes sz;
  HS(hs_required_sizes(&cfg, &sz));
  hs_ctx* ctx = nullptr;
  HS(hs_create(&cfg, &ctx));
  void* pool = nullptr;
  uint64_t stride = 0;
  int32_t rows = 0;
  HS(hs_host_pool(ctx, &pool, &stride, &rows));
  EXPECT(rows == H && stride == (uint64_t)H * rb, "pool shape %d rows, stride %llu", rows, (unsigned long long)stride);
  for (int r = 0; r < R; ++r)
    for (int x = 0; x < H; ++x)
      for (int b = 0; b < rb; ++b) static_cast<uint8_t*>(pool)[r * stride + (uint64_t)x * rb + b] = row_byte(r, x, b);

  hs_device_views v;
  std::memset(&v, 0, sizeof(v));
  HIP(hipMalloc(&v.hot, sz.hot_bytes));
  HIP(hipMalloc((void**)&v.slot_tok, sz.slot_tok_bytes));
  HIP(hipMalloc((void**)&v.stamp, sz.stamp_bytes));
  HIP(hipMalloc((void**)&v.lru_order, sz.lru_order_bytes));
  HIP(hipMalloc((void**)&v.page, sz.page_bytes));
  HIP(hipMalloc((void**)&v.step, sz.step_bytes));
  HIP(hipMalloc((void**)&v.epoch, sz.epoch_bytes));
  v.hot_bytes = sz.hot_bytes;
  v.slot_tok_bytes = sz.slot_tok_bytes;
  v.stamp_bytes = sz.stamp_bytes;
  v.lru_order_bytes = sz.lru_order_bytes;
  v.page_bytes = sz.page_bytes;
  v.step_bytes = sz.step_bytes;
  v.epoch_bytes = sz.epoch_bytes;
  HS(hs_bind_device(ctx, &v));
  HS(hs_reset(ctx, nullptr, -1, nullptr));

  int32_t *d_topk, *d_out, *d_miss, *d_status;
  void* d_gather;
  HIP(hipMalloc((void**)&d_topk, sz.topk_bytes));
  HIP(hipMalloc((void**)&d_out, sz.out_bytes));
  HIP(hipMalloc((void**)&d_miss, R * sizeof(int32_t)));
  HIP(hipMalloc((void**)&d_status, R * sizeof(int32_t)));
  HIP(hipMalloc(&d_gather, sz.gather_bytes));

  std::vector<int32_t> topk((size_t)R * k), out((size_t)R * k), miss(R), status(R), slot_tok((size_t)R * B),
      page((size_t)R * H), prev_slot_tok((size_t)R * B, -1);
  std::vector<uint8_t> gather(sz.gather_bytes);
  const uint64_t snap_bytes = sz.state_tables_bytes + sz.state_rows_bytes;
  void* d_snap = nullptr;
  HIP(hipMalloc(&d_snap, snap_bytes));
  const int snap_step = steps / 2;
  std::vector<std::vector<int32_t>> outs_after;  // outputs of the steps after the snapshot
  std::vector<uint8_t> state_end, state_replay;
  for (int t = 0; t < steps; ++t) {
    if (t == snap_step) HS(hs_export_state(ctx, d_snap, snap_bytes, HS_STATE_TABLES | HS_STATE_ROWS, nullptr));
    // a sliding window of distinct ids per request
    for (int r = 0; r < R; ++r) {
      const int base = (t * 23 + r * 101) % H;
      for (int i = 0; i < k; ++i) topk[(size_t)r * k + i] = (base + i * 3) % H;
    }
    HIP(hipMemcpy(d_topk, topk.data(), sz.topk_bytes, hipMemcpyHostToDevice));
    HS(hs_resolve(ctx, d_topk, nullptr, d_out, d_miss, d_status, d_gather, nullptr));
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(out.data(), d_out, sz.out_bytes, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(miss.data(), d_miss, R * sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(status.data(), d_status, R * sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(slot_tok.data(), v.slot_tok, sz.slot_tok_bytes, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(page.data(), v.page, sz.page_bytes, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(gather.data(), d_gather, sz.gather_bytes, hipMemcpyDeviceToHost));
    for (int r = 0; r < R; ++r) {
      EXPECT(status[r] == 0, "step %d request %d: status %d", t, r, status[r]);
      std::set<int32_t> resident(prev_slot_tok.begin() + (size_t)r * B, prev_slot_tok.begin() + (size_t)(r + 1) * B);
      int expected_miss = 0;
      for (int i = 0; i < k; ++i) {
        const int32_t x = topk[(size_t)r * k + i], s = out[(size_t)r * k + i];
        expected_miss += resident.count(x) == 0;
        EXPECT(s >= 0 && s < B, "step %d request %d: id %d resolved to %d", t, r, x, s);
        EXPECT(slot_tok[(size_t)r * B + s] == x, "step %d request %d: slot %d holds %d, not %d", t, r, s,
               slot_tok[(size_t)r * B + s], x);
        EXPECT(page[(size_t)r * H + x] == s, "step %d request %d: page[%d] = %d, not %d", t, r, x,
               page[(size_t)r * H + x], s);
        const uint8_t* g = &gather[((size_t)r * k + i) * rb];
        for (int b = 0; b < rb; ++b)
          EXPECT(g[b] == row_byte(r, x, b), "step %d request %d: gathered row of id %d differs at byte %d", t, r, x, b);
      }
      EXPECT(miss[r] == expected_miss, "step %d request %d: %d misses, expected %d", t, r, miss[r], expected_miss);
      int mapped = 0;
      for (int x = 0; x < H; ++x) mapped += page[(size_t)r * H + x] >= 0;
      int occupied = 0;
      for (int s = 0; s < B; ++s) occupied += slot_tok[(size_t)r * B + s] >= 0;
      EXPECT(mapped == occupied, "step %d request %d: %d page entries for %d occupied slots", t, r, mapped, occupied);
    }
    prev_slot_tok = slot_tok;
    if (t >= snap_step) outs_after.push_back(out);
  }
  // the state after the last step, then the same steps again from the imported snapshot
  state_end.resize(snap_bytes);
  state_replay.resize(snap_bytes);
  void* d_end = nullptr;
  HIP(hipMalloc(&d_end, snap_bytes));
  HS(hs_export_state(ctx, d_end, snap_bytes, HS_STATE_TABLES | HS_STATE_ROWS, nullptr));
  HIP(hipDeviceSynchronize());
  HIP(hipMemcpy(state_end.data(), d_end, snap_bytes, hipMemcpyDeviceToHost));
  HS(hs_import_state(ctx, d_snap, snap_bytes, HS_STATE_TABLES | HS_STATE_ROWS, nullptr));
  for (int t = snap_step; t < steps; ++t) {
    for (int r = 0; r < R; ++r) {
      const int base = (t * 23 + r * 101) % H;
      for (int i = 0; i < k; ++i) topk[(size_t)r * k + i] = (base + i * 3) % H;
    }
    HIP(hipMemcpy(d_topk, topk.data(), sz.topk_bytes, hipMemcpyHostToDevice));
    HS(hs_resolve(ctx, d_topk, nullptr, d_out, d_miss, d_status, d_gather, nullptr));
    HIP(hipMemcpy(out.data(), d_out, sz.out_bytes, hipMemcpyDeviceToHost));
    EXPECT(out == outs_after[(size_t)(t - snap_step)], "replayed step %d: outputs differ after the import", t);
  }
  HS(hs_export_state(ctx, d_end, snap_bytes, HS_STATE_TABLES | HS_STATE_ROWS, nullptr));
  HIP(hipDeviceSynchronize());
  HIP(hipMemcpy(state_replay.data(), d_end, snap_bytes, hipMemcpyDeviceToHost));
  EXPECT(state_end == state_replay, "the replayed state differs from the state of the first run");
  HIP(hipFree(d_end));
  HIP(hipFree(d_snap));
  HIP(hipFree(d_gather));
  HIP(hipFree(d_status));
  HIP(hipFree(d_miss));
  HIP(hipFree(d_out));
  HIP(hipFree(d_topk));
  HIP(hipFree(v.step));
  HIP(hipFree(v.epoch));
  HIP(hipFree(v.page));
  HIP(hipFree(v.lru_order));
  HIP(hipFree(v.stamp));
  HIP(hipFree(v.slot_tok));
  HIP(hipFree(v.hot));
  hs_destroy(ctx);
  std::printf("c client: %d steps x %d requests consistent through the C ABI, snapshot replay identical\n", steps, R);
  return 0;
}
