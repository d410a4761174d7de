// C ABI of the HiSparse swap-in path: argument checks, the pinned host pool, launches.
#include "hisparse.h"
#include "hs_internal.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

struct hs_ctx {
  hs_config cfg;
  int32_t H;             // host rows per request
  hs::Layout layout;          // the rank layout: what a context of this shape needs at least
  hs::Layout layout_plain;    // launches without a gather output: the direct layout where it fits
  hs::Layout layout_gather;   // launches with one (fused gather, trial)
  hs::Layout layout_plain_direct, layout_gather_direct;  // the same before the bound tables' alignment is known
  uint32_t lds_cap;           // LDS a resolve workgroup may take on this device
  int device;
  void* pool_host;       // pinned, mapped host pool
  void* pool_dev;        // its device address
  uint64_t pool_bytes;
  bool bound;
  hs_device_views views;
};

namespace {

thread_local char g_err[512] = "";

// Device address of the static plan array of each device (hs_step_static), taken once per device by the first
// hs_create made while that device is current.
std::mutex g_static_plan_mu;
std::vector<void*> g_static_plan;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return HS_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HS_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Validates cfg and derives the host rows and LDS layout. Host-only.
int check_config(const hs_config* cfg, int32_t* H_out, hs::Layout* L_out) {
  if (!cfg) return fail(HS_E_INVALID, "config is NULL");
  if (cfg->num_requests < 1 || cfg->num_requests > 65535)
    return fail(HS_E_INVALID, "num_requests must be in [1, 65535] (got %d)", cfg->num_requests);
  if (cfg->top_k < 1 || cfg->top_k > hs::kMaxTopK)
    return fail(HS_E_INVALID, "top_k must be in [1, %d] (got %d)", hs::kMaxTopK, cfg->top_k);
  if (cfg->device_buffer_size < cfg->top_k || cfg->device_buffer_size > hs::kMaxSlots)
    return fail(HS_E_INVALID, "device_buffer_size must be in [top_k, %d] (got %d, top_k %d)", hs::kMaxSlots,
                cfg->device_buffer_size, cfg->top_k);
  if (cfg->row_bytes < 16 || cfg->row_bytes % 16 != 0 || cfg->row_bytes > (1 << 20))
    return fail(HS_E_INVALID, "row_bytes must be a multiple of 16 in [16, 1 MiB] (got %d)", cfg->row_bytes);
  if (cfg->tail_tokens < 0) return fail(HS_E_INVALID, "tail_tokens must be >= 0 (got %d)", cfg->tail_tokens);
  if (cfg->max_context < 0) return fail(HS_E_INVALID, "max_context must be >= 0 (got %d)", cfg->max_context);
  if (cfg->eviction_policy != HS_EVICT_LRU && cfg->eviction_policy != HS_EVICT_FIFO)
    return fail(HS_E_INVALID, "eviction_policy must be HS_EVICT_LRU (0) or HS_EVICT_FIFO (1) (got %d)",
                cfg->eviction_policy);
  int64_t H = cfg->max_context;
  if (H == 0) {
    const double want = std::ceil((double)cfg->host_to_device_ratio * (double)cfg->device_buffer_size);
    if (!(cfg->host_to_device_ratio > 0.0f) || !std::isfinite(want) || want > 2147483647.0)
      return fail(HS_E_INVALID, "host_to_device_ratio must be > 0 and give at most 2^31-1 rows (got %g)",
                  (double)cfg->host_to_device_ratio);
    H = (int64_t)want;
  }
  if (H < 1) return fail(HS_E_INVALID, "host rows per request must be >= 1");
  // The pool (R * H * row_bytes) is the one size that can pass 64 bits: bound it well below that, so no size
  // or offset derived from it wraps (the allocation itself fails long before).
  uint64_t pool = 0;
  if (__builtin_mul_overflow((uint64_t)cfg->num_requests, (uint64_t)H, &pool) ||
      __builtin_mul_overflow(pool, (uint64_t)cfg->row_bytes, &pool) || pool > (1ull << 56))
    return fail(HS_E_INVALID, "the host pool (%d requests x %lld rows x %d bytes) exceeds 2^56 bytes",
                cfg->num_requests, (long long)H, cfg->row_bytes);
  // one workgroup's LDS: each kind of launch (with and without a gather output) takes the direct layout where
  // it fits and the rank layout otherwise (its flat bitmaps, or past their LDS the two-level ones); 1 KiB of
  // the 160 KiB of a gfx950 compute unit stays for the kernels' static LDS
  const int k = cfg->top_k, B = cfg->device_buffer_size, T = cfg->tail_tokens;
  const hs::Layout L = hs::rank_layout(k, B, (int)H, hs::kLdsCap);
  const uint32_t need = std::max(hs::launch_layout(k, B, (int)H, T, false, hs::kLdsCap).total,
                                 hs::launch_layout(k, B, (int)H, T, true, hs::kLdsCap).total);
  if (need > hs::kLdsCap)
    return fail(HS_E_INVALID,
                "this shape needs %u bytes of LDS per workgroup (top_k %d, buffer %d, host rows %lld), "
                "more than the 159 KiB one resolve workgroup may use on gfx950",
                need, k, B, (long long)H);
  *H_out = (int32_t)H;
  *L_out = L;
  return HS_OK;
}

void fill_sizes(const hs_config* cfg, int32_t H, const hs::Layout& L, hs_sizes* s) {
  const uint64_t R = (uint64_t)cfg->num_requests, k = (uint64_t)cfg->top_k, B = (uint64_t)cfg->device_buffer_size;
  const uint64_t rb = (uint64_t)cfg->row_bytes, T = (uint64_t)cfg->tail_tokens;
  s->host_rows = H;
  s->host_pool_bytes = R * (uint64_t)H * rb;
  s->hot_bytes = R * B * rb;
  s->tail_bytes = R * T * rb;
  s->slot_tok_bytes = R * B * 4;
  s->stamp_bytes = R * B * 4;
  s->lru_order_bytes = R * B * 2;
  s->page_bytes = R * (uint64_t)H * 4;
  s->step_bytes = R * 4;
  s->epoch_bytes = R * 4;
  s->topk_bytes = R * k * 4;
  s->out_bytes = R * k * 4;
  s->gather_bytes = R * k * rb;
  s->plan_bytes = R * 4 * k * 4;
  s->trial_bytes = R * (uint64_t)hs::trial_words((int)k, (int)B) * 4;
  // what launches take on a device that allows the full 159 KiB (the direct layout where it fits)
  const int kk = cfg->top_k, BB = cfg->device_buffer_size, TT = cfg->tail_tokens;
  const hs::Layout lp = hs::launch_layout(kk, BB, (int)H, TT, false, hs::kLdsCap);
  const hs::Layout lg = hs::launch_layout(kk, BB, (int)H, TT, true, hs::kLdsCap);
  s->lds_bytes_rank = L.total;
  s->sparse_rank = L.sparse;
  uint64_t tables = 0, rows = 0;
  for (const uint64_t b : {s->slot_tok_bytes, s->stamp_bytes, s->lru_order_bytes, s->page_bytes, s->step_bytes})
    tables += (b + 255) & ~255ull;
  for (const uint64_t b : {s->hot_bytes, s->tail_bytes}) rows += (b + 255) & ~255ull;
  s->state_tables_bytes = tables;
  s->state_rows_bytes = rows;
  s->lds_bytes_launch = lp.total;
  s->lds_bytes_launch_gather = lg.total;
  s->lds_bytes = std::max(lp.total, lg.total);
  s->token_slot_table = (lp.direct ? 1u : 0u) | (lg.direct ? 2u : 0u);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_ready(hs_ctx* ctx) {
  if (!ctx) return fail(HS_E_INVALID, "context is NULL");
  if (!ctx->bound) return fail(HS_E_STATE, "device buffers not bound (call hs_bind_device first)");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != ctx->device)
    return fail(HS_E_STATE, "the context belongs to device %d but device %d is current", ctx->device, dev);
  return HS_OK;
}

// A buffer handed to the kernels must be device (or managed) memory of the context's device.
int check_device_buffer(const hs_ctx* ctx, const void* p, const char* name) {
  hipPointerAttribute_t at{};
  hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(HS_E_INVALID, "buffer '%s' is not memory the HIP runtime knows (%s)", name, hipGetErrorString(e));
  }
  if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged)
    return fail(HS_E_INVALID, "buffer '%s' is not device memory", name);
  if (at.device != ctx->device)
    return fail(HS_E_INVALID, "buffer '%s' lives on device %d, the context on device %d", name, at.device, ctx->device);
  return HS_OK;
}

}  // namespace

extern "C" {

int hs_required_sizes(const hs_config* cfg, hs_sizes* out) {
  if (!out) return fail(HS_E_INVALID, "sizes output is NULL");
  int32_t H;
  hs::Layout L;
  int rc = check_config(cfg, &H, &L);
  if (rc) return rc;
  fill_sizes(cfg, H, L, out);
  return ok();
}

int hs_create(const hs_config* cfg, hs_ctx** out) {
  if (!out) return fail(HS_E_INVALID, "context output is NULL");
  *out = nullptr;
  int32_t H;
  hs::Layout L;
  int rc = check_config(cfg, &H, &L);
  if (rc) return rc;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int lds_max = 0;
  e = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(max shared memory per block)");
  // the device's own limit: a direct layout that does not fit under it falls back to the rank layout
  const uint32_t cap = std::min<uint32_t>(hs::kLdsCap, lds_max > 1024 ? (uint32_t)lds_max - 1024u : 0u);
  const hs::Layout lp = hs::launch_layout(cfg->top_k, cfg->device_buffer_size, (int)H, cfg->tail_tokens, false, cap);
  const hs::Layout lg = hs::launch_layout(cfg->top_k, cfg->device_buffer_size, (int)H, cfg->tail_tokens, true, cap);
  if (std::max(lp.total, lg.total) > cap)
    return fail(HS_E_INVALID, "this shape needs %u bytes of LDS per workgroup, the device allows %d",
                std::max(lp.total, lg.total), lds_max);
  // The cap on dynamic LDS is an attribute of the kernels, shared by every context on the device: set it to
  // the most any context may use, so a later context of a smaller shape cannot lower it under this one.
  e = hs::set_lds_limits(cap, cap);
  if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute(resolve kernel LDS)");
  {
    std::lock_guard<std::mutex> lock(g_static_plan_mu);
    if ((int)g_static_plan.size() <= dev) g_static_plan.resize((size_t)dev + 1, nullptr);
    if (!g_static_plan[(size_t)dev]) {
      void* p = nullptr;
      e = hs::static_plan_address(&p);
      if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(static plan)");
      g_static_plan[(size_t)dev] = p;
    }
  }

  hs_ctx* ctx = new (std::nothrow) hs_ctx();
  if (!ctx) return fail(HS_E_NOMEM, "out of host memory for the context");
  ctx->cfg = *cfg;
  ctx->H = H;
  ctx->layout = hs::rank_layout(cfg->top_k, cfg->device_buffer_size, (int)H, cap);
  ctx->layout_plain = lp;
  ctx->layout_gather = lg;
  ctx->layout_plain_direct = lp;
  ctx->layout_gather_direct = lg;
  ctx->lds_cap = cap;
  ctx->device = dev;
  ctx->pool_bytes = (uint64_t)cfg->num_requests * (uint64_t)H * (uint64_t)cfg->row_bytes;
  // Pinned host memory mapped into the GPU's address space; the resolve kernel reads missed rows
  // from it directly over the host link. Coherent: host writes made after a kernel has read the
  // pool are seen by later kernels.
  e = hipHostMalloc(&ctx->pool_host, ctx->pool_bytes, hipHostMallocMapped | hipHostMallocCoherent);
  if (e != hipSuccess || !ctx->pool_host) {
    (void)hipGetLastError();
    delete ctx;
    return fail(HS_E_NOMEM, "hipHostMalloc of a %llu-byte pinned host pool failed: %s",
                (unsigned long long)(cfg->num_requests * (uint64_t)H * (uint64_t)cfg->row_bytes),
                hipGetErrorString(e));
  }
  e = hipHostGetDevicePointer(&ctx->pool_dev, ctx->pool_host, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(ctx->pool_host);
    delete ctx;
    return hip_fail(e, "hipHostGetDevicePointer");
  }
  *out = ctx;
  return ok();
}

int hs_host_pool(hs_ctx* ctx, void** host_base, uint64_t* request_stride_bytes, int32_t* host_rows) {
  if (!ctx) return fail(HS_E_INVALID, "context is NULL");
  if (host_base) *host_base = ctx->pool_host;
  if (request_stride_bytes) *request_stride_bytes = (uint64_t)ctx->H * (uint64_t)ctx->cfg.row_bytes;
  if (host_rows) *host_rows = ctx->H;
  return ok();
}

int hs_bind_device(hs_ctx* ctx, const hs_device_views* v) {
  if (!ctx) return fail(HS_E_INVALID, "context is NULL");
  if (!v) return fail(HS_E_INVALID, "views are NULL");
  hs_sizes s;
  fill_sizes(&ctx->cfg, ctx->H, ctx->layout, &s);
  struct Need { const void* p; uint64_t have, need; const char* name; uintptr_t align; };
  const Need needs[] = {
      {v->hot, v->hot_bytes, s.hot_bytes, "hot", 16},
      {v->slot_tok, v->slot_tok_bytes, s.slot_tok_bytes, "slot_tok", 4},
      {v->stamp, v->stamp_bytes, s.stamp_bytes, "stamp", 4},
      {v->lru_order, v->lru_order_bytes, s.lru_order_bytes, "lru_order", 2},
      {v->page, v->page_bytes, s.page_bytes, "page", 4},
      {v->step, v->step_bytes, s.step_bytes, "step", 4},
      {v->epoch, v->epoch_bytes, s.epoch_bytes, "epoch", 4},
  };
  for (const Need& n : needs) {
    if (!n.p) return fail(HS_E_INVALID, "device buffer '%s' is NULL", n.name);
    if (n.have < n.need)
      return fail(HS_E_INVALID, "device buffer '%s' has %llu bytes, needs %llu", n.name, (unsigned long long)n.have,
                  (unsigned long long)n.need);
    if (!aligned(n.p, n.align)) return fail(HS_E_INVALID, "device buffer '%s' is not %d-byte aligned", n.name,
                                             (int)n.align);
    const int rc = check_device_buffer(ctx, n.p, n.name);
    if (rc) return rc;
  }
  if (ctx->cfg.tail_tokens > 0) {
    if (!v->tail) return fail(HS_E_INVALID, "device buffer 'tail' is NULL but tail_tokens = %d", ctx->cfg.tail_tokens);
    if (v->tail_bytes < s.tail_bytes)
      return fail(HS_E_INVALID, "device buffer 'tail' has %llu bytes, needs %llu", (unsigned long long)v->tail_bytes,
                  (unsigned long long)s.tail_bytes);
    if (!aligned(v->tail, 16)) return fail(HS_E_INVALID, "device buffer 'tail' is not 16-byte aligned");
    const int rc = check_device_buffer(ctx, v->tail, "tail");
    if (rc) return rc;
  }
  // The direct kernel reads and writes each request's slot table and stamps in 16-byte pieces and its order
  // list in 8-byte ones: with tables less aligned than that, launches take the rank layout.
  const bool tables16 = aligned(v->slot_tok, 16) && aligned(v->stamp, 16) && aligned(v->lru_order, 8);
  hs::Layout lp = ctx->layout_plain_direct, lg = ctx->layout_gather_direct;
  if (!tables16) {
    if (lp.direct) lp = ctx->layout;
    if (lg.direct) lg = ctx->layout;
    if (std::max(lp.total, lg.total) > ctx->lds_cap)
      return fail(HS_E_INVALID, "this shape needs 16-byte aligned slot_tok and stamp and an 8-byte aligned "
                                "lru_order (its rank layout does not fit in LDS)");
  }
  ctx->layout_plain = lp;
  ctx->layout_gather = lg;
  ctx->views = *v;
  ctx->bound = true;
  return ok();
}

int hs_reset(hs_ctx* ctx, const int32_t* d_request_ids, int32_t n, void* stream) {
  int rc = check_ready(ctx);
  if (rc) return rc;
  int blocks;
  if (d_request_ids) {
    if (n < 0) return fail(HS_E_INVALID, "n must be >= 0 when request ids are given (got %d)", n);
    blocks = n;
  } else {
    if (n >= 0) return fail(HS_E_INVALID, "request ids are NULL: pass n < 0 to reset every request");
    blocks = ctx->cfg.num_requests;
  }
  hs::ResetArgs a{};
  a.R = ctx->cfg.num_requests;
  a.B = ctx->cfg.device_buffer_size;
  a.H = ctx->H;
  a.ids = d_request_ids;
  a.slot_tok = ctx->views.slot_tok;
  a.stamp = ctx->views.stamp;
  a.order = ctx->views.lru_order;
  a.page = ctx->views.page;
  a.step = ctx->views.step;
  a.epoch = ctx->views.epoch;
  hipError_t e = hs::launch_reset(a, blocks, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reset launch");
  return ok();
}

}  // extern "C"

namespace {

int resolve_common(hs_ctx* ctx, const int32_t* d_topk, const int32_t* d_tail0, int32_t* d_out, int32_t* d_miss,
                   int32_t* d_status, void* d_gather, int32_t* d_plan, int32_t plan_flags, int32_t* d_trial,
                   void* stream) {
  int rc = check_ready(ctx);
  if (rc) return rc;
  if (!d_topk || !d_out || !d_miss || !d_status)
    return fail(HS_E_INVALID, "topk, out, miss and status must not be NULL");
  if (d_gather && !aligned(d_gather, 16)) return fail(HS_E_INVALID, "gather output is not 16-byte aligned");
  if (ctx->cfg.tail_tokens == 0 && d_tail0)
    return fail(HS_E_INVALID, "tail0 given but the context has no tail (tail_tokens = 0)");
  hs::ResolveArgs a{};
  a.R = ctx->cfg.num_requests;
  a.k = ctx->cfg.top_k;
  a.B = ctx->cfg.device_buffer_size;
  a.H = ctx->H;
  a.T = ctx->cfg.tail_tokens;
  a.row16 = ctx->cfg.row_bytes / 16;
  a.policy = ctx->cfg.eviction_policy;
  // fused row copy: about 128K 16-byte host loads in flight over the whole chip saturate the host link
  // (measured: more in flight only queues); at most 1024 threads per request, then up to 4 loads each
  {
    const int per_request = (131072 + a.R - 1) / a.R;
    a.copy_threads = per_request < 256 ? 256 : per_request > hs::kThreads ? hs::kThreads : per_request;
    const int u = (per_request + hs::kThreads - 1) / hs::kThreads;
    a.copy_unroll = u <= 1 ? 1 : u == 2 ? 2 : 4;
  }
  a.L = d_gather ? ctx->layout_gather : ctx->layout_plain;
  a.host = (const hs::v4u*)ctx->pool_dev;
  a.hot = (hs::v4u*)ctx->views.hot;
  a.tail = (const hs::v4u*)ctx->views.tail;
  a.slot_tok = ctx->views.slot_tok;
  a.stamp = ctx->views.stamp;
  a.order = ctx->views.lru_order;
  a.page = ctx->views.page;
  a.step = ctx->views.step;
  a.topk = d_topk;
  a.tail0 = d_tail0;
  a.out = d_out;
  a.miss = d_miss;
  a.status = d_status;
  a.gather = (hs::v4u*)d_gather;
  a.plan = d_plan;
  a.plan_sources = (plan_flags & HS_PLAN_ROW_SOURCES) ? 1 : 0;
  a.trial = d_trial;
  a.epoch = ctx->views.epoch;
  a.trial_words = hs::trial_words(a.k, a.B);
  if (d_trial && !aligned(d_trial, 16)) return fail(HS_E_INVALID, "trial buffer is not 16-byte aligned");
  hipError_t e = hs::launch_resolve(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, d_trial ? "trial launch" : d_plan ? "plan launch" : "resolve launch");
  return ok();
}

}  // namespace

extern "C" {

int hs_resolve(hs_ctx* ctx, const int32_t* d_topk, const int32_t* d_tail0, int32_t* d_out, int32_t* d_miss,
               int32_t* d_status, void* d_gather, void* stream) {
  return resolve_common(ctx, d_topk, d_tail0, d_out, d_miss, d_status, d_gather, nullptr, 0, nullptr, stream);
}

int hs_plan(hs_ctx* ctx, const int32_t* d_topk, const int32_t* d_tail0, int32_t* d_out, int32_t* d_miss,
            int32_t* d_status, int32_t* d_plan, int32_t flags, void* stream) {
  if (!d_plan) return fail(HS_E_INVALID, "plan buffer must not be NULL");
  if (flags & ~HS_PLAN_ROW_SOURCES) return fail(HS_E_INVALID, "unknown plan flags 0x%x", (unsigned)flags);
  return resolve_common(ctx, d_topk, d_tail0, d_out, d_miss, d_status, nullptr, d_plan, flags, nullptr, stream);
}

int hs_trial(hs_ctx* ctx, const int32_t* d_topk, const int32_t* d_tail0, int32_t* d_out, int32_t* d_miss,
             int32_t* d_status, void* d_gather, int32_t* d_trial, void* stream) {
  if (!d_trial || !d_gather) return fail(HS_E_INVALID, "trial and gather buffers must not be NULL");
  return resolve_common(ctx, d_topk, d_tail0, d_out, d_miss, d_status, d_gather, nullptr, 0, d_trial, stream);
}

int hs_commit(hs_ctx* ctx, const int32_t* d_trial, const void* d_gather, const int32_t* d_accept, int32_t* d_status,
              void* stream) {
  int rc = check_ready(ctx);
  if (rc) return rc;
  if (!d_trial || !d_gather) return fail(HS_E_INVALID, "trial and gather buffers must not be NULL");
  if (!aligned(d_gather, 16) || !aligned(d_trial, 16))
    return fail(HS_E_INVALID, "trial and gather buffers must be 16-byte aligned");
  hs::CommitArgs a{};
  a.R = ctx->cfg.num_requests;
  a.k = ctx->cfg.top_k;
  a.B = ctx->cfg.device_buffer_size;
  a.H = ctx->H;
  a.row16 = ctx->cfg.row_bytes / 16;
  a.trial_words = hs::trial_words(a.k, a.B);
  a.trial = d_trial;
  a.accept = d_accept;
  a.epoch = ctx->views.epoch;
  a.gather = (const hs::v4u*)d_gather;
  a.status = d_status;
  a.hot = (hs::v4u*)ctx->views.hot;
  a.slot_tok = ctx->views.slot_tok;
  a.stamp = ctx->views.stamp;
  a.order = ctx->views.lru_order;
  a.page = ctx->views.page;
  a.step = ctx->views.step;
  hipError_t e = hs::launch_commit(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "commit launch");
  return ok();
}

int hs_copy(hs_ctx* ctx, const int32_t* d_plan, const int32_t* d_miss, void* d_gather, void* stream) {
  int rc = check_ready(ctx);
  if (rc) return rc;
  if (!d_plan || !d_miss) return fail(HS_E_INVALID, "plan and miss must not be NULL");
  if (d_gather && !aligned(d_gather, 16)) return fail(HS_E_INVALID, "gather output is not 16-byte aligned");
  hs::CopyArgs a{};
  a.R = ctx->cfg.num_requests;
  a.k = ctx->cfg.top_k;
  a.B = ctx->cfg.device_buffer_size;
  a.H = ctx->H;
  a.T = ctx->cfg.tail_tokens;
  a.row16 = ctx->cfg.row_bytes / 16;
  a.rows = std::max(1, hs::kGatherChunks / a.row16);
  a.workgroups = hs::kCopyWorkgroups;
  a.plan = d_plan;
  a.miss = d_miss;
  a.host = (const hs::v4u*)ctx->pool_dev;
  a.hot = (hs::v4u*)ctx->views.hot;
  a.tail = (const hs::v4u*)ctx->views.tail;
  a.gather = (hs::v4u*)d_gather;
  a.page = ctx->views.page;
  hipError_t e = hs::launch_copy(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "copy launch");
  return ok();
}

int hs_step_static(hs_ctx* ctx, const int32_t* d_topk, const int32_t* d_tail0, int32_t* d_out, int32_t* d_miss,
                   int32_t* d_status, void* d_gather, void* stream) {
  int rc = check_ready(ctx);
  if (rc) return rc;
  const uint64_t need = (uint64_t)ctx->cfg.num_requests * 4ull * (uint64_t)ctx->cfg.top_k * 4ull;
  if (need > hs::kStaticPlanBytes)
    return fail(HS_E_INVALID,
                "the plan of %d requests x top_k %d takes %llu bytes, more than the %llu of the static plan; use "
                "hs_plan and hs_copy with a plan buffer",
                ctx->cfg.num_requests, ctx->cfg.top_k, (unsigned long long)need,
                (unsigned long long)hs::kStaticPlanBytes);
  void* plan = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_static_plan_mu);
    if ((size_t)ctx->device < g_static_plan.size()) plan = g_static_plan[(size_t)ctx->device];
  }
  if (!plan) return fail(HS_E_STATE, "no static plan address for device %d", ctx->device);
  if (d_gather && !aligned(d_gather, 16)) return fail(HS_E_INVALID, "gather output is not 16-byte aligned");
  rc = resolve_common(ctx, d_topk, d_tail0, d_out, d_miss, d_status, nullptr, (int32_t*)plan,
                      d_gather ? HS_PLAN_ROW_SOURCES : 0, nullptr, stream);
  if (rc) return rc;
  return hs_copy(ctx, (const int32_t*)plan, d_miss, d_gather, stream);
}

int hs_gather(hs_ctx* ctx, const int32_t* d_out, void* d_gather, void* stream) {
  int rc = check_ready(ctx);
  if (rc) return rc;
  if (!d_out || !d_gather) return fail(HS_E_INVALID, "out and gather must not be NULL");
  if (!aligned(d_gather, 16)) return fail(HS_E_INVALID, "gather output is not 16-byte aligned");
  hs::GatherArgs a{};
  a.R = ctx->cfg.num_requests;
  a.k = ctx->cfg.top_k;
  a.B = ctx->cfg.device_buffer_size;
  a.T = ctx->cfg.tail_tokens;
  a.row16 = ctx->cfg.row_bytes / 16;
  a.rows = std::max(1, hs::kGatherChunks / a.row16);
  a.out = d_out;
  a.hot = (const hs::v4u*)ctx->views.hot;
  a.tail = (const hs::v4u*)ctx->views.tail;
  a.gather = (hs::v4u*)d_gather;
  hipError_t e = hs::launch_gather(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return ok();
}

int hs_offload(hs_ctx* ctx, const void* d_rows, const int32_t* d_pos, int32_t n, int32_t* d_status, void* stream) {
  int rc = check_ready(ctx);
  if (rc) return rc;
  if (n < 0) return fail(HS_E_INVALID, "n must be >= 0 (got %d)", n);
  if (n > 0 && (!d_rows || !d_pos)) return fail(HS_E_INVALID, "rows and pos must not be NULL");
  if (d_rows && !aligned(d_rows, 16)) return fail(HS_E_INVALID, "rows are not 16-byte aligned");
  if ((int64_t)n * (ctx->cfg.row_bytes / 16) > INT32_MAX) return fail(HS_E_INVALID, "n is too large");
  hs::OffloadArgs a{};
  a.R = ctx->cfg.num_requests;
  a.B = ctx->cfg.device_buffer_size;
  a.H = ctx->H;
  a.row16 = ctx->cfg.row_bytes / 16;
  a.n = n;
  a.rows = (const hs::v4u*)d_rows;
  a.pos = d_pos;
  a.status = d_status;
  a.host = (hs::v4u*)ctx->pool_dev;
  a.hot = (hs::v4u*)ctx->views.hot;
  a.page = ctx->views.page;
  a.epoch = ctx->views.epoch;
  hipError_t e = hs::launch_offload(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "offload launch");
  return ok();
}

int hs_advance_tail(hs_ctx* ctx, int32_t* d_tail0, const int32_t* d_n, int32_t* d_status, void* stream) {
  int rc = check_ready(ctx);
  if (rc) return rc;
  if (ctx->cfg.tail_tokens == 0) return fail(HS_E_INVALID, "the context has no device tail (tail_tokens = 0)");
  if (!d_tail0 || !d_n) return fail(HS_E_INVALID, "tail0 and n must not be NULL");
  hs::AdvanceTailArgs a{};
  a.R = ctx->cfg.num_requests;
  a.B = ctx->cfg.device_buffer_size;
  a.H = ctx->H;
  a.T = ctx->cfg.tail_tokens;
  a.row16 = ctx->cfg.row_bytes / 16;
  a.tail0 = d_tail0;
  a.n = d_n;
  a.status = d_status;
  a.tail = (const hs::v4u*)ctx->views.tail;
  a.host = (hs::v4u*)ctx->pool_dev;
  a.hot = (hs::v4u*)ctx->views.hot;
  a.page = ctx->views.page;
  a.epoch = ctx->views.epoch;
  hipError_t e = hs::launch_advance_tail(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "advance-tail launch");
  return ok();
}

int hs_rebuild_order(hs_ctx* ctx, void* stream) {
  int rc = check_ready(ctx);
  if (rc) return rc;
  hs::RebuildArgs a{};
  a.R = ctx->cfg.num_requests;
  a.B = ctx->cfg.device_buffer_size;
  a.stamp = ctx->views.stamp;
  a.order = ctx->views.lru_order;
  hipError_t e = hs::launch_rebuild_order(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rebuild-order launch");
  return ok();
}

}  // extern "C"

namespace {

// The sections of a state snapshot, in their order, each at a 256-byte aligned offset: what they hold on the
// device, their size, and whether they are tables (HS_STATE_TABLES) or rows (HS_STATE_ROWS).
struct Section { void* dev; uint64_t bytes; uint32_t kind; };

int state_sections(hs_ctx* ctx, uint32_t what, Section* sec, int* n, uint64_t* total) {
  if (what == 0 || (what & ~(uint32_t)(HS_STATE_TABLES | HS_STATE_ROWS)))
    return fail(HS_E_INVALID, "what must be HS_STATE_TABLES, HS_STATE_ROWS or both (got 0x%x)", (unsigned)what);
  hs_sizes s;
  fill_sizes(&ctx->cfg, ctx->H, ctx->layout, &s);
  const hs_device_views& v = ctx->views;
  const Section all[] = {
      {v.slot_tok, s.slot_tok_bytes, HS_STATE_TABLES}, {v.stamp, s.stamp_bytes, HS_STATE_TABLES},
      {v.lru_order, s.lru_order_bytes, HS_STATE_TABLES}, {v.page, s.page_bytes, HS_STATE_TABLES},
      {v.step, s.step_bytes, HS_STATE_TABLES}, {v.hot, s.hot_bytes, HS_STATE_ROWS},
      {v.tail, s.tail_bytes, HS_STATE_ROWS},
  };
  *n = 0;
  *total = 0;
  for (const Section& x : all) {
    if (!(x.kind & what)) continue;
    sec[(*n)++] = x;
    *total += (x.bytes + 255) & ~255ull;
  }
  return HS_OK;
}

int copy_state(hs_ctx* ctx, void* snap, uint64_t snap_bytes, uint32_t what, bool to_snapshot, void* stream) {
  int rc = check_ready(ctx);
  if (rc) return rc;
  if (!snap) return fail(HS_E_INVALID, "snapshot buffer is NULL");
  Section sec[7];
  int n = 0;
  uint64_t total = 0;
  rc = state_sections(ctx, what, sec, &n, &total);
  if (rc) return rc;
  if (snap_bytes < total)
    return fail(HS_E_INVALID, "snapshot buffer has %llu bytes, needs %llu", (unsigned long long)snap_bytes,
                (unsigned long long)total);
  if (!aligned(snap, 256)) return fail(HS_E_INVALID, "snapshot buffer is not 256-byte aligned");
  rc = check_device_buffer(ctx, snap, "snapshot");
  if (rc) return rc;
  uint64_t off = 0;
  for (int i = 0; i < n; ++i) {
    if (sec[i].bytes) {
      char* p = static_cast<char*>(snap) + off;
      hipError_t e = to_snapshot
                         ? hipMemcpyAsync(p, sec[i].dev, sec[i].bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream)
                         : hipMemcpyAsync(sec[i].dev, p, sec[i].bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync of a state section");
    }
    off += (sec[i].bytes + 255) & ~255ull;
  }
  if (!to_snapshot) {
    hipError_t e = hs::launch_bump_epoch(ctx->views.epoch, ctx->cfg.num_requests, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "epoch launch");
  }
  return ok();
}

}  // namespace

extern "C" {

int hs_export_state(hs_ctx* ctx, void* d_dst, uint64_t dst_bytes, uint32_t what, void* stream) {
  return copy_state(ctx, d_dst, dst_bytes, what, true, stream);
}

int hs_import_state(hs_ctx* ctx, const void* d_src, uint64_t src_bytes, uint32_t what, void* stream) {
  return copy_state(ctx, const_cast<void*>(d_src), src_bytes, what, false, stream);
}

void hs_destroy(hs_ctx* ctx) {
  if (!ctx) return;
  if (ctx->pool_host) (void)hipHostFree(ctx->pool_host);
  delete ctx;
}

const char* hs_last_error(void) { return g_err; }

}  // extern "C"
