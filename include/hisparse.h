/*
 * hisparse.h — C ABI of the HiSparse swap-in path on MI355X (gfx950).
 *
 * The swap-in step, per request and decode step, as the pages describe it
 * ("HiSparse: Turbocharging Sparse Attention with Hierarchical Memory",
 * section 2, the swap-in kernel; 「HiSparse：階層化メモリシステムによる
 * スパースアテンションの加速」, section 「効率的なSwap-inカーネル」):
 *   (1) find which of the top-k selected KV tokens miss the hot device buffer,
 *   (2) choose LRU eviction victims,
 *   (3) update the page table and fetch the missed rows from host memory.
 * The hybrid variant ("vLLM GLM 5.3 最適化: Hybrid HiSparse オフローディング",
 * section 2 Mixed Residency) adds a device-resident tail whose tokens resolve
 * in place, and a fused gather of every selected row.
 *
 * Rules fixed by this library where the pages say only "LRU":
 *   - eviction candidates are the slots not hit this step, taken in ascending
 *     (last-use step, slot index); an empty slot has last-use step -1;
 *   - the j-th smallest missed token id takes the j-th victim;
 *   - hit slots and newly filled slots get last-use step = the request's step.
 *
 * Memory and ownership
 *   - The library owns the host KV pool: pinned, mapped host memory of
 *     num_requests x host_rows x row_bytes bytes, request-major. The caller
 *     fills it (hs_host_pool) before resolving.
 *   - The caller owns every device buffer (hs_device_views) and the stream.
 *     Device buffers are plain device pointers; the library checks their sizes
 *     against the configuration and never frees them.
 *   - A context is not thread-safe. All device work of a call is enqueued on
 *     the given stream (NULL = the default stream) and the call returns without
 *     waiting for it: hs_resolve and hs_gather never synchronise with the host
 *     and keep the step counters on the device, so a captured HIP graph can
 *     replay them.
 *
 * Errors
 *   - Every int-returning call returns HS_OK (0) or a negative HS_E_* code
 *     after synchronous host-side checks; hs_last_error() then describes it.
 *   - Bad data found on the device (ids out of range, repeated ids, a corrupt
 *     state table) never traps: it sets bits in the per-request status output
 *     and the affected entries resolve to -1.
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HS_OK 0
#define HS_E_INVALID (-1) /* bad argument: null pointer, size out of range, buffer too small, B < k ... */
#define HS_E_NOMEM (-2)   /* the pinned host pool could not be allocated */
#define HS_E_HIP (-3)     /* a HIP runtime call failed (no device, launch failure, attribute) */
#define HS_E_STATE (-4)   /* call out of order (e.g. resolve before hs_bind_device), or made while another
                             device than the context's is current */

/* Per-request status bits written by hs_resolve. */
#define HS_STATUS_BAD_ID 1    /* an id outside [0, host_rows), or >= tail0 but outside the tail window */
#define HS_STATUS_DUP_ID 2    /* an id repeated within the request's selection (first occurrence wins) */
#define HS_STATUS_BAD_STATE 4 /* the request's slot table or LRU order held an impossible value: nothing
                                 was changed for this request and every output is -1 */
#define HS_STATUS_STALE 8     /* hs_commit: the request changed since the trial (another step, a reset, an
                                 offload, a tail advance or an imported state); it was not applied */

/*
 * Configuration. top_k, device_buffer_size and host_to_device_ratio are the
 * three keys of the HiSparse launch configuration printed on the pages
 * (「HiSparse：階層化メモリシステムによるスパースアテンションの加速」, section
 * 「ベンチマークテスト」, and "HiSparse: Turbocharging Sparse Attention with
 * Hierarchical Memory", section 3 launch scripts: top_k 2048,
 * device_buffer_size 4096 or 6144, host_to_device_ratio 8 or 10).
 * Beyond the per-field ranges, a shape is accepted only if one resolve
 * workgroup's LDS fits in 159 KiB for launches with and without a gather
 * output, and the host pool (R x H x row_bytes) in 2^56 bytes;
 * hs_required_sizes and hs_create return HS_E_INVALID otherwise. A launch
 * takes one of two layouts. Where a uint16 token -> slot entry for each of
 * the H host rows fits (the direct layout: about 8k + 5B + T / 8 +
 * 6 * ceil(H / 32) + max(2H, 6 * ceil(H / 32) + 4k, 4k + 2B) bytes, 4k more
 * with a gather output, and B <= 8192), it tests each selected id against the
 * slot table directly.
 * Elsewhere it ranks the selected ids in bitmaps over token ids (the rank
 * layout: about 21k + 7B + 10 * ceil(H / 32) bytes, plus 4k more where that
 * still fits, which saves the kernel a pass; at k = 2048 and B = 4096 that
 * allows about 290,000 host rows). Past that the same ranks run over compact
 * ids: a coarse bitmap with one bit per 32 host rows numbers the 32-row words
 * that hold a selected id, and the bitmaps cover only those words (the sparse
 * rank layout: about 39k + 7B + 6 * ceil(H / 1024) bytes; at k = 2048 and
 * B = 4096 up to about 10.5 million host rows). hs_sizes reports the bytes of
 * each and which rank layout the shape takes.
 */
typedef struct hs_config {
  int32_t num_requests;       /* R, 1 .. 65535 */
  int32_t top_k;              /* k, 1 .. 8192: selected ids per request and step */
  int32_t device_buffer_size; /* B, k .. 65535: hot slots per request (B >= k so a step never runs out) */
  float host_to_device_ratio; /* host rows per request = ceil(ratio * B) when max_context == 0 */
  int32_t row_bytes;          /* bytes per KV row, a positive multiple of 16 (576 bf16 = 1152) */
  int32_t max_context;        /* > 0: host rows per request (overrides the ratio) */
  int32_t tail_tokens;        /* T >= 0: device-resident tail rows per request (Mixed residency) */
  int32_t eviction_policy;    /* HS_EVICT_LRU (default) or HS_EVICT_FIFO */
} hs_config;

/*
 * Eviction policies. LRU is the method's ("HiSparse: Turbocharging Sparse Attention with Hierarchical
 * Memory", section 2). The pages compare it with another strategy they do not name; FIFO is offered as
 * that alternative: victims are taken the same way, but a hit does not refresh its slot's stamp, so a
 * slot's stamp is the step it was filled.
 */
#define HS_EVICT_LRU 0
#define HS_EVICT_FIFO 1

/*
 * Device buffers (caller-owned). Sizes are in bytes and must be at least what
 * hs_required_sizes reports; pointers must be 16-byte aligned (hot, tail,
 * gather output) or 4-byte aligned (tables). H = host rows per request.
 * The tables are written by the library; a caller that writes them itself
 * (hs_import_state aside) must leave a consistent state, and must not then
 * commit a trial made before the write. Out-of-range
 * entries are caught (HS_STATUS_BAD_STATE); a slot table holding one token in
 * two slots is not: a step that selects that token reports either slot.
 */
typedef struct hs_device_views {
  void* hot;            uint64_t hot_bytes;       /* [R][B][row_bytes] hot buffer rows */
  void* tail;           uint64_t tail_bytes;      /* [R][T][row_bytes] resident tail ring (token x in row
                                                     x mod T); NULL when T == 0 */
  int32_t* slot_tok;    uint64_t slot_tok_bytes;  /* [R][B] token held by each slot, -1 = empty */
  int32_t* stamp;       uint64_t stamp_bytes;     /* [R][B] last-use step of each slot, -1 = empty */
  uint16_t* lru_order;  uint64_t lru_order_bytes; /* [R][B] slots in ascending (stamp, slot) (library-maintained) */
  int32_t* page;        uint64_t page_bytes;      /* [R][H] slot of each token, -1 = not in the hot buffer */
  int32_t* step;        uint64_t step_bytes;      /* [R] step counter of each request */
  int32_t* epoch;       uint64_t epoch_bytes;     /* [R] change counter of each request (library-maintained, any
                                                     initial contents): hs_reset, hs_offload, hs_advance_tail and
                                                     hs_import_state advance it; hs_commit refuses a trial made
                                                     under another value */
} hs_device_views;

typedef struct hs_sizes {
  int32_t host_rows;         /* H */
  uint64_t host_pool_bytes;  /* R * H * row_bytes */
  uint64_t hot_bytes, tail_bytes, slot_tok_bytes, stamp_bytes, lru_order_bytes, page_bytes, step_bytes;
  uint64_t topk_bytes;       /* [R][k] int32 input of one step */
  uint64_t out_bytes;        /* [R][k] int32 output of one step */
  uint64_t gather_bytes;     /* [R][k][row_bytes] gather output */
  uint64_t plan_bytes;       /* [R][4][k] int32 plan of hs_plan (miss list, evicted tokens, row sources) */
  uint64_t trial_bytes;      /* trial records of hs_trial / hs_commit */
  uint32_t lds_bytes;        /* LDS a resolve workgroup of this shape takes at most (the larger of the two below) */
  uint32_t lds_bytes_launch;        /* LDS a resolve / plan launch without a gather output takes (device
                                       allowing 159 KiB): the direct layout where it fits, else the rank layout */
  uint32_t lds_bytes_launch_gather; /* the same for a launch with a gather output (fused gather, trial) */
  uint32_t token_slot_table;        /* bit 0: launches without a gather output use the direct layout;
                                       bit 1: launches with one do */
  uint32_t lds_bytes_rank;          /* LDS of the rank layout of this shape (whether or not launches take it) */
  uint32_t sparse_rank;             /* 1: that rank layout is the two-level one (contexts past the flat
                                       bitmaps' LDS) */
  uint64_t epoch_bytes;             /* [R] int32 change counters */
  uint64_t state_tables_bytes;      /* snapshot of the tables (HS_STATE_TABLES), see hs_export_state */
  uint64_t state_rows_bytes;        /* snapshot of the hot and tail rows (HS_STATE_ROWS) */
} hs_sizes;

typedef struct hs_ctx hs_ctx;

/* Sizes every buffer needs for cfg. Host-only; validates cfg like hs_create. */
int hs_required_sizes(const hs_config* cfg, hs_sizes* out);

/* Validate cfg, allocate the pinned mapped host pool on the current HIP device
 * (contents undefined until the caller fills it) and return a context. The context belongs to that device:
 * every later call on it must be made while the same device is current (else HS_E_STATE). */
int hs_create(const hs_config* cfg, hs_ctx** out);

/* Host address of the pool: request r's row x starts at
 * host_base + r * request_stride_bytes + x * row_bytes. */
int hs_host_pool(hs_ctx* ctx, void** host_base, uint64_t* request_stride_bytes, int32_t* host_rows);

/* Register the caller's device buffers. Each must be device (or managed) memory of the context's device,
 * at least the size hs_required_sizes gives and aligned to its element (16 bytes for hot and tail);
 * HS_E_INVALID names the first that is not. Must precede reset/resolve/gather. The per-call device
 * buffers (ids, outputs, plans, trial records, gather outputs) are not checked this way: they must be
 * device memory of the same device too. */
int hs_bind_device(hs_ctx* ctx, const hs_device_views* views);

/* Reset requests to the empty state: slot table, stamps and page table -1, LRU order = slot order,
 * step 0. Hot rows are left as they are. d_request_ids: device int32[n]; NULL with n < 0 resets all.
 * Ids outside [0, R) are skipped. */
int hs_reset(hs_ctx* ctx, const int32_t* d_request_ids, int32_t n, void* stream);

/*
 * One decode step for every request (one workgroup per request).
 *   d_topk    [R][k] int32: selected token ids; -1 = padding.
 *   d_tail0   [R] int32 or NULL: first device-resident token of each request; a token x with
 *             tail0 <= x < tail0 + T resolves to B + (x mod T) and takes no slot. The device tail is a
 *             ring of T rows per request: token x of the window [tail0, tail0 + T) is in row x mod T.
 *   d_out     [R][k] int32: slot of each id (hit or newly filled), B + tail row for a resident id,
 *             -1 for padding or a bad id.
 *   d_miss    [R] int32: misses (rows fetched from the host pool) of each request.
 *   d_status  [R] int32: HS_STATUS_* bits of this step.
 *   d_gather  [R][k][row_bytes] or NULL: when given, row i of request r receives the row d_out names
 *             (hot slot, tail row, or the fetched row); zeros for -1 (fused resolve + gather).
 * Inputs must not alias outputs or state.
 */
int hs_resolve(hs_ctx* ctx, const int32_t* d_topk, const int32_t* d_tail0, int32_t* d_out, int32_t* d_miss,
               int32_t* d_status, void* d_gather, void* stream);

/*
 * The same step split in two, so the row copy can overlap other work: the pages name better overlap of
 * the swap-in I/O as the way to cut its cost ("HiSparse: Turbocharging Sparse Attention with Hierarchical
 * Memory", section 4 future work; 「HiSparse：階層化メモリシステムによるスパースアテンションの加速」, section
 * 「今後の展望」).
 * hs_plan makes every decision of the step: outputs, slot table, stamps, LRU order and step counters are
 * final when it completes. d_plan [R][4][k] int32 receives, for request r, the missed tokens in ascending id
 * order (d_plan[r][0][0..m)), their slots (d_plan[r][1][0..m)), the tokens those slots held before (d_plan[r][2]
 * [0..m), -1 for an empty slot) and, with flags HS_PLAN_ROW_SOURCES, for every position i of the selection,
 * where its row is (d_plan[r][3][i]: a slot in [0, B), B + a tail row, -1 for none, or -2 - j for the j-th
 * miss); without it d_plan[r][3] is not written. Unknown flag bits are refused (HS_E_INVALID).
 * hs_copy then moves the rows and publishes the step in the page table: each missed row is copied from the
 * host pool into its slot, the evicted tokens' page entries become -1 and the missed tokens' entries their
 * slots (the page table is not read on the decode path, so its scattered updates ride with the link-bound
 * copy instead of the plan). Without d_gather the copy runs on a bounded grid of 128 one-wave workgroups,
 * which holds the host link's rate and leaves the compute units to work on other streams (with fewer requests
 * than workgroups, the step's missed rows are shared out evenly over them). With d_gather (nullable,
 * [R][k][row_bytes], 16-byte aligned) it also writes every selected row there, as hs_resolve's fused gather
 * does, in workgroups spread over the whole chip (the missed rows straight from the host pool, and into their
 * slots from the positions that gather them); that needs a plan made with HS_PLAN_ROW_SOURCES (with another
 * plan the gathered rows and the new slots' rows are undefined, never an access out of bounds; the page table
 * and every other table are still exact).
 * hs_copy reads d_plan and d_miss as hs_plan left them: on another stream it must be ordered after the plan
 * (an event recorded after hs_plan, waited on by the copy's stream). Until hs_copy completes, the hot rows of
 * this step's new slots are stale and the page table does not show the step. Two plans may run back to back,
 * but the copy of a step must complete before the copy of the next step and before any call other than
 * hs_plan reads or writes the context's state.
 */
#define HS_PLAN_ROW_SOURCES 1 /* hs_plan flag: also record each position's row source (for a gathering hs_copy) */
int hs_plan(hs_ctx* ctx, const int32_t* d_topk, const int32_t* d_tail0, int32_t* d_out, int32_t* d_miss,
            int32_t* d_status, int32_t* d_plan, int32_t flags, void* stream);
int hs_copy(hs_ctx* ctx, const int32_t* d_plan, const int32_t* d_miss, void* d_gather, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the split step, hs_plan then hs_copy (with HS_PLAN_ROW_SOURCES when d_gather is
 * given), in one call whose plan lives in the library's own static device array instead of a caller's plan
 * buffer. Arguments and results are those of hs_resolve (d_gather nullable). The array holds HS_STATIC_PLAN_BYTES
 * per device, kept until the process ends and shared by every call on that device: a context whose plan
 * (R x 4 x top_k int32) is larger is refused with HS_E_INVALID, and calls that overlap on one device (other
 * streams, other threads, other contexts) race. The array keeps the last call's plan; nothing in it has to
 * start at zero. Allocates nothing.
 */
#define HS_STATIC_PLAN_BYTES (8u << 20)
int hs_step_static(hs_ctx* ctx, const int32_t* d_topk, const int32_t* d_tail0, int32_t* d_out, int32_t* d_miss,
                   int32_t* d_status, void* d_gather, void* stream);

/*
 * A retryable step, for speculative decoding: the vLLM page names a per-step resolver plan that can be
 * retried and shares the request's hot state ("vLLM GLM 5.3 最適化: Hybrid HiSparse オフローディング",
 * section vLLM エコシステムとの統合).
 * hs_trial resolves a step exactly as hs_resolve would (same d_out, d_miss, d_status) but changes no state
 * at all: no table, stamp, step counter or hot row. Every selected row goes to d_gather
 * [R][k][row_bytes] (required), missed rows straight from the host pool, so the step can be verified
 * from d_gather. d_trial (hs_sizes.trial_bytes, 16-byte aligned) receives one record per request.
 * hs_commit applies the records of the requests with d_accept[r] != 0 (all when d_accept is NULL): LRU
 * order, stamps, slot and page tables, step counter, and the missed rows copied from d_gather into their
 * victim slots (HBM to HBM). Requests not accepted keep their state, so a trial is rolled back by not
 * committing it and retried by calling hs_trial again. A record made at another step than the request's
 * current one, or before a reset, offload, tail advance or state import of that request (the change counter
 * in hs_device_views.epoch differs), is not applied and sets HS_STATUS_STALE in d_status[r] (optional, [R]).
 * d_gather must still hold what hs_trial wrote.
 */
int hs_trial(hs_ctx* ctx, const int32_t* d_topk, const int32_t* d_tail0, int32_t* d_out, int32_t* d_miss,
             int32_t* d_status, void* d_gather, int32_t* d_trial, void* stream);
int hs_commit(hs_ctx* ctx, const int32_t* d_trial, const void* d_gather, const int32_t* d_accept, int32_t* d_status,
              void* stream);

/*
 * Offload of device rows to the host pool: HiSparse keeps inactive KV in host memory and only a hot buffer
 * on the GPU (「HiSparse：階層化メモリシステムによるスパースアテンションの加速」, section 「HiSparseの設計」;
 * "HiSparse: Turbocharging Sparse Attention with Hierarchical Memory", section 2), and the vLLM variant
 * copies finished prefix pages to host memory ahead of eviction ("vLLM GLM 5.3 最適化: Hybrid HiSparse
 * オフローディング", section 1 Full Residency).
 * For every request r, the n rows d_rows[r][0..n) ([R][n][row_bytes], device, 16-byte aligned) become host
 * rows d_pos[r] .. d_pos[r] + n - 1 of its pool, written by the GPU over the host link. When such a token
 * currently sits in a hot slot, the slot's row is replaced too, so every slot keeps holding its token's
 * row. Rows that would fall outside [0, host_rows) are skipped and set HS_STATUS_BAD_ID in d_status[r]
 * (optional; not written otherwise). Stream-ordered with resolves: a later resolve fetches the new rows.
 */
int hs_offload(hs_ctx* ctx, const void* d_rows, const int32_t* d_pos, int32_t n, int32_t* d_status, void* stream);

/*
 * Tail migration (Mixed residency: under memory pressure the older part of a request's device tail moves
 * to host memory, "vLLM GLM 5.3 最適化: Hybrid HiSparse オフローディング", section 2). For every request r,
 * the n = clamp(d_n[r], 0, T) tokens d_tail0[r] .. d_tail0[r] + n - 1 leave the tail: their ring rows are
 * written to their host-pool rows over the host link (and to the hot slot of a token that has one), then
 * d_tail0[r] advances by n, in place. Those tokens then resolve through the hot buffer; the ring rows they
 * free belong to the tokens entering the window at its end, which the caller writes. d_status[r]
 * (optional) gets HS_STATUS_BAD_ID if a leaving token lies outside [0, host_rows) (its row is skipped),
 * else 0. Requires tail_tokens > 0.
 */
int hs_advance_tail(hs_ctx* ctx, int32_t* d_tail0, const int32_t* d_n, int32_t* d_status, void* stream);

/* Unfused gather: d_gather[r][i] = the row d_out[r][i] names (as in hs_resolve), zeros for -1 or for
 * an index outside [0, B + T). d_out [R][k] int32, d_gather [R][k][row_bytes]. */
int hs_gather(hs_ctx* ctx, const int32_t* d_out, void* d_gather, void* stream);

/*
 * Snapshots of a context's device state, for tests, benchmarks and the retryable step ("vLLM GLM 5.3 最適化:
 * Hybrid HiSparse オフローディング", section vLLM エコシステムとの統合: a per-step resolver plan that shares the
 * request's hot state and can be retried).
 * what selects HS_STATE_TABLES (slot table, stamps, LRU order list, page table, step counters), HS_STATE_ROWS
 * (hot rows and device tail rows) or both. The snapshot (device memory of the context's device, 256-byte
 * aligned, at least hs_sizes.state_tables_bytes and/or .state_rows_bytes) holds the selected buffers in the
 * order slot_tok, stamp, lru_order, page, step, hot, tail, each at the next 256-byte aligned offset, byte for
 * byte as the bound buffers hold them. Both calls are stream-ordered device-to-device copies and allocate
 * nothing. hs_import_state writes the snapshot back (it must come from a context of the same configuration,
 * with the same what) and then advances every request's change counter, so no trial made before the import
 * can be committed after it. HS_E_INVALID for a bad what, a small or misaligned buffer, or one that is not
 * device memory of the context's device.
 */
#define HS_STATE_TABLES 1u
#define HS_STATE_ROWS 2u
int hs_export_state(hs_ctx* ctx, void* d_dst, uint64_t dst_bytes, uint32_t what, void* stream);
int hs_import_state(hs_ctx* ctx, const void* d_src, uint64_t src_bytes, uint32_t what, void* stream);

/* Rebuild every request's LRU order list from its stamps (ascending (stamp, slot)). Call it after a caller
 * writes slot_tok / stamp / page / step itself without the order list (hs_import_state restores the order list
 * with the rest). */
int hs_rebuild_order(hs_ctx* ctx, void* stream);

/* Free the host pool and the context (device buffers belong to the caller). NULL is ignored. */
void hs_destroy(hs_ctx* ctx);

/* Message of the last failing call in this thread ("" if none). */
const char* hs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_H */
