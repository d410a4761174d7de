// Internal declarations shared by the C ABI (hs_api.cpp) and the kernels (hs_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

constexpr int kThreads = 1024;            // resolve workgroup: 16 wave64s
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kLdsCap = 159u * 1024u;  // LDS one resolve workgroup may use (gfx950 has 160 KiB per CU)
constexpr int kMaxTopK = 8192;
constexpr int kMaxSlots = 65535;          // slot ids fit the uint16 LRU order list

typedef unsigned int v4u __attribute__((ext_vector_type(4)));  // one 16-byte chunk of a row

// LDS carve-up of one resolve workgroup (byte offsets; every section 16-byte aligned). Two layouts:
//
// Rank layout (resolve_kernel, every accepted shape): the selected ids and the ids found in a slot are kept
// as bitmaps over token ids, separate arrays of 32-bit words (consecutive words in consecutive LDS banks,
// which spreads the random lookups); a selected id's rank among the selected ids is a prefix count plus a
// popcount. Candidates (selected, not resident in the device tail) are the selected bits outside the tail
// window, which is one contiguous id range, so they need no bitmap of their own. Sections reused once dead:
// the rank -> first position table holds the victim list from phase 4 on, the per-position ranks hold the
// missed ids from phase 5 on, and the prefix counts of the selected set become those of the misses.
//
// Sparse rank layout (resolve_kernel's two-level form, for contexts whose bitmaps over token ids do not fit):
// the same ranks, over a compact id space. A coarse bitmap marks the 32-token words that hold a selected id;
// its prefix counts number those words 0, 1, ... (at most one per selected id), and a selected id x becomes
// 32 * (number of x's word) + (x mod 32), which keeps the ids' order. The rank layout's bitmaps then run over
// at most k words, and the device tail's ids have a bitmap of their own over the same compact words.
//
// Direct layout (resolve_direct_kernel, where it fits): a uint16 token -> slot table with one entry per host
// row, never cleared. Each slot writes its index under its token; an id x then hits slot s = t2s[x] exactly
// when s < B and the slot table holds x at s, so garbage left in the table by earlier work is harmless. Only
// the missed ids need a bitmap (for their ascending-id ranks). A selection that repeats an id is ranked as in
// the rank layout, with its arrays placed inside the table's region, dead by then.
struct Layout {
  // rank layout
  uint32_t ids, cls, rank_slot, rank, ord, hbits;
  // both
  uint32_t stok, sflag, sel, selpre, first, mpre, vict, mtok, gsrc, misc;
  // direct layout
  uint32_t mbits, rbits, t2s;
  uint32_t bm_end;  // rank layout: end of the bitmaps (adjacent from sel on, cleared together)
  uint32_t direct;  // 1: direct layout
  uint32_t words;   // bitmap words = ceil(H / 32); sparse: the most compact words, min(k, ceil(H / 32))
  uint32_t total;
  // sparse rank layout: the coarse bitmap over 32-token words and its uint16 prefix counts
  uint32_t sparse, coarse, cpre, cwords;
};

inline uint32_t align16(uint64_t x) { return (uint32_t)((x + 15) & ~uint64_t(15)); }

// misc words: one slot array of wave totals per block scan, per-wave flag words, then single words
constexpr int kMiscWords = 8 * kWaves + 8;

inline Layout make_layout(int k, int B, int H) {
  Layout L{};
  L.words = (uint32_t)(((uint64_t)H + 31) / 32);
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) { uint32_t o = (uint32_t)off; off = align16(off + bytes); return o; };
  L.ids = take(4ull * k);
  L.cls = take(1ull * k);
  L.rank_slot = take(4ull * k);
  L.rank = take(4ull * k);
  L.stok = take(4ull * B);
  L.ord = take(2ull * B);
  L.sflag = take(1ull * B);
  L.sel = take(4ull * L.words);     // selected ids (candidates and resident)
  L.hbits = take(4ull * L.words);   // candidate ids found in a slot
  L.bm_end = (uint32_t)off;
  L.selpre = take(2ull * L.words);  // uint16 prefix counts (k <= 8192)
  L.first = take(4ull * k);
  L.mpre = L.selpre;
  L.vict = L.first;
  L.gsrc = take(4ull * k);
  L.misc = take(4ull * kMiscWords);
  // The missed tokens get an array of their own when it still fits: then a selection without repeated ids
  // reads each hit slot from rank_slot while pairing, with no pass of its own. Otherwise they reuse rank_slot,
  // dead once every position has taken its slot in that pass.
  if (align16(off + 4ull * k) <= kLdsCap) L.mtok = take(4ull * k);
  else L.mtok = L.rank_slot;
  L.total = (uint32_t)off;
  return L;
}

// The sparse rank layout for k, B, H: the rank layout's arrays with bitmaps over at most min(k, ceil(H / 32))
// compact words, a bitmap of the resident ids over the same words, and the coarse bitmap (one bit per 32 host
// rows) with its prefix counts.
inline Layout make_sparse_layout(int k, int B, int H) {
  Layout L{};
  const uint64_t W = ((uint64_t)H + 31) / 32;
  L.words = (uint32_t)(W < (uint64_t)k ? W : (uint64_t)k);
  L.cwords = (uint32_t)((W + 31) / 32);
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) { uint32_t o = (uint32_t)off; off = align16(off + bytes); return o; };
  L.ids = take(4ull * k);
  L.cls = take(1ull * k);
  L.rank_slot = take(4ull * k);
  L.rank = take(4ull * k);
  L.stok = take(4ull * B);
  L.ord = take(2ull * B);
  L.sflag = take(1ull * B);
  L.sel = take(4ull * L.words);
  L.hbits = take(4ull * L.words);
  L.rbits = take(4ull * L.words);
  L.coarse = take(4ull * L.cwords);
  L.bm_end = (uint32_t)off;
  L.cpre = take(2ull * L.cwords);
  L.selpre = take(2ull * L.words);
  L.first = take(4ull * k);
  L.mpre = L.selpre;
  L.vict = L.first;
  L.gsrc = take(4ull * k);
  L.misc = take(4ull * kMiscWords);
  if (align16(off + 4ull * k) <= kLdsCap) L.mtok = take(4ull * k);
  else L.mtok = L.rank_slot;
  L.total = (uint32_t)(off > 0xffffffffull ? 0xffffffffull : off);
  L.sparse = 1;
  return L;
}

// The rank layout a context of this shape takes: the flat one where it fits in cap, else the sparse one.
inline Layout rank_layout(int k, int B, int H, uint64_t cap) {
  const Layout F = make_layout(k, B, H);
  return F.total <= cap ? F : make_sparse_layout(k, B, H);
}

// Ids and slots per thread of the direct kernel: (2, 4) for k <= 2048 and B <= 4096, else (8, 8); it holds at
// most three bitmap words per thread and clears its two bitmaps with at most two 16-byte stores per thread.
constexpr int kDirectMaxSlots = 8 * kThreads;

// The direct layout for k, B, H (tail of T rows), or one with direct == 0 where the direct kernel cannot take
// the shape: it does not fit in cap bytes, B is not a multiple of 4 or passes the kernel's limit, or the
// bitmaps pass the per-thread limits above. The per-position row sources only for launches that gather rows.
// The token -> slot table has a spare entry at index H, where slots without a valid token write.
inline Layout make_direct_layout(int k, int B, int H, int T, bool gather, uint64_t cap) {
  Layout L{};
  L.words = (uint32_t)(((uint64_t)H + 31) / 32);
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) { uint32_t o = (uint32_t)off; off = align16(off + bytes); return o; };
  L.stok = take(4ull * B);
  L.sflag = take(4ull * (((uint64_t)B + 3) / 4));   // one byte per slot, read and or-ed as 32-bit words
  L.mbits = take(4ull * L.words);
  L.rbits = take(4ull * (((uint64_t)T + 31) / 32));
  L.mpre = take(2ull * L.words);
  L.vict = take(4ull * k);
  L.mtok = take(4ull * k);
  L.gsrc = gather ? take(4ull * k) : 0u;
  L.misc = take(4ull * kMiscWords);
  // the table's region, holding the repeat path's arrays once the table is dead, then a plan launch's
  // evicted tokens and the staged new order
  const uint64_t region = off;
  L.t2s = (uint32_t)region;
  L.sel = take(4ull * L.words);
  L.selpre = take(2ull * L.words);
  L.first = take(4ull * k);
  const uint64_t table = align16(2ull * (uint64_t)H + 2);
  if (off < region + table) off = region + table;
  // the region also takes, once the table is dead, a plan's evicted tokens (4k) and the staged new order (2B)
  const uint64_t staged = align16(4ull * k) + 2ull * B;
  if (off < region + staged) off = region + staged;
  L.total = (uint32_t)off;
  const bool bitmaps_ok = L.words <= 3u * kThreads && (L.mpre - L.mbits) <= 2u * 16u * kThreads;
  L.direct = (off <= cap && B <= kDirectMaxSlots && B % 4 == 0 && bitmaps_ok) ? 1u : 0u;
  return L;
}

// The layout a launch takes: the direct one where it fits, else the rank one (flat, or sparse beyond it).
inline Layout launch_layout(int k, int B, int H, int T, bool gather, uint64_t cap) {
  const Layout D = make_direct_layout(k, B, H, T, gather, cap);
  return D.direct ? D : rank_layout(k, B, H, cap);
}

struct ResolveArgs {
  int32_t R, k, B, H, T, row16;
  int32_t policy;   // 0 LRU, 1 FIFO
  int32_t copy_threads, copy_unroll;  // fused row copy: threads per workgroup and loads in flight each
  Layout L;
  const v4u* host;  // device address of the pinned pool [R][H][row16]
  v4u* hot;         // [R][B][row16]
  const v4u* tail;  // [R][T][row16]
  int32_t* slot_tok;
  int32_t* stamp;
  uint16_t* order;
  int32_t* page;
  int32_t* step;
  const int32_t* topk;
  const int32_t* tail0;
  int32_t* out;
  int32_t* miss;
  int32_t* status;
  v4u* gather;
  int32_t* plan;    // non-null: plan-only launch, [R][4][k] (missed tokens, their victim slots, the tokens
                    // the victims held (-1: empty), and with plan_sources the source of each position's row: slot,
                    // B + tail row, -1 none, -2 - j the j-th miss)
  int32_t plan_sources;
  int32_t* trial;   // non-null: trial launch, [R][trial_words]
  const int32_t* epoch;  // [R] change counters (a trial records its request's)
  int64_t trial_words;
};

// Words of one request's trial record: 4 header words, 4 lists of k, the new order as B uint16, rounded
// up to 16 bytes.
inline int64_t trial_words(int k, int B) { return ((4 + 4ll * k + (B + 1) / 2) + 3) & ~3ll; }

struct CommitArgs {
  int32_t R, k, B, H, row16;
  int64_t trial_words;
  const int32_t* trial;
  const int32_t* accept;  // [R] or nullptr (all)
  const int32_t* epoch;   // [R] change counters: a record made under another value is stale
  const v4u* gather;      // [R][k][row16]
  int32_t* status;        // [R] or nullptr
  v4u* hot;
  int32_t* slot_tok;
  int32_t* stamp;
  uint16_t* order;
  int32_t* page;
  int32_t* step;
};

struct CopyArgs {
  int32_t R, k, B, H, T, row16;
  int32_t rows;         // with a gather: selected rows per workgroup
  int32_t workgroups;   // without a gather: the most workgroups the copy may take
  int32_t slices;       // set by the launch: workgroups per request (> 1 only with fewer requests than workgroups)
  const int32_t* plan;  // [R][4][k]
  const int32_t* miss;  // [R]
  const v4u* host;
  v4u* hot;
  int32_t* page;        // [R][H]: the plan's page-table updates are applied here
  const v4u* tail;      // [R][T][row16] or nullptr
  v4u* gather;          // [R][k][row16] or nullptr (no gather)
};

struct OffloadArgs {
  int32_t R, B, H, row16, n;
  const v4u* rows;     // [R][n][row16] device rows
  const int32_t* pos;  // [R] first token of each request's rows
  int32_t* status;     // [R] or nullptr
  v4u* host;           // device address of the pinned pool
  v4u* hot;
  const int32_t* page;
  int32_t* epoch;      // [R] change counters, advanced
};

struct AdvanceTailArgs {
  int32_t R, B, H, T, row16;
  int32_t* tail0;      // [R], advanced in place
  const int32_t* n;    // [R]
  int32_t* status;     // [R] or nullptr
  const v4u* tail;     // [R][T][row16] ring
  v4u* host;
  v4u* hot;
  const int32_t* page;
  int32_t* epoch;      // [R] change counters, advanced where the window moves
};

struct RebuildArgs {
  int32_t R, B;
  const int32_t* stamp;
  uint16_t* order;
};

struct ResetArgs {
  int32_t R, B, H;
  const int32_t* ids;  // nullptr: workgroup b resets request b
  int32_t* slot_tok;
  int32_t* stamp;
  uint16_t* order;
  int32_t* page;
  int32_t* step;
  int32_t* epoch;      // [R] change counters, advanced (nullptr: leave them)
};

// copy_kernel and copy_balanced_kernel: 16-byte host loads each thread keeps in flight, threads per workgroup
// (one wave) and the number of workgroups (measured: 128 one-wave workgroups hold the host link's rate within 2 %
// of the best grid, and disturb HBM-bound work on other streams far less than fewer, larger workgroups with as
// many loads in flight)
constexpr int kCopyUnroll = 8;
constexpr int kCopyWorkgroups = 128;
constexpr int kCopyThreads = 64;
constexpr int kBatchRows = 512;  // the balanced copy (fewer requests than workgroups): rows located per batch

// gather_kernel: threads per workgroup, 16-byte loads in flight per thread, and the chunks one workgroup
// covers (its row count is the largest that fits, at least one). Measured with 1152-byte rows, TB/s on the
// 256-, 32- and 64-request (device tail) workloads: 128 x 2 (3 rows per workgroup) 6.11-6.16 / 5.55 /
// 5.89-5.90; 256 x 3 6.02-6.05 / 5.43-5.44 / 5.77-5.79; 128 x 4 6.09-6.10 / 5.41-5.43 / 5.69; 256 x 2
// 5.98-6.00 / 5.46 / 5.87; 512 x 1 6.07 / 5.42-5.43 / 5.18-5.20. The gathering copy (hs_copy with a gather
// output) is the same at every shape.
constexpr int kGatherThreads = 128;
constexpr int kGatherUnroll = 2;
constexpr int kGatherChunks = kGatherThreads * kGatherUnroll;

struct GatherArgs {
  int32_t R, k, B, T, row16;
  int32_t rows;  // selected rows per workgroup
  const int32_t* out;
  const v4u* hot;
  const v4u* tail;
  v4u* gather;
};

// The plan of hs_step_static lives in a file-scope device array of this many bytes (one copy per device, held
// until the process ends); static_plan_address gives its device address on the current device.
constexpr uint64_t kStaticPlanBytes = 8ull << 20;
hipError_t static_plan_address(void** ptr);

hipError_t launch_resolve(const ResolveArgs& a, hipStream_t s);
hipError_t launch_reset(const ResetArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_bump_epoch(int32_t* epoch, int R, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_copy(const CopyArgs& a, hipStream_t s);
hipError_t launch_rebuild_order(const RebuildArgs& a, hipStream_t s);
hipError_t launch_commit(const CommitArgs& a, hipStream_t s);
hipError_t launch_offload(const OffloadArgs& a, hipStream_t s);
hipError_t launch_advance_tail(const AdvanceTailArgs& a, hipStream_t s);
hipError_t set_lds_limits(uint32_t resolve_bytes, uint32_t rebuild_bytes);

}  // namespace hs
