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

// LDS carve-up of one resolve workgroup (byte offsets; every section 16-byte aligned). The token sets are
// kept as separate arrays of 32-bit words (consecutive words in consecutive LDS banks, which spreads the
// random lookups). Sections reused once dead: the rank -> first position table holds the victim list from
// phase 4 on, the per-position ranks hold the missed ids from phase 5 on, and the prefix counts of the
// selected set become the prefix counts of the misses.
struct Layout {
  uint32_t ids, cls, rank_slot, rank, stok, ord, sflag, sel, cbits, hbits, selpre, first, mpre, vict, mtok, gsrc,
      misc;
  uint32_t bm_end;  // end of the three bitmaps (sel, cbits, hbits are adjacent and cleared together)
  uint32_t t2s;     // token -> slot table (uint16 per host row) of the direct layout
  uint32_t direct;  // 1: direct layout (t2s valid; rank_slot, rank, first and selpre live inside it)
  uint32_t words;   // bitmap words = ceil(H / 32)
  uint32_t total;
};

inline uint32_t align16(uint64_t x) { return (uint32_t)((x + 15) & ~uint64_t(15)); }

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
  L.cbits = take(4ull * L.words);   // candidate ids (not resident)
  L.hbits = take(4ull * L.words);   // candidate ids found in a slot
  L.bm_end = (uint32_t)off;
  L.selpre = take(2ull * L.words);  // uint16 prefix counts (k <= 8192)
  L.first = take(4ull * k);
  L.mpre = L.selpre;
  L.vict = L.first;
  L.gsrc = take(4ull * k);
  L.misc = take(4ull * (4 * kWaves + 8));
  // The missed tokens get an array of their own when it still fits: then a selection without repeated ids
  // reads each hit slot from rank_slot while pairing, with no pass of its own. Otherwise they reuse rank_slot,
  // dead once every position has taken its slot in that pass.
  if (align16(off + 4ull * k) <= kLdsCap) L.mtok = take(4ull * k);
  else L.mtok = L.rank_slot;
  L.total = (uint32_t)off;
  return L;
}

// The direct layout, where it fits in cap bytes (else the layout above): every host row of the request has a
// uint16 entry in a token -> slot table, so a slot holding a selected token writes its index under the token
// itself and the selected ids need no ranks. Nothing reads an entry whose token has no hit bit, so the table
// is never cleared. A launch whose selection repeats an id still ranks (the lowest position holding an id
// keeps it): the rank arrays and the selected set's prefix counts then live inside the table's region, which
// that launch does not use otherwise. The miss prefixes, the victim list and the missed tokens get arrays of
// their own; the per-position row sources only when the launch gathers rows.
inline Layout make_direct_layout(int k, int B, int H, bool gather, uint64_t cap) {
  Layout L{};
  L.words = (uint32_t)(((uint64_t)H + 31) / 32);
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) { uint32_t o = (uint32_t)off; off = align16(off + bytes); return o; };
  L.ids = take(4ull * k);
  L.cls = take(1ull * k);
  L.stok = take(4ull * B);
  L.ord = take(2ull * B);
  L.sflag = take(1ull * B);
  L.sel = take(4ull * L.words);
  L.cbits = take(4ull * L.words);
  L.hbits = take(4ull * L.words);
  L.bm_end = (uint32_t)off;
  L.mpre = take(2ull * L.words);
  L.vict = take(4ull * k);
  L.mtok = take(4ull * k);
  L.gsrc = gather ? take(4ull * k) : 0u;  // unused without a gather (a plan launch writes the sources out)
  L.misc = take(4ull * (4 * kWaves + 8));
  // the table's region, with the rank path's arrays inside it
  const uint64_t region = off;
  L.t2s = (uint32_t)region;
  L.rank_slot = take(4ull * k);
  L.rank = take(4ull * k);
  L.first = take(4ull * k);
  L.selpre = take(2ull * L.words);
  const uint64_t table = align16(2ull * (uint64_t)H);
  if (off < region + table) off = region + table;
  L.total = (uint32_t)off;
  L.direct = 1u;
  if (off > cap) return make_layout(k, B, H);
  return L;
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
  int32_t* plan;    // non-null: plan-only launch, [R][3][k] (missed tokens, their victim slots, the source of
                    // each position's row: slot, B + tail row, -1 none, -2 - j the j-th miss)
  int32_t* trial;   // non-null: trial launch, [R][trial_words]
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
  const int32_t* plan;  // [R][3][k]
  const int32_t* miss;  // [R]
  const v4u* host;
  v4u* hot;
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
};

// gather_kernel: threads per workgroup, 16-byte loads in flight per thread, and the chunks one workgroup
// covers (its row count is the largest that fits, at least one)
constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 3;
constexpr int kGatherChunks = kGatherThreads * kGatherUnroll;

struct GatherArgs {
  int32_t R, k, B, T, row16;
  int32_t rows;  // selected rows per workgroup
  const int32_t* out;
  const v4u* hot;
  const v4u* tail;
  v4u* gather;
};

hipError_t launch_resolve(const ResolveArgs& a, hipStream_t s);
hipError_t launch_reset(const ResetArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_copy(const CopyArgs& a, hipStream_t s);
hipError_t launch_rebuild_order(const RebuildArgs& a, hipStream_t s);
hipError_t launch_commit(const CommitArgs& a, hipStream_t s);
hipError_t launch_offload(const OffloadArgs& a, hipStream_t s);
hipError_t launch_advance_tail(const AdvanceTailArgs& a, hipStream_t s);
hipError_t set_lds_limits(uint32_t resolve_bytes, uint32_t rebuild_bytes);

}  // namespace hs
