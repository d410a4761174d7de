// HIP kernels of the HiSparse swap-in path for gfx950 (MI355X).
//
// One 1024-thread workgroup per request performs one decode step of the swap-in kernel the pages describe
// ("HiSparse: Turbocharging Sparse Attention with Hierarchical Memory", section 2, steps 1-3;
// 「HiSparse：階層化メモリシステムによるスパースアテンションの加速」, section 「効率的なSwap-inカーネル」), with the
// device-resident tail and the fused gather of "vLLM GLM 5.3 最適化: Hybrid HiSparse オフローディング", section 2
// Mixed Residency. Two kernels do it, by LDS layout.
//
// resolve_direct_kernel (where a uint16 token -> slot entry for every host row fits in LDS):
//   A  coalesced loads of the selected ids, the slot table, the LRU order list and the stamps, all issued before
//      any is consumed; each slot writes its index under its token in the (never cleared) token -> slot table;
//   B  each selected id is tested from its own side: it hits slot s = t2s[x] exactly when s < B and slot s
//      holds x, so stale table entries cannot fake a hit; a hit marks its slot, a miss its bit in a bitmap
//      of missed ids (an already-set bit or flag means the selection repeats an id, which is then ranked as
//      in the rank kernel: the lowest position keeps it);
//   C  one block scan ranks the misses (ascending id, popcounts of the bitmap) and the non-hit slots in LRU
//      order; the first m of these are the victims, the others open the new order;
//   D  the used slots' stamp rows go out (whole rows, 16 bytes per lane); the j-th missed id takes the j-th
//      victim: outputs, page table (fused), the LDS slot table; a second scan closes the new order with the
//      slots used this step, in slot order; the slot-table rows go out;
//   E  the missed rows are copied from mapped pinned host memory (and every selected row gathered when fused).
// Ids, order entries and stamps stay in registers from A to D. The new order is staged in LDS and written at
// the end in one 8-byte store per thread, and a plan's victim lists go out densely after C: the kernel's phases
// wait mostly on their vector-memory instructions, so each phase issues as few as it can. Six barriers.
//
// resolve_kernel (every shape, the rank layout):
//   phase 0  the same loads, staged in LDS; ids classified and put into a bitmap of selected ids;
//   phase 1  popcount prefix over the bitmap's words, so the rank of a selected id is one lookup;
//   phase 2  every selected position takes its id's rank and, when phase 0 saw an id twice, bids for it (the
//            lowest position wins, without order-dependent atomics) while every slot tests its token against
//            the bitmap: a hit, recorded under the token's rank and marked in a hit bitmap;
//   phase 3  one block scan ranks the misses (selected ids outside the tail window and not hit) and the
//            non-hit slots in LRU order, as in C above;
//   phase 4  as D above (where B is four slots per thread, the stamps and slot-table entries go back as whole
//            16-byte rows, the stamp rows right after phase 3; elsewhere one store per used slot);
//   phase 5  as E above.
// Scans run over thread-contiguous chunks: a DPP scan inside each wave, one exchange of the 16 wave totals
// through LDS, which each wave scans again in one DPP row. No result depends on the order of LDS atomics
// (they are OR and MIN only, and which of two equal ids a bit or flag records is never used).
//
// The LRU order list keeps each request's slots sorted by (stamp, slot). After a step, the non-victim
// candidates keep their stamps and relative order, and every hit or victim slot now carries stamp t, larger
// than any older stamp, so appending them in slot order keeps the list sorted. Empty slots (stamp -1) start at
// the front in slot order after a reset.
//
// FIFO replacement (the alternative to LRU a request can be configured with) takes victims the same way, but
// a hit does not refresh its stamp: hits keep their place in the list and only the victims, stamped t, move to
// its end.
#include "hs_internal.h"

#include <climits>

namespace hs {

namespace {

enum : int8_t { C_PAD = 0, C_BAD = 1, C_DUP = 2, C_RES = 3, C_CAND = 4 };

constexpr int kStatusBadId = 1, kStatusDupId = 2, kStatusBadState = 4, kStatusStale = 8;
constexpr int kUnroll = 4;  // 16-byte loads each thread keeps in flight in the gather loop
constexpr int kCommitUnroll = 2;  // the same in the commit's row copy (measured: 2 beats 4 and 8)
constexpr int kTailUnroll = 8;    // chunks each thread moves per pass when the tail window advances

// misc words in LDS: one slot array of wave totals per block scan, per-wave flag words, then single words
constexpr int kMiscScanSel = 0, kMiscScanRank = kWaves, kMiscScanTail = 2 * kWaves, kMiscWaveBad = 3 * kWaves,
              kMiscWaveRep = 4 * kWaves, kMiscWaveSt = 5 * kWaves, kMiscStatus = 8 * kWaves,
              kMiscRepeat = 8 * kWaves + 1, kMiscBad = 8 * kWaves + 2, kMiscDummy = 8 * kWaves + 4;
static_assert(kMiscDummy + 4 <= kMiscWords, "misc words (the dummy takes 16 bytes)");

// The tail is a ring of T rows, token x in row x mod T. For a resident x (t0 <= x < t0 + T) that row is
// (t0 mod T + (x - t0)) mod T: ring_base gives t0 mod T (0 without a tail), once per wave on uniform values,
// and ring_row wraps the sum, which stays below 2T, once.
__device__ __forceinline__ uint32_t ring_base(bool has_tail, int32_t t0, int32_t T) {
  if (!has_tail || T <= 0) return 0u;
  const int32_t m = t0 % T;
  return (uint32_t)(m < 0 ? m + T : m);
}
__device__ __forceinline__ uint32_t ring_row(uint32_t base, uint32_t offset, int32_t T) {
  const uint32_t e = base + offset;
  return e >= (uint32_t)T ? e - (uint32_t)T : e;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2, 4, 8 inside each row of 16
// lanes, then the row broadcasts of lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive prefix sum of one value per thread over the workgroup. sh: kWaves ints used by this call only.
// After the exchange, lanes 0..15 of every wave hold the 16 wave totals and scan them in one DPP row; the
// wave's offset and the block total are two lane reads of that row.
static_assert(kWaves == 16, "the wave totals fill one DPP row");
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int lane, int wave, int* total) {
  const int inc = wave_incl_scan(v);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int x = lane < kWaves ? sh[lane] : 0;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  const int w = __builtin_amdgcn_readfirstlane(wave);
  const int pre = w > 0 ? __builtin_amdgcn_readlane(x, w - 1) : 0;
  *total = __builtin_amdgcn_readlane(x, kWaves - 1);
  return pre + inc - v;
}

// True in every lane when any of the 16 per-wave flag words at f is set (they are written before a barrier).
__device__ __forceinline__ bool any_wave_flag(const int32_t* f, int lane) {
  return __ballot(lane < kWaves && f[lane < kWaves ? lane : 0] != 0) != 0ull;
}

// OR of v over the wave (v holds status bits 0..3).
__device__ __forceinline__ int wave_or_bits(int v) {
  int o = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) o |= __ballot((v >> b) & 1) != 0ull ? (1 << b) : 0;
  return o;
}

__device__ __forceinline__ uint32_t below(int32_t x) { return (1u << (x & 31)) - 1u; }

// Bits of bitmap word w (tokens 32w .. 32w + 31) that lie in [lo, hi), a window already clipped to [0, H)
// (so every difference below fits in 32 bits).
__device__ __forceinline__ uint32_t window_bits(int w, int32_t lo, int32_t hi) {
  const int a = min(max(lo - 32 * w, 0), 32), b = min(max(hi - 32 * w, 0), 32);
  const uint32_t below_b = b >= 32 ? ~0u : (1u << b) - 1u, below_a = a >= 32 ? ~0u : (1u << a) - 1u;
  return below_b & ~below_a;
}

// Element i of an array whose byte size stays below 4 GiB (per-request rows of k or B entries): the byte
// offset is formed in 32 bits, so a store takes the scalar-base + 32-bit-offset form.
template <class T>
__device__ __forceinline__ T& at(T* base, uint32_t i) {
  return *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + i * (uint32_t)sizeof(T));
}

__device__ __forceinline__ v4u load_host(const v4u* p) { return __builtin_nontemporal_load(p); }

// Missed rows from the host pool into their slots, flattened over (miss, 16-byte chunk): thread tid of nt
// copies chunks tid, tid + nt, ..., keeping U loads in flight.
template <int U>
__device__ __forceinline__ void copy_missed_rows(const v4u* hostr, v4u* hotr, const int32_t* mtok, const int32_t* vict,
                                                 int total, int row16, int tid, int nt) {
  for (int c0 = tid; c0 < total; c0 += nt * U) {
    v4u v[U];
    size_t dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * nt;
      if (c < total) {
        const int j = c / row16, q = c - j * row16;
        v[u] = load_host(hostr + (size_t)mtok[j] * row16 + q);
        dst[u] = (size_t)vict[j] * row16 + q;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * nt;
      if (c < total) hotr[dst[u]] = v[u];
    }
  }
}

constexpr int kFused = 0, kPlan = 1, kTrial = 2;
constexpr int kTrialHead = 4;

// Trial record of one request (int32 words): [m, first tail position of the new order, step, epoch], then
// k missed tokens, k victim slots, k evicted tokens (-1: slot was empty), k positions in the selection,
// then the new LRU order as B uint16.
__device__ __forceinline__ int32_t* trial_rec(const ResolveArgs& a, int r) { return a.trial + (size_t)r * a.trial_words; }

__device__ __forceinline__ void trial_header(const ResolveArgs& a, int r, int m, int tail_start, int step) {
  int32_t* rec = trial_rec(a, r);
  rec[0] = m;
  rec[1] = tail_start;
  rec[2] = step;
  rec[3] = a.epoch[r];
}

// A request whose state tables hold impossible values: every output -1 (zero rows gathered), no miss, status
// HS_STATUS_BAD_STATE; nothing of its state is changed.
template <int kMode>
__device__ __forceinline__ void refuse_request(const ResolveArgs& a, int r, int tid) {
  const size_t rk = (size_t)r * a.k;
  for (int i = tid; i < a.k; i += kThreads) a.out[rk + i] = -1;
  if (kMode == kPlan && a.plan_sources)
    for (int i = tid; i < a.k; i += kThreads) a.plan[4 * rk + 3 * (size_t)a.k + i] = -1;
  if (kMode != kPlan && a.gather) {
    v4u* gr = a.gather + rk * a.row16;
    const v4u z = {0u, 0u, 0u, 0u};
    for (int c = tid; c < a.k * a.row16; c += kThreads) gr[c] = z;
  }
  if (tid == 0) { a.miss[r] = 0; a.status[r] = kStatusBadState; }
  if (kMode == kTrial && tid == 0) trial_header(a, r, 0, 0, -1);
}

// Phase E / 5: the rows of a fused or trial launch. Without a gather output, the missed rows go from the host
// pool into their slots; with one, every selected row goes to the output (a miss's straight from the host
// pool, also into its slot unless this is a trial), as gsrc says: slot, B + tail row, -1 none, -2 - j miss j.
// mtok, vict and gsrc are LDS arrays made visible by a barrier before the call.
template <int kMode>
__device__ __forceinline__ void rows_phase(const ResolveArgs& a, int r, int m, const int32_t* mtok,
                                           const int32_t* vict, const int32_t* gsrc, int tid) {
  const int row16 = a.row16, k = a.k, B = a.B;
  const v4u* hostr = a.host + (size_t)r * a.H * (size_t)row16;
  v4u* hotr = a.hot + (size_t)r * B * (size_t)row16;
  if (a.gather == nullptr) {
    // The host link is saturated with about 128K 16-byte loads in flight over the whole chip; more than that
    // only queues and costs throughput, so the host sizes (copy_threads, copy_unroll) per request.
    const int total = m * row16, nt = a.copy_threads;
    if (tid < nt) {
      if (a.copy_unroll == 1) copy_missed_rows<1>(hostr, hotr, mtok, vict, total, row16, tid, nt);
      else if (a.copy_unroll == 2) copy_missed_rows<2>(hostr, hotr, mtok, vict, total, row16, tid, nt);
      else copy_missed_rows<4>(hostr, hotr, mtok, vict, total, row16, tid, nt);
    }
    return;
  }
  const int total = k * row16;
  const v4u* tailr = a.tail + (size_t)r * a.T * row16;
  v4u* gr = a.gather + (size_t)r * k * (size_t)row16;
  for (int c0 = tid; c0 < total; c0 += kThreads * kUnroll) {
    v4u v[kUnroll];
    long long hot_dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * kThreads;
      hot_dst[u] = -1;
      v[u] = v4u{0u, 0u, 0u, 0u};
      if (c < total) {
        const int i = c / row16, q = c - i * row16;
        const int g = gsrc[i];
        if (g <= -2) {
          const int j = -2 - g;
          v[u] = load_host(hostr + (size_t)mtok[j] * row16 + q);
          if (kMode != kTrial) hot_dst[u] = (long long)vict[j] * row16 + q;
        } else if (g >= B) {
          v[u] = tailr[(size_t)(g - B) * row16 + q];
        } else if (g >= 0) {
          v[u] = hotr[(size_t)g * row16 + q];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * kThreads;
      if (c < total) {
        // streamed in a fused step (nothing reads the output back in this launch, and it leaves less to
        // write back when the launch ends); plain in a trial, whose commit reads the missed rows back
        if (kMode == kTrial) gr[c] = v[u];
        else __builtin_nontemporal_store(v[u], gr + c);
        if (hot_dst[u] >= 0) hotr[hot_dst[u]] = v[u];
      }
    }
  }
}

}  // namespace

// kMode selects what a launch does with the step it has ranked:
//   kFused: commit the step and copy the rows (hs_resolve);
//   kPlan:  commit the step, except the page table, and write the miss list (token, victim slot, evicted
//           token), and on request each position's row source, to a.plan instead of copying rows; copy_kernel
//           then moves the rows and updates the page table, possibly on another stream (hs_plan);
//   kTrial: commit nothing; write a trial record (the new LRU order and, per miss, token, victim slot,
//           evicted token and position) and gather every selected row, the missed ones straight from the
//           host pool; commit_kernel applies accepted records later (hs_trial / hs_commit).
// kFifo: FIFO replacement instead of LRU (hits keep their stamps and their place in the order list).
// kSparse: the two-level bitmaps of the sparse rank layout (contexts past the flat bitmaps' LDS): every bitmap
// below runs over compact words, word number vw(x) for a selected id x, the same bit x mod 32 within it.
template <int kMode, bool kFifo, bool kSparse>
__global__ __launch_bounds__(kThreads) void resolve_kernel(ResolveArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Layout& L = a.L;
  int32_t* ids = (int32_t*)(smem + L.ids);
  int8_t* cls = (int8_t*)(smem + L.cls);
  int32_t* rank_slot = (int32_t*)(smem + L.rank_slot);  // rank of a selected id -> slot that holds it (hit)
  int32_t* rnk = (int32_t*)(smem + L.rank);  // position -> rank of its id, then -> its slot (hit) or -1
  int32_t* stok = (int32_t*)(smem + L.stok);
  uint16_t* ord = (uint16_t*)(smem + L.ord);
  uint8_t* sflag = smem + L.sflag;  // 1: hit this step, 2: victim this step
  uint32_t* sel = (uint32_t*)(smem + L.sel);
  uint32_t* hbits = (uint32_t*)(smem + L.hbits);
  uint16_t* selpre = (uint16_t*)(smem + L.selpre);
  uint16_t* mpre = (uint16_t*)(smem + L.mpre);
  int32_t* first = (int32_t*)(smem + L.first);        // rank -> lowest position holding that id
  int32_t* vict = (int32_t*)(smem + L.vict);
  int32_t* mtok = (int32_t*)(smem + L.mtok);
  int32_t* gsrc = (int32_t*)(smem + L.gsrc);
  int32_t* misc = (int32_t*)(smem + L.misc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  // where the new LRU order goes: the request's order list, or the trial record
  uint16_t* new_order = kMode == kTrial
                            ? reinterpret_cast<uint16_t*>(a.trial + (size_t)r * a.trial_words + kTrialHead + 4 * a.k)
                            : a.order + (size_t)r * a.B;
  const int k = a.k, B = a.B, H = a.H, T = a.T;
  int W = (int)L.words;  // sparse: the compact words in use, known once the coarse bitmap is counted
  const bool has_tail = a.tail0 != nullptr;
  constexpr bool fifo = kFifo;
  const int32_t t0 = has_tail ? a.tail0[r] : 0;
  uint32_t* coarse = (uint32_t*)(smem + L.coarse);  // sparse: one bit per 32-token word holding a selected id
  uint16_t* cpre = (uint16_t*)(smem + L.cpre);      // sparse: compact words before each coarse word
  uint32_t* rbits = (uint32_t*)(smem + L.rbits);    // sparse: resident ids, over the compact words
  // the bitmap word of a selected id: its 32-token word, or in the sparse layout that word's compact number
  auto vw = [&](int32_t x) -> int {
    if constexpr (kSparse) {
      const int c_ = x >> 10;
      return (int)cpre[c_] + __popc(coarse[c_] & ((1u << ((x >> 5) & 31)) - 1u));
    } else {
      return x >> 5;
    }
  };
  const int32_t t = a.step[r];
  const size_t rk = (size_t)r * k, rB = (size_t)r * B, rH = (size_t)r * H;
  // per-request bases (uniform): with at(), stores take the scalar-base form with no 64-bit address arithmetic
  // per lane
  int32_t* const out_r = a.out + rk;
  int32_t* const page_r = a.page + rH;
  int32_t* const stamp_r = a.stamp + rB;
  int32_t* const slot_tok_r = a.slot_tok + rB;
  int32_t* const plan_r = a.plan + 4 * rk;  // used by plan launches only
  const bool sources = kMode == kPlan && a.plan_sources != 0;
  // thread-contiguous chunks of bitmap words and of slots / order positions
  int cw = (W + kThreads - 1) / kThreads, w0 = min(W, tid * cw), w1 = min(W, w0 + cw);
  const int cb = (B + kThreads - 1) / kThreads, s0 = min(B, tid * cb), s1 = min(B, s0 + cb);
  // x - t0 is exact in uint32 once x >= t0, whatever the signs
  auto resident = [&](int32_t x) { return has_tail && x >= t0 && (uint32_t)x - (uint32_t)t0 < (uint32_t)T; };
  // the tail window clipped to the host rows (uniform), and the candidates of a bitmap word: selected ids
  // outside it
  const int32_t win_lo = has_tail ? (int32_t)min<int64_t>(max<int64_t>(t0, 0), H) : 0;
  const int32_t win_hi = has_tail ? (int32_t)min<int64_t>(max<int64_t>((int64_t)t0 + T, 0), H) : 0;
  // words that the window touches at all (uniform); elsewhere the mask is zero and is not computed
  const int win_w0 = win_lo >> 5, win_w1 = win_hi > win_lo ? (win_hi - 1) >> 5 : -1;
  auto wmask = [&](int w) { return (w >= win_w0 && w <= win_w1) ? window_bits(w, win_lo, win_hi) : 0u; };
  auto cand_word = [&](int w) {
    if constexpr (kSparse) return sel[w] & ~rbits[w];
    else return has_tail ? sel[w] & ~wmask(w) : sel[w];
  };
  int st = 0;

  // ---- phase 0: stage and classify, and build the bitmap of selected ids. The first round of every global
  // load of the phase is issued before any of them is consumed (one HBM round trip for the common shapes), as
  // 16-byte vectors when the sizes allow; LDS scratch is cleared, behind a barrier, while they are in flight,
  // so each id goes into the bitmap straight from the register it arrives in.
  int bad = 0, repeat = 0;
  const bool vecB = (B & 3) == 0 && ((reinterpret_cast<uintptr_t>(a.slot_tok + rB) & 15) == 0) &&
                    ((reinterpret_cast<uintptr_t>(a.order + rB) & 7) == 0);
  const bool veck = (k & 3) == 0 && ((reinterpret_cast<uintptr_t>(a.topk + rk) & 15) == 0);
  const int n4B = vecB ? (B >> 2) : 0, n4k = veck ? (k >> 2) : 0;
  // B = 4 x threads with aligned rows: thread tid owns slots 4 tid .. 4 tid + 3, and writes their stamps and
  // slot-table entries back as whole 16-byte rows (the old stamps loaded with the first round of loads): one
  // store instruction per wave for each table instead of one masked instruction per slot. (Staging the new
  // order in LDS for 8-byte stores, as the direct layout does, measured slower here: its extra barrier costs
  // more than the stores it saves.)
  const bool stamp_rows = kMode != kTrial && B == 4 * kThreads && vecB &&
                          (reinterpret_cast<uintptr_t>(stamp_r) & 15) == 0;
  const int4* st4 = reinterpret_cast<const int4*>(a.slot_tok + rB);
  const uint2* or4 = reinterpret_cast<const uint2*>(a.order + rB);
  const int4* tk4 = reinterpret_cast<const int4*>(a.topk + rk);
  int4 y0 = make_int4(-1, -1, -1, -1), x0 = make_int4(-1, -1, -1, -1);
  uint2 o0 = make_uint2(0u, 0u);
  if (tid < n4B) { y0 = st4[tid]; o0 = or4[tid]; }
  if (tid < n4k) x0 = tk4[tid];
  v4u sp0 = {0u, 0u, 0u, 0u};  // the old stamps of the thread's four slots, for the stamp rows
  if (stamp_rows) sp0 = reinterpret_cast<const v4u*>(stamp_r)[tid];
  {
    // the two bitmaps are adjacent, each padded to 16 bytes: cleared together in 16-byte stores
    uint4* bm = reinterpret_cast<uint4*>(smem + L.sel);
    const int n16 = (int)((L.bm_end - L.sel) >> 4);
    for (int q = tid; q < n16; q += kThreads) bm[q] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid == 0) { misc[kMiscStatus] = 0; misc[kMiscRepeat] = 0; misc[kMiscBad] = 0; }
  __syncthreads();

  auto stage4 = [&](int i, int4 y, uint2 o) {
    reinterpret_cast<int4*>(stok)[i] = y;
    reinterpret_cast<uint2*>(ord)[i] = o;
    reinterpret_cast<uint32_t*>(sflag)[i] = 0u;
    const int yy[4] = {y.x, y.y, y.z, y.w};
    const uint32_t oo[4] = {o.x & 0xffffu, o.x >> 16, o.y & 0xffffu, o.y >> 16};
#pragma unroll
    for (int c = 0; c < 4; ++c) bad |= ((uint32_t)yy[c] + 1u > (uint32_t)H) | (oo[c] >= (uint32_t)B);  // y in [-1, H)
  };
  // without branches: -1 is padding; outside [0, H), or at or past the tail start but outside the tail, is a
  // bad id; inside the tail is resident; anything else is a candidate for the hot buffer
  auto classify = [&](int32_t x) -> int8_t {
    const bool past = has_tail && x >= t0;
    const bool res = past && (uint32_t)x - (uint32_t)t0 < (uint32_t)T;
    const bool badid = x != -1 && (x < 0 || x >= H || (past && !res));
    st |= badid ? kStatusBadId : 0;
    return x == -1 ? C_PAD : badid ? C_BAD : res ? C_RES : C_CAND;
  };
  // a selected id (candidate or resident) goes into the bitmap; finding its bit already set means the
  // selection repeats an id. Without branches: an id that is not selected ORs nothing into word 0.
  auto mark = [&](int32_t x, int8_t c) {
    const bool s = c == C_CAND || c == C_RES;
    if constexpr (kSparse) {  // the coarse bit of x's word; the id's own bit waits for the compact numbering
      atomicOr(&coarse[s ? (x >> 10) : 0], s ? 1u << ((x >> 5) & 31) : 0u);
    } else {
      const int wi = s ? (x >> 5) : 0;
      const uint32_t bit = s ? 1u << (x & 31) : 0u;
      const uint32_t old = atomicOr(&sel[wi], bit);
      repeat |= (old & bit) != 0u;
    }
  };
  auto ids4 = [&](int i, int4 x) {
    reinterpret_cast<int4*>(ids)[i] = x;
    reinterpret_cast<int4*>(rank_slot)[i] = make_int4(-1, -1, -1, -1);
    const int32_t xs[4] = {x.x, x.y, x.z, x.w};
    int8_t c[4];
    int wi[4];
    uint32_t bit[4], old[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c[u] = classify(xs[u]);
      const bool s = c[u] == C_CAND || c[u] == C_RES;
      wi[u] = s ? (kSparse ? (xs[u] >> 10) : (xs[u] >> 5)) : 0;
      bit[u] = s ? 1u << (kSparse ? ((xs[u] >> 5) & 31) : (xs[u] & 31)) : 0u;
    }
    reinterpret_cast<uint32_t*>(cls)[i] = (uint32_t)(uint8_t)c[0] | ((uint32_t)(uint8_t)c[1] << 8) |
                                          ((uint32_t)(uint8_t)c[2] << 16) | ((uint32_t)(uint8_t)c[3] << 24);
    // what mark does, for four ids at once: every atomic is issued before the first result is looked at
    uint32_t* const bm = kSparse ? coarse : sel;
#pragma unroll
    for (int u = 0; u < 4; ++u) old[u] = atomicOr(&bm[wi[u]], bit[u]);
    if constexpr (!kSparse) {
      uint32_t rep = 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u) rep |= old[u] & bit[u];
      repeat |= rep != 0u;
    }
  };

  if (tid < n4B) stage4(tid, y0, o0);
  for (int i = tid + kThreads; i < n4B; i += kThreads) stage4(i, st4[i], or4[i]);
  if (!vecB) {
    for (int s = tid; s < B; s += kThreads) {
      const int32_t y = a.slot_tok[rB + s];
      const uint16_t o = a.order[rB + s];
      stok[s] = y;
      ord[s] = o;
      sflag[s] = 0;
      bad |= (y < -1 || y >= H || (int)o >= B);
    }
  }
  if (tid < n4k) ids4(tid, x0);
  for (int i = tid + kThreads; i < n4k; i += kThreads) ids4(i, tk4[i]);
  if (!veck) {
    for (int i = tid; i < k; i += kThreads) {
      const int32_t x = a.topk[rk + i];
      const int8_t c = classify(x);
      ids[i] = x;
      cls[i] = c;
      rank_slot[i] = -1;
      mark(x, c);
    }
  }
  if constexpr (kSparse) {
    // number the marked 32-token words in id order (a block scan of the coarse words' popcounts), then put
    // each selected id into the bitmaps over its compact word; finding its bit set means a repeated id
    __syncthreads();
    const int CW = (int)L.cwords;
    const int ccw = (CW + kThreads - 1) / kThreads, c0 = min(CW, tid * ccw), c1 = min(CW, c0 + ccw);
    int cnt = 0;
    for (int w = c0; w < c1; ++w) cnt += __popc(coarse[w]);
    int n_words;
    int run = block_excl_scan(cnt, misc + kMiscScanSel, lane, wave, &n_words);
    for (int w = c0; w < c1; ++w) {
      cpre[w] = (uint16_t)run;
      run += __popc(coarse[w]);
    }
    W = min(n_words, (int)L.words);  // n_words <= k: every marked word holds a selected id
    cw = (W + kThreads - 1) / kThreads;
    w0 = min(W, tid * cw);
    w1 = min(W, w0 + cw);
    __syncthreads();
    for (int i = tid; i < k; i += kThreads) {
      const int8_t c = cls[i];
      if (c == C_CAND || c == C_RES) {
        const int32_t x = ids[i];
        const int v = vw(x);
        const uint32_t bit = 1u << (x & 31);
        const uint32_t old = atomicOr(&sel[v], bit);
        repeat |= (old & bit) != 0u;
        if (c == C_RES) atomicOr(&rbits[v], bit);
      }
    }
  }
  // one barrier publishes both flags (every writer stores the same 1)
  if (repeat) misc[kMiscRepeat] = 1;
  if (bad) misc[kMiscBad] = 1;
  __syncthreads();
  bad = misc[kMiscBad];
  const bool repeats = misc[kMiscRepeat] != 0;  // rare: only then do positions bid for their id's rank
  if (repeats && !bad) {
    for (int i = tid; i < k; i += kThreads) first[i] = INT_MAX;
    __syncthreads();
  }
  // a thread whose chunk is four whole slots (B = 4 x threads) reads its slot-table entries, order entries
  // and slot flags with one LDS access each, 16-, 8- and 4-byte aligned; likewise a whole chunk of two or
  // four bitmap words is one 8- or 16-byte access, its uint16 prefixes one 4- or 8-byte store
  const bool whole4 = cb == 4 && s1 - s0 == 4;
  const bool wvec = (cw == 2 || cw == 4) && w1 - w0 == cw;
  auto load_words = [&](const uint32_t* bm, uint32_t (&v)[4]) {
    if (cw == 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(bm + w0);
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
      const uint2 q = *reinterpret_cast<const uint2*>(bm + w0);
      v[0] = q.x; v[1] = q.y; v[2] = 0u; v[3] = 0u;
    }
  };
  // prefixes of a whole chunk: run, then run plus the popcounts of the words before each
  auto store_prefixes = [&](uint16_t* pre, const uint32_t (&v)[4], int run) {
    const uint32_t p0 = (uint32_t)run, p1 = p0 + __popc(v[0]), p2 = p1 + __popc(v[1]), p3 = p2 + __popc(v[2]);
    if (cw == 4)
      *reinterpret_cast<uint2*>(pre + w0) = make_uint2((p0 & 0xffffu) | (p1 << 16), (p2 & 0xffffu) | (p3 << 16));
    else
      *reinterpret_cast<uint32_t*>(pre + w0) = (p0 & 0xffffu) | (p1 << 16);
  };

  if (bad) {
    // impossible state: leave the request untouched
    refuse_request<kMode>(a, r, tid);
    return;
  }

  // ---- phase 1: prefix counts of the selected bitmap (the rank of a selected id is one lookup)
  {
    int cnt = 0;
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    if (wvec) {
      load_words(sel, v);
      cnt = __popc(v[0]) + __popc(v[1]) + __popc(v[2]) + __popc(v[3]);
    } else {
      for (int w = w0; w < w1; ++w) cnt += __popc(sel[w]);
    }
    int n_sel;
    int run = block_excl_scan(cnt, misc + kMiscScanSel, lane, wave, &n_sel);
    if (wvec) {
      store_prefixes(selpre, v, run);
    } else {
      for (int w = w0; w < w1; ++w) {
        selpre[w] = (uint16_t)run;
        run += __popc(sel[w]);
      }
    }
    __syncthreads();
  }

  // ---- phase 2: ranks and the hit test in one pass. Every selected position records the rank of its id and,
  // if the selection repeats an id, bids for it (the lowest position holding an id wins); every slot whose
  // token is selected records itself under that token's rank and marks the token hit.
  for (int i = tid; i < k; i += kThreads) {
    const int8_t c = cls[i];
    if (c == C_CAND || c == C_RES) {
      const int32_t x = ids[i];
      const int v = vw(x);
      const int q = (int)selpre[v] + __popc(sel[v] & below(x));
      rnk[i] = q;
      if (repeats) atomicMin(&first[q], i);
    }
  }
  auto probe_slot = [&](int s, int32_t y) {
    if (y < 0 || resident(y)) return;  // empty, or resident (a resident id takes no slot)
    int v = y >> 5;
    if constexpr (kSparse) {  // no selected id in y's 32-token word: not selected
      if (!(coarse[y >> 10] & (1u << ((y >> 5) & 31)))) return;
      v = vw(y);
    }
    const uint32_t word = sel[v];
    if (word & (1u << (y & 31))) {
      rank_slot[(int)selpre[v] + __popc(word & below(y))] = s;
      sflag[s] = 1;
      atomicOr(&hbits[v], 1u << (y & 31));
    }
  };
  if (whole4) {
    const int4 y4 = *reinterpret_cast<const int4*>(stok + s0);
    probe_slot(s0, y4.x);
    probe_slot(s0 + 1, y4.y);
    probe_slot(s0 + 2, y4.z);
    probe_slot(s0 + 3, y4.w);
  } else {
    for (int s = s0; s < s1; ++s) probe_slot(s, stok[s]);
  }
  __syncthreads();
  // Repeats: a position that lost its rank's bid holds a repeated id. From here on a position's cls and rnk
  // entries are read and written by its own thread only, so rnk takes the position's slot (hit) or -1, and
  // phase 3 needs no barrier before it: it reads bitmaps, slot flags and the order list, final above.
  // Without repeats, and with the missed tokens in an array of their own (rank_slot then lives through the
  // pairing), this pass is left to the pairing, which reads the hit slot under the position's rank.
  const bool settle = repeats || L.mtok == L.rank_slot;
  for (int i = tid; settle && i < k; i += kThreads) {
    const int8_t c = cls[i];
    if (c == C_CAND || c == C_RES) {
      const int q = rnk[i];
      if (repeats && first[q] != i) {
        cls[i] = C_DUP;
        st |= kStatusDupId;
      } else {
        rnk[i] = rank_slot[q];
      }
    }
  }
  if (st) atomicOr(&misc[kMiscStatus], st);

  auto used = [&](uint32_t f) { return fifo ? f == 2u : f != 0u; };

  // ---- phase 3: ranks of the misses (ascending id) and of the non-hit slots in LRU order, in one scan
  // (misses in the low 16 bits: m <= k <= 8192; candidates in the high 16 bits: <= B <= 65535)
  int m, ncand;
  {
    int cm = 0, cc = 0;
    uint32_t mw[4] = {0u, 0u, 0u, 0u};  // a whole chunk's missed-id words, kept for the prefixes below
    if (wvec) {
      uint32_t hw[4];
      load_words(sel, mw);
      load_words(hbits, hw);
      if constexpr (kSparse) {
        uint32_t rw[4];
        load_words(rbits, rw);
#pragma unroll
        for (int u = 0; u < 4; ++u) mw[u] &= ~rw[u];
      } else {
        const bool touched = has_tail && w0 + cw > win_w0 && w0 <= win_w1;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (touched) mw[u] &= ~window_bits(w0 + u, win_lo, win_hi);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        mw[u] &= ~hw[u];
        cm += __popc(mw[u]);
      }
    } else {
      for (int w = w0; w < w1; ++w) cm += __popc(cand_word(w) & ~hbits[w]);
    }
    // a whole chunk keeps its four slots and their flags in registers for the victim pass below: no flag it
    // reads there is written in between (each slot sits at one position of the order)
    int sl4[4] = {0, 0, 0, 0};
    uint32_t fl4[4] = {0u, 0u, 0u, 0u};
    if (whole4) {
      const uint2 o = *reinterpret_cast<const uint2*>(ord + s0);
      sl4[0] = (int)(o.x & 0xffffu);
      sl4[1] = (int)(o.x >> 16);
      sl4[2] = (int)(o.y & 0xffffu);
      sl4[3] = (int)(o.y >> 16);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        fl4[u] = sflag[sl4[u]];
        cc += !(fl4[u] & 1u);
      }
    } else {
      for (int p = s0; p < s1; ++p) cc += !(sflag[ord[p]] & 1);
    }
    int tot;
    const int pre = block_excl_scan(cm | (cc << 16), misc + kMiscScanRank, lane, wave, &tot);
    m = tot & 0xffff;
    ncand = (int)((uint32_t)tot >> 16);
    if (m > ncand) {
      // more misses than free slots: only possible with a corrupt slot table
      refuse_request<kMode>(a, r, tid);
      return;
    }
    int run = pre & 0xffff;
    if (wvec) {
      store_prefixes(mpre, mw, run);
    } else {
      for (int w = w0; w < w1; ++w) {
        mpre[w] = (uint16_t)run;
        run += __popc(cand_word(w) & ~hbits[w]);
      }
    }
    // LRU: the new order opens with the candidates that stay; FIFO: with every slot that stays (hits keep
    // their place), position p moving up by the number of victims before it
    int runC = (int)((uint32_t)pre >> 16);
    auto place = [&](int p, int slot, uint32_t flag) {
      if (flag & 1u) {
        if (fifo) at(new_order, p - min(m, runC)) = (uint16_t)slot;
        return;
      }
      if (runC < m) {
        vict[runC] = slot;
        sflag[slot] = 2;
      } else {
        at(new_order, fifo ? p - m : runC - m) = (uint16_t)slot;
      }
      ++runC;
    };
    if (whole4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) place(s0 + u, sl4[u], fl4[u]);
    } else {
      for (int p = s0; p < s1; ++p) {
        const int slot = ord[p];
        place(p, slot, sflag[slot]);
      }
    }
  }
  __syncthreads();
  const uint32_t t0m = ring_base(has_tail, t0, T);  // x mod T = (t0m + x - t0) mod T for a resident x
  // the slot flags are final: the stamp rows go out now, ahead of the pairing (every row, used slots or not:
  // measured faster than predicating the store on the row holding a used slot)
  uint32_t f4 = 0u;  // a whole chunk's four flags, one byte each
  if (whole4) f4 = *reinterpret_cast<const uint32_t*>(sflag + s0);
  if (stamp_rows) {
    v4u ns = sp0;
    if (used(f4 & 0xffu)) ns.x = (uint32_t)t;
    if (used((f4 >> 8) & 0xffu)) ns.y = (uint32_t)t;
    if (used((f4 >> 16) & 0xffu)) ns.z = (uint32_t)t;
    if (used(f4 >> 24)) ns.w = (uint32_t)t;
    __builtin_nontemporal_store(ns, reinterpret_cast<v4u*>(stamp_r) + tid);
  }

  // ---- phase 4: pair misses with victims: outputs and page table; the victims' new tokens go to the LDS
  // copy of the slot table, written back below as coalesced rows
  for (int i = tid; i < k; i += kThreads) {
    const int8_t c = cls[i];
    const int32_t x = ids[i];
    int32_t o = -1, g = -1;
    const bool cand = c == C_CAND;
    int32_t hit = -1;
    if (cand) hit = settle ? rnk[i] : rank_slot[rnk[i]];
    if (cand && hit < 0) {  // a miss
      const int w = vw(x);
      const uint32_t cwd = cand_word(w);
      const int j = (int)mpre[w] + __popc(cwd & ~hbits[w] & below(x));
      const int v = vict[j];
      const int32_t y = stok[v];  // each victim belongs to exactly one miss
      if (kMode == kTrial) {
        int32_t* rec = trial_rec(a, r);
        rec[kTrialHead + j] = x;
        rec[kTrialHead + k + j] = v;
        rec[kTrialHead + 2 * k + j] = y;
        rec[kTrialHead + 3 * k + j] = i;
      } else if (kMode == kPlan) {
        at(plan_r, 2 * k + j) = y;  // the copy updates the page table
      } else {
        if (y >= 0) page_r[y] = -1;  // H rows may pass 4 GiB of page table: 64-bit offsets here
        page_r[x] = v;
      }
      stok[v] = x;
      mtok[j] = x;
      o = v;
      g = -2 - j;
    } else if (cand) {  // a hit
      o = hit;
      g = o;
    } else if (c == C_RES) {
      o = B + (int32_t)ring_row(t0m, (uint32_t)x - (uint32_t)t0, T);  // the tail is a ring: x in row x mod T
      g = o;
    }
    at(out_r, i) = o;
    if (kMode != kPlan && a.gather != nullptr) gsrc[i] = g;  // read by the gather below
    if (sources) at(plan_r, 3 * k + i) = g;  // where position i's row comes from (hs_copy's gather)
  }
  // the slots used this step close the new order in slot order: hits and victims (LRU) or victims only
  // (FIFO); the scan's barrier also publishes the LDS writes above
  const int tail_start = fifo ? B - m : ncand - m;
  {
    int ch = 0;
    if (whole4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) ch += used((f4 >> (8 * u)) & 0xffu);
    } else {
      for (int s = s0; s < s1; ++s) ch += used(sflag[s]);
    }
    int tot;
    int pos = tail_start + block_excl_scan(ch, misc + kMiscScanTail, lane, wave, &tot);
    auto append = [&](int s) {
      if (pos < B) at(new_order, pos) = (uint16_t)s;  // pos < B always holds for a permutation
      ++pos;
    };
    if (whole4) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (used((f4 >> (8 * u)) & 0xffu)) append(s0 + u);
    } else {
      for (int s = s0; s < s1; ++s)
        if (used(sflag[s])) append(s);
    }
  }
  // stamps of hit and victim slots, and the victims' slot-table entries: whole rows that hold a victim, or
  // with consecutive lanes on consecutive slots
  if (stamp_rows) {
    if ((f4 & 0x02020202u) != 0u)
      __builtin_nontemporal_store(*reinterpret_cast<const v4u*>(stok + s0), reinterpret_cast<v4u*>(slot_tok_r) + tid);
  } else if (kMode != kTrial) {
    for (int s = tid; s < B; s += kThreads) {
      const uint8_t f = sflag[s];
      if (fifo ? f == 2 : f != 0) at(stamp_r, s) = t;
      if (f == 2) at(slot_tok_r, s) = stok[s];
    }
  }

  if (kMode == kPlan) {
    for (int j = tid; j < m; j += kThreads) {
      at(plan_r, j) = mtok[j];
      at(plan_r, k + j) = vict[j];
    }
    if (tid == 0) {
      a.step[r] = t + 1;
      a.miss[r] = m;
      a.status[r] = misc[kMiscStatus];
    }
    return;
  }

  if (kMode == kTrial && tid == 0) trial_header(a, r, m, tail_start, t);

  // ---- phase 5: rows (the block scan above ended with a barrier, so mtok and gsrc are visible)
  rows_phase<kMode>(a, r, m, mtok, vict, gsrc, tid);

  if (tid == 0) {
    if (kMode != kTrial) a.step[r] = t + 1;
    a.miss[r] = m;
    a.status[r] = misc[kMiscStatus];
  }
}

// Raw buffer access (gfx9 family): a per-request descriptor in scalar registers and a 32-bit byte offset per
// lane. An offset at or past the descriptor's size reads 0 and writes nothing, so a lane's access is
// predicated by its offset rather than by a branch around it.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
constexpr uint32_t kNoAccess = 0x80000000u;  // past every per-request array (each is below 2 GiB)

__device__ __forceinline__ rsrc_t buf(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0); }
__device__ __forceinline__ v2u ld64(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0); }
__device__ __forceinline__ v4u ld128(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0); }
// Stores of whole rows and lists (outputs, order list, stamps, slot table, plan and trial records) are streamed
// (the non-temporal hint): nothing reads them again in the launch, and they leave less dirty data in L2 for the
// write-back at its end (measured: plan chain 9.4 -> 9.0 us at 256 requests). The scattered page-table stores
// keep the default policy, under which they are much cheaper.
constexpr int kStream = 2;  // the non-temporal bit of the buffer instructions' cache-policy operand
__device__ __forceinline__ void st16(uint32_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, (int)off, 0, kStream);
}
__device__ __forceinline__ void st32(uint32_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kStream);
}
// the same with a uniform byte offset added to the lane's (valid lane offsets stay inside the buffer with it;
// kNoAccess plus it stays past the end)
__device__ __forceinline__ void st32_at(uint32_t v, rsrc_t r, uint32_t off, uint32_t uniform_off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, (int)uniform_off, kStream);
}
__device__ __forceinline__ void st32_scattered(uint32_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void st64(v2u v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kStream);
}
__device__ __forceinline__ void st128(v4u v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kStream);
}

// The direct-layout resolve (see the top of this file): kIPT selected ids per thread (position tid + u * 1024),
// kSPT slots and LRU order positions per thread (one contiguous chunk, kSPT a multiple of 4). The host takes it
// only where B is a multiple of 4 and the slot table, stamps and order list are 16-byte aligned, so every chunk
// of four slots is one 16-byte access. Accesses that only some lanes make are predicated through their address:
// a global one by a buffer offset out of range, an LDS store by the dummy words after the misc words.
template <int kMode, bool kFifo, int kIPT, int kSPT>
__global__ __launch_bounds__(kThreads) void resolve_direct_kernel(ResolveArgs a) {
  static_assert(kSPT % 4 == 0, "slot chunks are whole groups of four");
  constexpr int kQ = kSPT / 4;
  extern __shared__ __align__(16) unsigned char smem[];
  const Layout& L = a.L;
  int32_t* stok = (int32_t*)(smem + L.stok);
  uint8_t* sflag = smem + L.sflag;           // 1: hit this step, 2: victim this step
  uint32_t* sflagw = (uint32_t*)(smem + L.sflag);
  uint32_t* mbits = (uint32_t*)(smem + L.mbits);  // missed ids (resident ids follow, at L.rbits)
  uint16_t* mpre = (uint16_t*)(smem + L.mpre);
  int32_t* vict = (int32_t*)(smem + L.vict);
  int32_t* mtok = (int32_t*)(smem + L.mtok);
  int32_t* gsrc = (int32_t*)(smem + L.gsrc);
  int32_t* misc = (int32_t*)(smem + L.misc);
  uint16_t* t2s = (uint16_t*)(smem + L.t2s);  // token -> slot that holds it (valid only where the slot agrees)
  // in the table's region, dead after the id tests (it holds at least 4k + 2B bytes): a plan launch's evicted
  // tokens by victim rank, and the new LRU order, staged so that it goes out as one 8-byte store per thread
  int32_t* evt = (int32_t*)(smem + L.t2s);
  uint16_t* nord_l = (uint16_t*)(smem + L.t2s + ((4u * (uint32_t)a.k + 15u) & ~15u));
  // LDS addresses a lane stores to when it has nothing to store
  unsigned char* const dummy = smem + L.misc + 4 * kMiscDummy;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const int k = a.k, B = a.B, H = a.H, T = a.T;
  const int W = (int)L.words;
  const bool has_tail = a.tail0 != nullptr;
  constexpr bool fifo = kFifo;
  const int32_t t0 = has_tail ? a.tail0[r] : 0;
  const int32_t t = a.step[r];
  const size_t rk = (size_t)r * k, rB = (size_t)r * B, rH = (size_t)r * H;
  const bool sources = kMode == kPlan && a.plan_sources != 0;
  const bool gathers = kMode != kPlan && a.gather != nullptr;
  const rsrc_t topk_b = buf(a.topk + rk, 4u * k);
  const rsrc_t stok_b = buf(a.slot_tok + rB, 4u * B);
  const rsrc_t ord_b = buf(a.order + rB, 2u * B);
  const rsrc_t stamp_b = buf(a.stamp + rB, 4u * B);
  const rsrc_t out_b = buf(a.out + rk, 4u * k);
  const rsrc_t page_b = buf(a.page + rH, 4u * H);
  const rsrc_t plan_b = buf(a.plan + 4 * rk, kMode == kPlan ? 16u * k : 0u);
  int32_t* const rec = kMode == kTrial ? a.trial + (size_t)r * a.trial_words : nullptr;
  const rsrc_t rec_b = buf(rec, kMode == kTrial ? (uint32_t)(4 * (kTrialHead + 4 * k)) : 0u);
  const rsrc_t nord_b = kMode == kTrial ? buf(rec + kTrialHead + 4 * k, 2u * B) : ord_b;  // the new LRU order
  const int s0 = tid * kSPT;  // this thread's slots and order positions: [s0, s0 + kSPT) within [0, B)
  bool inq[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) inq[q] = s0 + 4 * q < B;

  // ---- A: every global load of the step issued before any is consumed (the stamps only at the very end)
  int32_t x[kIPT];
#pragma unroll
  for (int u = 0; u < kIPT; ++u) {
    const int i = tid + u * kThreads;
    const uint32_t v = ld32(topk_b, 4u * (uint32_t)i);  // past k: out of range
    x[u] = i < k ? (int32_t)v : -1;
  }
  v4u yq[kQ], sq[kQ];
  v2u oq[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) yq[q] = ld128(stok_b, 4u * (uint32_t)(s0 + 4 * q));
#pragma unroll
  for (int q = 0; q < kQ; ++q) oq[q] = ld64(ord_b, 2u * (uint32_t)(s0 + 4 * q));
  if (kMode != kTrial) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) sq[q] = ld128(stamp_b, 4u * (uint32_t)(s0 + 4 * q));
  }
  // the ring row of a resident id x is x mod T = (t0 mod T + (x - t0)) mod T: one modulo per wave, on uniform
  // values, instead of one per id (none without a tail)
  const uint32_t t0m = ring_base(has_tail, t0, T);
  // scratch cleared while the loads are in flight: the missed-id and resident-id bitmaps (adjacent; at most
  // two 16-byte stores per thread), and this chunk's slot flags
  {
    const int n16 = (int)((L.mpre - L.mbits) >> 4);
    uint4* bm = reinterpret_cast<uint4*>(smem + L.mbits);
    uint4* d16 = reinterpret_cast<uint4*>(dummy);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int q = tid + c * kThreads;
      *(q < n16 ? bm + q : d16) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  int32_t y[kSPT];
  uint32_t o[kSPT];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    y[4 * q] = inq[q] ? (int32_t)yq[q].x : -1;
    y[4 * q + 1] = inq[q] ? (int32_t)yq[q].y : -1;
    y[4 * q + 2] = inq[q] ? (int32_t)yq[q].z : -1;
    y[4 * q + 3] = inq[q] ? (int32_t)yq[q].w : -1;
    o[4 * q] = oq[q].x & 0xffffu;
    o[4 * q + 1] = oq[q].x >> 16;
    o[4 * q + 2] = oq[q].y & 0xffffu;
    o[4 * q + 3] = oq[q].y >> 16;
    *reinterpret_cast<uint32_t*>(inq[q] ? (unsigned char*)(sflagw + (s0 >> 2) + q) : dummy) = 0u;
    *reinterpret_cast<v4u*>(inq[q] ? (unsigned char*)(stok + s0 + 4 * q) : dummy) = yq[q];
  }
  // stage the slot table; each slot writes its index under its token (a slot with no valid token writes
  // into the spare entry past the table)
  int bad = 0;
#pragma unroll
  for (int u = 0; u < kSPT; ++u) {
    const bool in = inq[u / 4];
    bad |= in && (((uint32_t)y[u] + 1u > (uint32_t)H) | (o[u] >= (uint32_t)B));  // y in [-1, H), order < B
    const bool tok = in && y[u] >= 0 && y[u] < H;
    t2s[tok ? y[u] : H] = (uint16_t)(s0 + u);
  }
  {
    const bool wbad = __ballot(bad) != 0ull;  // every lane takes part in the ballot
    if (lane == 0) misc[kMiscWaveBad + wave] = wbad;
  }
  __syncthreads();  // (1)
  if (any_wave_flag(misc + kMiscWaveBad, lane)) {
    refuse_request<kMode>(a, r, tid);  // impossible state: leave the request untouched
    return;
  }

  // ---- B: classify the ids and test each against the slot table from its own side. Every predicate is
  // evaluated in full (bitwise, no short circuit) and every choice is a select, so no lane branches.
  int st = 0;
  bool cand[kIPT], res[kIPT], hit[kIPT];
  uint32_t hs[kIPT];
#pragma unroll
  for (int u = 0; u < kIPT; ++u) {
    // -1 is padding; outside [0, H), or at or past the tail start but outside the tail, is a bad id; inside
    // the tail is resident; anything else is a candidate for the hot buffer
    const int32_t xv = x[u];
    const bool pad = xv == -1;
    const bool in_h = (uint32_t)xv < (uint32_t)H;
    const bool past = has_tail & (xv >= t0);
    const bool in_t = (uint32_t)xv - (uint32_t)t0 < (uint32_t)T;  // exact in uint32 once x >= t0
    const bool badid = !pad & (!in_h | (past & !in_t));
    st |= badid ? kStatusBadId : 0;
    res[u] = in_h & past & in_t;
    cand[u] = in_h & !past;
  }
#pragma unroll
  for (int u = 0; u < kIPT; ++u) hs[u] = t2s[cand[u] ? x[u] : 0];
  int32_t held[kIPT];
#pragma unroll
  for (int u = 0; u < kIPT; ++u) held[u] = stok[hs[u] < (uint32_t)B ? hs[u] : 0u];
  bool rep = false;
  {
    // one OR per id: a hit marks its slot's flag byte, a miss its bit among the missed ids, a resident id
    // its bit in the tail window; finding it already set means the id is repeated. Byte offsets in LDS.
    uint32_t off[kIPT], bit[kIPT], old[kIPT];
#pragma unroll
    for (int u = 0; u < kIPT; ++u) {
      const uint32_t xv = (uint32_t)x[u], ri = xv - (uint32_t)t0;
      hit[u] = cand[u] & (hs[u] < (uint32_t)B) & (held[u] == x[u]);
      const uint32_t o_hit = L.sflag + (hs[u] & ~3u), b_hit = 1u << ((hs[u] & 3u) << 3);
      const uint32_t o_miss = L.mbits + ((xv >> 5) << 2), b_miss = 1u << (xv & 31u);
      const uint32_t o_res = L.rbits + ((ri >> 5) << 2), b_res = 1u << (ri & 31u);
      uint32_t o = hit[u] ? o_hit : o_miss, b = hit[u] ? b_hit : b_miss;
      o = res[u] ? o_res : o;
      b = res[u] ? b_res : b;
      off[u] = (cand[u] | res[u]) ? o : L.mbits;
      bit[u] = (cand[u] | res[u]) ? b : 0u;
    }
#pragma unroll
    for (int u = 0; u < kIPT; ++u) old[u] = atomicOr(reinterpret_cast<uint32_t*>(smem + off[u]), bit[u]);
#pragma unroll
    for (int u = 0; u < kIPT; ++u) rep |= (old[u] & bit[u]) != 0u;
  }
  {
    const bool wrep = __ballot(rep) != 0ull;  // every lane takes part in the ballots
    const int wst = wave_or_bits(st);
    if (lane == 0) {
      misc[kMiscWaveRep + wave] = wrep;
      misc[kMiscWaveSt + wave] = wst;
    }
  }
  __syncthreads();  // (2)

  const bool repeats = any_wave_flag(misc + kMiscWaveRep, lane);
  if (repeats) {
    // Rare: some id is selected twice. The lowest position holding it keeps it: the selected ids are ranked
    // in a bitmap with prefix counts and every position bids for its id's rank, in the table's region (the
    // table is dead now). Bits and flags set above are the same for every copy of an id, so only the losers
    // change, and they only in this thread's registers.
    uint32_t* sel = (uint32_t*)(smem + L.sel);
    uint16_t* selpre = (uint16_t*)(smem + L.selpre);
    int32_t* first = (int32_t*)(smem + L.first);
    for (int w = tid; w < W; w += kThreads) sel[w] = 0u;
    for (int q = tid; q < k; q += kThreads) first[q] = INT_MAX;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kIPT; ++u)
      if (cand[u] || res[u]) atomicOr(&sel[x[u] >> 5], 1u << (x[u] & 31));
    __syncthreads();
    const int cw = (W + kThreads - 1) / kThreads, w0 = min(W, tid * cw), w1 = min(W, w0 + cw);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(sel[w]);
    int n_sel;
    int run = block_excl_scan(cnt, misc + kMiscScanSel, lane, wave, &n_sel);
    for (int w = w0; w < w1; ++w) {
      selpre[w] = (uint16_t)run;
      run += __popc(sel[w]);
    }
    __syncthreads();
    int q[kIPT];
#pragma unroll
    for (int u = 0; u < kIPT; ++u) {
      q[u] = 0;
      if (cand[u] || res[u]) {
        q[u] = (int)selpre[x[u] >> 5] + __popc(sel[x[u] >> 5] & below(x[u]));
        atomicMin(&first[q[u]], tid + u * kThreads);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kIPT; ++u)
      if ((cand[u] || res[u]) && first[q[u]] != tid + u * kThreads) cand[u] = res[u] = hit[u] = false;  // a repeat
  }

  // ---- C: ranks of the misses (ascending id) and of the non-hit slots in LRU order, in one scan
  // (misses in the low 16 bits: m <= k <= 8192; candidates in the high 16 bits: <= B <= 8192). This thread's
  // words of the missed-id bitmap: up to three (W <= 3072 for any direct layout).
  const int cw = (W + kThreads - 1) / kThreads, w0 = tid * cw;
  uint32_t mw[3];
#pragma unroll
  for (int e = 0; e < 3; ++e) {
    const int w = w0 + e;
    const bool inw = e < cw && w < W;
    mw[e] = mbits[inw ? w : 0];
    mw[e] = inw ? mw[e] : 0u;
  }
  int m, ncand;
  {
    const int cm = __popc(mw[0]) + __popc(mw[1]) + __popc(mw[2]);
    uint32_t fl[kSPT];
    int cc = 0;
#pragma unroll
    for (int u = 0; u < kSPT; ++u) {
      fl[u] = inq[u / 4] ? (uint32_t)sflag[o[u]] : 1u;  // past the end: not a candidate
      cc += !(fl[u] & 1u);
    }
    int tot;
    const int pre = block_excl_scan(cm | (cc << 16), misc + kMiscScanRank, lane, wave, &tot);  // (3)
    m = tot & 0xffff;
    ncand = (int)((uint32_t)tot >> 16);
    if (m > ncand) {
      // more misses than free slots: only possible with a corrupt slot table
      refuse_request<kMode>(a, r, tid);
      return;
    }
    const uint32_t p0 = (uint32_t)(pre & 0xffff), p1 = p0 + __popc(mw[0]), p2 = p1 + __popc(mw[1]);
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      const int w = w0 + e;
      const bool inw = e < cw && w < W;
      *reinterpret_cast<uint16_t*>(inw ? (unsigned char*)(mpre + w) : dummy) = (uint16_t)(e == 0 ? p0 : e == 1 ? p1 : p2);
    }
    // LRU: the new order opens with the candidates that stay; FIFO: with every slot that stays (hits keep
    // their place), position p moving up by the number of victims before it. A victim's evicted token leaves
    // the page table here already, so these scattered stores start draining early (a plan records it for the
    // copy, which updates the page table).
    int runC = (int)((uint32_t)pre >> 16);
#pragma unroll
    for (int u = 0; u < kSPT; ++u) {
      const int p = s0 + u;
      const uint32_t slot = o[u];
      const bool in = inq[u / 4];
      const bool nonhit = in & !(fl[u] & 1u);
      const bool isv = nonhit & (runC < m);
      const uint32_t dv = (uint32_t)(dummy - smem);
      *reinterpret_cast<int32_t*>(smem + (isv ? L.vict + 4u * (uint32_t)runC : dv)) = (int32_t)slot;
      smem[isv ? L.sflag + slot : dv] = 2;
      if (kMode == kFused) {
        const int32_t yo = stok[isv ? slot : 0u];
        st32_scattered(0xffffffffu, page_b, (isv & (yo >= 0)) ? 4u * (uint32_t)yo : kNoAccess);
      } else if (kMode == kPlan) {  // the token the victim held, for the plan's evicted-token list
        const int32_t yo = stok[isv ? slot : 0u];
        *reinterpret_cast<int32_t*>(isv ? (unsigned char*)(evt + runC) : dummy) = yo;
      }
      const bool keep = fifo ? (in & !isv) : (nonhit & !isv);
      const int np = fifo ? (nonhit ? p - m : p - min(m, runC)) : runC - m;
      *(keep ? nord_l + np : reinterpret_cast<uint16_t*>(dummy)) = (uint16_t)slot;
      runC += nonhit ? 1 : 0;
    }
  }
  __syncthreads();  // (4)
  if (kMode == kPlan) {
    // the plan's victim and evicted-token lists, dense by victim rank (staged in LDS by the victim pass): only
    // the waves holding ranks below m store anything, and the stores drain while the pairing runs
    for (int j = tid; j < m; j += kThreads) {
      const uint32_t jo = 4u * (uint32_t)j;
      st32_at((uint32_t)vict[j], plan_b, jo, 4u * (uint32_t)k);
      st32_at((uint32_t)evt[j], plan_b, jo, 8u * (uint32_t)k);
    }
  }
  // the slots used this step (hits and victims under LRU, victims under FIFO) are final: their stamps become t,
  // and the stamp rows go out now, to drain while the pairing runs
  auto used = [&](uint32_t f) { return fifo ? f == 2u : f != 0u; };
  uint32_t fw[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    fw[q] = sflagw[inq[q] ? (s0 >> 2) + q : 0];
    fw[q] = inq[q] ? fw[q] : 0u;
  }
  if (kMode != kTrial) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const uint32_t f = fw[q];
      v4u ns;
      ns.x = used(f & 0xffu) ? (uint32_t)t : sq[q].x;
      ns.y = used((f >> 8) & 0xffu) ? (uint32_t)t : sq[q].y;
      ns.z = used((f >> 16) & 0xffu) ? (uint32_t)t : sq[q].z;
      ns.w = used(f >> 24) ? (uint32_t)t : sq[q].w;
      st128(ns, stamp_b, inq[q] ? 4u * (uint32_t)(s0 + 4 * q) : kNoAccess);
    }
  }

  // ---- D: the j-th missed id takes the j-th victim: outputs, the new tokens' page entries (fused; a plan leaves
  // them to the copy), the LDS slot table
  {
    bool mi[kIPT];
    uint32_t mp[kIPT], mb[kIPT];
#pragma unroll
    for (int u = 0; u < kIPT; ++u) {
      mi[u] = cand[u] & !hit[u];
      const int w = mi[u] ? x[u] >> 5 : 0;
      mp[u] = mpre[w];
      mb[u] = mbits[w];
    }
    int j[kIPT], v[kIPT];
#pragma unroll
    for (int u = 0; u < kIPT; ++u) {
      j[u] = mi[u] ? (int)mp[u] + __popc(mb[u] & below(x[u])) : 0;
      v[u] = vict[j[u]];
    }
    int32_t yv[kIPT];
    if (kMode == kTrial) {
#pragma unroll
      for (int u = 0; u < kIPT; ++u) yv[u] = stok[mi[u] ? v[u] : 0];
    }
#pragma unroll
    for (int u = 0; u < kIPT; ++u) {
      const int i = tid + u * kThreads;
      const bool pos = i < k;
      // the output: a miss's victim, a hit's slot, a resident id's ring row B + x mod T, else -1
      int32_t ov = res[u] ? B + (int32_t)ring_row(t0m, (uint32_t)x[u] - (uint32_t)t0, T) : -1;
      ov = hit[u] ? (int32_t)hs[u] : ov;
      ov = mi[u] ? v[u] : ov;
      const int32_t g = mi[u] ? -2 - j[u] : ov;  // where the row comes from
      st32((uint32_t)ov, out_b, pos ? 4u * (uint32_t)i : kNoAccess);
      if (sources) st32((uint32_t)g, plan_b, pos ? 4u * (uint32_t)(3 * k + i) : kNoAccess);
      if (gathers) *reinterpret_cast<int32_t*>(pos ? (unsigned char*)(gsrc + i) : dummy) = g;
      if (kMode == kTrial) {
        const uint32_t jo = mi[u] ? 4u * (uint32_t)(kTrialHead + j[u]) : kNoAccess;
        st32((uint32_t)x[u], rec_b, jo);
        st32((uint32_t)v[u], rec_b, jo + 4u * k);
        st32((uint32_t)yv[u], rec_b, jo + 8u * k);
        st32((uint32_t)i, rec_b, jo + 12u * k);
      } else if (kMode == kFused) {
        st32_scattered((uint32_t)v[u], page_b, mi[u] ? 4u * (uint32_t)x[u] : kNoAccess);
      } else {
        st32((uint32_t)x[u], plan_b, mi[u] ? 4u * (uint32_t)j[u] : kNoAccess);  // the miss list's token
      }
      *reinterpret_cast<int32_t*>(mi[u] ? (unsigned char*)(stok + v[u]) : dummy) = x[u];  // one miss per victim
      if (kMode != kPlan) *reinterpret_cast<int32_t*>(mi[u] ? (unsigned char*)(mtok + j[u]) : dummy) = x[u];
    }
  }
  // the slots used this step close the new order in slot order: hits and victims (LRU) or victims only
  // (FIFO); the scan's barrier also publishes the LDS writes above
  const int tail_start = fifo ? B - m : ncand - m;
  {
    int ch = 0;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int b = 0; b < 4; ++b) ch += used((fw[q] >> (8 * b)) & 0xffu);
    int tot;
    int pos = tail_start + block_excl_scan(ch, misc + kMiscScanTail, lane, wave, &tot);  // (5)
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bool u = used((fw[q] >> (8 * b)) & 0xffu);
        *(u ? nord_l + pos : reinterpret_cast<uint16_t*>(dummy)) = (uint16_t)(s0 + 4 * q + b);
        pos += u ? 1 : 0;
      }
  }
  // the slot table written back as whole rows, 16 bytes per lane: the victims' entries hold their new tokens
  if (kMode != kTrial) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const uint32_t off = inq[q] ? 4u * (uint32_t)(s0 + 4 * q) : kNoAccess;
      st128(*reinterpret_cast<const v4u*>(stok + (inq[q] ? s0 + 4 * q : 0)), stok_b, off);
    }
  }
  // the new order, complete in LDS after this barrier: this thread's four entries per chunk in one store
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const v2u ov = *reinterpret_cast<const v2u*>(nord_l + (inq[q] ? s0 + 4 * q : 0));
    st64(ov, nord_b, inq[q] ? 2u * (uint32_t)(s0 + 4 * q) : kNoAccess);
  }
  const int status = [&] {
    int v = lane < kWaves ? misc[kMiscWaveSt + lane] : 0;
    return wave_or_bits(v) | (repeats ? kStatusDupId : 0);
  }();

  if (kMode == kPlan) {
    if (tid == 0) {
      a.step[r] = t + 1;
      a.miss[r] = m;
      a.status[r] = status;
    }
    return;
  }

  if (kMode == kTrial && tid == 0) trial_header(a, r, m, tail_start, t);

  // ---- E: rows (the block scan above ended with a barrier, so mtok and gsrc are visible)
  rows_phase<kMode>(a, r, m, mtok, vict, gsrc, tid);

  if (tid == 0) {
    if (kMode != kTrial) a.step[r] = t + 1;
    a.miss[r] = m;
    a.status[r] = status;
  }
}

__global__ __launch_bounds__(1024) void reset_kernel(ResetArgs a) {
  const int r = a.ids ? a.ids[blockIdx.x] : (int)blockIdx.x;
  if (r < 0 || r >= a.R) return;
  const size_t rB = (size_t)r * a.B, rH = (size_t)r * a.H;
  for (int s = threadIdx.x; s < a.B; s += blockDim.x) {
    a.slot_tok[rB + s] = -1;
    a.stamp[rB + s] = -1;
    a.order[rB + s] = (uint16_t)s;
  }
  for (int x = threadIdx.x; x < a.H; x += blockDim.x) a.page[rH + x] = -1;
  if (threadIdx.x == 0) {
    a.step[r] = 0;
    a.epoch[r] += 1;  // a pending trial of this request is stale now
  }
}

// Every request's change counter advances by one (after an imported state).
__global__ __launch_bounds__(256) void bump_epoch_kernel(int32_t* epoch, int R) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < R) epoch[r] += 1;
}

hipError_t launch_bump_epoch(int32_t* epoch, int R, hipStream_t s) {
  hipLaunchKernelGGL(bump_epoch_kernel, dim3((R + 255) / 256), dim3(256), 0, s, epoch, R);
  return hipGetLastError();
}

// Workgroup (b, r) gathers rows [b*rows, b*rows + rows) of request r's selection into one contiguous
// stretch of the output: every thread first loads its kGatherUnroll chunks (16 bytes each; the slot or tail
// index of each comes from the output array), then stores them non-temporally, so each wave keeps several
// HBM reads in flight and the output is written once, in order. Entries with no row (-1) give zeros.
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherArgs a) {
  const int r = blockIdx.y;
  const int i0 = blockIdx.x * a.rows;
  const int row16 = a.row16;
  const int n = min(a.rows, a.k - i0) * row16;
  const int32_t* outr = a.out + (size_t)r * a.k + i0;
  const v4u* hotr = a.hot + (size_t)r * a.B * row16;
  const v4u* tailr = a.tail ? a.tail + (size_t)r * a.T * row16 : nullptr;
  v4u* gr = a.gather + ((size_t)r * a.k + i0) * row16;
  for (int c0 = threadIdx.x; c0 < n; c0 += kGatherThreads * kGatherUnroll) {
    int o[kGatherUnroll], q[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int c = c0 + u * kGatherThreads;
      const int i = (int)((unsigned)c / (unsigned)row16);
      q[u] = c - i * row16;
      o[u] = c < n ? outr[i] : -1;
    }
    v4u v[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      v[u] = v4u{0u, 0u, 0u, 0u};
      if (o[u] >= 0 && o[u] < a.B) v[u] = __builtin_nontemporal_load(hotr + (size_t)o[u] * row16 + q[u]);
      else if (o[u] >= a.B && o[u] - a.B < a.T)
        v[u] = __builtin_nontemporal_load(tailr + (size_t)(o[u] - a.B) * row16 + q[u]);
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int c = c0 + u * kGatherThreads;
      if (c < n) __builtin_nontemporal_store(v[u], gr + c);
    }
  }
}

// The page-table updates of request r's plan: the evicted tokens leave it, the missed tokens point at their
// slots (no token is both in one step). Thread t of n handles misses t, t + n, ...
__device__ __forceinline__ void plan_page_updates(const CopyArgs& a, int r, int m, int t, int n) {
  const int32_t* p = a.plan + (size_t)r * 4 * a.k;
  int32_t* page = a.page + (size_t)r * a.H;
  for (int j = t; j < m; j += n) {
    const int32_t x = p[j], v = p[a.k + j], y = p[2 * a.k + j];
    if (y >= 0 && y < a.H) page[y] = -1;
    if (x >= 0 && x < a.H && v >= 0 && v < a.B) page[x] = v;
  }
}

// The copy with fewer requests than workgroups: every workgroup takes the same number of missed rows, whatever
// their requests. Each workgroup scans the requests' miss counts into a prefix table in LDS; workgroup w of G
// copies the rows [w M / G, (w + 1) M / G) of the M missed rows of the step, in request order, located in
// batches of kBatchRows (one lane per row finds the row's request in the prefix table by binary search). The
// chunk loop then reads each row's token and slot from the plan, as copy_kernel does (cache-resident after the
// row's first chunk), with kCopyUnroll host loads in flight per lane; the batch's page-table updates follow.
// Splitting each request over R / G workgroups instead leaves the requests with the most misses to set the
// end: measured 2-3 % slower at 32 requests and twice as slow for one request. (With many requests, binding
// workgroups to requests disturbs HBM-bound work on other streams less, so copy_kernel keeps that case.)
__global__ __launch_bounds__(kCopyThreads) void copy_balanced_kernel(CopyArgs a) {
  __shared__ int32_t pre[kCopyWorkgroups + 1];  // pre[r]: missed rows of the requests before r
  __shared__ int32_t brow[kBatchRows], bj[kBatchRows];  // a batch row's request and miss index
  const int lane = threadIdx.x;
  const int R = a.R, k = a.k, row16 = a.row16;
  int run = 0;
  for (int r0 = 0; r0 < R; r0 += kCopyThreads) {
    const int r = r0 + lane;
    int m = r < R ? a.miss[r] : 0;
    m = (m > 0 && m <= k) ? m : 0;  // a refused or impossible count copies nothing, as in copy_kernel
    const int inc = wave_incl_scan(m);
    if (r < R) pre[r + 1] = run + inc;
    run += __builtin_amdgcn_readlane(inc, kCopyThreads - 1);
  }
  if (lane == 0) pre[0] = 0;
  __syncthreads();
  const int M = run, G = gridDim.x, w = blockIdx.x;
  const int lo = (int)((int64_t)M * w / G), hi = (int)((int64_t)M * (w + 1) / G);
  for (int b0 = lo; b0 < hi; b0 += kBatchRows) {
    const int nb = min(kBatchRows, hi - b0);
    for (int i = lane; i < nb; i += kCopyThreads) {
      const int g = b0 + i;
      int rl = 0, rh = R;  // pre[rl] <= g < pre[rh]: the row's request is the last rl with pre[rl] <= g
      while (rh - rl > 1) {
        const int mid = (rl + rh) >> 1;
        if (pre[mid] <= g) rl = mid;
        else rh = mid;
      }
      brow[i] = rl;
      bj[i] = g - pre[rl];  // < the request's miss count <= k
    }
    __syncthreads();
    const int total = nb * row16;
    for (int c0 = lane; c0 < total; c0 += kCopyThreads * kCopyUnroll) {
      v4u v[kCopyUnroll];
      int64_t dst[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int c = c0 + u * kCopyThreads;
        dst[u] = -1;
        if (c < total) {
          const int i = c / row16, q = c - i * row16;
          const int r = brow[i], j = bj[i];
          const int32_t* p = a.plan + (size_t)r * 4 * k;
          const int x = p[j], sl = p[k + j];
          if (x >= 0 && x < a.H && sl >= 0 && sl < a.B) {
            v[u] = load_host(a.host + ((size_t)r * a.H + x) * row16 + q);
            dst[u] = ((int64_t)r * a.B + sl) * row16 + q;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u)
        if (dst[u] >= 0) a.hot[dst[u]] = v[u];
    }
    for (int i = lane; i < nb; i += kCopyThreads) {  // the batch's page-table updates
      const int r = brow[i], j = bj[i];
      const int32_t* p = a.plan + (size_t)r * 4 * k;
      const int32_t x = p[j], v = p[k + j], y = p[2 * k + j];
      int32_t* page = a.page + (size_t)r * a.H;
      if (y >= 0 && y < a.H) page[y] = -1;
      if (x >= 0 && x < a.H && v >= 0 && v < a.B) page[x] = v;
    }
    __syncthreads();  // every lane is done with the batch's table before the next batch overwrites it
  }
}

// Rows of a plan on a bounded grid of one-wave workgroups, where there are at least as many requests as
// workgroups (or more than the balanced copy's table holds). With at least as many requests as workgroups,
// workgroup w takes requests w, w + gridDim.x, ...; with fewer, each request gets
// `slices` workgroups (gridDim.x = R * slices) that share its chunks. A workgroup copies its requests' missed
// rows from the pinned host pool into their victim slots, flattened over (miss, 16-byte chunk): each pass of the
// slices over a request covers slices * kCopyThreads * kCopyUnroll consecutive chunks, each thread keeping
// kCopyUnroll host loads in flight. Then it applies its share of those requests' page-table updates.
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(CopyArgs a) {
  const int row16 = a.row16;
  const int S = a.slices, per = gridDim.x / S;  // per: workgroups per slice (the request stride)
  const int sl = blockIdx.x / per;              // this workgroup's slice of each of its requests
  const int span = kCopyThreads * kCopyUnroll;  // chunks one workgroup covers per pass
  for (int r = blockIdx.x - sl * per; r < a.R; r += per) {
    const int m = a.miss[r];
    if (m <= 0 || m > a.k) continue;
    const int total = m * row16;
    const size_t rk = (size_t)r * a.k;
    const int32_t* ptok = a.plan + rk * 4;
    const int32_t* pslot = ptok + a.k;
    const v4u* hostr = a.host + (size_t)r * a.H * row16;
    v4u* hotr = a.hot + (size_t)r * a.B * row16;
    for (int c0 = sl * span + threadIdx.x; c0 < total; c0 += S * span) {
      v4u v[kCopyUnroll];
      int64_t dst[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int c = c0 + u * kCopyThreads;
        dst[u] = -1;
        if (c < total) {
          const int j = c / row16, q = c - j * row16;
          const int x = ptok[j], s = pslot[j];
          if (x >= 0 && x < a.H && s >= 0 && s < a.B) {
            v[u] = load_host(hostr + (size_t)x * row16 + q);
            dst[u] = (int64_t)s * row16 + q;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u)
        if (dst[u] >= 0) hotr[dst[u]] = v[u];
    }
    plan_page_updates(a, r, m, sl * kCopyThreads + threadIdx.x, S * kCopyThreads);
  }
}

// A plan's rows and the gather of every selected row, in the gather kernel's tiles: workgroup (b, r) fills
// positions [b*rows, b*rows + rows) of request r's gather output, each 16-byte chunk from where the plan says
// the position's row is: a missed row from the host pool (also written to its victim slot), a hot slot, a tail
// row, or zeros. The host loads spread over every workgroup of the chip rather than one per request. The
// page-table updates are shared out over the request's workgroups too.
__global__ __launch_bounds__(kGatherThreads) void copy_gather_kernel(CopyArgs a) {
  const int r = blockIdx.y;
  const int i0 = blockIdx.x * a.rows;
  const int row16 = a.row16, k = a.k, B = a.B;
  const int n = min(a.rows, k - i0) * row16;
  const int m = a.miss[r];
  const size_t rk = (size_t)r * k;
  const int32_t* ptok = a.plan + rk * 4;
  const int32_t* pslot = ptok + k;
  const int32_t* psrc = ptok + 3 * k + i0;
  const v4u* hostr = a.host + (size_t)r * a.H * row16;
  v4u* hotr = a.hot + (size_t)r * B * row16;
  const v4u* tailr = a.tail ? a.tail + (size_t)r * a.T * row16 : nullptr;
  v4u* gr = a.gather + (rk + i0) * row16;
  for (int c0 = threadIdx.x; c0 < n; c0 += kGatherThreads * kGatherUnroll) {
    v4u v[kGatherUnroll];
    int64_t slot_dst[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int c = c0 + u * kGatherThreads;
      v[u] = v4u{0u, 0u, 0u, 0u};
      slot_dst[u] = -1;
      if (c >= n) continue;
      const int i = (int)((unsigned)c / (unsigned)row16), q = c - i * row16;
      const int g = psrc[i];
      if (g <= -2) {
        const int j = -2 - g;
        if (j < m && m <= k) {
          const int x = ptok[j], s = pslot[j];
          if (x >= 0 && x < a.H && s >= 0 && s < B) {
            v[u] = load_host(hostr + (size_t)x * row16 + q);
            slot_dst[u] = (int64_t)s * row16 + q;
          }
        }
      } else if (g >= B) {
        if (g - B < a.T) v[u] = __builtin_nontemporal_load(tailr + (size_t)(g - B) * row16 + q);
      } else if (g >= 0) {
        v[u] = __builtin_nontemporal_load(hotr + (size_t)g * row16 + q);
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int c = c0 + u * kGatherThreads;
      if (c >= n) continue;
      __builtin_nontemporal_store(v[u], gr + c);
      if (slot_dst[u] >= 0) hotr[slot_dst[u]] = v[u];
    }
  }
  if (m > 0 && m <= k) plan_page_updates(a, r, m, blockIdx.x * kGatherThreads + threadIdx.x, gridDim.x * kGatherThreads);
}

// Applies accepted trial records: the new LRU order, stamp t for the hit and victim slots (the new order's
// tail), the victims' slot-table and page-table entries, the step counter, and each missed row copied from
// the gather output (where the trial put it) into its victim slot. A record whose step or epoch no longer
// matches the request's is stale and is not applied: another step, a reset, an offload, a tail advance or an
// imported state came in between, and the rows it gathered may no longer be the host pool's.
__global__ __launch_bounds__(1024) void commit_kernel(CommitArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint8_t* used = smem;  // B flags: slot in the new order's tail
  // the misses' victim slots and gather positions, staged for the row copy (after the B flags, 4-aligned)
  int32_t* lslot = reinterpret_cast<int32_t*>(smem + ((a.B + 3) & ~3));
  int32_t* lpos = lslot + a.k;
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int k = a.k, B = a.B, H = a.H;
  const int32_t* rec = a.trial + (size_t)r * a.trial_words;
  const uint16_t* nord = reinterpret_cast<const uint16_t*>(rec + kTrialHead + 4 * k);
  const int32_t* tok = rec + kTrialHead;
  const int32_t* slot = tok + k;
  const int32_t* evicted = slot + k;
  const int32_t* pos = evicted + k;
  const size_t rB = (size_t)r * B, rH = (size_t)r * H, rk = (size_t)r * k;
  // One round of independent loads: the accept flag, the record's header, the request's step and change
  // counter, four order entries and one miss entry per thread (a miss entry is read before m is known, from
  // the record's k entries, and used only below m). The flags are cleared while they are in flight.
  const int acc = a.accept ? a.accept[r] : 1;
  const int m = rec[0], u0 = rec[1], t = rec[2], rec_epoch = rec[3];
  const int cur_step = a.step[r], cur_epoch = a.epoch[r];
  int o0[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o0[u] = tid + u * nt < B ? nord[tid + u * nt] : B;
  int x0 = -1, v0 = -1, y0 = -1, i0 = -1;
  if (tid < k) { x0 = tok[tid]; v0 = slot[tid]; y0 = evicted[tid]; i0 = pos[tid]; }
  for (int s = tid; s < B; s += nt) used[s] = 0;
  if (acc == 0) {
    if (a.status && tid == 0) a.status[r] = 0;
    return;
  }
  if (t < 0 || cur_step != t || cur_epoch != rec_epoch || m < 0 || m > k || u0 < 0 || u0 > B) {
    if (a.status && tid == 0) a.status[r] = kStatusStale;
    return;
  }
  // the victims' table entries, and their slots and gather positions staged for the row copy
  auto miss_entry = [&](int j, int x, int v, int y, int i) {
    const bool ok = x >= 0 && x < H && v >= 0 && v < B;
    lslot[j] = ok && i >= 0 && i < k ? v : -1;  // a row only for a sound entry
    lpos[j] = i;
    if (!ok) return;
    if (y >= 0 && y < H) a.page[rH + y] = -1;
    a.page[rH + x] = v;
    a.slot_tok[rB + v] = x;
  };
  if (tid < m) miss_entry(tid, x0, v0, y0, i0);
  for (int j = tid + nt; j < m; j += nt) miss_entry(j, tok[j], slot[j], evicted[j], pos[j]);
  __syncthreads();  // the staged slots and positions, and the cleared flags
  // the new order and its tail's flags
  auto place = [&](int p, int o) {
    if (p >= B || o >= B) return;  // past the end, or a corrupt record
    a.order[rB + p] = (uint16_t)o;
    if (p >= u0) used[o] = 1;
  };
#pragma unroll
  for (int u = 0; u < 4; ++u) place(tid + u * nt, o0[u]);
  // four strided entries per thread at a time, all loaded before any is stored: the record and the order
  // list are both global memory, so a store could otherwise hold back the next entry's load
  for (int p0 = tid + 4 * nt; p0 < B; p0 += 4 * nt) {
    int o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = p0 + u * nt < B ? nord[p0 + u * nt] : B;
#pragma unroll
    for (int u = 0; u < 4; ++u) place(p0 + u * nt, o[u]);
  }
  // missed rows, gather output -> victim slots, while the table stores drain: the slot and position of a
  // chunk come from LDS, kCommitUnroll 16-byte loads in flight per thread
  const int row16 = a.row16, total = m * row16;
  for (int c0 = tid; c0 < total; c0 += nt * kCommitUnroll) {
    v4u val[kCommitUnroll];
    int64_t dst[kCommitUnroll];
#pragma unroll
    for (int u = 0; u < kCommitUnroll; ++u) {
      const int c = c0 + u * nt;
      dst[u] = -1;
      if (c < total) {
        const int j = c / row16, q = c - j * row16;
        const int v = lslot[j];
        if (v >= 0) {
          val[u] = a.gather[(rk + lpos[j]) * row16 + q];
          dst[u] = (int64_t)(rB + v) * row16 + q;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCommitUnroll; ++u)
      if (dst[u] >= 0) a.hot[dst[u]] = val[u];
  }
  __syncthreads();  // the tail's flags
  for (int s = tid; s < B; s += nt)
    if (used[s]) a.stamp[rB + s] = t;
  if (tid == 0) {
    a.step[r] = t + 1;
    if (a.status) a.status[r] = 0;
  }
}

// The plan of hs_step_static (the split step in one call, for callers that cannot allocate): kernels reach it
// only through the device address static_plan_address returns, never through its name in host code.
static __device__ __align__(256) int32_t scratch[kStaticPlanBytes / 4];

hipError_t static_plan_address(void** ptr) { return hipGetSymbolAddress(ptr, HIP_SYMBOL(scratch)); }

hipError_t launch_commit(const CommitArgs& a, hipStream_t s) {
  const size_t lds = (size_t)((a.B + 3) & ~3) + 8 * (size_t)a.k;  // flags, then slots and positions
  hipLaunchKernelGGL(commit_kernel, dim3(a.R), dim3(1024), lds, s, a);
  return hipGetLastError();
}

// Offload: n device rows of request r become host-pool rows pos[r] .. pos[r] + n - 1 (16-byte stores over
// the host link into the mapped pool); a row whose token sits in a hot slot is written there too, so the
// slot keeps holding its token's row. Rows that would fall outside [0, H) are skipped and reported.
__global__ __launch_bounds__(256) void offload_kernel(OffloadArgs a) {
  const int r = blockIdx.y;
  const int row16 = a.row16, n = a.n;
  const int p0 = a.pos[r];
  const int total = n * row16;
  const size_t rH = (size_t)r * a.H, rB = (size_t)r * a.B;
  const v4u* src = a.rows + (size_t)r * n * row16;
  v4u* hostr = a.host + rH * row16;
  v4u* hotr = a.hot + rB * row16;
  bool skipped = false;
  const int stride = gridDim.x * blockDim.x;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
    const int j = c / row16, q = c - j * row16;
    const int64_t x = (int64_t)p0 + j;
    if (x < 0 || x >= a.H) {
      skipped = true;
      continue;
    }
    const v4u v = src[c];
    hostr[(size_t)x * row16 + q] = v;  // plain stores: non-temporal ones to host memory run ~10 % slower
    const int s = a.page[rH + x];
    if (s >= 0 && s < a.B) hotr[(size_t)s * row16 + q] = v;
  }
  if (a.status && skipped) a.status[r] = kStatusBadId;  // same value from every thread that skipped
  if (blockIdx.x == 0 && threadIdx.x == 0) a.epoch[r] += 1;  // a pending trial of this request is stale now
}

hipError_t launch_offload(const OffloadArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const int64_t chunks = (int64_t)a.n * a.row16;
  int g = (int)((chunks + 255) / 256);
  if (g > 64) g = 64;
  hipLaunchKernelGGL(offload_kernel, dim3(g, a.R), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Advances request r's device tail window by n[r] tokens (clamped to [0, T]): the leaving tokens
// tail0 .. tail0+n-1 have their ring rows (x mod T) written to their host-pool rows over the host link, and
// to their hot slot if they have one; then tail0 moves. One workgroup per request, so tail0 is updated in
// place after every thread has read it.
__global__ __launch_bounds__(1024) void advance_tail_kernel(AdvanceTailArgs a) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const int T = a.T, row16 = a.row16;
  const int32_t t0 = a.tail0[r];
  int n = a.n[r];
  n = n < 0 ? 0 : n > T ? T : n;
  const size_t rH = (size_t)r * a.H, rB = (size_t)r * a.B;
  const v4u* tailr = a.tail + (size_t)r * T * row16;
  v4u* hostr = a.host + rH * row16;
  v4u* hotr = a.hot + rB * row16;
  int skipped = 0;
  // the ring row of token t0 + j is (t0 mod T) + j, wrapped once (j < n <= T)
  const int t0m = (int)((((int64_t)t0 % T) + T) % T);
  // kTailUnroll chunks per thread per pass, every load (the ring row and the token's page entry) issued before
  // any store (measured with 64 rows per request on 64 requests: 93.9 us one chunk at a time, 91.7 us with 8)
  const int total = n * row16, nt = blockDim.x;
  for (int c0 = tid; c0 < total; c0 += nt * kTailUnroll) {
    v4u v[kTailUnroll];
    int64_t xs[kTailUnroll];
    int ss[kTailUnroll], qs[kTailUnroll];
#pragma unroll
    for (int u = 0; u < kTailUnroll; ++u) {
      const int c = c0 + u * nt;
      xs[u] = -1;
      ss[u] = -1;
      qs[u] = 0;
      if (c < total) {
        const int j = c / row16, q = c - j * row16;
        const int64_t x = (int64_t)t0 + j;
        if (x < 0 || x >= a.H) {
          skipped = 1;
          continue;
        }
        const uint32_t e = (uint32_t)t0m + (uint32_t)j;  // < 2T, exact in uint32
        const uint32_t ring = e >= (uint32_t)T ? e - (uint32_t)T : e;
        v[u] = tailr[(size_t)ring * row16 + q];
        ss[u] = a.page[rH + x];
        xs[u] = x;
        qs[u] = q;
      }
    }
#pragma unroll
    for (int u = 0; u < kTailUnroll; ++u) {
      if (xs[u] < 0) continue;
      hostr[(size_t)xs[u] * row16 + qs[u]] = v[u];  // plain stores: non-temporal ones to host memory run ~10 % slower
      if (ss[u] >= 0 && ss[u] < a.B) hotr[(size_t)ss[u] * row16 + qs[u]] = v[u];
    }
  }
  skipped = __syncthreads_or(skipped);
  if (tid == 0) {
    a.tail0[r] = t0 + n;
    if (a.status) a.status[r] = skipped ? kStatusBadId : 0;
    if (n > 0) a.epoch[r] += 1;  // a pending trial of this request is stale now
  }
}

hipError_t launch_advance_tail(const AdvanceTailArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(advance_tail_kernel, dim3(a.R), dim3(1024), 0, s, a);
  return hipGetLastError();
}

// Rebuilds request r's LRU order list from its stamps: the rank of slot s is the number of slots with a
// smaller (stamp, slot) key, counted against all B stamps staged in LDS. Used after a caller imports
// tables that did not carry the order list; O(B^2 / 1024) per thread, off the decode path.
__global__ __launch_bounds__(1024) void rebuild_order_kernel(RebuildArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* st = (int32_t*)smem;
  const int r = blockIdx.x;
  const size_t rB = (size_t)r * a.B;
  for (int s = threadIdx.x; s < a.B; s += blockDim.x) st[s] = a.stamp[rB + s];
  __syncthreads();
  for (int s = threadIdx.x; s < a.B; s += blockDim.x) {
    const int32_t mine = st[s];
    int rank = 0;
    for (int u = 0; u < a.B; ++u) {
      const int32_t o = st[u];
      rank += (o < mine) || (o == mine && u < s);
    }
    a.order[rB + rank] = (uint16_t)s;
  }
}

hipError_t launch_rebuild_order(const RebuildArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(rebuild_order_kernel, dim3(a.R), dim3(1024), (size_t)a.B * 4, s, a);
  return hipGetLastError();
}

hipError_t set_lds_limits(uint32_t resolve_bytes, uint32_t rebuild_bytes) {
  const void* resolve_variants[] = {
      (const void*)resolve_kernel<kFused, false, false>, (const void*)resolve_kernel<kFused, true, false>,
      (const void*)resolve_kernel<kPlan, false, false>,  (const void*)resolve_kernel<kPlan, true, false>,
      (const void*)resolve_kernel<kTrial, false, false>, (const void*)resolve_kernel<kTrial, true, false>,
      (const void*)resolve_kernel<kFused, false, true>, (const void*)resolve_kernel<kFused, true, true>,
      (const void*)resolve_kernel<kPlan, false, true>,  (const void*)resolve_kernel<kPlan, true, true>,
      (const void*)resolve_kernel<kTrial, false, true>, (const void*)resolve_kernel<kTrial, true, true>,
      (const void*)resolve_direct_kernel<kFused, false, 2, 4>, (const void*)resolve_direct_kernel<kFused, true, 2, 4>,
      (const void*)resolve_direct_kernel<kPlan, false, 2, 4>,  (const void*)resolve_direct_kernel<kPlan, true, 2, 4>,
      (const void*)resolve_direct_kernel<kTrial, false, 2, 4>, (const void*)resolve_direct_kernel<kTrial, true, 2, 4>,
      (const void*)resolve_direct_kernel<kFused, false, 8, 8>, (const void*)resolve_direct_kernel<kFused, true, 8, 8>,
      (const void*)resolve_direct_kernel<kPlan, false, 8, 8>,  (const void*)resolve_direct_kernel<kPlan, true, 8, 8>,
      (const void*)resolve_direct_kernel<kTrial, false, 8, 8>, (const void*)resolve_direct_kernel<kTrial, true, 8, 8>,
  };
  hipError_t e = hipSuccess;
  for (const void* f : resolve_variants) {
    e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)resolve_bytes);
    if (e != hipSuccess) return e;
  }
  e = hipFuncSetAttribute((const void*)commit_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)rebuild_bytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)rebuild_order_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)rebuild_bytes);
}

template <int kMode, bool kFifo>
static void launch_mode_policy(const ResolveArgs& a, hipStream_t s) {
  const dim3 grid(a.R), block(kThreads);
  if (!a.L.direct && a.L.sparse)
    hipLaunchKernelGGL((resolve_kernel<kMode, kFifo, true>), grid, block, a.L.total, s, a);
  else if (!a.L.direct) hipLaunchKernelGGL((resolve_kernel<kMode, kFifo, false>), grid, block, a.L.total, s, a);
  else if (a.k <= 2 * kThreads && a.B <= 4 * kThreads)
    hipLaunchKernelGGL((resolve_direct_kernel<kMode, kFifo, 2, 4>), grid, block, a.L.total, s, a);
  else hipLaunchKernelGGL((resolve_direct_kernel<kMode, kFifo, 8, 8>), grid, block, a.L.total, s, a);
}

template <int kMode>
static void launch_mode(const ResolveArgs& a, hipStream_t s) {
  if (a.policy == 1) launch_mode_policy<kMode, true>(a, s);
  else launch_mode_policy<kMode, false>(a, s);
}

hipError_t launch_resolve(const ResolveArgs& a, hipStream_t s) {
  if (a.L.direct && (a.B > kDirectMaxSlots || a.k > 8 * kThreads)) return hipErrorInvalidValue;
  if (a.trial) launch_mode<kTrial>(a, s);
  else if (a.plan) launch_mode<kPlan>(a, s);
  else launch_mode<kFused>(a, s);
  return hipGetLastError();
}

hipError_t launch_copy(const CopyArgs& a, hipStream_t s) {
  if (a.gather) {
    if ((size_t)a.R * a.k * a.row16 == 0) return hipSuccess;
    if (a.rows < 1) return hipErrorInvalidValue;
    const unsigned bx = (unsigned)((a.k + a.rows - 1) / a.rows);
    hipLaunchKernelGGL(copy_gather_kernel, dim3(bx, (unsigned)a.R), dim3(kGatherThreads), 0, s, a);
    return hipGetLastError();
  }
  if (a.R < 1) return hipSuccess;
  // every request the same number of workgroups: slices per request with fewer requests than workgroups,
  // else one workgroup per request up to the bound
  const int wg = a.workgroups < 1 ? 1 : a.workgroups;
  if (a.R < wg && a.R <= kCopyWorkgroups) {  // fewer requests than workgroups: rows shared out evenly
    hipLaunchKernelGGL(copy_balanced_kernel, dim3(wg), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
  }
  CopyArgs b = a;
  b.slices = a.R < wg ? wg / a.R : 1;
  const int g = a.R < wg ? a.R * b.slices : wg;
  hipLaunchKernelGGL(copy_kernel, dim3(g), dim3(kCopyThreads), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_reset(const ResetArgs& a, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(reset_kernel, dim3(n_blocks), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  if ((size_t)a.R * a.k * a.row16 == 0) return hipSuccess;
  if (a.rows < 1) return hipErrorInvalidValue;
  const unsigned bx = (unsigned)((a.k + a.rows - 1) / a.rows);
  hipLaunchKernelGGL(gather_kernel, dim3(bx, (unsigned)a.R), dim3(kGatherThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs
