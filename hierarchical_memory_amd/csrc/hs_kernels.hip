// HIP kernels of the HiSparse swap-in path for gfx950 (MI355X).
//
// resolve_kernel: one 1024-thread workgroup per request performs one decode
// step of the swap-in kernel the pages describe ("HiSparse: Turbocharging
// Sparse Attention with Hierarchical Memory", section 2, steps 1-3;
// 「HiSparse：階層化メモリシステムによるスパースアテンションの加速」, section
// 「効率的なSwap-inカーネル」), with the device-resident tail and the fused
// gather of "vLLM GLM 5.3 最適化: Hybrid HiSparse オフローディング", section 2
// Mixed Residency:
//   phase 0  coalesced loads of the selected ids, the slot->token table and the
//            LRU order list into LDS; ids classified (padding, bad, resident,
//            candidate); LDS scratch cleared;
//   phase 1  candidate and resident ids inserted into an LDS hash (id -> first
//            position), so repeats are found with set semantics;
//   phase 2  every slot probes the hash with its token: a hit;
//   phase 3  missed ids set bits in an LDS bitmap over token ids;
//   phase 4  wave-segmented ballot/popcount scans: the rank of every missed id
//            among the misses (ascending id) and of every non-hit slot in the
//            LRU order (the first m are the victims); the new LRU order is
//            written as the surviving candidates followed by the hit and
//            victim slots in slot order;
//   phase 5  j-th missed id -> j-th victim: page table, slot table and stamps;
//   phase 6  wavefronts copy the missed rows, 16 bytes per lane, straight from
//            mapped pinned host memory into the HBM slots (and every selected
//            row into the gather output when fused).
// No step of the result depends on the order of LDS atomics: the hash is used
// only as a set with min-position, and every rank comes from a prefix count.
//
// The LRU order list keeps each request's slots sorted by (stamp, slot). After
// a step, the non-victim candidates keep their stamps and relative order, and
// every hit or victim slot now carries stamp t, larger than any older stamp, so
// appending them in slot order keeps the list sorted. Empty slots (stamp -1)
// start at the front in slot order after a reset.
#include "hs_internal.h"

#include <climits>

namespace hs {

namespace {

enum : int8_t { C_PAD = 0, C_BAD = 1, C_DUP = 2, C_RES = 3, C_CAND = 4, C_HIT = 5, C_MISS = 6 };

constexpr int kStatusBadId = 1, kStatusDupId = 2, kStatusBadState = 4;
constexpr int kUnroll = 4;  // 16-byte loads each thread keeps in flight in the copy loops

// misc words in LDS
constexpr int kMiscTotW = 0, kMiscTotC = kWaves, kMiscTotH = 2 * kWaves, kMiscStatus = 3 * kWaves;

__device__ __forceinline__ uint32_t hash_slot(int32_t x, uint32_t bits) {
  return ((uint32_t)x * 0x9E3779B1u) >> (32u - bits);
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int n = __shfl_up(v, d, 64);
    if (lane >= d) v += n;
  }
  return v;
}

__device__ __forceinline__ int hash_find(const int32_t* hkey, int32_t x, uint32_t bits, uint32_t mask) {
  uint32_t h = hash_slot(x, bits);
  while (true) {
    const int32_t kx = hkey[h];
    if (kx == x) return (int)h;
    if (kx == -1) return -1;
    h = (h + 1) & mask;
  }
}

__device__ __forceinline__ v4u load_host(const v4u* p) { return __builtin_nontemporal_load(p); }

}  // namespace

// kPlanOnly: stop after phase 5 and write the miss list (token, victim slot) to a.plan instead of
// copying rows; copy_kernel then moves the rows, possibly on another stream.
template <bool kPlanOnly>
__global__ __launch_bounds__(kThreads) void resolve_kernel(ResolveArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Layout& L = a.L;
  int32_t* ids = (int32_t*)(smem + L.ids);
  int8_t* cls = (int8_t*)(smem + L.cls);
  int32_t* pos_slot = (int32_t*)(smem + L.pos_slot);
  int32_t* stok = (int32_t*)(smem + L.stok);
  uint16_t* ord = (uint16_t*)(smem + L.ord);
  uint8_t* sflag = smem + L.sflag;  // bit 0: hit this step, bit 1: victim this step
  uint32_t* bitmap = (uint32_t*)(smem + L.bitmap);
  uint16_t* wpre = (uint16_t*)(smem + L.wpre);
  int32_t* hkey = (int32_t*)(smem + L.hash_key);
  int32_t* hpos = (int32_t*)(smem + L.hash_pos);
  int32_t* vict = (int32_t*)(smem + L.vict);
  int32_t* mtok = (int32_t*)(smem + L.mtok);
  int32_t* gsrc = (int32_t*)(smem + L.gsrc);
  int32_t* misc = (int32_t*)(smem + L.misc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const int k = a.k, B = a.B, H = a.H, T = a.T;
  const uint32_t hbits = L.hash_bits, hmask = (1u << hbits) - 1u;
  const int W = (int)L.words;
  const bool has_tail = a.tail0 != nullptr;
  const int32_t t0 = has_tail ? a.tail0[r] : 0;
  const int32_t t = a.step[r];
  const size_t rk = (size_t)r * k, rB = (size_t)r * B, rH = (size_t)r * H;
  int st = 0;

  // ---- phase 0: stage and classify
  int bad = 0;
  for (int s = tid; s < B; s += kThreads) {
    const int32_t y = a.slot_tok[rB + s];
    const uint16_t o = a.order[rB + s];
    stok[s] = y;
    ord[s] = o;
    sflag[s] = 0;
    bad |= (y < -1 || y >= H || (int)o >= B);
  }
  for (int i = tid; i < k; i += kThreads) {
    const int32_t x = a.topk[rk + i];
    int8_t c;
    if (x == -1) c = C_PAD;
    else if (x < 0 || x >= H) { c = C_BAD; st |= kStatusBadId; }
    else if (has_tail && x >= t0) {
      if ((int64_t)x - (int64_t)t0 < (int64_t)T) c = C_RES;
      else { c = C_BAD; st |= kStatusBadId; }
    } else c = C_CAND;
    ids[i] = x;
    cls[i] = c;
    pos_slot[i] = -1;
  }
  for (uint32_t h = tid; h <= hmask; h += kThreads) { hkey[h] = -1; hpos[h] = INT_MAX; }
  for (int w = tid; w < W; w += kThreads) bitmap[w] = 0u;
  if (tid == 0) misc[kMiscStatus] = 0;
  bad = __syncthreads_or(bad);

  if (bad) {
    // impossible state: leave the request untouched
    for (int i = tid; i < k; i += kThreads) a.out[rk + i] = -1;
    if (a.gather) {
      v4u* gr = a.gather + rk * a.row16;
      const v4u z = {0u, 0u, 0u, 0u};
      for (int c = tid; c < k * a.row16; c += kThreads) gr[c] = z;
    }
    if (tid == 0) { a.miss[r] = 0; a.status[r] = kStatusBadState; }
    return;
  }

  // ---- phase 1: hash of candidate and resident ids (value = first position)
  for (int i = tid; i < k; i += kThreads) {
    const int8_t c = cls[i];
    if (c == C_CAND || c == C_RES) {
      const int32_t x = ids[i];
      uint32_t h = hash_slot(x, hbits);
      while (true) {
        const int32_t old = atomicCAS(&hkey[h], -1, x);
        if (old == -1 || old == x) { atomicMin(&hpos[h], i); break; }
        h = (h + 1) & hmask;
      }
    }
  }
  __syncthreads();

  // ---- phase 2: repeats, then the hit test: every slot probes the set with its token
  for (int i = tid; i < k; i += kThreads) {
    const int8_t c = cls[i];
    if (c == C_CAND || c == C_RES) {
      const int h = hash_find(hkey, ids[i], hbits, hmask);
      if (hpos[h] != i) { cls[i] = C_DUP; st |= kStatusDupId; }
    }
  }
  for (int s = tid; s < B; s += kThreads) {
    const int32_t y = stok[s];
    if (y < 0) continue;
    if (has_tail && y >= t0 && (int64_t)y - (int64_t)t0 < (int64_t)T) continue;  // resident: not a hit
    const int h = hash_find(hkey, y, hbits, hmask);
    if (h >= 0) {
      pos_slot[hpos[h]] = s;
      sflag[s] = 1;
    }
  }
  __syncthreads();

  // ---- phase 3: misses into the id bitmap
  if (st) atomicOr(&misc[kMiscStatus], st);
  for (int i = tid; i < k; i += kThreads) {
    if (cls[i] == C_CAND) {
      if (pos_slot[i] >= 0) cls[i] = C_HIT;
      else {
        cls[i] = C_MISS;
        const int32_t x = ids[i];
        atomicOr(&bitmap[x >> 5], 1u << (x & 31));
      }
    }
  }
  __syncthreads();

  // ---- phase 4: ranks. Each wave owns a contiguous segment of the bitmap words and of the LRU order.
  const int segW = ((W + kWaves * 64 - 1) / (kWaves * 64)) * 64;
  const int segB = ((B + kWaves * 64 - 1) / (kWaves * 64)) * 64;
  const int w_lo = wave * segW, w_hi = min(W, w_lo + segW);
  const int p_lo = wave * segB, p_hi = min(B, p_lo + segB);
  {
    int my = 0;
    for (int base = w_lo; base < w_hi; base += 64) {
      const int w = base + lane;
      if (w < w_hi) my += __popc(bitmap[w]);
    }
    const int totW = wave_incl_scan(my, lane);
    int totC = 0;
    for (int base = p_lo; base < p_hi; base += 64) {
      const int p = base + lane;
      const bool f = p < p_hi && !(sflag[ord[p]] & 1);
      totC += __popcll(__ballot(f));
    }
    if (lane == 63) misc[kMiscTotW + wave] = totW;
    if (lane == 0) misc[kMiscTotC + wave] = totC;
  }
  __syncthreads();
  int preW = 0, m = 0, preC = 0, ncand = 0;
  for (int w2 = 0; w2 < kWaves; ++w2) {
    const int aW = misc[kMiscTotW + w2], aC = misc[kMiscTotC + w2];
    if (w2 < wave) { preW += aW; preC += aC; }
    m += aW;
    ncand += aC;
  }
  if (m > ncand) {
    // more misses than free slots: only possible with a corrupt slot table
    for (int i = tid; i < k; i += kThreads) a.out[rk + i] = -1;
    if (a.gather) {
      v4u* gr = a.gather + rk * a.row16;
      const v4u z = {0u, 0u, 0u, 0u};
      for (int c = tid; c < k * a.row16; c += kThreads) gr[c] = z;
    }
    if (tid == 0) { a.miss[r] = 0; a.status[r] = kStatusBadState; }
    return;
  }
  {
    int run = preW;
    for (int base = w_lo; base < w_hi; base += 64) {
      const int w = base + lane;
      const int v = (w < w_hi) ? __popc(bitmap[w]) : 0;
      const int inc = wave_incl_scan(v, lane);
      if (w < w_hi) wpre[w] = (uint16_t)(run + inc - v);
      run += __shfl(inc, 63, 64);
    }
    int runC = preC;
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int base = p_lo; base < p_hi; base += 64) {
      const int p = base + lane;
      const int slot = p < p_hi ? (int)ord[p] : 0;
      const bool f = p < p_hi && !(sflag[slot] & 1);
      const uint64_t mask = __ballot(f);
      const int rank = runC + __popcll(mask & lt);
      if (f) {
        if (rank < m) { vict[rank] = slot; sflag[slot] = 2; }
        else a.order[rB + (rank - m)] = (uint16_t)slot;
      }
      runC += __popcll(mask);
    }
  }
  __syncthreads();

  // ---- phase 5: pair misses with victims; page table, slot table, stamps, outputs
  for (int i = tid; i < k; i += kThreads) {
    const int8_t c = cls[i];
    const int32_t x = ids[i];
    int32_t o = -1, g = -1;
    if (c == C_MISS) {
      const int w = x >> 5;
      const int j = (int)wpre[w] + __popc(bitmap[w] & ((1u << (x & 31)) - 1u));
      const int v = vict[j];
      const int32_t y = stok[v];
      if (y >= 0) a.page[rH + y] = -1;
      a.page[rH + x] = v;
      a.slot_tok[rB + v] = x;
      a.stamp[rB + v] = t;
      if (kPlanOnly) {
        a.plan[rk * 2 + j] = x;
        a.plan[rk * 2 + a.k + j] = v;
      } else {
        mtok[j] = x;
      }
      o = v;
      g = -2 - j;
    } else if (c == C_HIT) {
      const int s = pos_slot[i];
      a.stamp[rB + s] = t;
      o = s;
      g = s;
    } else if (c == C_RES) {
      o = B + (x - t0);
      g = o;
    }
    a.out[rk + i] = o;
    gsrc[i] = g;
  }
  // hit and victim slots close the new LRU order, in slot order
  {
    int cnt = 0;
    for (int base = p_lo; base < p_hi; base += 64) {
      const int s = base + lane;
      cnt += __popcll(__ballot(s < p_hi && sflag[s] != 0));
    }
    if (lane == 0) misc[kMiscTotH + wave] = cnt;
  }
  __syncthreads();
  {
    int run = ncand - m;
    for (int w2 = 0; w2 < wave; ++w2) run += misc[kMiscTotH + w2];
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int base = p_lo; base < p_hi; base += 64) {
      const int s = base + lane;
      const bool f = s < p_hi && sflag[s] != 0;
      const uint64_t mask = __ballot(f);
      const int pos = run + __popcll(mask & lt);
      if (f && pos < B) a.order[rB + pos] = (uint16_t)s;  // pos < B always holds for a permutation
      run += __popcll(mask);
    }
  }

  if (kPlanOnly) {
    if (tid == 0) {
      a.step[r] = t + 1;
      a.miss[r] = m;
      a.status[r] = misc[kMiscStatus];
    }
    return;
  }

  // ---- phase 6: rows
  const int row16 = a.row16;
  const v4u* hostr = a.host + rH * (size_t)row16;
  v4u* hotr = a.hot + rB * (size_t)row16;
  if (a.gather == nullptr) {
    const int total = m * row16;
    for (int c0 = tid; c0 < total; c0 += kThreads * kUnroll) {
      v4u v[kUnroll];
      size_t dst[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * kThreads;
        if (c < total) {
          const int j = c / row16, q = c - j * row16;
          v[u] = load_host(hostr + (size_t)mtok[j] * row16 + q);
          dst[u] = (size_t)vict[j] * row16 + q;
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * kThreads;
        if (c < total) hotr[dst[u]] = v[u];
      }
    }
  } else {
    const int total = k * row16;
    const v4u* tailr = a.tail + (size_t)r * T * row16;
    v4u* gr = a.gather + rk * (size_t)row16;
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
            hot_dst[u] = (long long)vict[j] * row16 + q;
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
          gr[c] = v[u];
          if (hot_dst[u] >= 0) hotr[hot_dst[u]] = v[u];
        }
      }
    }
  }

  if (tid == 0) {
    a.step[r] = t + 1;
    a.miss[r] = m;
    a.status[r] = misc[kMiscStatus];
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
  if (threadIdx.x == 0) a.step[r] = 0;
}

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const size_t total = (size_t)a.R * a.k * a.row16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
    const size_t ri = c / (size_t)a.row16;
    const int q = (int)(c - ri * (size_t)a.row16);
    const int r = (int)(ri / (size_t)a.k);
    const int o = a.out[ri];
    v4u v = {0u, 0u, 0u, 0u};
    if (o >= 0 && o < a.B) v = a.hot[((size_t)r * a.B + o) * a.row16 + q];
    else if (o >= a.B && o - a.B < a.T) v = a.tail[((size_t)r * a.T + (o - a.B)) * a.row16 + q];
    a.gather[c] = v;
  }
}

// Rows of a plan: workgroup (g, r) copies every gridDim.x-th group of 16-byte chunks of request r's
// missed rows from the pinned host pool into their victim slots.
__global__ __launch_bounds__(256) void copy_kernel(CopyArgs a) {
  const int r = blockIdx.y;
  const int m = a.miss[r];
  if (m <= 0 || m > a.k) return;
  const int row16 = a.row16;
  const int total = m * row16;
  const size_t rk = (size_t)r * a.k;
  const int32_t* ptok = a.plan + rk * 2;
  const int32_t* pslot = ptok + a.k;
  const v4u* hostr = a.host + (size_t)r * a.H * row16;
  v4u* hotr = a.hot + (size_t)r * a.B * row16;
  const int stride = gridDim.x * blockDim.x;
  for (int c0 = blockIdx.x * blockDim.x + threadIdx.x; c0 < total; c0 += stride * kUnroll) {
    v4u v[kUnroll];
    long long dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * stride;
      dst[u] = -1;
      if (c < total) {
        const int j = c / row16, q = c - j * row16;
        const int x = ptok[j], s = pslot[j];
        if (x >= 0 && x < a.H && s >= 0 && s < a.B) {
          v[u] = load_host(hostr + (size_t)x * row16 + q);
          dst[u] = (long long)s * row16 + q;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (dst[u] >= 0) hotr[dst[u]] = v[u];
  }
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
  hipError_t e = hipFuncSetAttribute((const void*)resolve_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)resolve_bytes);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)resolve_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)resolve_bytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)rebuild_order_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)rebuild_bytes);
}

hipError_t launch_resolve(const ResolveArgs& a, hipStream_t s) {
  if (a.plan) hipLaunchKernelGGL(resolve_kernel<true>, dim3(a.R), dim3(kThreads), a.L.total, s, a);
  else hipLaunchKernelGGL(resolve_kernel<false>, dim3(a.R), dim3(kThreads), a.L.total, s, a);
  return hipGetLastError();
}

hipError_t launch_copy(const CopyArgs& a, hipStream_t s) {
  // about 2048 workgroups over the whole chip whatever the number of requests
  int g = (2048 + a.R - 1) / a.R;
  if (g < 1) g = 1;
  if (g > 64) g = 64;
  hipLaunchKernelGGL(copy_kernel, dim3(g, a.R), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reset(const ResetArgs& a, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(reset_kernel, dim3(n_blocks), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const size_t total = (size_t)a.R * a.k * a.row16;
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs
