// Workgroup-level building blocks shared by the select kernels and the fused
// decode-step kernels (256-thread workgroups, wave64).
#pragma once

#include "common.h"

namespace ekv {

constexpr int kBlk = 256;
constexpr int kTopkLdsKeys = 16384;  // 64 KiB of LDS keys; longer rows read U from global

// Inclusive prefix sum over a 256-thread block; `sh` holds 4 ints of LDS.
__device__ __forceinline__ int block_incl_scan(int x, int* sh) {
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  x = wave_incl_scan_i32(x);
  if (lane == kWave - 1) sh[w] = x;
  __syncthreads();
  int add = 0;
  for (int i = 0; i < w; ++i) add += sh[i];
  __syncthreads();
  return x + add;
}

// fp32 -> uint32 with the same order (-0 folded onto +0 so they tie).
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x == 0.0f) x = 0.0f;
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A thread's run of kPer consecutive 32-bit entries src[p0 .. p0 + kPer) in
// registers, entries at or past lim read as zero.  The runs of a wave's lanes
// lie 4 kPer bytes apart, so every load instruction touches a separate cache
// line per lane: 16-byte loads need a quarter of the instructions (and of the
// cache-line lookups) of 4-byte ones.  They are used when the runs are 16-byte
// aligned (src aligned and p0 a multiple of 4: the same for every lane of a
// launch whose p0 are multiples of kPer); otherwise one load per entry.
template <int kPer, typename V>
__device__ __forceinline__ void load_run(const V* __restrict__ src, int p0, int lim,
                                         V (&dst)[kPer]) {
  static_assert(sizeof(V) == 4, "32-bit entries");
  const bool vec = kPer % 4 == 0 && (p0 & 3) == 0 && ((uintptr_t)src & 15) == 0;
  if (vec) {
#pragma unroll
    for (int j = 0; j < kPer; j += 4) {
      if (p0 + j + 3 < lim) {
        const uint4 w = *reinterpret_cast<const uint4*>(src + p0 + j);
        dst[j] = __builtin_bit_cast(V, w.x);
        dst[j + 1] = __builtin_bit_cast(V, w.y);
        dst[j + 2] = __builtin_bit_cast(V, w.z);
        dst[j + 3] = __builtin_bit_cast(V, w.w);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[j + i] = p0 + j + i < lim ? src[p0 + j + i] : V(0);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) dst[i] = p0 + i < lim ? src[p0 + i] : V(0);
  }
}

// LDS scratch of one top-k selection (keys of rows up to kCap pages).
template <int kCap = kTopkLdsKeys>
struct alignas(16) TopkLds {
  static constexpr int kKeyCap = kCap;
  uint32_t keys[kCap];
  int hist[2048];
  int scan_sh[4];
  int s_digit, s_above, s_cnt;
};

// Top-k pages of one (row, KV head): the min(k, n) largest bounds U[0..n),
// ties to the lower page index, written ascending to out[0..k).  k < n.
// Called by all 256 threads of the workgroup.
// kCoherentU: U was written by other workgroups of the same launch with
// device-coherent stores; read it with device-coherent loads.
template <bool kLds, bool kCoherentU, typename Lds>
__device__ __forceinline__ void topk_block(const float* __restrict__ U, int n, int k,
                                           int32_t* __restrict__ out, Lds& sm) {
  uint32_t* keys = sm.keys;
  int* hist = sm.hist;
  int* scan_sh = sm.scan_sh;
  int& s_digit = sm.s_digit;
  int& s_above = sm.s_above;
  int& s_cnt = sm.s_cnt;
  constexpr int kSelBlock = kBlk;
  auto load_u = [&](int p) -> float {
    if constexpr (kCoherentU)
      return __hip_atomic_load(U + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      return U[p];
  };
  if constexpr (kLds) {
    for (int p = threadIdx.x; p < n; p += kSelBlock) keys[p] = order_key(load_u(p));
    __syncthreads();
  }
  auto key_of = [&](int p) -> uint32_t {
    if constexpr (kLds) return keys[p];
    else return order_key(load_u(p));
  };

  // radix select of the k-th largest key over the keys' actual range [lo, hi]:
  // each pass splits the current range into <= 2048 bins of 2^shift keys (so
  // nearly equal bounds do not pile into one LDS counter), picks the bin that
  // holds the k-th largest key and narrows [lo, hi] to it
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
  for (int p = threadIdx.x; p < n; p += kSelBlock) {
    const uint32_t key = key_of(p);
    kmn = min(kmn, key);
    kmx = max(kmx, key);
  }
  kmn = wave_min_u32(kmn);
  kmx = wave_max_u32(kmx);
  if (threadIdx.x % kWave == 0) {
    hist[threadIdx.x / kWave] = (int)kmn;
    hist[4 + threadIdx.x / kWave] = (int)kmx;
  }
  __syncthreads();
  uint32_t lo = min(min((uint32_t)hist[0], (uint32_t)hist[1]), min((uint32_t)hist[2], (uint32_t)hist[3]));
  uint32_t hi = max(max((uint32_t)hist[4], (uint32_t)hist[5]), max((uint32_t)hist[6], (uint32_t)hist[7]));
  __syncthreads();
  int remaining = k;
  bool cut = false;  // every key >= lo is selected
  for (int pass = 0; pass < 4; ++pass) {
    const uint32_t span = hi - lo;
    const int width = span == 0u ? 0 : 32 - __clz((int)span);
    const int shift = width > 11 ? width - 11 : 0;
    for (int i = threadIdx.x; i < 2048; i += kSelBlock) hist[i] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < n; p += kSelBlock) {
      const uint32_t key = key_of(p);
      if (key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> shift], 1);
    }
    __syncthreads();
    // thread t owns digits 2047-8t down to 2040-8t
    const int dhi = 2047 - threadIdx.x * 8;
    int local = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) local += hist[dhi - i];
    const int incl = block_incl_scan(local, scan_sh);
    const int excl = incl - local;
    if (excl < remaining && remaining <= incl) {
      int acc = excl;
      for (int i = 0; i < 8; ++i) {
        const int hcount = hist[dhi - i];
        if (acc + hcount >= remaining) {
          s_digit = dhi - i;
          s_above = acc;
          s_cnt = hcount;
          break;
        }
        acc += hcount;
      }
    }
    __syncthreads();
    const uint32_t nlo = lo + ((uint32_t)s_digit << shift);
    const uint32_t top = shift == 0 ? nlo : nlo + ((1u << shift) - 1u);
    hi = top < hi ? top : hi;
    lo = nlo;
    remaining -= s_above;
    cut = (s_cnt == remaining);
    __syncthreads();
    if (cut || shift == 0) break;
  }
  // selected: key > T, or key == T among the first `remaining` such pages;
  // with `cut`, every key >= T is selected
  const uint32_t T = lo;
  const int chunk = (n + kSelBlock - 1) / kSelBlock;
  const int p0 = threadIdx.x * chunk;
  const int p1 = min(n, p0 + chunk);
  int cg = 0, ce = 0;
  for (int p = p0; p < p1; ++p) {
    const uint32_t key = key_of(p);
    if (cut ? key >= T : key > T) ++cg;
    else if (!cut && key == T) ++ce;
  }
  const int gt_incl = block_incl_scan(cg, scan_sh);
  const int eq_incl = block_incl_scan(ce, scan_sh);
  int eq_seen = eq_incl - ce;
  int pos = (gt_incl - cg) + min(eq_seen, remaining);
  for (int p = p0; p < p1; ++p) {
    const uint32_t key = key_of(p);
    if (cut ? key >= T : key > T) {
      out[pos++] = p;
    } else if (!cut && key == T) {
      if (eq_seen < remaining) out[pos++] = p;
      ++eq_seen;
    }
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) { return wave_incl_scan_i32(x); }

// Workgroup top-k with the keys in registers (kPerThread consecutive pages per
// thread, n <= 256 * kPerThread, k < n): range-adaptive radix passes over a
// double-buffered LDS histogram (the next pass's buffer is cleared while the
// current one is read), three barriers per pass, and one ordered placement.
struct alignas(16) TopkRegLds {
  int hist[2][2048];
  int wsum[4];
  int wsum2[4];
  uint32_t mm[8];
  int s_digit, s_above, s_cnt;
  // the few keys of the threshold bin, ranked exactly (topk_threshold)
  uint32_t cand_key[kWave];
  int cand_page[kWave];
  int cand_n;
  uint32_t res_T;
  int res_rem;
};

// Inclusive prefix sum over a 256-thread block with LDS-only barriers (global
// loads in flight stay in flight); `sh` holds 4 ints of LDS.
__device__ __forceinline__ int block_incl_scan_lds(int x, int* sh) {
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  x = wave_incl_scan_i32(x);
  if (lane == kWave - 1) sh[w] = x;
  lds_barrier();
  int add = 0;
  for (int i = 0; i < w; ++i) add += sh[i];
  lds_barrier();
  return x + add;
}

// Threshold of a top-k selection: every key > T is selected, and of the keys
// equal to T the first `rem` in page order (cut: every key >= T, rem unused).
struct TopkThr {
  uint32_t T;
  int rem;
  bool cut;
};

// Top-k threshold over order keys in registers (thread t holds pages
// t * kPerThread + i for i < nv; k < n <= 256 * kPerThread): range-adaptive
// radix passes as in topk_reg_keys, but as soon as the bin that holds the k-th
// key has at most 64 keys they are gathered into LDS and one wave ranks them
// exactly (by key, then page), which replaces the remaining passes.  Only LDS
// and registers are used, so the barriers are LDS-only: global loads the
// caller issued before stay in flight.
template <int kPerThread>
__device__ __forceinline__ TopkThr topk_threshold(const uint32_t (&key)[kPerThread], int nv, int k,
                                                 TopkRegLds& sm) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int p0 = tid * kPerThread;
  // the first histogram buffer is cleared here, the second during pass 0
  for (int i = tid; i < 2048; i += kBlk) sm.hist[0][i] = 0;
  if (tid == 0) sm.cand_n = 0;
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if (i < nv) {
      kmn = min(kmn, key[i]);
      kmx = max(kmx, key[i]);
    }
  kmn = wave_min_u32(kmn);
  kmx = wave_max_u32(kmx);
  if (lane == 0) {
    sm.mm[wave] = kmn;
    sm.mm[4 + wave] = kmx;
  }
  lds_barrier();
  uint32_t lo = min(min(sm.mm[0], sm.mm[1]), min(sm.mm[2], sm.mm[3]));
  uint32_t hi = max(max(sm.mm[4], sm.mm[5]), max(sm.mm[6], sm.mm[7]));
  int remaining = k;
  bool cut = false;
  for (int pass = 0; pass < 4; ++pass) {
    int* hist = sm.hist[pass & 1];
    int* next = sm.hist[(pass + 1) & 1];
    const uint32_t span = hi - lo;
    const int width = span == 0u ? 0 : 32 - __clz((int)span);
    const int shift = width > 11 ? width - 11 : 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      if (i < nv && key[i] >= lo && key[i] <= hi) atomicAdd(&hist[(key[i] - lo) >> shift], 1);
    lds_barrier();                                     // (1) histogram complete
    const int4* h4 = reinterpret_cast<const int4*>(hist + 2040 - 8 * tid);
    const int4 a = h4[0], b = h4[1];
    const int bins[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};  // bins[7] = highest digit
    reinterpret_cast<int4*>(next + 2040 - 8 * tid)[0] = make_int4(0, 0, 0, 0);
    reinterpret_cast<int4*>(next + 2040 - 8 * tid)[1] = make_int4(0, 0, 0, 0);
    int local = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) local += bins[i];
    int incl = wave_incl_scan(local);
    if (lane == kWave - 1) sm.wsum[wave] = incl;
    lds_barrier();                                     // (2) wave totals
    for (int w = 0; w < wave; ++w) incl += sm.wsum[w];
    const int excl = incl - local;
    if (excl < remaining && remaining <= incl) {
      int acc = excl;
      bool found = false;
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        if (!found && acc + bins[i] >= remaining) {
          sm.s_digit = 2040 - 8 * tid + i;
          sm.s_above = acc;
          sm.s_cnt = bins[i];
          found = true;
        }
        if (!found) acc += bins[i];
      }
    }
    lds_barrier();                                     // (3) chosen bin
    const int digit = sm.s_digit, above = sm.s_above, cnt = sm.s_cnt;
    const uint32_t nlo = lo + ((uint32_t)digit << shift);
    const uint32_t top = shift == 0 ? nlo : nlo + ((1u << shift) - 1u);
    hi = top < hi ? top : hi;
    lo = nlo;
    remaining -= above;
    cut = (cnt == remaining);
    if (cut || shift == 0) break;
    if (cnt <= kWave) {
      // the bin's keys (at most 64), in any order; the wsum of this pass has
      // been read by every thread (barrier 3), the LDS below is not used yet
#pragma unroll
      for (int i = 0; i < kPerThread; ++i)
        if (i < nv && key[i] >= lo && key[i] <= hi) {
          const int slot = atomicAdd(&sm.cand_n, 1);
          sm.cand_key[slot] = key[i];
          sm.cand_page[slot] = p0 + i;
        }
      lds_barrier();
      if (wave == 0) {
        // rank = keys before this one in the order (larger key, then lower
        // page); lane j's key and page come back through readlane, so the
        // loop has no memory access
        const bool live = lane < cnt;
        const uint32_t mk = live ? sm.cand_key[lane] : 0u;
        const int mp = live ? sm.cand_page[lane] : 0;
        int rank = 0;
        for (int j = 0; j < cnt; ++j) {
          const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mk, j);
          const int pj = __builtin_amdgcn_readlane(mp, j);
          rank += (kj > mk || (kj == mk && pj < mp)) ? 1 : 0;
        }
        // the remaining-th key of the bin is the threshold; keys above it in
        // the bin are all selected, of those equal to it the first rem
        const uint64_t at = __ballot(live && rank == remaining - 1);
        const int src = __ffsll((long long)at) - 1;
        const uint32_t T = (uint32_t)__builtin_amdgcn_readlane((int)mk, src);
        const int gt = __popcll(__ballot(live && mk > T));
        if (lane == 0) {
          sm.res_T = T;
          sm.res_rem = remaining - gt;
        }
      }
      lds_barrier();
      return TopkThr{sm.res_T, sm.res_rem, false};
    }
  }
  return TopkThr{lo, remaining, cut};
}

// The selection itself, on keys already in registers: thread t holds the
// order keys of pages t * kPerThread + i for i < nv (n pages in all, k < n);
// the selected pages are written ascending to out[0 .. k) (global or LDS).
template <int kPerThread, typename OutT>
__device__ __forceinline__ void topk_reg_keys(const uint32_t (&key)[kPerThread], int nv, int k,
                                              OutT* __restrict__ out, TopkRegLds& sm);

template <int kPerThread, bool kCoherentU>
__device__ __forceinline__ void topk_block_reg(const float* __restrict__ U, int n, int k,
                                               int32_t* __restrict__ out, TopkRegLds& sm) {
  const int p0 = threadIdx.x * kPerThread;
  const int nv = max(0, min(kPerThread, n - p0));
  uint32_t key[kPerThread];
  if constexpr (kCoherentU) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      float u = 0.0f;
      if (i < nv) u = __hip_atomic_load(U + p0 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      key[i] = order_key(u);
    }
  } else {
    float u[kPerThread];
    load_run<kPerThread>(U, p0, n, u);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) key[i] = order_key(u[i]);
  }
  topk_reg_keys<kPerThread>(key, nv, k, out, sm);
}

template <int kPerThread, typename OutT>
__device__ __forceinline__ void topk_reg_keys(const uint32_t (&key)[kPerThread], int nv, int k,
                                              OutT* __restrict__ out, TopkRegLds& sm) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int p0 = tid * kPerThread;
  // clear both histogram buffers; min / max of the keys
  for (int i = tid; i < 2 * 2048; i += kBlk) (&sm.hist[0][0])[i] = 0;
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if (i < nv) {
      kmn = min(kmn, key[i]);
      kmx = max(kmx, key[i]);
    }
  kmn = wave_min_u32(kmn);
  kmx = wave_max_u32(kmx);
  if (lane == 0) {
    sm.mm[wave] = kmn;
    sm.mm[4 + wave] = kmx;
  }
  __syncthreads();
  uint32_t lo = min(min(sm.mm[0], sm.mm[1]), min(sm.mm[2], sm.mm[3]));
  uint32_t hi = max(max(sm.mm[4], sm.mm[5]), max(sm.mm[6], sm.mm[7]));
  int remaining = k;
  bool cut = false;
  for (int pass = 0; pass < 4; ++pass) {
    int* hist = sm.hist[pass & 1];
    int* next = sm.hist[(pass + 1) & 1];
    const uint32_t span = hi - lo;
    const int width = span == 0u ? 0 : 32 - __clz((int)span);
    const int shift = width > 11 ? width - 11 : 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      if (i < nv && key[i] >= lo && key[i] <= hi) atomicAdd(&hist[(key[i] - lo) >> shift], 1);
    __syncthreads();                                     // (1) histogram complete
    // thread t owns digits 2047-8t .. 2040-8t; clear the other buffer meanwhile
    const int4* h4 = reinterpret_cast<const int4*>(hist + 2040 - 8 * tid);
    const int4 a = h4[0], b = h4[1];
    const int bins[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};  // bins[7] = highest digit
    reinterpret_cast<int4*>(next + 2040 - 8 * tid)[0] = make_int4(0, 0, 0, 0);
    reinterpret_cast<int4*>(next + 2040 - 8 * tid)[1] = make_int4(0, 0, 0, 0);
    int local = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) local += bins[i];
    int incl = wave_incl_scan(local);
    if (lane == kWave - 1) sm.wsum[wave] = incl;
    __syncthreads();                                     // (2) wave totals
    for (int w = 0; w < wave; ++w) incl += sm.wsum[w];
    const int excl = incl - local;
    if (excl < remaining && remaining <= incl) {
      int acc = excl;
      bool found = false;
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        if (!found && acc + bins[i] >= remaining) {
          sm.s_digit = 2040 - 8 * tid + i;
          sm.s_above = acc;
          sm.s_cnt = bins[i];
          found = true;
        }
        if (!found) acc += bins[i];
      }
    }
    __syncthreads();                                     // (3) chosen bin
    const int digit = sm.s_digit, above = sm.s_above, cnt = sm.s_cnt;
    const uint32_t nlo = lo + ((uint32_t)digit << shift);
    const uint32_t top = shift == 0 ? nlo : nlo + ((1u << shift) - 1u);
    hi = top < hi ? top : hi;
    lo = nlo;
    remaining -= above;
    cut = (cnt == remaining);
    if (cut || shift == 0) break;
  }
  // ordered placement: every key > T, and the first `remaining` keys == T
  // (branch-free: per-key flags, running positions, one masked store per key)
  const uint32_t T = lo;
  bool gt[kPerThread], eq[kPerThread];
  int cg = 0, ce = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const bool v = i < nv;
    gt[i] = v && (cut ? key[i] >= T : key[i] > T);
    eq[i] = v && !cut && key[i] == T;
    cg += gt[i] ? 1 : 0;
    ce += eq[i] ? 1 : 0;
  }
  int gi = wave_incl_scan(cg);
  int ei = wave_incl_scan(ce);
  __syncthreads();  // wsum reuse: every thread has read the last pass's totals
  if (lane == kWave - 1) {
    sm.wsum[wave] = gi;
    sm.wsum2[wave] = ei;
  }
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    gi += sm.wsum[w];
    ei += sm.wsum2[w];
  }
  int eq_seen = ei - ce;
  int pos = (gi - cg) + min(eq_seen, remaining);
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const bool take = gt[i] || (eq[i] && eq_seen < remaining);
    if (take) out[pos] = p0 + i;
    pos += take ? 1 : 0;
    eq_seen += eq[i] ? 1 : 0;
  }
}

// Metadata of one (physical page pi, KV head g) tile with nv valid tokens,
// computed by one wave (all 64 lanes call it): exact per-coordinate min/max,
// mean and population variance (two passes, fp64 sums, one rounding to fp32).
template <typename T, int D, typename M = float>
__device__ __forceinline__ void meta_tile(const T* __restrict__ K, int Hkv, int P, int pi, int g,
                                          int nv, T* __restrict__ kmin, T* __restrict__ kmax,
                                          M* __restrict__ mean, M* __restrict__ var) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kLpr = D / kVec;      // lanes per key row
  constexpr int kRows = kWave / kLpr; // rows per wave instruction
  constexpr int kBatch = 8;           // rows per lane loaded together
  const int lane = threadIdx.x % kWave;
  const size_t tile_off = ((size_t)pi * Hkv + g) * (size_t)P * D;
  const T* src = K + tile_off;
  const int c = lane % kLpr;
  const int r0 = lane / kLpr;

  float mn[kVec], mx[kVec];
  double sm[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) {
    mn[v] = __builtin_huge_valf();
    mx[v] = -__builtin_huge_valf();
    sm[v] = 0.0;
  }
  // rows in batches of kBatch, all loads of a batch in flight together
  for (int t0 = r0; t0 < nv; t0 += kRows * kBatch) {
    uint4 w[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int t = t0 + i * kRows;
      if (t < nv) w[i] = load16(src + (size_t)t * D + c * kVec);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (t0 + i * kRows >= nv) break;
      float x[kVec];
      Elem<T>::unpack(w[i], x);
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        mn[v] = fminf(mn[v], x[v]);
        mx[v] = fmaxf(mx[v], x[v]);
        sm[v] += (double)x[v];
      }
    }
  }
#pragma unroll
  for (int o = kLpr; o < kWave; o <<= 1) {
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      mn[v] = fminf(mn[v], __shfl_xor(mn[v], o, kWave));
      mx[v] = fmaxf(mx[v], __shfl_xor(mx[v], o, kWave));
      sm[v] += __shfl_xor(sm[v], o, kWave);
    }
  }
  double mu[kVec], sq[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) {
    mu[v] = sm[v] / (double)nv;
    sq[v] = 0.0;
  }
  for (int t0 = r0; t0 < nv; t0 += kRows * kBatch) {
    uint4 w[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int t = t0 + i * kRows;
      if (t < nv) w[i] = load16(src + (size_t)t * D + c * kVec);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (t0 + i * kRows >= nv) break;
      float x[kVec];
      Elem<T>::unpack(w[i], x);
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        const double dlt = (double)x[v] - mu[v];
        sq[v] = fma(dlt, dlt, sq[v]);
      }
    }
  }
#pragma unroll
  for (int o = kLpr; o < kWave; o <<= 1) {
#pragma unroll
    for (int v = 0; v < kVec; ++v) sq[v] += __shfl_xor(sq[v], o, kWave);
  }
  if (r0 != 0) return;

  const size_t m_off = ((size_t)pi * Hkv + g) * D + c * kVec;
  if constexpr (sizeof(T) == 2) {
    // min/max of bf16 values are bf16 values: repack the top halves
    uint32_t wn[4], wx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wn[i] = (__float_as_uint(mn[2 * i]) >> 16) | (__float_as_uint(mn[2 * i + 1]) & 0xffff0000u);
      wx[i] = (__float_as_uint(mx[2 * i]) >> 16) | (__float_as_uint(mx[2 * i + 1]) & 0xffff0000u);
    }
    *reinterpret_cast<uint4*>(kmin + m_off) = make_uint4(wn[0], wn[1], wn[2], wn[3]);
    *reinterpret_cast<uint4*>(kmax + m_off) = make_uint4(wx[0], wx[1], wx[2], wx[3]);
  } else {
    *reinterpret_cast<float4*>(kmin + m_off) = make_float4(mn[0], mn[1], mn[2], mn[3]);
    *reinterpret_cast<float4*>(kmax + m_off) = make_float4(mx[0], mx[1], mx[2], mx[3]);
  }
  if (mean != nullptr) {
    if constexpr (sizeof(M) == 2) {
      // compact moments: each fp64 value rounded once to bf16, two per word
      uint32_t wm[kVec / 2], wv[kVec / 2];
#pragma unroll
      for (int i = 0; i < kVec / 2; ++i) {
        wm[i] = bf16_bits_rn(mu[2 * i]) | (bf16_bits_rn(mu[2 * i + 1]) << 16);
        wv[i] = bf16_bits_rn(sq[2 * i] / nv) | (bf16_bits_rn(sq[2 * i + 1] / nv) << 16);
      }
      if constexpr (kVec == 8) {
        *reinterpret_cast<uint4*>(mean + m_off) = make_uint4(wm[0], wm[1], wm[2], wm[3]);
        *reinterpret_cast<uint4*>(var + m_off) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      } else {
        *reinterpret_cast<uint2*>(mean + m_off) = make_uint2(wm[0], wm[1]);
        *reinterpret_cast<uint2*>(var + m_off) = make_uint2(wv[0], wv[1]);
      }
    } else {
#pragma unroll
      for (int v = 0; v < kVec; v += 4) {
        *reinterpret_cast<float4*>(mean + m_off + v) =
            make_float4((float)mu[v], (float)mu[v + 1], (float)mu[v + 2], (float)mu[v + 3]);
        *reinterpret_cast<float4*>(var + m_off + v) = make_float4(
            (float)(sq[v] / nv), (float)(sq[v + 1] / nv), (float)(sq[v + 2] / nv),
            (float)(sq[v + 3] / nv));
      }
    }
  }
}

}  // namespace ekv
